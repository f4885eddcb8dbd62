"""GPU parity of mtp_kv_append / mtp_kv_restore against the oracle's commit
(the cache as if only the accepted verify rows had been written).

Bar: bit-exact.  Every cache row is compared except the rows of rejected
positions below cap, whose contents no reader may use (a linear cache's
length, or a rotating cache's window, ends before them).  Snapshot rows that
no write destroyed must still hold their fill (nothing copied lazily)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, dev, host, log

pytestmark = pytest.mark.gpu

bv = pytest.importorskip("bit_verify_gemm_amd")

FILL = 0x5A5A


def u16(t):
    return host(t).view(np.uint16)


def make(seed, NL, B, Hkv, cap, D, M, pad=0):
    rng = np.random.default_rng(seed)
    ck = rng.integers(0, 65536, (NL, B, Hkv, cap, D), dtype=np.uint16)
    cv = rng.integers(0, 65536, (NL, B, Hkv, cap, D), dtype=np.uint16)
    # new rows as a fused projection would give them: Hkv * D columns of a
    # wider row (pad extra columns after them)
    nk = rng.integers(0, 65536, (NL, B, M, Hkv * D + pad), dtype=np.uint16)
    nv = rng.integers(0, 65536, (NL, B, M, Hkv * D + pad), dtype=np.uint16)
    return ck, cv, nk, nv


def rows_of(n, Hkv, D):
    NL, B, M, _ = n.shape
    return np.ascontiguousarray(n[..., :Hkv * D]).reshape(NL, B, M, Hkv, D)


def compare(got, want, roll, hi, cap, what):
    """All rows equal except rows p in [roll[b], hi[b]) with p < cap."""
    NL, B, Hkv, _, D = want.shape
    for b in range(B):
        mask = np.ones(cap, bool)
        for p in range(max(int(roll[b]), 0), min(int(hi[b]), cap)):
            mask[p] = False
        g, w = got[:, b][:, :, mask], want[:, b][:, :, mask]
        if not np.array_equal(g, w):
            bad = np.argwhere(g != w)[:4].tolist()
            raise AssertionError(f"{what}: sequence {b} differs at {bad}")


def run(seed, NL, B, Hkv, cap, D, M, ring, base, roll, pad=0):
    what = f"kv NL={NL} B={B} Hkv={Hkv} cap={cap} D={D} M={M} ring={ring} base={base} roll={roll}"
    log(what)
    ck, cv, nk, nv = make(seed, NL, B, Hkv, cap, D, M, pad)
    gk, gv = dev(ck), dev(cv)
    tk, tv = dev(nk)[..., :Hkv * D], dev(nv)[..., :Hkv * D]
    base_t = torch.tensor(base, dtype=torch.int64, device=DEV)
    roll_t = torch.tensor(roll, dtype=torch.int64, device=DEV)
    snap = None
    if ring:
        snap = bv.kv_snapshot(gk, M)
        snap[0].fill_(FILL)
        snap[1].fill_(FILL)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    bv.kv_append(gk, gv, tk, tv, base_t, ring, snap, err)
    rk, rv = rows_of(nk, Hkv, D), rows_of(nv, Hkv, D)
    full = [b + M for b in base]
    # after the write: the oracle's commit of all M rows, bit for bit
    assert np.array_equal(u16(gk), oracle.kv_commit(ck, rk, base, full, ring)), what + " append K"
    assert np.array_equal(u16(gv), oracle.kv_commit(cv, rv, base, full, ring)), what + " append V"
    if ring:
        sk, sv = u16(snap[0]), u16(snap[1])
        for b in range(B):
            for m in range(M):
                p = base[b] + m
                if p >= cap:   # destroyed position p - cap was copied out
                    assert np.array_equal(sk[:, b, :, m], ck[:, b, :, p % cap]), what + " snapshot"
                    assert np.array_equal(sv[:, b, :, m], cv[:, b, :, p % cap]), what + " snapshot"
                else:          # nothing destroyed: nothing copied
                    assert (sk[:, b, :, m] == FILL).all() and (sv[:, b, :, m] == FILL).all(), \
                        what + " lazy snapshot"
    bv.kv_restore(gk, gv, M, base_t, roll_t, ring, snap, err)
    wk = oracle.kv_commit(ck, rk, base, roll, ring)
    wv = oracle.kv_commit(cv, rv, base, roll, ring)
    compare(u16(gk), wk, roll, full, cap, what + " restore K")
    compare(u16(gv), wv, roll, full, cap, what + " restore V")
    assert int(host(err)[0]) == 0, what + " err set"


@pytest.mark.parametrize("ring", [0, 1])
@pytest.mark.parametrize("D,M", [(128, 8), (64, 4), (256, 16), (8, 1), (512, 3)])
def test_append_restore_matches_oracle(ring, D, M):
    cap = 40
    if ring:
        base, roll = [37, 100, 3], [38, 100 + M, 3]      # crossing the end, wrapped, no wrap
    else:
        base, roll = [0, cap - M, 17], [1, cap, 17 + M // 2]
    run(D * 10 + M + ring, 3, 3, 4, cap, D, M, ring, base, roll)


def test_ring_fully_overwritten_and_padded_rows():
    # M == cap: every row of the ring is replaced (and given back), new rows
    # taken from a wider fused row
    run(5, 2, 2, 3, 64, 128, 64, 1, [64, 1000], [65, 1030], pad=3 * 128)


def test_linear_reject_all_needs_no_work():
    # committing to base: a linear cache keeps the written rows (they are
    # past the length); only rows below base are compared
    run(6, 1, 4, 8, 256, 128, 8, 0, [0, 10, 100, 248], [0, 10, 100, 248])


def test_repeated_steps_follow_the_oracle():
    # ten verify steps on one rotating and one linear cache; each step's
    # rollback is the next step's base, kept on the device throughout
    rng = np.random.default_rng(21)
    NL, B, Hkv, D, M = 2, 3, 2, 64, 6
    for ring, cap in ((1, 23), (0, 80)):
        ck, cv, _, _ = make(22 + ring, NL, B, Hkv, cap, D, M)
        gk, gv = dev(ck), dev(cv)
        snap = bv.kv_snapshot(gk, M) if ring else None
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        length = np.zeros(B, np.int64)
        base_t = torch.zeros(B, dtype=torch.int64, device=DEV)
        for step in range(10):
            nk = rng.integers(0, 65536, (NL, B, M, Hkv * D), dtype=np.uint16)
            nv = rng.integers(0, 65536, (NL, B, M, Hkv * D), dtype=np.uint16)
            roll = length + rng.integers(1, M + 1, B)
            roll_t = torch.tensor(roll, dtype=torch.int64, device=DEV)
            bv.kv_append(gk, gv, dev(nk), dev(nv), base_t, ring, snap, err)
            bv.kv_restore(gk, gv, M, base_t, roll_t, ring, snap, err)
            ck = oracle.kv_commit(ck, rows_of(nk, Hkv, D), length, roll, ring)
            cv = oracle.kv_commit(cv, rows_of(nv, Hkv, D), length, roll, ring)
            length, base_t = roll, roll_t
        for b in range(B):
            live = oracle.kv_live_rows(cap, ring, int(length[b]))
            rows = sorted(live)
            assert np.array_equal(u16(gk)[:, b][:, :, rows], ck[:, b][:, :, rows]), f"ring={ring} K"
            assert np.array_equal(u16(gv)[:, b][:, :, rows], cv[:, b][:, :, rows]), f"ring={ring} V"
        assert int(host(err)[0]) == 0
        log("ring", ring, "lengths after ten steps", length.tolist())


def test_rollback_from_greedy_accept():
    # the accept call's out_rollback drives the restore directly
    M, V, Hkv, D, cap = 8, 1000, 4, 128, 50
    base = 45
    rng = np.random.default_rng(31)
    logits = rng.standard_normal((M, V)).astype(np.float32)
    g = logits.argmax(axis=1)
    drafts = g[:M - 1].copy()
    drafts[3] = (drafts[3] + 1) % V                   # three drafts accepted
    _, _, rb = bv.accept_greedy(dev(logits), dev(drafts.astype(np.int32)), base_len=base)
    ck, cv, nk, nv = make(32, 1, 1, Hkv, cap, D, M)
    gk, gv = dev(ck), dev(cv)
    snap = bv.kv_snapshot(gk, M)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    base_t = torch.tensor([base], dtype=torch.int64, device=DEV)
    bv.kv_append(gk, gv, dev(nk), dev(nv), base_t, True, snap, err)
    bv.kv_restore(gk, gv, M, base_t, rb.reshape(1), True, snap, err)
    roll = int(host(rb).reshape(-1)[0])
    assert roll == base + 4
    want = oracle.kv_commit(ck, rows_of(nk, Hkv, D), [base], [roll], 1)
    compare(u16(gk), want, [roll], [base + M], cap, "greedy-driven restore")
    assert int(host(err)[0]) == 0


def test_out_of_range_positions_are_flagged():
    # a linear cache without room, a negative base and a rollback outside
    # [base, base + M]: rows that fit are written, the rest skipped, the
    # rollback clamped, and err is raised
    NL, B, Hkv, cap, D, M = 1, 3, 2, 20, 64, 8
    ck, cv, nk, nv = make(41, NL, B, Hkv, cap, D, M)
    gk, gv = dev(ck), dev(cv)
    base = [16, -3, 4]
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    base_t = torch.tensor(base, dtype=torch.int64, device=DEV)
    bv.kv_append(gk, gv, dev(nk), dev(nv), base_t, False, None, err)
    assert int(host(err)[0]) != 0
    want = oracle.kv_commit(ck, rows_of(nk, Hkv, D), base, [b + M for b in base], 0)
    assert np.array_equal(u16(gk), want)
    # rotating cache: a rollback below base and one above base + M are clamped
    ck, cv, nk, nv = make(42, NL, 2, Hkv, cap, D, M)
    gk, gv = dev(ck), dev(cv)
    snap = bv.kv_snapshot(gk, M)
    err.zero_()
    base_t = torch.tensor([30, 50], dtype=torch.int64, device=DEV)
    bv.kv_append(gk, gv, dev(nk), dev(nv), base_t, True, snap, err)
    assert int(host(err)[0]) == 0
    bv.kv_restore(gk, gv, M, base_t, torch.tensor([2, 99], dtype=torch.int64, device=DEV), True,
                  snap, err)
    assert int(host(err)[0]) != 0
    want = oracle.kv_commit(ck, rows_of(nk, Hkv, D), [30, 50], [30, 58], 1)
    assert np.array_equal(u16(gk), want)


def test_layer_stack_at_full_size():
    # 62 layers, 16 KV heads of dim 128, a 1031-row ring (1024-key window
    # plus 7 verify rows), 8 rows written past the wrap, all drafts rejected
    NL, B, Hkv, cap, D, M = 62, 1, 16, 1031, 128, 8
    base, roll = [5000], [5001]
    run(51, NL, B, Hkv, cap, D, M, 1, base, roll)
