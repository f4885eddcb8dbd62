"""CPU-side checks of the C ABI: the library loads, exports every entry point
that include/mtp_verify.h declares, and rejects bad arguments on the host
before enqueueing anything (no GPU work is launched by these tests)."""
import ctypes
import os
import re

import pytest

import bit_verify_gemm_amd as bv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mtp_verify.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mtp_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("mtp_verify_gemm", "mtp_verify_moe", "mtp_accept_greedy", "mtp_accept_rejection"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = bv.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_abi_version():
    assert bv.abi_version() == 8


def test_packed_sizes():
    # one 2304-byte block per (16 rows, 256 K): codes 16*256/2 + scales 256
    assert bv.packed_weight_bytes(14336, 4096) == 14336 * 4096 // 2 + 14336 * 4096 // 16
    assert bv.packed_weight_bytes(1, 32) == 2304
    assert bv.packed_weight_bytes(17, 288) == 4 * 2304
    assert bv.packed_weight_bytes(0, 32) == 0
    assert bv.packed_weight_bytes(16, 48) == 0


def test_workspace_queries():
    assert bv.gemm_workspace_bytes(262144, 256) == 0              # one K slice: no split
    assert bv.gemm_workspace_bytes(5120, 17408) > 0               # long K is split
    assert bv.gemm_workspace_bytes(0, 32) == 0
    assert bv.gemm_workspace_bytes(10, 33) == 0
    assert bv.moe_workspace_bytes(8, 2048, 768, 128, 8) > 8 * 8 * 2048 * 4
    assert bv.accept_workspace_bytes(8, 262144) > 0
    assert bv.accept_workspace_bytes(65, 10) == 0


P = ctypes.c_void_p
FAKE = ctypes.c_void_p(0x10000)        # aligned, never dereferenced (checks fail first)
FAKE_ODD = ctypes.c_void_p(0x10001)


def gemm(**kw):
    a = dict(fmt=1, M=4, N=64, K=256, x=FAKE, ldx=256, packed=FAKE, g=1.0, y=FAKE,
             ldy=64, yb=None, ldyb=0, ws=None, wsb=0, stream=None)
    a.update(kw)
    return bv.lib().mtp_verify_gemm(a["fmt"], a["M"], a["N"], a["K"], a["x"], a["ldx"],
                                    a["packed"], a["g"], a["y"], a["ldy"], a["yb"],
                                    a["ldyb"], a["ws"], a["wsb"], a["stream"])


BIG = dict(M=16, N=5120, K=17408, ldx=17408, ldy=5120)   # K split over workgroups


@pytest.mark.parametrize("kw,code", [
    (dict(fmt=3), -4), (dict(M=0), -2), (dict(M=17), -2), (dict(K=100), -2), (dict(K=0), -2),
    (dict(N=0), -2), (dict(x=None), -1), (dict(packed=None), -1), (dict(y=None), -1),
    (dict(ldx=128), -2), (dict(ldx=260), -3), (dict(x=FAKE_ODD), -3),
    (dict(packed=FAKE_ODD), -3), (dict(ldy=10), -2), (BIG, -5),
    (dict(BIG, ws=ctypes.c_void_p(0x100010), wsb=1 << 30), -3),
    (dict(M=2, ldx=1 << 30), -2),                        # rows span 2 GiB
    (dict(M=16, ldx=((1 << 30) // 15 + 8) & ~7), -2),
])
def test_gemm_rejects_bad_arguments(kw, code):
    assert gemm(**kw) == code
    assert bv.lib().mtp_last_error()


def pack(**kw):
    a = dict(fmt=1, count=1, N=64, K=256, codes=FAKE, scales=ctypes.c_void_p(0x20000),
             packed=ctypes.c_void_p(0x40000), stream=None)
    a.update(kw)
    return bv.lib().mtp_pack_weights(a["fmt"], a["count"], a["N"], a["K"], a["codes"],
                                     a["scales"], a["packed"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(fmt=0), -4), (dict(K=48), -2), (dict(N=0), -2), (dict(count=0), -2),
    (dict(codes=None), -1), (dict(packed=None), -1), (dict(scales=FAKE_ODD), -3),
    (dict(packed=ctypes.c_void_p(0x10100)), -2),            # overlaps the codes
    (dict(count=1 << 20, N=1 << 20, K=4096), -2),           # more blocks than one launch
])
def test_pack_rejects_bad_arguments(kw, code):
    assert pack(**kw) == code
    assert bv.lib().mtp_last_error()


def test_accept_rejects_bad_arguments():
    L = bv.lib()
    ws = ctypes.c_void_p(0x100000)
    need = bv.accept_workspace_bytes(4, 100)
    # M out of range
    assert L.mtp_accept_greedy(FAKE, 0, 100, 100, FAKE, 0, FAKE, FAKE, FAKE, ws, need, None) == -2
    # ldl < V
    assert L.mtp_accept_greedy(FAKE, 4, 100, 50, FAKE, 0, FAKE, FAKE, FAKE, ws, need, None) == -2
    # missing drafts with M > 1
    assert L.mtp_accept_greedy(FAKE, 4, 100, 100, None, 0, FAKE, FAKE, FAKE, ws, need, None) == -1
    # workspace too small
    assert L.mtp_accept_greedy(FAKE, 4, 100, 100, FAKE, 0, FAKE, FAKE, FAKE, ws, need - 1, None) == -5
    # negative / NaN temperature
    assert L.mtp_accept_rejection(FAKE, 4, 100, 100, FAKE, 100, FAKE, FAKE, -1.0, 0.9, 0, FAKE,
                                  FAKE, FAKE, ws, need, None) == -7
    assert L.mtp_accept_rejection(FAKE, 4, 100, 100, FAKE, 100, FAKE, FAKE, float("nan"), 0.9, 0,
                                  FAKE, FAKE, FAKE, ws, need, None) == -7
    # missing uniforms / draft probabilities at T > 0
    assert L.mtp_accept_rejection(FAKE, 4, 100, 100, FAKE, 100, FAKE, None, 0.6, 0.9, 0, FAKE,
                                  FAKE, FAKE, ws, need, None) == -1
    assert L.mtp_accept_rejection(FAKE, 4, 100, 100, None, 100, FAKE, FAKE, 0.6, 0.9, 0, FAKE,
                                  FAKE, FAKE, ws, need, None) == -1


def test_accept_greedy_static_rejects_bad_arguments():
    L = bv.lib()
    FAKE = ctypes.c_void_p(0x1000)
    args = lambda M=4, V=100, ldl=100, logits=FAKE, d=FAKE, t=FAKE: (  # noqa: E731
        logits, M, V, ldl, d, 0, t, FAKE, FAKE, None)
    assert L.mtp_accept_greedy_static(*args(M=0)) == -2
    assert L.mtp_accept_greedy_static(*args(M=65)) == -2
    assert L.mtp_accept_greedy_static(*args(V=0)) == -2
    assert L.mtp_accept_greedy_static(*args(ldl=99)) == -2
    assert L.mtp_accept_greedy_static(*args(logits=None)) == -1
    assert L.mtp_accept_greedy_static(*args(d=None)) == -1
    assert L.mtp_accept_greedy_static(*args(t=None)) == -1
    assert L.mtp_accept_greedy_static(*args(logits=ctypes.c_void_p(0x1002))) == -3
    assert b"mtp_accept_greedy_static" in L.mtp_last_error()


def test_moe_rejects_bad_arguments():
    L = bv.lib()
    ws = ctypes.c_void_p(0x100000)
    need = bv.moe_workspace_bytes(8, 2048, 768, 128, 8)
    args = [1, 8, 2048, 768, 128, 8, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE,
            None, ws, need, None]

    def call(**kw):
        a = list(args)
        idx = {"fmt": 0, "T": 1, "H": 2, "F": 3, "E": 4, "topk": 5, "x": 6, "gu": 9, "dn": 11,
               "wsb": 16}
        for k, v in kw.items():
            a[idx[k]] = v
        return L.mtp_verify_moe(*a)

    assert call(fmt=0) == -4
    assert call(T=0) == -2
    assert call(T=200, topk=8) == -2
    assert call(H=100) == -2
    assert call(F=40) == -2
    assert call(x=None) == -1
    assert call(gu=None) == -1
    assert call(dn=FAKE_ODD) == -3
    assert call(wsb=need - 1) == -5


def test_accept_sampled_rejects_bad_arguments():
    L = bv.lib()
    B, M, V = 2, 4, 100
    need = bv.accept_sampled_workspace_bytes(B, M, V, 40, False)
    assert need > 0 and bv.accept_sampled_workspace_bytes(B, M, V, 0, False) == 0
    # the one-launch path penalises in registers; the chained kernels (a large
    # top_k over a large vocabulary) keep penalised copies of the rows
    assert bv.accept_sampled_workspace_bytes(B, M, V, 40, True) == need
    big = 1 << 18
    assert (bv.accept_sampled_workspace_bytes(1, 4, big, 600, True) >=
            bv.accept_sampled_workspace_bytes(1, 4, big, 600, False) + 4 * 4 * big)
    ws = ctypes.c_void_p(0x100000)

    def call(params, B=B, M=M, V=V, drafts=FAKE, q=FAKE, qi=None, qp=None, Kq=0, ws_bytes=need,
             uniforms=FAKE, tid=None, tpr=None):
        return L.mtp_accept_sampled(FAKE, B, M, V, V, None, None, 0, drafts, q, V, qi, qp, Kq,
                                    uniforms, ctypes.cast(ctypes.pointer(params), ctypes.c_void_p),
                                    None, FAKE, FAKE, FAKE, tid, tpr, ws, ws_bytes, None)

    ok = bv.Sampler(temperature=0.6, top_k=40)
    assert call(bv.Sampler(temperature=-1.0, top_k=40)) == -7
    assert call(bv.Sampler(temperature=float("nan"), top_k=40)) == -7
    assert call(bv.Sampler(top_p=float("nan"), top_k=40)) == -7
    assert call(bv.Sampler(top_k=0)) == -7
    assert call(bv.Sampler(top_k=1025)) == -7
    assert call(bv.Sampler(top_k=40, repeat_penalty=0.0)) == -7
    assert call(bv.Sampler(top_k=40, penalty_last_n=4097)) == -7
    assert call(ok, B=0) == -2
    assert call(ok, B=1025) == -2
    assert call(ok, M=65) == -2
    assert call(ok, drafts=None) == -1
    assert call(ok, q=None) == -1                        # neither dense nor sparse q
    assert call(ok, q=None, qi=FAKE, qp=FAKE, Kq=0) == -2
    assert call(ok, q=None, qi=FAKE, qp=FAKE, Kq=1025) == -2
    assert call(ok, uniforms=None) == -1
    assert call(ok, tid=FAKE) == -1                      # ids without probs
    assert call(ok, ws_bytes=need - 1) == -5
    assert L.mtp_accept_sampled(FAKE, B, M, V, V, None, None, 0, FAKE, FAKE, V, None, None, 0,
                                FAKE, None, None, FAKE, FAKE, FAKE, None, None, ws, need,
                                None) == -1              # no params
    assert bv.lib().mtp_last_error()


def test_kv_calls_reject_bad_arguments():
    L = bv.lib()

    def app(NL=2, B=1, Hkv=4, cap=64, D=128, ring=1, kn=FAKE, ld=512, M=8, base=FAKE, sk=FAKE,
            k=FAKE):
        return L.mtp_kv_append(k, FAKE, NL, B, Hkv, cap, D, ring, kn, FAKE, ld, M, base, sk, FAKE,
                               None, None)

    def res(M=8, roll=ctypes.c_void_p(0x20000), base=FAKE, ring=1, sk=FAKE, D=128):
        return L.mtp_kv_restore(FAKE, FAKE, 2, 1, 4, 64, D, ring, M, base, roll, sk, FAKE, None,
                                None)

    assert app(NL=0) == -2
    assert app(NL=1 << 12, B=1 << 12, Hkv=2) == -2       # more than 2^24 heads
    assert app(D=0) == -2 and app(D=12) == -2 and app(D=520) == -2
    assert app(M=0) == -2 and app(M=65) == -2
    assert app(cap=7) == -2                               # cap below M
    assert app(ring=2) == -7
    assert app(k=None) == -1 and app(base=None) == -1 and app(kn=None) == -1
    assert app(sk=None) == -1                             # a ring needs its snapshots
    assert app(ld=511) == -2 and app(ld=500) == -2        # below Hkv * D, not a multiple of 8
    assert app(kn=FAKE_ODD) == -3 and app(k=FAKE_ODD) == -3
    assert res(roll=None) == -1
    assert res(roll=FAKE) == -7                           # rollback aliases base_len
    assert L.mtp_kv_restore(FAKE, FAKE, 2, 3, 4, 64, 128, 1, 8, FAKE,
                            ctypes.c_void_p(0x10000 + 16), FAKE, FAKE, None, None) == -7  # partial overlap
    assert res(sk=None) == -1 and res(M=0) == -2 and res(D=4) == -2
    assert "mtp_kv_restore" in bv.lib().mtp_last_error().decode()


def test_read_probe_rejects_bad_arguments():
    L = bv.lib()
    n = bv.read_probe_shapes()
    assert n >= 1
    assert L.mtp_read_probe(FAKE, 16, FAKE, n, None) == -7
    assert L.mtp_read_probe(None, 16, FAKE, 0, None) == -1
    assert L.mtp_read_probe(FAKE, 16, None, 0, None) == -1
    assert L.mtp_read_probe(FAKE_ODD, 16, FAKE, 0, None) == -3
    assert L.mtp_read_probe(FAKE, 17, FAKE, 0, None) == -3


def test_depth_observe_device_rejects_bad_arguments_on_the_host():
    # every check below fails before anything is enqueued (no GPU needed)
    L = bv.lib()
    buf = (ctypes.c_double * 64)()
    cnt = (ctypes.c_int32 * 2)()
    P = ctypes.cast
    r = P(buf, ctypes.c_void_p)
    c = P(cnt, ctypes.c_void_p)
    f = L.mtp_depth_observe_device
    assert f(None, r, 4, 1, c, 1.0, None, None, None, None, None) == -1
    assert f(r, r, 4, 1, None, 1.0, None, None, None, None, None) == -1
    assert f(r, r, 4, 1, c, 1.0, None, c, None, None, None) == -1      # choice needs cost
    assert f(r, r, 0, 1, c, 1.0, None, None, None, None, None) == -2
    assert f(r, r, 64, 1, c, 1.0, None, None, None, None, None) == -2
    assert f(r, r, 4, -1, c, 1.0, None, None, None, None, None) == -2
    assert f(r, r, 4, 1, c, 1.5, None, None, None, None, None) == -7
