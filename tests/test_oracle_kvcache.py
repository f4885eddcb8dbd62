"""Pins of the KV-cache commit oracle (Ollama mtp.go commit log, snapshot
rework: committing a verify batch restores the caches to the accepted count).

Rows are tagged with their position (every element of position p's row
encodes p and its column), so what a row holds can be read back without the
oracle's own indexing."""
import numpy as np
import pytest

import oracle


def tagged_rows(NL, B, M, Hkv, D, base):
    """new_rows[l][b][m][h][d] = tag(position base[b] + m, l, h, d)."""
    r = np.zeros((NL, B, M, Hkv, D), np.uint16)
    for l in range(NL):
        for b in range(B):
            for m in range(M):
                for h in range(Hkv):
                    r[l, b, m, h] = tag(base[b] + m, l, h, np.arange(D))
    return r


def tag(p, l, h, d):
    return ((p * 7 + l * 3 + h) * 16 + d) % 65521


def test_ring_by_hand():
    # cap 4, positions 0..5 written one by one: rows hold 4, 5, 2, 3.
    cap, D = 4, 2
    cache = np.full((1, 1, 1, cap, D), 0xFFFF, np.uint16)
    for p in range(6):
        rows = tagged_rows(1, 1, 1, 1, D, [p])
        cache = oracle.kv_commit(cache, rows, [p], [p + 1], ring=1)
    held = [4, 5, 2, 3]
    for row, p in enumerate(held):
        assert list(cache[0, 0, 0, row]) == [tag(p, 0, 0, d) for d in range(D)]


def test_linear_by_hand():
    # cap 6, base 2, four rows, two accepted: rows 2 and 3 written, 4 and 5 untouched.
    cap, D = 6, 3
    before = np.full((1, 1, 1, cap, D), 0xAAAA, np.uint16)
    rows = tagged_rows(1, 1, 4, 1, D, [2])
    after = oracle.kv_commit(before, rows, [2], [4], ring=0)
    for row in range(cap):
        want = [tag(row, 0, 0, d) for d in range(D)] if row in (2, 3) else [0xAAAA] * D
        assert list(after[0, 0, 0, row]) == want
    # positions at or past cap are not stored by a linear cache
    full = oracle.kv_commit(before, tagged_rows(1, 1, 6, 1, D, [2]), [2], [8], ring=0)
    assert list(full[0, 0, 0, 5]) == [tag(5, 0, 0, d) for d in range(D)]


@pytest.mark.parametrize("ring", [0, 1])
def test_commit_to_base_changes_nothing(ring):
    rng = np.random.default_rng(3)
    cache = rng.integers(0, 65536, (2, 3, 2, 9, 8), dtype=np.uint16)
    rows = rng.integers(0, 65536, (2, 3, 5, 2, 8), dtype=np.uint16)
    base = [0, 4, 7] if ring else [0, 2, 4]
    out = oracle.kv_commit(cache, rows, base, base, ring)
    assert np.array_equal(out, cache)


@pytest.mark.parametrize("ring", [0, 1])
def test_two_writes_equal_one(ring):
    # accepting n1 rows, then n2 more from the new base, equals accepting n1 + n2 at once
    rng = np.random.default_rng(5)
    NL, B, Hkv, cap, D, M = 2, 2, 3, 11, 8, 6
    cache = rng.integers(0, 65536, (NL, B, Hkv, cap, D), dtype=np.uint16)
    rows = rng.integers(0, 65536, (NL, B, M, Hkv, D), dtype=np.uint16)
    base = np.array([3, 9]) if ring else np.array([1, 4])
    n1 = np.array([2, 4])
    one = oracle.kv_commit(cache, rows, base, base + M, ring)
    step = oracle.kv_commit(cache, rows, base, base + n1, ring)
    rest = np.zeros_like(rows)
    for b in range(B):
        rest[:, b, :M - n1[b]] = rows[:, b, n1[b]:]
    two = oracle.kv_commit(step, rest, base + n1, base + M, ring)
    assert np.array_equal(one, two)


def test_wide_ring_is_linear():
    rng = np.random.default_rng(7)
    cache = rng.integers(0, 65536, (1, 2, 2, 16, 8), dtype=np.uint16)
    rows = rng.integers(0, 65536, (1, 2, 5, 2, 8), dtype=np.uint16)
    base, roll = [3, 10], [6, 15]
    assert np.array_equal(oracle.kv_commit(cache, rows, base, roll, 1),
                          oracle.kv_commit(cache, rows, base, roll, 0))


@pytest.mark.parametrize("cap", [5, 8, 13])
def test_ring_live_window_holds_its_positions(cap):
    # write positions 0 .. P-1 in verify batches of varying acceptance; the
    # live window of the last cap positions must read back by tag.
    rng = np.random.default_rng(cap)
    NL, B, Hkv, D, M = 1, 1, 2, 4, 4
    cache = np.zeros((NL, B, Hkv, cap, D), np.uint16)
    length = 0
    for _ in range(12):
        rows = tagged_rows(NL, B, M, Hkv, D, [length])
        acc = int(rng.integers(1, M + 1))
        cache = oracle.kv_commit(cache, rows, [length], [length + acc], ring=1)
        length += acc
    live = oracle.kv_live_rows(cap, 1, length)
    assert len(live) == min(cap, length)
    for row, p in live.items():
        for h in range(Hkv):
            assert list(cache[0, 0, h, row]) == [tag(p, 0, h, d) for d in range(D)]


def test_rollback_is_clamped():
    rng = np.random.default_rng(9)
    cache = rng.integers(0, 65536, (1, 2, 1, 10, 8), dtype=np.uint16)
    rows = rng.integers(0, 65536, (1, 2, 3, 1, 8), dtype=np.uint16)
    lo = oracle.kv_commit(cache, rows, [4, 4], [1, 99], ring=0)
    ref = oracle.kv_commit(cache, rows, [4, 4], [4, 7], ring=0)
    assert np.array_equal(lo, ref)
