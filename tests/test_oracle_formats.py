"""Pins for the oracle's element decoders, against library routines and the
published format tables -- never against the oracle itself."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_all_codes_match_torch():
    # torch's float8_e4m3fn is the OCP E4M3 "FN" variant (bias 7, no inf,
    # 0x7F/0xFF NaN): an implementation independent of the oracle.
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = ref.to(torch.float64).numpy()
    got = np.array([oracle.e4m3(b) for b in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    # spot values of the format
    assert oracle.e4m3(0x01) == 2.0 ** -9
    assert oracle.e4m3(0x08) == 2.0 ** -6
    assert oracle.e4m3(0x38) == 1.0
    assert oracle.e4m3(0x7E) == 448.0


def test_e2m1_matches_spec_table():
    with open(os.path.join(GOLDEN, "e2m1_table.json")) as f:
        tab = json.load(f)
    got = [oracle.e2m1(c) for c in range(16)]
    assert got == tab["values"]
    # sign bit: codes 8..15 are the negatives of 0..7 (code 8 is -0)
    for c in range(8):
        assert oracle.e2m1(c + 8) == -oracle.e2m1(c)
    assert np.signbit(oracle.e2m1(8))
    # every magnitude is a half-integer of {0,1,2,3,4,6,8,12}/2
    assert sorted({abs(2 * v) for v in got}) == [0, 1, 2, 3, 4, 6, 8, 12]


def test_f16_all_codes_match_numpy():
    bits = np.arange(65536, dtype=np.uint32)
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    got = np.array([oracle.f16(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_bf16_all_codes_match_torch():
    bits = np.arange(65536, dtype=np.int32)
    ref = torch.from_numpy(bits.astype(np.uint16).view(np.int16)).view(torch.bfloat16)
    ref = ref.to(torch.float64).numpy()
    got = np.array([oracle.bf16(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def _bf16_values_nonneg():
    """All finite non-negative bf16 values as exact Fractions, ascending."""
    out = []
    for b in range(0x7F80):
        u = np.array([b << 16], dtype=np.uint32).view(np.float32)[0]
        out.append((Fraction(float(u)), b))
    return out


def test_bf16_rne_against_bruteforce_nearest():
    # Independent rounding: pick the nearest representable bf16 by search over
    # the sorted value list, ties to the even bit pattern.
    vals = _bf16_values_nonneg()
    keys = [v for v, _ in vals]
    import bisect
    rng = np.random.default_rng(7)
    samples = list(rng.standard_normal(3000) * np.exp2(rng.integers(-140, 120, 3000)))
    # exact ties and near-ties
    for b in (0x3F80, 0x3F81, 0x4000, 0x0001, 0x0080, 0x7F7E):
        lo = float(keys[b]) if b < len(keys) else None
        hi = float(keys[b + 1])
        mid = (Fraction(lo) + Fraction(hi)) / 2
        samples += [float(mid), np.nextafter(float(mid), 0), np.nextafter(float(mid), 1e300)]
    for v in samples:
        a = Fraction(abs(float(v)))
        i = bisect.bisect_left(keys, a)
        if i == len(keys):
            expect = 0x7F80 if a > keys[-1] + (keys[-1] - keys[-2]) / 2 else vals[-1][1]
        else:
            cands = [vals[i]]
            if i > 0:
                cands.append(vals[i - 1])
            best = min(cands, key=lambda t: (abs(t[0] - a), t[1] & 1))
            expect = best[1]
        if v < 0 or (v == 0 and np.signbit(v)):
            expect |= 0x8000
        assert oracle.bf16_rne(float(v)) == expect, (v, hex(expect))


def test_bf16_rne_matches_torch_on_fp32_inputs():
    # For inputs that are exact fp32 values, torch's fp32->bf16 cast is a single
    # nearest-even rounding as well.
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_rne(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(ref, got)


def test_oracle_reproduces_its_golden_file():
    import importlib.util
    spec = importlib.util.spec_from_file_location("make_golden",
                                                  os.path.join(GOLDEN, "make_golden.py"))
    mg = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mg)
    with open(os.path.join(GOLDEN, "oracle_small.json")) as f:
        stored = json.load(f)
    assert mg.cases() == stored
