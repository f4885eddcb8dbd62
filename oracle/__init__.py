"""CPU oracle for the verification pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never loads it, and the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, serial fp64 sums, pthreads over
output columns); this module only marshals numpy arrays through ctypes.  See
the header of ``oracle.c`` for the definitions and the passages they follow.

Readings the pages leave open (they name neither): the SiLU activation and
the bf16 rounding of the MoE intermediate, and the bf16 rounding of the first
product in the tiny chained verify pass.  The oracle's arithmetic for them is
pinned all the same: the MoE against an independent composition (library
element decoders, numpy products, a bf16 rounding checked against brute-force
nearest-even) and invariants; the chained pass is a composition of the
pinned GEMM, bf16-rounding and greedy oracles.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

FMT_NVFP4 = 1
FMT_Q4_0 = 2

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
             "-pthread"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        lib.orc_kv_write.restype = None
        lib.orc_kv_write.argtypes = [P, i64, ctypes.c_int, ctypes.c_int, i64, P, i64, ctypes.c_int]
        lib.orc_e2m1.restype = ctypes.c_double
        lib.orc_e2m1.argtypes = [ctypes.c_uint32]
        lib.orc_e4m3.restype = ctypes.c_double
        lib.orc_e4m3.argtypes = [ctypes.c_uint32]
        lib.orc_f16.restype = ctypes.c_double
        lib.orc_f16.argtypes = [ctypes.c_uint32]
        lib.orc_bf16.restype = ctypes.c_double
        lib.orc_bf16.argtypes = [ctypes.c_uint32]
        lib.orc_bf16_rne.restype = ctypes.c_uint16
        lib.orc_bf16_rne.argtypes = [ctypes.c_double]
        lib.orc_weight.restype = ctypes.c_double
        lib.orc_weight.argtypes = [ctypes.c_int, ctypes.c_int, P, P, f32, i64, i64]
        lib.orc_gemm.restype = ctypes.c_int
        lib.orc_gemm.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, i64,
                                 P, P, f32, P, i64, P, P, ctypes.c_int]
        lib.orc_moe.restype = ctypes.c_int
        lib.orc_moe.argtypes = [ctypes.c_int] * 6 + [P] * 9 + [P, P, P, P, P, ctypes.c_int]
        lib.orc_argmax.restype = i32
        lib.orc_argmax.argtypes = [P, ctypes.c_int]
        lib.orc_accept_greedy.restype = ctypes.c_int
        lib.orc_accept_greedy.argtypes = [P, ctypes.c_int, ctypes.c_int, i64, P, i64, P, P, P]
        lib.orc_accept_sampled.restype = ctypes.c_int
        lib.orc_accept_sampled.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, i64, P, P,
                                           i64, P, P, i64, P, P, ctypes.c_int, P, P, P, P, P, P,
                                           P, P]
        lib.orc_verify_attention.restype = ctypes.c_int
        lib.orc_verify_attention.argtypes = [ctypes.c_int] * 5 + [i64, P, P, P, ctypes.c_double,
                                                                   P, P, ctypes.c_int]
        lib.orc_choose_draft_depth.restype = ctypes.c_int
        lib.orc_choose_draft_depth.argtypes = [P, P, ctypes.c_int, P]
        lib.orc_depth_observe.restype = None
        lib.orc_depth_observe.argtypes = [P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_double]
        lib.orc_depth_estimate.restype = None
        lib.orc_depth_estimate.argtypes = [P, P, ctypes.c_int, P]
        lib.orc_accept_rejection.restype = ctypes.c_int
        lib.orc_accept_rejection.argtypes = [P, ctypes.c_int, ctypes.c_int, i64, P, i64, P, P,
                                             f32, f32, i64, P, P, P, P]
        _lib = lib
        return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _threads(n=None):
    if n:
        return int(n)
    return max(1, min(16, os.cpu_count() or 1))


# ---------------------------------------------------------------------------
# element decoders (scalar; for pins)
# ---------------------------------------------------------------------------

def e2m1(code: int) -> float:
    return _load().orc_e2m1(int(code))


def e4m3(byte: int) -> float:
    return _load().orc_e4m3(int(byte))


def f16(bits: int) -> float:
    return _load().orc_f16(int(bits))


def bf16(bits: int) -> float:
    return _load().orc_bf16(int(bits))


def bf16_rne(v: float) -> int:
    return int(_load().orc_bf16_rne(float(v)))


def weight(w: dict, n: int, k: int) -> float:
    codes = np.ascontiguousarray(w["codes"])
    scales = np.ascontiguousarray(w["scales"])
    return _load().orc_weight(w["format"], w["K"], _ptr(codes), _ptr(scales),
                              float(w.get("g", 1.0)), int(n), int(k))


# ---------------------------------------------------------------------------
# verify GEMM
# ---------------------------------------------------------------------------

def gemm(w: dict, x: np.ndarray, cols=None, with_bound: bool = True, nthreads=None):
    """y[m][c] = sum_k x[m][k] * w(cols[c], k) in fp64.  x: uint16 bf16 bits
    [M][K].  Returns (y, b) as float64 [M][len(cols)] (b = sum |x*w|, or None)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.uint16)
    M, K = x.shape
    assert K == w["K"]
    codes = np.ascontiguousarray(w["codes"], dtype=np.uint8)
    scales = np.ascontiguousarray(w["scales"])
    if cols is None:
        ncols = w["N"]
        colsarr = None
    else:
        colsarr = np.ascontiguousarray(cols, dtype=np.int64)
        ncols = len(colsarr)
    y = np.zeros((M, ncols), np.float64)
    b = np.zeros((M, ncols), np.float64) if with_bound else None
    rc = lib.orc_gemm(w["format"], M, w["N"], K, _ptr(x), K, _ptr(codes), _ptr(scales),
                      float(w.get("g", 1.0)), _ptr(colsarr), ncols, _ptr(y), _ptr(b),
                      _threads(nthreads))
    if rc != 0:
        raise ValueError("orc_gemm rejected its arguments")
    return y, b


# ---------------------------------------------------------------------------
# MoE
# ---------------------------------------------------------------------------

def moe(cfg: dict, nthreads=None, with_preact: bool = False):
    """Returns (out[T][H], outb[T][H], h[T*topk][F] bf16 bits), plus the
    gate/up pre-activations a[T*topk][2F] and their error scale ab (sum of
    |x*w|) when with_preact is set."""
    lib = _load()
    T, H, F, E, topk = cfg["T"], cfg["H"], cfg["F"], cfg["E"], cfg["topk"]
    gu, dn = cfg["gate_up"], cfg["down"]
    assert gu["format"] == dn["format"]
    x = np.ascontiguousarray(cfg["x"], dtype=np.uint16)
    ids = np.ascontiguousarray(cfg["ids"], dtype=np.int32)
    gw = np.ascontiguousarray(cfg["gw"], dtype=np.float32)
    arrs = [np.ascontiguousarray(a) for a in (gu["codes"], gu["scales"], dn["codes"], dn["scales"])]
    gug = None if gu.get("g") is None else np.ascontiguousarray(gu["g"], dtype=np.float32)
    dng = None if dn.get("g") is None else np.ascontiguousarray(dn["g"], dtype=np.float32)
    out = np.zeros((T, H), np.float64)
    outb = np.zeros((T, H), np.float64)
    h = np.zeros((T * topk, F), np.uint16)
    a = np.zeros((T * topk, 2 * F), np.float64) if with_preact else None
    ab = np.zeros((T * topk, 2 * F), np.float64) if with_preact else None
    rc = lib.orc_moe(gu["format"], T, H, F, E, topk, _ptr(x), _ptr(ids), _ptr(gw),
                     _ptr(arrs[0]), _ptr(arrs[1]), _ptr(gug), _ptr(arrs[2]), _ptr(arrs[3]),
                     _ptr(dng), _ptr(out), _ptr(outb), _ptr(h), _ptr(a), _ptr(ab),
                     _threads(nthreads))
    if rc != 0:
        raise ValueError("orc_moe rejected its arguments")
    if with_preact:
        return out, outb, h, a, ab
    return out, outb, h


# ---------------------------------------------------------------------------
# acceptance
# ---------------------------------------------------------------------------

def argmax(row: np.ndarray) -> int:
    row = np.ascontiguousarray(row, dtype=np.float32)
    return int(_load().orc_argmax(_ptr(row), row.shape[0]))


def accept_greedy(logits: np.ndarray, drafts: np.ndarray, base_len: int = 0):
    lib = _load()
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    M, V = logits.shape
    d = np.ascontiguousarray(drafts if drafts is not None and len(drafts) else np.zeros(1),
                             dtype=np.int32)
    tokens = np.zeros(M, np.int32)
    counts = np.zeros(2, np.int32)
    rb = np.zeros(1, np.int64)
    rc = lib.orc_accept_greedy(_ptr(logits), M, V, V, _ptr(d), int(base_len), _ptr(tokens),
                               _ptr(counts), _ptr(rb))
    if rc != 0:
        raise ValueError("orc_accept_greedy rejected its arguments")
    return tokens, counts, int(rb[0])


def accept_rejection(logits: np.ndarray, q: np.ndarray, drafts: np.ndarray, u: np.ndarray,
                     temperature: float, top_p: float, base_len: int = 0,
                     with_margins: bool = False):
    lib = _load()
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    M, V = logits.shape
    if M > 1:
        q = np.ascontiguousarray(q, dtype=np.float32)
        assert q.shape == (M - 1, V)
        d = np.ascontiguousarray(drafts, dtype=np.int32)
    else:
        q = np.zeros((1, V), np.float32)
        d = np.zeros(1, np.int32)
    u = np.ascontiguousarray(u, dtype=np.float32)
    assert u.shape[0] >= M
    tokens = np.zeros(M, np.int32)
    counts = np.zeros(2, np.int32)
    rb = np.zeros(1, np.int64)
    margins = np.zeros(M + 1, np.float64)
    rc = lib.orc_accept_rejection(_ptr(logits), M, V, V, _ptr(q), V, _ptr(d), _ptr(u),
                                  float(temperature), float(top_p), int(base_len), _ptr(tokens),
                                  _ptr(counts), _ptr(rb), _ptr(margins))
    if rc != 0:
        raise ValueError("orc_accept_rejection rejected its arguments")
    if with_margins:
        return tokens, counts, int(rb[0]), margins
    return tokens, counts, int(rb[0])


# Sampler parameters of accept_sampled (the fields of orc_sampler, in order).
SAMPLER_FIELDS = ("temperature", "top_p", "min_p", "top_k", "repeat_penalty",
                  "presence_penalty", "frequency_penalty", "penalty_last_n")
SAMPLER_DEFAULTS = dict(temperature=1.0, top_p=1.0, min_p=0.0, top_k=0, repeat_penalty=1.0,
                        presence_penalty=0.0, frequency_penalty=0.0, penalty_last_n=0)


class _Sampler(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_p", ctypes.c_float),
                ("min_p", ctypes.c_float), ("top_k", ctypes.c_int32),
                ("repeat_penalty", ctypes.c_float), ("presence_penalty", ctypes.c_float),
                ("frequency_penalty", ctypes.c_float), ("penalty_last_n", ctypes.c_int32)]


def sampler(**kw) -> dict:
    s = dict(SAMPLER_DEFAULTS)
    for k, v in kw.items():
        if k not in s:
            raise KeyError(k)
        s[k] = v
    return s


def accept_sampled(logits: np.ndarray, drafts: np.ndarray, u: np.ndarray, params: dict,
                   q: np.ndarray | None = None, q_sparse=None, history=None,
                   base_len=None, with_target: bool = False, with_margins: bool = False):
    """Sampled acceptance of B sequences (see orc_accept_sampled).
    logits [B][M][V]; drafts [B][M-1]; u [B][M]; q dense [B][M-1][V] or
    q_sparse = (ids [B][M-1][K], probs [B][M-1][K]); history: list of B int
    sequences (or None); base_len [B].  Returns tokens [B][M], counts [B][2],
    rollback [B] (+ target p' [B][M][V], + margins [B][M+1])."""
    lib = _load()
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    B, M, V = logits.shape
    d = np.ascontiguousarray(drafts if M > 1 else np.zeros((B, 1)), dtype=np.int32)
    u = np.ascontiguousarray(u, dtype=np.float32)
    assert u.shape == (B, M)
    qd, qi, qp, Kq, ldq = None, None, None, 0, 0
    if M > 1:
        if q is not None:
            qd = np.ascontiguousarray(q, dtype=np.float32)
            assert qd.shape == (B, M - 1, V)
            ldq = V
        else:
            qi = np.ascontiguousarray(q_sparse[0], dtype=np.int32)
            qp = np.ascontiguousarray(q_sparse[1], dtype=np.float32)
            assert qi.shape == qp.shape and qi.shape[:2] == (B, M - 1)
            Kq = qi.shape[2]
    hist, hlen, ldh = None, None, 0
    if history is not None:
        hlen = np.array([len(h) for h in history], np.int32)
        ldh = max(1, int(hlen.max()))
        hist = np.zeros((B, ldh), np.int32)
        for b, h in enumerate(history):
            hist[b, :len(h)] = h
    bl = np.ascontiguousarray(np.zeros(B) if base_len is None else base_len, dtype=np.int64)
    s = _Sampler(**{k: params[k] for k in SAMPLER_FIELDS})
    tokens = np.zeros((B, M), np.int32)
    counts = np.zeros((B, 2), np.int32)
    rb = np.zeros(B, np.int64)
    tp = np.zeros((B, M, V), np.float64) if with_target else None
    margins = np.zeros((B, M + 1), np.float64)
    rc = lib.orc_accept_sampled(B, M, V, _ptr(logits), V, _ptr(hist), _ptr(hlen), ldh, _ptr(d),
                                _ptr(qd), ldq, _ptr(qi), _ptr(qp), Kq, _ptr(u),
                                ctypes.cast(ctypes.pointer(s), ctypes.c_void_p), _ptr(bl),
                                _ptr(tokens), _ptr(counts), _ptr(rb), _ptr(tp), _ptr(margins))
    if rc != 0:
        raise ValueError("orc_accept_sampled rejected its arguments")
    out = [tokens, counts, rb]
    if with_target:
        out.append(tp)
    if with_margins:
        out.append(margins)
    return tuple(out)


def choose_draft_depth(accept_prob, cost):
    """(d, rates): the depth maximising E(d) / cost[d] (see oracle.c)."""
    lib = _load()
    a = np.ascontiguousarray(accept_prob, dtype=np.float64)
    c = np.ascontiguousarray(cost, dtype=np.float64)
    dmax = len(c) - 1
    assert len(a) >= dmax
    rate = np.zeros(dmax + 1, np.float64)
    d = lib.orc_choose_draft_depth(_ptr(a if len(a) else np.zeros(1)), _ptr(c), dmax, _ptr(rate))
    if d < 0:
        raise ValueError("orc_choose_draft_depth rejected its arguments")
    return int(d), rate


def depth_observe(reached, accepted, d, a, keep=1.0):
    lib = _load()
    lib.orc_depth_observe(_ptr(reached), _ptr(accepted), len(reached), int(d), int(a), float(keep))


def depth_estimate(reached, accepted):
    lib = _load()
    prob = np.zeros(len(reached), np.float64)
    lib.orc_depth_estimate(_ptr(reached), _ptr(accepted), len(reached), _ptr(prob))
    return prob


def verify_attention(q, k, v, L, scale=None, nthreads=None):
    """(out, bound): causal attention of the M verify rows (see oracle.c).
    q uint16 (bf16 bits) [M][Hq][D]; k, v [Hkv][ldk][D]."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    M, Hq, D = q.shape
    Hkv, ldk, _ = k.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o = np.zeros((M, Hq, D), np.float64)
    ob = np.zeros((M, Hq, D), np.float64)
    rc = lib.orc_verify_attention(M, Hq, Hkv, D, int(L), ldk, _ptr(q), _ptr(k), _ptr(v),
                                  float(scale), _ptr(o), _ptr(ob), _threads(nthreads))
    if rc != 0:
        raise ValueError("orc_verify_attention rejected its arguments")
    return o, ob


def kv_commit(cache: np.ndarray, new_rows: np.ndarray, base, rollback, ring: int) -> np.ndarray:
    """The cache after a verify write of M rows at base[b] committed to
    rollback[b] (Ollama mtp.go commit log, snapshot rework): a copy of
    ``cache`` [NL][B][Hkv][cap][D] (uint16 bf16 bits) that received only the
    first rollback[b] - base[b] rows of ``new_rows`` [NL][B][M][Hkv][D].
    ``rollback`` is clamped into [base, base + M] as the library does."""
    out = np.array(cache, dtype=np.uint16, copy=True, order="C")
    NL, B, Hkv, cap, D = out.shape
    rows = np.ascontiguousarray(new_rows, dtype=np.uint16)
    M = rows.shape[2]
    lib = _load()
    for b in range(B):
        n = int(min(max(int(rollback[b]) - int(base[b]), 0), M))
        for l in range(NL):
            for h in range(Hkv):
                head = out[l, b, h]
                src = np.ascontiguousarray(rows[l, b, :, h, :])
                lib.orc_kv_write(_ptr(head), cap, D, ring, int(base[b]), _ptr(src), D, n)
    return out


def kv_live_rows(cap: int, ring: int, length: int) -> dict:
    """Row -> position of every live position of a cache holding positions
    0 .. length-1: all of them for a linear cache, the last cap for a
    rotating one."""
    lo = max(0, length - cap) if ring else 0
    hi = length if ring else min(length, cap)
    return {(p % cap if ring else p): p for p in range(lo, hi)}
