"""Helpers for the GPU parity tests: host arrays -> device tensors, and the
GEMM tolerance.  Inputs always come from workloads.py or the oracle; no
expected value ever comes from the HIP path."""
import sys

import numpy as np
import torch

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def pack_gpu(bv, w: dict, count: int = 1) -> torch.Tensor:
    """Device copy of the source-layout weights of `w`, packed by the library."""
    return bv.pack_weights(w["format"], dev(w["codes"]), dev(w["scales"]), w["N"], w["K"],
                           count=count)


def gemm_gpu(bv, w: dict, x: np.ndarray, ldx_pad: int = 0, ldy_pad: int = 0, want_bf16=False,
             packed=None):
    """Run mtp_verify_gemm on device copies of (w, x); returns host y (and
    y_bf16 bits)."""
    M, K = x.shape
    N = w["N"]
    if ldx_pad:
        xp = np.zeros((M, K + ldx_pad), np.uint16)
        xp[:, :K] = x
        xd = dev(xp)
    else:
        xd = dev(x)
    y = torch.full((M, N + ldy_pad), float("nan"), dtype=torch.float32, device=DEV)
    yb = torch.zeros((M, N + ldy_pad), dtype=torch.int16, device=DEV) if want_bf16 else None
    if packed is None:
        packed = pack_gpu(bv, w)
    bv.verify_gemm(w["format"], xd, packed, N, K, float(w.get("g", 1.0)), y=y, y_bf16=yb)
    yh = host(y)[:, :N].astype(np.float64)
    if want_bf16:
        return yh, host(yb)[:, :N].view(np.uint16)
    return yh


def assert_gemm_close(y, y_ref, b_ref, what=""):
    err = np.abs(y - y_ref)
    tol = 1e-3 * b_ref + 1e-5
    bad = ~(err <= tol)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first at "
                             f"{tuple(i)}: gpu={y[tuple(i)]!r} oracle={y_ref[tuple(i)]!r} "
                             f"bound={b_ref[tuple(i)]!r}")
    return float((err / np.maximum(b_ref, 1e-30)).max())
