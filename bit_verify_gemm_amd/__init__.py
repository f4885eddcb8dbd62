"""Python binding of libmtpverify (the MTP verification pass on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/mtp_verify.h``.  PyTorch
supplies device memory and the current stream.  If the library has not been
built this module raises on first use; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "FMT_NVFP4", "FMT_Q4_0", "MAX_M", "MtpError", "lib", "abi_version",
    "packed_weight_bytes", "pack_weights", "gemm_workspace_bytes", "gemm_workspace",
    "gemm_plan_info",
    "moe_workspace_bytes", "accept_workspace_bytes", "accept_workspace",
    "Sampler", "accept_sampled", "accept_sampled_workspace", "accept_sampled_workspace_bytes",
    "choose_draft_depth", "DepthStats", "DepthStatsDevice", "verify_attention", "attention_workspace_bytes",
    "kv_snapshot", "kv_append", "kv_restore", "read_probe",
    "read_probe_shapes",
    "verify_gemm", "verify_moe", "accept_greedy", "accept_greedy_static", "accept_rejection",
    "LIB_PATH",
]

FMT_NVFP4 = 1
FMT_Q4_0 = 2
MAX_M = 16

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmtpverify.so")

_lock = threading.Lock()
_lib = None


class MtpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libmtpverify.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                ctypes.c_size_t)
        L.mtp_abi_version.restype = i32
        L.mtp_abi_version.argtypes = []
        L.mtp_last_error.restype = ctypes.c_char_p
        L.mtp_last_error.argtypes = []
        L.mtp_packed_weight_bytes.restype = sz
        L.mtp_packed_weight_bytes.argtypes = [i32, i32]
        L.mtp_pack_weights.restype = i32
        L.mtp_pack_weights.argtypes = [i32, i32, i32, i32, P, P, P, P]
        L.mtp_gemm_plan_info.restype = i32
        L.mtp_gemm_plan_info.argtypes = [i32, i32, i32, i32, P, i32]
        L.mtp_gemm_workspace_bytes.restype = sz
        L.mtp_gemm_workspace_bytes.argtypes = [i32, i32]
        L.mtp_verify_gemm.restype = i32
        L.mtp_verify_gemm.argtypes = [i32, i32, i32, i32, P, i64, P, f32, P, i64, P, i64, P, sz, P]
        L.mtp_moe_workspace_bytes.restype = sz
        L.mtp_moe_workspace_bytes.argtypes = [i32] * 5
        L.mtp_verify_moe.restype = i32
        L.mtp_verify_moe.argtypes = [i32] * 6 + [P] * 3 + [P, P, P, P] + [P, P, P, sz, P]
        L.mtp_accept_workspace_bytes.restype = sz
        L.mtp_accept_workspace_bytes.argtypes = [i32, i32]
        L.mtp_accept_greedy.restype = i32
        L.mtp_accept_greedy.argtypes = [P, i32, i32, i64, P, i64, P, P, P, P, sz, P]
        L.mtp_accept_greedy_static.restype = i32
        L.mtp_accept_greedy_static.argtypes = [P, i32, i32, i64, P, i64, P, P, P, P]
        L.mtp_accept_rejection.restype = i32
        L.mtp_accept_rejection.argtypes = [P, i32, i32, i64, P, i64, P, P, f32, f32, i64, P, P, P,
                                           P, sz, P]
        L.mtp_accept_sampled_workspace_bytes.restype = sz
        L.mtp_accept_sampled_workspace_bytes.argtypes = [i32] * 5
        L.mtp_accept_sampled.restype = i32
        L.mtp_accept_sampled.argtypes = [P, i32, i32, i32, i64, P, P, i64, P, P, i64, P, P, i32,
                                         P, P, P, P, P, P, P, P, P, sz, P]
        L.mtp_verify_attention_workspace_bytes.restype = sz
        L.mtp_verify_attention_workspace_bytes.argtypes = [i32] * 5
        L.mtp_verify_attention.restype = i32
        L.mtp_verify_attention.argtypes = [P, P, P, i64, i32, i32, i32, i32, i32, f32, P, P, sz, P]
        L.mtp_kv_append.restype = i32
        L.mtp_kv_append.argtypes = [P, P, i32, i32, i32, i64, i32, i32, P, P, i64, i32, P, P, P,
                                    P, P]
        L.mtp_kv_restore.restype = i32
        L.mtp_kv_restore.argtypes = [P, P, i32, i32, i32, i64, i32, i32, i32, P, P, P, P, P, P]
        L.mtp_read_probe.restype = i32
        L.mtp_read_probe.argtypes = [P, sz, P, i32, P]
        D = ctypes.c_double
        L.mtp_choose_draft_depth.restype = i32
        L.mtp_choose_draft_depth.argtypes = [P, P, i32, P]
        L.mtp_depth_observe.restype = i32
        L.mtp_depth_observe.argtypes = [P, P, i32, i32, i32, D]
        L.mtp_depth_estimate.restype = i32
        L.mtp_depth_estimate.argtypes = [P, P, i32, P]
        L.mtp_depth_observe_device.restype = i32
        L.mtp_depth_observe_device.argtypes = [P, P, i32, i32, P, D, P, P, P, P, P]
        _lib = L
        return L


def abi_version() -> int:
    return int(lib().mtp_abi_version())


def _check(status: int):
    if status != 0:
        raise MtpError(status, lib().mtp_last_error().decode(errors="replace"))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _ld(t):
    return int(t.stride(0)) if t is not None and t.dim() >= 2 else 0


def packed_weight_bytes(N: int, K: int) -> int:
    return int(lib().mtp_packed_weight_bytes(N, K))


def pack_weights(fmt: int, codes: torch.Tensor, scales: torch.Tensor, N: int, K: int,
                 count: int = 1, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Repack `count` stacked source matrices (codes [count*N][K/2] uint8,
    scales [count*N][K/bs]) into the packed layout the GEMM reads."""
    nb = packed_weight_bytes(N, K) * count
    if out is None:
        out = torch.empty(nb, dtype=torch.uint8, device=codes.device)
    _check(lib().mtp_pack_weights(fmt, count, N, K, _ptr(codes), _ptr(scales), _ptr(out),
                                  _stream(stream)))
    return out


def gemm_workspace_bytes(N: int, K: int) -> int:
    return int(lib().mtp_gemm_workspace_bytes(N, K))


PLAN_FIELDS = ("T", "P", "S", "ppj", "J", "KG", "TW", "TG", "G", "grid", "threads", "lds",
               "ws_bytes", "PP")


def gemm_plan_info(fmt: int, M: int, N: int, K: int) -> dict:
    """The launch shape mtp_verify_gemm uses (diagnostic; enqueues nothing)."""
    info = (ctypes.c_int32 * len(PLAN_FIELDS))()
    _check(lib().mtp_gemm_plan_info(fmt, M, N, K, ctypes.cast(info, ctypes.c_void_p),
                                    len(PLAN_FIELDS)))
    return dict(zip(PLAN_FIELDS, list(info)))


def gemm_workspace(N: int, K: int, device) -> torch.Tensor | None:
    """A zero-filled workspace for mtp_verify_gemm on N x K (None if not needed).
    Keep it for later calls: the library leaves it zero after every call."""
    nb = gemm_workspace_bytes(N, K)
    return torch.zeros(nb, dtype=torch.uint8, device=device) if nb else None


def moe_workspace_bytes(T: int, H: int, F: int, E: int, topk: int) -> int:
    return int(lib().mtp_moe_workspace_bytes(T, H, F, E, topk))


def accept_workspace_bytes(M: int, V: int) -> int:
    return int(lib().mtp_accept_workspace_bytes(M, V))


def accept_workspace(M: int, V: int, device) -> torch.Tensor:
    """A zero-filled workspace for the accept calls on M x V logits (it may
    be kept for later calls of either kind and any shape that fits)."""
    return torch.zeros(accept_workspace_bytes(M, V), dtype=torch.uint8, device=device)


def _workspace(nbytes: int, device, ws):
    if nbytes == 0:
        return ws
    if ws is None or _nbytes(ws) < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws


def verify_gemm(fmt: int, x: torch.Tensor, packed: torch.Tensor, N: int, K: int,
                global_scale: float = 1.0, y: torch.Tensor | None = None,
                y_bf16: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                want_fp32: bool = True, stream=None):
    """y[M][N] = x[M][K] . W.  x: bf16 (or its uint16/int16 bits) [M][>=K] on
    the GPU; packed: from pack_weights.  Returns (y, y_bf16); allocates the
    outputs it is not given.  ws must come from gemm_workspace (zero-filled)."""
    M = x.shape[0]
    dev = x.device
    if y is None and want_fp32:
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
    if ws is None and gemm_workspace_bytes(N, K):
        ws = gemm_workspace(N, K, dev)
    _check(lib().mtp_verify_gemm(fmt, M, N, K, _ptr(x), _ld(x), _ptr(packed),
                                 float(global_scale), _ptr(y), _ld(y), _ptr(y_bf16), _ld(y_bf16),
                                 _ptr(ws), _nbytes(ws), _stream(stream)))
    return y, y_bf16


def verify_moe(fmt: int, x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor,
               gu_packed: torch.Tensor, dn_packed: torch.Tensor, E: int, F: int,
               gu_global=None, dn_global=None, out: torch.Tensor | None = None,
               h_out: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None):
    """Routed MoE verify pass over packed experts (pack_weights with count=E);
    returns out [T][H] fp32 (and h_out if given)."""
    T, H = x.shape
    topk = topk_ids.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=x.device)
    ws = _workspace(moe_workspace_bytes(T, H, F, E, topk), x.device, ws)
    _check(lib().mtp_verify_moe(fmt, T, H, F, E, topk, _ptr(x), _ptr(topk_ids), _ptr(topk_w),
                                _ptr(gu_packed), _ptr(gu_global), _ptr(dn_packed),
                                _ptr(dn_global), _ptr(out), _ptr(h_out),
                                _ptr(ws), _nbytes(ws), _stream(stream)))
    return out, h_out


def _accept_outputs(M, dev, outs):
    if outs is not None:
        return outs
    return (torch.empty(M, dtype=torch.int32, device=dev),
            torch.empty(2, dtype=torch.int32, device=dev),
            torch.empty(1, dtype=torch.int64, device=dev))


def accept_greedy(logits: torch.Tensor, draft_ids: torch.Tensor | None, base_len: int = 0,
                  outs=None, ws: torch.Tensor | None = None, stream=None):
    """Returns (tokens[M] int32, counts[2] int32, rollback[1] int64) on the GPU."""
    M, V = logits.shape
    tok, cnt, rb = _accept_outputs(M, logits.device, outs)
    if ws is None or _nbytes(ws) < accept_workspace_bytes(M, V):
        ws = accept_workspace(M, V, logits.device)
    _check(lib().mtp_accept_greedy(_ptr(logits), M, V, _ld(logits), _ptr(draft_ids),
                                   int(base_len), _ptr(tok), _ptr(cnt), _ptr(rb), _ptr(ws),
                                   _nbytes(ws), _stream(stream)))
    return tok, cnt, rb


def accept_greedy_static(logits: torch.Tensor, draft_ids: torch.Tensor | None,
                         base_len: int = 0, outs=None, stream=None):
    """mtp_accept_greedy on the library's static scratch (no workspace).
    Returns (tokens[M] int32, counts[2] int32, rollback[1] int64) on the GPU."""
    M, V = logits.shape
    tok, cnt, rb = _accept_outputs(M, logits.device, outs)
    _check(lib().mtp_accept_greedy_static(_ptr(logits), M, V, _ld(logits), _ptr(draft_ids),
                                          int(base_len), _ptr(tok), _ptr(cnt), _ptr(rb),
                                          _stream(stream)))
    return tok, cnt, rb


def accept_rejection(logits: torch.Tensor, draft_probs: torch.Tensor | None,
                     draft_ids: torch.Tensor | None, uniforms: torch.Tensor, temperature: float,
                     top_p: float, base_len: int = 0, outs=None, ws: torch.Tensor | None = None,
                     stream=None):
    """Returns (tokens[M] int32, counts[2] int32, rollback[1] int64) on the GPU."""
    M, V = logits.shape
    tok, cnt, rb = _accept_outputs(M, logits.device, outs)
    if ws is None or _nbytes(ws) < accept_workspace_bytes(M, V):
        ws = accept_workspace(M, V, logits.device)
    _check(lib().mtp_accept_rejection(_ptr(logits), M, V, _ld(logits), _ptr(draft_probs),
                                      _ld(draft_probs), _ptr(draft_ids), _ptr(uniforms),
                                      float(temperature), float(top_p), int(base_len), _ptr(tok),
                                      _ptr(cnt), _ptr(rb), _ptr(ws), _nbytes(ws),
                                      _stream(stream)))
    return tok, cnt, rb


class Sampler(ctypes.Structure):
    """mtp_sampler: the sampler pipeline's parameters (see mtp_verify.h)."""
    _fields_ = [("temperature", ctypes.c_float), ("top_p", ctypes.c_float),
                ("min_p", ctypes.c_float), ("top_k", ctypes.c_int32),
                ("repeat_penalty", ctypes.c_float), ("presence_penalty", ctypes.c_float),
                ("frequency_penalty", ctypes.c_float), ("penalty_last_n", ctypes.c_int32)]

    def __init__(self, temperature=1.0, top_p=1.0, min_p=0.0, top_k=40, repeat_penalty=1.0,
                 presence_penalty=0.0, frequency_penalty=0.0, penalty_last_n=0):
        super().__init__(temperature, top_p, min_p, top_k, repeat_penalty, presence_penalty,
                         frequency_penalty, penalty_last_n)

    @property
    def penalties(self) -> bool:
        return self.penalty_last_n > 0 and (self.repeat_penalty != 1.0 or
                                            self.presence_penalty != 0.0 or
                                            self.frequency_penalty != 0.0)


def accept_sampled_workspace_bytes(B: int, M: int, V: int, top_k: int, penalties: bool) -> int:
    return int(lib().mtp_accept_sampled_workspace_bytes(B, M, V, top_k, int(bool(penalties))))


def accept_sampled_workspace(B: int, M: int, V: int, top_k: int, penalties: bool,
                             device) -> torch.Tensor:
    """A zero-filled workspace for mtp_accept_sampled (its head holds counters
    that each call leaves zero)."""
    return torch.zeros(max(accept_sampled_workspace_bytes(B, M, V, top_k, penalties), 1),
                       dtype=torch.uint8, device=device)


def accept_sampled(logits: torch.Tensor, draft_ids: torch.Tensor | None, uniforms: torch.Tensor,
                   params: Sampler, draft_probs: torch.Tensor | None = None,
                   draft_topk: tuple | None = None, history: torch.Tensor | None = None,
                   history_len: torch.Tensor | None = None, base_len: torch.Tensor | None = None,
                   want_target: bool = False, outs=None, ws: torch.Tensor | None = None,
                   stream=None):
    """Sampled acceptance of B sequences.  logits [B][M][V] (or [B*M][V] views
    with uniforms [B][M] giving B); draft_ids [B][M-1]; draft_probs dense
    [B][M-1][V] or draft_topk = (ids [B][M-1][Kq], probs [B][M-1][Kq]);
    history [B][ldh] with history_len [B]; base_len [B] int64.  Returns
    (tokens [B][M], counts [B][2], rollback [B]) and, with want_target, the
    targets' sparse ids and probabilities [B][M][K]."""
    B, M = uniforms.shape
    V = logits.shape[-1]
    z = logits.reshape(B * M, V) if logits.dim() == 3 else logits
    dev = z.device
    K = min(int(params.top_k), V)
    if outs is None:
        outs = (torch.empty((B, M), dtype=torch.int32, device=dev),
                torch.empty((B, 2), dtype=torch.int32, device=dev),
                torch.empty(B, dtype=torch.int64, device=dev))
    tok, cnt, rb = outs
    tid = tpr = None
    if want_target:
        tid = torch.empty((B, M, K), dtype=torch.int32, device=dev)
        tpr = torch.empty((B, M, K), dtype=torch.float32, device=dev)
    need = accept_sampled_workspace_bytes(B, M, V, int(params.top_k), params.penalties)
    if ws is None or _nbytes(ws) < need:
        ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    q = qi = qp = None
    ldq, Kq = 0, 0
    if M > 1:
        if draft_probs is not None:
            q = draft_probs.reshape(B * (M - 1), -1)
            ldq = _ld(q)
        else:
            qi, qp = draft_topk
            Kq = int(qi.shape[-1])
    ldh = _ld(history) if history is not None else 0
    _check(lib().mtp_accept_sampled(_ptr(z), B, M, V, _ld(z), _ptr(history), _ptr(history_len),
                                    ldh, _ptr(draft_ids), _ptr(q), ldq, _ptr(qi), _ptr(qp), Kq,
                                    _ptr(uniforms), ctypes.cast(ctypes.pointer(params),
                                                                ctypes.c_void_p),
                                    _ptr(base_len), _ptr(tok), _ptr(cnt), _ptr(rb), _ptr(tid),
                                    _ptr(tpr), _ptr(ws), _nbytes(ws), _stream(stream)))
    if want_target:
        return tok, cnt, rb, tid, tpr
    return tok, cnt, rb


def _host_ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def choose_draft_depth(accept_prob, cost):
    """(d, rates): the draft depth with the most expected committed tokens per
    unit of cost (mtp_choose_draft_depth).  accept_prob [dmax], cost [dmax+1]."""
    import numpy as np
    c = np.ascontiguousarray(cost, dtype=np.float64)
    dmax = len(c) - 1
    a = np.ascontiguousarray(accept_prob, dtype=np.float64)[:dmax]
    rate = np.zeros(dmax + 1, np.float64)
    d = int(lib().mtp_choose_draft_depth(_host_ptr(a) if dmax else None, _host_ptr(c), dmax,
                                         _host_ptr(rate)))
    if d < 0:
        raise MtpError(d, "mtp_choose_draft_depth: bad arguments")
    return d, rate


class DepthStats:
    """Live per-position acceptance (mtp_depth_observe / mtp_depth_estimate)."""

    def __init__(self, dmax: int, keep: float = 1.0):
        import numpy as np
        self.dmax, self.keep = int(dmax), float(keep)
        self.reached = np.zeros(self.dmax, np.float64)
        self.accepted = np.zeros(self.dmax, np.float64)

    def observe(self, depth: int, n_accepted: int):
        _check(lib().mtp_depth_observe(_host_ptr(self.reached), _host_ptr(self.accepted),
                                       self.dmax, int(depth), int(n_accepted), self.keep))

    def estimate(self):
        import numpy as np
        prob = np.zeros(self.dmax, np.float64)
        _check(lib().mtp_depth_estimate(_host_ptr(self.reached), _host_ptr(self.accepted),
                                        self.dmax, _host_ptr(prob)))
        return prob


class DepthStatsDevice:
    """Live per-position acceptance kept on the GPU (mtp_depth_observe_device):
    observe() enqueues the update from an accept call's counts and the next
    depth choice on the stream; nothing is read back unless asked for."""

    def __init__(self, dmax: int, cost, device, keep: float = 1.0):
        self.dmax, self.keep = int(dmax), float(keep)
        self.reached = torch.zeros(self.dmax, dtype=torch.float64, device=device)
        self.accepted = torch.zeros(self.dmax, dtype=torch.float64, device=device)
        self.prob = torch.zeros(self.dmax, dtype=torch.float64, device=device)
        self.cost = torch.as_tensor(cost, dtype=torch.float64).to(device).contiguous()
        if self.cost.numel() != self.dmax + 1:
            raise ValueError("cost needs dmax + 1 entries")
        self.choice = torch.zeros(1, dtype=torch.int32, device=device)
        self.err = torch.zeros(1, dtype=torch.int32, device=device)

    def observe(self, depth: int, counts: torch.Tensor, stream=None):
        _check(lib().mtp_depth_observe_device(
            _ptr(self.reached), _ptr(self.accepted), self.dmax, int(depth), _ptr(counts),
            self.keep, _ptr(self.cost), _ptr(self.choice), _ptr(self.prob), _ptr(self.err),
            _stream(stream)))


def attention_workspace_bytes(M: int, Hq: int, Hkv: int, D: int, L: int) -> int:
    return int(lib().mtp_verify_attention_workspace_bytes(M, Hq, Hkv, D, L))


def kv_snapshot(k_cache: torch.Tensor, M: int):
    """Snapshot buffers (K, V) [NL][B][Hkv][M][D] for a rotating cache
    k_cache [NL][B][Hkv][cap][D]; only rows a verify write destroys are
    ever written into them."""
    NL, B, Hkv, _, D = k_cache.shape
    return (torch.empty((NL, B, Hkv, M, D), dtype=k_cache.dtype, device=k_cache.device),
            torch.empty((NL, B, Hkv, M, D), dtype=k_cache.dtype, device=k_cache.device))


def kv_append(k_cache: torch.Tensor, v_cache: torch.Tensor, k_new: torch.Tensor,
              v_new: torch.Tensor, base_len: torch.Tensor, ring: bool, snapshot=None,
              err: torch.Tensor | None = None, stream=None):
    """Write the M verify rows k_new / v_new ([NL][B][M] rows of Hkv * D bf16,
    rows ld_new = k_new.stride(2) elements apart) into k_cache / v_cache
    [NL][B][Hkv][cap][D] at positions base_len[b] .. (device int64 [B]),
    copying out of a rotating cache only the rows that the write destroys."""
    NL, B, Hkv, cap, D = k_cache.shape
    M = k_new.shape[2]
    ld = int(k_new.stride(2)) if M > 1 else Hkv * D
    for t in (k_new, v_new):
        if (tuple(t.shape[:3]) != (NL, B, M) or t.shape[3] < Hkv * D or t.stride(3) != 1
                or (M > 1 and t.stride(2) != ld) or (B > 1 and t.stride(1) != M * ld)
                or (NL > 1 and t.stride(0) != B * M * ld)):
            raise ValueError("k_new and v_new must be [NL][B][M] rows of >= Hkv * D elements, "
                             "the rows ld_new apart with the same strides")
    sk, sv = snapshot if snapshot is not None else (None, None)
    _check(lib().mtp_kv_append(_ptr(k_cache), _ptr(v_cache), NL, B, Hkv, cap, D, int(bool(ring)),
                               _ptr(k_new), _ptr(v_new), ld, M, _ptr(base_len), _ptr(sk),
                               _ptr(sv), _ptr(err), _stream(stream)))


def kv_restore(k_cache: torch.Tensor, v_cache: torch.Tensor, M: int, base_len: torch.Tensor,
               rollback: torch.Tensor, ring: bool, snapshot=None,
               err: torch.Tensor | None = None, stream=None):
    """Commit the last kv_append to rollback[b] (device int64 [B], e.g. an
    accept call's out_rollback): a rotating cache gets back the rows that
    the dropped positions overwrote; a linear cache needs no work."""
    NL, B, Hkv, cap, D = k_cache.shape
    sk, sv = snapshot if snapshot is not None else (None, None)
    _check(lib().mtp_kv_restore(_ptr(k_cache), _ptr(v_cache), NL, B, Hkv, cap, D,
                                int(bool(ring)), int(M), _ptr(base_len), _ptr(rollback),
                                _ptr(sk), _ptr(sv), _ptr(err), _stream(stream)))


def read_probe_shapes() -> int:
    """Number of launch shapes of the read-bandwidth probe."""
    return int(lib().mtp_read_probe(None, 0, None, -1, None))


def read_probe(src: torch.Tensor, sink: torch.Tensor, shape: int = 0, stream=None):
    """Read every byte of the contiguous device tensor ``src`` once in launch
    shape ``shape`` (a bandwidth measurement aid); ``sink`` is a device
    int32 tensor."""
    _check(lib().mtp_read_probe(_ptr(src), _nbytes(src), _ptr(sink), int(shape), _stream(stream)))


def verify_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, L: int,
                     scale: float | None = None, out: torch.Tensor | None = None,
                     ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Causal attention of the M verify rows q [M][Hq][D] (bf16) over the
    cache k_cache / v_cache [Hkv][ldk][D] (bf16; positions 0 .. L+M-1 hold
    keys, the verify tokens' own at L ..).  Returns out [M][Hq][D] fp32."""
    M, Hq, D = q.shape
    Hkv, ldk, _ = k_cache.shape
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    if out is None:
        out = torch.empty((M, Hq, D), dtype=torch.float32, device=q.device)
    need = attention_workspace_bytes(M, Hq, Hkv, D, L)
    if ws is None or _nbytes(ws) < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().mtp_verify_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), ldk, M, Hq, Hkv, D,
                                      int(L), float(scale), _ptr(out), _ptr(ws), _nbytes(ws),
                                      _stream(stream)))
    return out
