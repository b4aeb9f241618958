"""Python binding of libmoegq (gathered affine-quantized MoE expert path, gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libmoegq.so``.  PyTorch supplies device memory (tensors) and the
current HIP stream.  There is no CPU fallback: without the built library the
import of any op raises.

Tensor conventions: bf16 activations/scales/biases are ``torch.bfloat16``;
packed words are ``torch.int32`` or ``torch.uint32`` holding the uint32 bit
patterns; indices are ``torch.int32``.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["MoegqError", "lib", "library_path", "gather_qmm", "quantized_matmul", "gather_qmm_workspace_bytes",
           "gather_qmm_mx", "gather_qmm_glu", "affine_qmm", "affine_qmm_glu", "affine_qmm_workspace",
           "switch_glu", "switch_glu_mode", "moe_decode", "moe_decode_static", "static_scratch_bytes", "moe_prefill", "moe_prefill_workspace_bytes",
           "moe_prefill_layout", "moe_prefill_tables", "moe_combine", "moe_combine_gated", "moe_combine_unfused", "sort_pairs",
           "schedule_tiles", "rms_norm", "sigmoid_gate", "route", "gather_mm", "kv_feed", "kv_feed_stacked",
           "selfcheck", "selfcheck_state", "probe_stream_read", "probe_mfma_bf16",
           "validate_indices", "workspace_bytes", "MODE_AUTO", "MODE_DECODE", "MODE_SORTED",
           "TILES_SCHEDULED", "TILES_NAIVE"]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libmoegq.so")

OK = 0
BF16, F16, F32, F64, I32, U32, I64 = range(7)
MODE_AUTO, MODE_DECODE, MODE_SORTED = 0, 1, 2
TILES_SCHEDULED, TILES_NAIVE = 0, 1
MX_MODES = {"mxfp4": (1, 4), "mxfp8": (2, 8)}     # mode code, element bits
OP_GATHER_QMM, OP_SWITCH_GLU_DECODE, OP_SWITCH_GLU_SORTED, OP_COMBINE_UNFUSED, OP_SELFCHECK, OP_SORT_PAIRS, \
    OP_MOE_DECODE, OP_GATHER_MM = range(8)

_DTYPE = {torch.bfloat16: BF16, torch.float16: F16, torch.float32: F32, torch.float64: F64,
          torch.int32: I32, torch.int64: I64}
if hasattr(torch, "uint32"):
    _DTYPE[torch.uint32] = U32


class MoegqError(ValueError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {lib().moegq_status_string(status).decode()} (status {status})")
        self.status = status


_LIB = None
_i64, _int, _p, _sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t

_SIGS = {
    "moegq_status_string": ([_int], ctypes.c_char_p),
    "moegq_version": ([], ctypes.c_char_p),
    "moegq_workspace_bytes": ([_int, _i64, _i64, _i64, _int], _sz),
    "moegq_gather_qmm_workspace_bytes": ([_i64, _i64, _i64, _i64, _i64, _int, _int, _int, _int], _sz),
    "moegq_gather_qmm_mx": ([_p, _int, _i64, _i64, _i64, _p, _p, _i64, _i64, _p, _i64, _p, _int, _i64, _int, _int,
                             _p, _p, _sz, _p], _int),
    "moegq_gather_qmm_mx_workspace_bytes": ([_i64, _i64, _i64, _i64, _int, _int], _sz),
    "moegq_gather_qmm": ([_p, _int, _i64, _i64, _i64, _p, _int, _p, _p, _i64, _i64, _p, _i64, _p, _int, _i64,
                          _int, _int, _int, _int, _p, _p, _sz, _p], _int),
    "moegq_gather_qmm_glu": ([_p, _int, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _i64, _i64, _p, _i64, _p, _int,
                              _i64, _int, _int, _int, _p, _p, _sz, _p], _int),
    "moegq_affine_qmm": ([_p, _int, _i64, _i64, _p, _int, _p, _p, _i64, _int, _int, _int, _p, _p, _p], _int),
    "moegq_affine_qmm_glu": ([_p, _i64, _i64, _p, _p, _p, _p, _p, _p, _i64, _int, _int, _p, _p], _int),
    "moegq_affine_qmm_ws": ([_p, _int, _i64, _i64, _p, _int, _p, _p, _i64, _int, _int, _int, _p, _p, _p, _sz, _p],
                            _int),
    "moegq_affine_qmm_glu_ws": ([_p, _i64, _i64, _p, _p, _p, _p, _p, _p, _i64, _int, _int, _p, _p, _sz, _p], _int),
    "moegq_affine_qmm_workspace_bytes": ([_i64, _i64, _i64, _int], _sz),
    "moegq_switch_glu": ([_p, _i64, _i64, _i64, _i64, _p, _i64, _p, _p, _p, _p, _p, _p, _p, _p, _p, _int, _int,
                          _int, _int, _int, _p, _p, _p, _sz, _p], _int),
    "moegq_switch_glu_mode": ([_i64, _i64, _i64], _int),
    "moegq_moe_decode": ([_p, _i64, _i64, _i64, _i64, _p, _i64, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _int,
                          _int, _p, _p, _p, _sz, _p], _int),
    "moegq_moe_decode_static": ([_p, _i64, _i64, _i64, _i64, _p, _i64, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                 _int, _int, _p, _p, _p], _int),
    "moegq_static_scratch_bytes": ([], _sz),
    "moegq_moe_prefill": ([_p, _i64, _i64, _i64, _i64, _p, _i64, _p] + [_p] * 21 + [_int, _int, _p, _p, _sz, _p],
                          _int),
    "moegq_moe_prefill_workspace_bytes": ([_i64, _i64, _i64, _i64, _i64, _int], _sz),
    "moegq_moe_prefill_layout": ([_i64, _i64, _i64, _i64, _i64, _int, _p, _p, _p], _int),
    "moegq_moe_combine": ([_p, _p, _p, _p, _i64, _i64, _i64, _p, _p], _int),
    "moegq_moe_combine_gated": ([_p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _p], _int),
    "moegq_moe_combine_unfused": ([_p, _p, _p, _p, _i64, _i64, _i64, _p, _p, _sz, _p], _int),
    "moegq_sort_pairs": ([_p, _int, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p, _sz, _p], _int),
    "moegq_schedule_tiles": ([_p, _i64, _i64, _int, _int, _p, _i64, _p, _p], _int),
    "moegq_rms_norm": ([_p, _p, _i64, _i64, ctypes.c_float, _p, _p], _int),
    "moegq_sigmoid_gate": ([_p, _p, _i64, _i64, _i64, _p, _p], _int),
    "moegq_route": ([_p, _i64, _i64, _i64, _p, _p, _p], _int),
    "moegq_gather_mm": ([_p, _i64, _i64, _i64, _p, _i64, _i64, _p, _i64, _p, _i64, _int, _p, _p, _sz, _p], _int),
    "moegq_kv_feed": ([_p, _p, _p, _i64, _i64, _i64, _i64, _p, _p], _int),
    "moegq_kv_feed_ld": ([_p, _i64, _p, _i64, _p, _i64, _i64, _i64, _p, _p], _int),
    "moegq_selfcheck": ([_p, _sz, _p], _int),
    "moegq_selfcheck_state": ([], _int),
    "moegq_probe_stream_read": ([_p, _i64, _p, _int, _p], _int),
    "moegq_probe_mfma_bf16": ([_int, _int, _p, _p], _int),
    "moegq_validate_indices": ([_p, _i64, _i64, _int, _p, _p], _int),
}


def lib():
    """The loaded libmoegq.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(library_path):
            raise ImportError(f"{library_path} is missing: build it with "
                              "`python -m moe_expert_gathered_amd.build` (there is no CPU fallback)")
        L = ctypes.CDLL(library_path)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _LIB = L
    return _LIB


def _check(status: int, where: str):
    if status != OK:
        raise MoegqError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt(t) -> int:
    return _DTYPE.get(t.dtype, -1)


def _wdt(t) -> int:
    # packed words travel as int32 or uint32 tensors holding the uint32 bits
    return U32 if t.dtype in (torch.int32, getattr(torch, "uint32", torch.int32)) else _dt(t)


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("moegq ops take device tensors")
        if t is not None and not t.is_contiguous():
            raise ValueError("moegq ops take contiguous tensors")


def _req(t, name, dtypes, shape=None):
    """Argument check of the binding: dtype (one of ``dtypes``) and, where
    given, the exact shape; a mismatch raises ValueError before anything is
    launched (the C entry points take raw pointers and cannot see either)."""
    if t is None:
        return
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


_BF = (torch.bfloat16,)
_IDX = (torch.int32,)
_WORDS = tuple(d for d in (torch.int32, getattr(torch, "uint32", None)) if d is not None)


def _req_matrix(trip, name, N, K, bits, gs, batch=()):
    """(words, scales, biases) of quantized rows: words [*batch, N, K*bits/32]
    int32/uint32, scales and biases [*batch, N, K/gs] bf16."""
    w, sc, bi = trip
    if K * bits % 32 or K % gs:
        raise ValueError(f"{name}: K={K} is not a whole number of words and groups")
    _req(w, name + " words", _WORDS, tuple(batch) + (N, K * bits // 32))
    _req(sc, name + " scales", _BF, tuple(batch) + (N, K // gs))
    _req(bi, name + " biases", _BF, tuple(batch) + (N, K // gs))


def _req_combine(y, inv, scores, shared, out):
    """Combine tail arguments: y [P, H] bf16 (P = T*top_k expert outputs),
    inv [P] int32 or None, scores [T, top_k] bf16, shared/out [T, H] bf16."""
    _req(scores, "scores", _BF)
    T, top_k = scores.shape
    _req(y, "y", _BF)
    if y.dim() != 2 or y.shape[0] < T * top_k:
        raise ValueError(f"y: shape {tuple(y.shape)}, expected [{T * top_k}, H]")
    H = y.shape[-1]
    _req(inv, "inv", _IDX, (T * top_k,))
    _req(shared, "shared", _BF, (T, H))
    _req(out, "out", _BF, (T, H))


def _req_experts(gate, up, down, E, H, I, bits, gs):
    _req_matrix(gate, "gate", I, H, bits, gs, (E,))
    _req_matrix(up, "up", I, H, bits, gs, (E,))
    _req_matrix(down, "down", H, I, bits, gs, (E,))


def workspace_bytes(op: int, P: int, E: int, N: int, bm: int = 0) -> int:
    return int(lib().moegq_workspace_bytes(op, P, E, N, bm))


def gather_qmm_workspace_bytes(P, E, M, N, K, x_dtype, transpose, bits, sorted_indices) -> int:
    return int(lib().moegq_gather_qmm_workspace_bytes(P, E, M, N, K, x_dtype, int(bool(transpose)), bits,
                                                      int(bool(sorted_indices))))


def _workspace(nbytes: int, device):
    if nbytes == 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def _gather_indices(x, w, rhs_indices, lhs_indices):
    """Flattened (lhs, rhs) pair indices over the broadcast index shape
    (marshalling only).  With x's batch a prefix of the index shape, the x
    batch of flat pair p is p // lhs_div and no lhs array is built."""
    xb, wb = tuple(x.shape[:-2]), tuple(w.shape[:-2])
    X = 1
    for d in xb:
        X *= d
    E = 1
    for d in wb:
        E *= d
    lhs_div = 1
    li = None
    if rhs_indices is None:
        rhs_indices = torch.arange(E, dtype=torch.int32, device=x.device).reshape(wb if wb else (1,))
    if lhs_indices is None:
        shape = tuple(torch.broadcast_shapes(xb, tuple(rhs_indices.shape)))
        bxp = (1,) * (len(shape) - len(xb)) + xb
        j = len(shape)
        while j > 0 and bxp[j - 1] == 1:
            j -= 1
        if tuple(bxp[:j]) == tuple(shape[:j]):
            # x's batch is a prefix of the index shape: the x row of flat pair p is p // prod(shape[j:])
            d = 1
            for v in shape[j:]:
                d *= v
            lhs_div = d
        else:
            lhs_full = torch.arange(X, dtype=rhs_indices.dtype, device=x.device).reshape(xb if xb else (1,))
            li = lhs_full.expand(shape).reshape(-1).contiguous()
        ri = rhs_indices.expand(shape).reshape(-1).contiguous()
    else:
        lb, rb = torch.broadcast_tensors(lhs_indices, rhs_indices)
        shape = tuple(lb.shape)
        li, ri = lb.reshape(-1).contiguous(), rb.reshape(-1).contiguous()
    return X, E, li, ri, lhs_div, shape


# ----------------------------------------------------------------------------- ops
def gather_qmm(x, w, scales, biases, rhs_indices=None, lhs_indices=None, transpose=True,
               group_size=64, bits=4, sorted_indices=False, out=None, workspace=None):
    """out[j] = x[lhs[j]] . dequant(w[rhs[j]])^T over the broadcast index shape.

    x: [*bx, M, K]; w: [E, N, K*bits/32] (or [*bw, N, Kw], flattened to E).
    With x of shape [B, 1, 1, K] and rhs [B, top_k] (the MoE decode layout)
    the x row of pair (b, k) is b, passed as lhs_div = top_k without building
    an index array.  Otherwise indices are broadcast (marshalling only).
    Output: index shape + [M, N], bf16 for bf16 activations, float32 for
    float16/float32 ones.  transpose=False takes w [E, K, N*bits/32] with
    groups along N.  workspace: an optional uint8 device tensor of at least
    gather_qmm_workspace_bytes(...) bytes (else one is allocated).
    """
    _req(scales, "scales", _BF)
    _req(biases, "biases", _BF)
    _dev(x, w, scales, biases, rhs_indices, lhs_indices, workspace)
    M, K = x.shape[-2], x.shape[-1]
    N = w.shape[-2] if transpose else w.shape[-1] * 32 // bits
    X, E, li, ri, lhs_div, shape = _gather_indices(x, w, rhs_indices, lhs_indices)
    P = int(ri.numel())
    idx_dt = _dt(ri)
    if li is not None and li.dtype != ri.dtype:
        raise ValueError("lhs and rhs indices must share a dtype")
    if out is None:
        # the promoted type: bf16 activations stay bf16, float16 and float32 give float32
        odt = torch.bfloat16 if x.dtype == torch.bfloat16 else torch.float32
        out = torch.empty(shape + (M, N), dtype=odt, device=x.device)
    need = gather_qmm_workspace_bytes(P, E, M, N, K, _dt(x), transpose, bits, sorted_indices)
    if workspace is not None and workspace.numel() >= need:
        ws, wsb = workspace, int(workspace.numel())
    else:
        ws, wsb = _workspace(need, x.device)
    st = lib().moegq_gather_qmm(_ptr(x), _dt(x), X, M, K, _ptr(w), _wdt(w), _ptr(scales), _ptr(biases), E, N,
                                _ptr(li), lhs_div, _ptr(ri), idx_dt, P, int(bool(sorted_indices)),
                                int(bool(transpose)), group_size, bits, _ptr(out), _ptr(ws), wsb, _stream())
    _check(st, "gather_qmm")
    return out


def gather_qmm_mx(x, w, scales, rhs_indices=None, lhs_indices=None, transpose=True, mode="mxfp8", out=None,
                  workspace=None):
    """gather_qmm for the mx modes ("mxfp4": E2M1 elements, 8 per word;
    "mxfp8": E4M3, 4 per word), one E8M0 scale byte per 32 elements along the
    packed axis (scales: uint8 tensor), no biases.  Indices and result type
    as gather_qmm."""
    _req(scales, "scales", (torch.uint8,))
    _dev(x, w, scales, rhs_indices, lhs_indices, workspace)
    code, bits = MX_MODES[mode]
    M, K = x.shape[-2], x.shape[-1]
    N = w.shape[-2] if transpose else w.shape[-1] * 32 // bits
    X, E, li, ri, lhs_div, shape = _gather_indices(x, w, rhs_indices, lhs_indices)
    P = int(ri.numel())
    if li is not None and li.dtype != ri.dtype:
        raise ValueError("lhs and rhs indices must share a dtype")
    if out is None:
        odt = torch.bfloat16 if x.dtype == torch.bfloat16 else torch.float32
        out = torch.empty(shape + (M, N), dtype=odt, device=x.device)
    need = int(lib().moegq_gather_qmm_mx_workspace_bytes(P, M, N, K, int(bool(transpose)), code))
    if workspace is not None and workspace.numel() >= need:
        ws, wsb = workspace, int(workspace.numel())
    else:
        ws, wsb = _workspace(need, x.device)
    st = lib().moegq_gather_qmm_mx(_ptr(x), _dt(x), X, M, K, _ptr(w), _ptr(scales), E, N, _ptr(li), lhs_div,
                                   _ptr(ri), _dt(ri), P, int(bool(transpose)), code, _ptr(out), _ptr(ws), wsb,
                                   _stream())
    _check(st, "gather_qmm_mx")
    return out


def quantized_matmul(x, w, scales, biases=None, transpose=True, group_size=64, bits=4, mode="affine", out=None):
    """x . dequant(w)^T (or x . dequant(w) without the transpose) with the
    leading batch axes of x [*bx, M, K] and w [*bw, rows, words] broadcast
    together; the result type is bf16 for bf16 activations, float32 for
    float16 and float32 ones.  mode "affine" (scales and biases, group_size,
    bits) or "mxfp4" / "mxfp8" (E8M0 scale bytes, no biases).  Runs as
    gather_qmm over the broadcast batch indices (marshalling only)."""
    xb, wb = tuple(x.shape[:-2]), tuple(w.shape[:-2])
    M = x.shape[-2]
    eb = bits if mode == "affine" else MX_MODES[mode][1]
    N = w.shape[-2] if transpose else w.shape[-1] * 32 // eb
    shape = tuple(torch.broadcast_shapes(xb, wb))
    x3 = x if x.dim() >= 3 else x.reshape((1,) * (3 - x.dim()) + tuple(x.shape))
    w3 = w if w.dim() >= 3 else w.reshape((1,) + tuple(w.shape))
    s3 = scales if scales.dim() >= 3 else scales.reshape((1,) + tuple(scales.shape))
    if mode != "affine":
        if biases is not None:
            raise ValueError("mx modes take no biases")
        res = gather_qmm_mx(x3, w3, s3, transpose=transpose, mode=mode, out=out)
        return res.reshape(shape + (M, N))
    b3 = biases if biases.dim() >= 3 else biases.reshape((1,) + tuple(biases.shape))
    res = gather_qmm(x3, w3, s3, b3, transpose=transpose, group_size=group_size, bits=bits,
                     out=out)
    return res.reshape(shape + (M, N))


def gather_mm(x, w, rhs_indices, lhs_indices=None, lhs_div=1, sorted_indices=False, out=None):
    """out[p] = x[row(p)] . w[rhs[p]]^T with unquantized bf16 experts.
    x: [X, M, K] (or [X, K] for M = 1) bf16; w: [E, N, K] bf16; rhs_indices [P]
    int32; the x batch of pair p is lhs_indices[p], or p // lhs_div.
    Returns [P, M, N] (M = 1: [P, N])."""
    _req(x, "x", _BF)
    _req(w, "w", _BF)
    _req(rhs_indices, "rhs_indices", _IDX)
    _req(lhs_indices, "lhs_indices", _IDX)
    _dev(x, w, rhs_indices, lhs_indices)
    squeeze = x.dim() == 2
    X, M, K = (x.shape[0], 1, x.shape[1]) if squeeze else tuple(x.shape)
    E, N = w.shape[0], w.shape[1]
    P = int(rhs_indices.numel())
    if out is None:
        out = torch.empty((P, N) if squeeze else (P, M, N), dtype=torch.bfloat16, device=x.device)
    ws, wsb = _workspace(workspace_bytes(OP_GATHER_MM, P, E, M, 0), x.device)
    st = lib().moegq_gather_mm(_ptr(x), X, M, K, _ptr(w), E, N, _ptr(lhs_indices), lhs_div, _ptr(rhs_indices), P,
                               int(bool(sorted_indices)), _ptr(out), _ptr(ws), wsb, _stream())
    _check(st, "gather_mm")
    return out


def gather_qmm_glu(x, gate, up, rhs_indices, lhs_indices=None, lhs_div=1, group_size=64, bits=4,
                   sorted_indices=False, out=None):
    """h[p] = bf16(silu(g) * u) over gathered experts, g/u = x[row(p)] . W[rhs[p]]^T.
    x: [X, M, K] (or [X, K] for M = 1); gate/up: (words [E, N, Kw], scales, biases);
    rhs_indices [P]; the x row of pair p is lhs_indices[p], or p // lhs_div."""
    _req(x, "x", _BF)
    _req(rhs_indices, "rhs_indices", _IDX)
    _req(lhs_indices, "lhs_indices", _IDX)
    if x.dim() == 2:
        X, K = x.shape
        M = 1
    else:
        X, M, K = x.shape
    E, N = gate[0].shape[0], gate[0].shape[1]
    _req_matrix(gate, "gate", N, K, bits, group_size, (E,))
    _req_matrix(up, "up", N, K, bits, group_size, (E,))
    _dev(x, *gate, *up, rhs_indices, lhs_indices)
    P = rhs_indices.numel()
    if out is None:
        out = torch.empty((P, M, N), dtype=torch.bfloat16, device=x.device)
    ws, wsb = _workspace(gather_qmm_workspace_bytes(P, E, M, N, K, BF16, True, bits, sorted_indices), x.device)
    st = lib().moegq_gather_qmm_glu(_ptr(x), _dt(x), X, M, K, *[_ptr(t) for t in gate], *[_ptr(t) for t in up], E,
                                    N, _ptr(lhs_indices), lhs_div, _ptr(rhs_indices), _dt(rhs_indices), P,
                                    int(bool(sorted_indices)), group_size, bits, _ptr(out), _ptr(ws), wsb,
                                    _stream())
    _check(st, "gather_qmm_glu")
    return out


def affine_qmm_workspace(M: int, N: int, K: int, glu: bool = False, device="cuda"):
    """A zero-filled workspace for affine_qmm / affine_qmm_glu at these sizes
    (None when the product takes none): K split over workgroups at 5..16 rows.
    Its layout depends on (N, K, glu) only: reusable by later calls with the
    same N, K and glu (any M up to 16) on one stream, not by other shapes."""
    n = int(lib().moegq_affine_qmm_workspace_bytes(M, N, K, int(bool(glu))))
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def affine_qmm(x, w, scales, biases, group_size=64, bits=4, transpose=True, residual=None, out=None,
               workspace=None):
    """out = x . dequant(w)^T (+ residual after rounding).  x [M, K], w [N, Kw].
    workspace: optional (affine_qmm_workspace): lets 5..16-row products split K."""
    M, K = x.shape
    N = w.shape[0]
    _req(x, "x", _BF)
    _req_matrix((w, scales, biases), "w", N, K, bits, group_size)
    _req(residual, "residual", _BF, (M, N))
    _dev(x, w, scales, biases, residual)
    _req(workspace, "workspace", (torch.uint8,))
    _dev(workspace)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    wsb = 0 if workspace is None else workspace.numel()
    st = lib().moegq_affine_qmm_ws(_ptr(x), _dt(x), M, K, _ptr(w), _wdt(w), _ptr(scales), _ptr(biases), N,
                                   int(bool(transpose)), group_size, bits, _ptr(residual), _ptr(out),
                                   _ptr(workspace), wsb, _stream())
    _check(st, "affine_qmm")
    return out


def affine_qmm_glu(x, gate, up, group_size=64, bits=4, out=None, workspace=None):
    """bf16(silu(x . Wg^T) * (x . Wu^T)); gate/up are (words, scales, biases).
    workspace: optional (affine_qmm_workspace(..., glu=True))."""
    M, K = x.shape
    N = gate[0].shape[0]
    _req(x, "x", _BF)
    _req_matrix(gate, "gate", N, K, bits, group_size)
    _req_matrix(up, "up", N, K, bits, group_size)
    _dev(x, *gate, *up)
    _req(workspace, "workspace", (torch.uint8,))
    _dev(workspace)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    wsb = 0 if workspace is None else workspace.numel()
    st = lib().moegq_affine_qmm_glu_ws(_ptr(x), M, K, *[_ptr(t) for t in gate], *[_ptr(t) for t in up], N,
                                       group_size, bits, _ptr(out), _ptr(workspace), wsb, _stream())
    _check(st, "affine_qmm_glu")
    return out


def switch_glu_mode(T: int, top_k: int, E: int) -> int:
    return int(lib().moegq_switch_glu_mode(T, top_k, E))


def switch_glu(x, idx, gate, up, down, group_size=64, bits=4, mode=MODE_AUTO, tile_mode=TILES_SCHEDULED,
               bm=0, y=None, inv=None):
    """Routed SwitchGLU.  Returns (y [T*top_k, H], inv [T*top_k] or None, mode used).
    DECODE: y in token order; SORTED: y expert-sorted and inv the inverse permutation."""
    T, H = x.shape
    top_k = idx.shape[1]
    E, I = gate[0].shape[0], gate[0].shape[1]
    _req(x, "x", _BF)
    _req(idx, "idx", _IDX, (T, top_k))
    _req_experts(gate, up, down, E, H, I, bits, group_size)
    _req(y, "y", _BF, (T * top_k, H))
    _req(inv, "inv", _IDX, (T * top_k,))
    _dev(x, idx, *gate, *up, *down, y, inv)
    P = T * top_k
    if mode == MODE_AUTO:
        mode = switch_glu_mode(T, top_k, E)
    if y is None:
        y = torch.empty((P, H), dtype=torch.bfloat16, device=x.device)
    if inv is None and mode == MODE_SORTED:
        inv = torch.empty(P, dtype=torch.int32, device=x.device)
    op = OP_SWITCH_GLU_SORTED if mode == MODE_SORTED else OP_SWITCH_GLU_DECODE
    ws, wsb = _workspace(workspace_bytes(op, P, E, I, bm), x.device)
    st = lib().moegq_switch_glu(_ptr(x), T, H, I, E, _ptr(idx), top_k, *[_ptr(t) for t in gate],
                                *[_ptr(t) for t in up], *[_ptr(t) for t in down], group_size, bits, mode,
                                tile_mode, bm, _ptr(y), _ptr(inv), _ptr(ws), wsb, _stream())
    _check(st, "switch_glu")
    return y, inv, mode


def moe_decode(x, idx, scores, gate, up, down, shared=None, group_size=64, bits=4, out=None, y=None,
               workspace=None):
    """Routed MoE decode layer in two kernels: gate/up + SiLU, then down fused
    with the combine tail.  Returns out [T, H] (y [T*top_k, H] filled if given)."""
    T, H = x.shape
    top_k = idx.shape[1]
    E, I = gate[0].shape[0], gate[0].shape[1]
    _req(x, "x", _BF)
    _req(idx, "idx", _IDX, (T, top_k))
    _req(scores, "scores", _BF, (T, top_k))
    _req(shared, "shared", _BF, (T, H))
    _req(y, "y", _BF, (T * top_k, H))
    _req(out, "out", _BF, (T, H))
    _req_experts(gate, up, down, E, H, I, bits, group_size)
    _dev(x, idx, scores, shared, *gate, *up, *down, y, out, workspace)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        ws, wsb = _workspace(workspace_bytes(OP_MOE_DECODE, T * top_k, E, I, 0), x.device)
    else:
        ws, wsb = workspace, workspace.numel()
    st = lib().moegq_moe_decode(_ptr(x), T, H, I, E, _ptr(idx), top_k, _ptr(scores), _ptr(shared),
                                *[_ptr(t) for t in gate], *[_ptr(t) for t in up], *[_ptr(t) for t in down],
                                group_size, bits, _ptr(out), _ptr(y), _ptr(ws), wsb, _stream())
    _check(st, "moe_decode")
    return out


def moe_decode_static(x, idx, scores, gate, up, down, shared=None, group_size=64, bits=4, out=None, y=None):
    """moe_decode without a workspace: the intermediate lives in the library's
    static per-GPU scratch (moegq_static_scratch_bytes() bytes); calls that
    overlap on one GPU race.  Returns out [T, H]."""
    T, H = x.shape
    top_k = idx.shape[1]
    E, I = gate[0].shape[0], gate[0].shape[1]
    _req(x, "x", _BF)
    _req(idx, "idx", _IDX, (T, top_k))
    _req(scores, "scores", _BF, (T, top_k))
    _req(shared, "shared", _BF, (T, H))
    _req(y, "y", _BF, (T * top_k, H))
    _req(out, "out", _BF, (T, H))
    _req_experts(gate, up, down, E, H, I, bits, group_size)
    _dev(x, idx, scores, shared, *gate, *up, *down, y, out)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    st = lib().moegq_moe_decode_static(_ptr(x), T, H, I, E, _ptr(idx), top_k, _ptr(scores), _ptr(shared),
                                       *[_ptr(t) for t in gate], *[_ptr(t) for t in up], *[_ptr(t) for t in down],
                                       group_size, bits, _ptr(out), _ptr(y), _stream())
    _check(st, "moe_decode_static")
    return out


def static_scratch_bytes() -> int:
    return int(lib().moegq_static_scratch_bytes())


def moe_prefill_workspace_bytes(T: int, top_k: int, E: int, H: int, I: int, has_shared: bool = True) -> int:
    return int(lib().moegq_moe_prefill_workspace_bytes(T, top_k, E, H, I, int(has_shared)))


ERR_SELFCHECK = -9
_CHECKED_DEVICES = set()


def _ensure_selfcheck(device):
    """Run the fused-vs-unfused combine self-check once per device before the
    first combine on it (it synchronizes, so never while a HIP graph is being
    captured).  MOEGQ_SELFCHECK=0 in the environment skips it."""
    dev = torch.device(device)
    key = dev.index if dev.index is not None else torch.cuda.current_device()
    if key in _CHECKED_DEVICES or os.environ.get("MOEGQ_SELFCHECK", "1") == "0":
        return
    if torch.cuda.is_current_stream_capturing():
        return
    _CHECKED_DEVICES.add(key)
    with torch.cuda.device(key):
        selfcheck(dev)


def probe_stream_read(buf, blocks: int, sink=None):
    """Diagnostic: one streaming read of every byte of the device tensor buf."""
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    _check(lib().moegq_probe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), blocks,
                                         _stream()), "probe_stream_read")
    return sink


def probe_mfma_bf16(iters: int, blocks: int, out) -> int:
    """Diagnostic: bf16 MFMA loop; returns the flops it performs."""
    _check(lib().moegq_probe_mfma_bf16(iters, blocks, _ptr(out), _stream()), "probe_mfma_bf16")
    return blocks * 4 * iters * 8 * 16384


def selfcheck_state() -> int:
    """The current device's last self-check result: 0 not run, 1 passed, 2 failed."""
    return int(lib().moegq_selfcheck_state())


def moe_prefill_layout(T: int, top_k: int, E: int, H: int, I: int, has_shared: bool = True) -> dict:
    """Byte offsets of moe_prefill's sort results and tile tables inside its
    workspace, the tables' capacities and the schedule parameters used on
    the current device (host query, no launch)."""
    off = (ctypes.c_int64 * 9)()
    caps = (ctypes.c_int64 * 2)()
    par = (ctypes.c_int32 * 4)()
    _check(lib().moegq_moe_prefill_layout(T, top_k, E, H, I, int(bool(has_shared)), off, caps, par),
           "moe_prefill_layout")
    names = ("inv", "lhs", "sorted_rhs", "counts", "offsets", "tiles", "small_tiles", "n_tiles", "tail")
    return dict(offsets=dict(zip(names, list(off))), caps=(caps[0], caps[1]), big=par[0], small=par[1],
                slots=par[2], col_blocks=par[3])


def moe_prefill_tables(workspace, T: int, top_k: int, E: int, H: int, I: int, has_shared: bool = True) -> dict:
    """Views into a moe_prefill workspace (uint8 device tensor) after a call:
    inv, lhs, sorted_rhs, counts, offsets, and the two tile tables cut to
    their counts (each tile = (row start, expert, valid rows))."""
    L = moe_prefill_layout(T, top_k, E, H, I, has_shared)
    o = L["offsets"]
    P = T * top_k
    extra = T if has_shared else 0

    def view(name, n):
        return workspace[o[name]:o[name] + 4 * n].view(torch.int32)

    n = view("n_tiles", 2).cpu()
    big = view("tiles", 3 * L["caps"][0]).view(-1, 3)[:int(n[0])]
    small = view("small_tiles", 3 * L["caps"][1]).view(-1, 3)[:int(n[1])]
    return dict(inv=view("inv", P), lhs=view("lhs", P + extra), sorted_rhs=view("sorted_rhs", P),
                counts=view("counts", E), offsets=view("offsets", E + 1), tiles=big, small_tiles=small,
                layout=L)


def moe_prefill(x, idx, scores, gate, up, down, shared=None, group_size=64, bits=4, out=None, workspace=None):
    """One MoE layer on the expert-sorted route: sort, routed SwitchGLU with the
    gated shared expert riding along, one-pass combine.  shared: None or
    (gate, up, down, gate_row), each a (words, scales, biases) triple.
    Returns out [T, H]."""
    T, H = x.shape
    top_k = idx.shape[1]
    E, I = gate[0].shape[0], gate[0].shape[1]
    _req(x, "x", _BF)
    _req(idx, "idx", _IDX, (T, top_k))
    _req(scores, "scores", _BF, (T, top_k))
    _req(out, "out", _BF, (T, H))
    _req_experts(gate, up, down, E, H, I, bits, group_size)
    _dev(x, idx, scores, *gate, *up, *down, out, workspace)
    sh = [None] * 12
    if shared is not None:
        if len(shared) != 4:
            raise ValueError("shared: (gate, up, down, gate_row) triples")
        Is = shared[0][0].shape[0]
        _req_matrix(shared[0], "shared gate", Is, H, bits, group_size)
        _req_matrix(shared[1], "shared up", Is, H, bits, group_size)
        _req_matrix(shared[2], "shared down", H, Is, bits, group_size)
        _req_matrix(shared[3], "shared gate row", 1, H, bits, group_size)
        sh = [t for trip in shared for t in trip]
        _dev(*sh)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _ensure_selfcheck(x.device)
    if workspace is None:
        ws, wsb = _workspace(moe_prefill_workspace_bytes(T, top_k, E, H, I, shared is not None), x.device)
    else:
        ws, wsb = workspace, workspace.numel()
    st = lib().moegq_moe_prefill(_ptr(x), T, H, I, E, _ptr(idx), top_k, _ptr(scores),
                                 *[_ptr(t) for t in gate], *[_ptr(t) for t in up], *[_ptr(t) for t in down],
                                 *[_ptr(t) for t in sh], group_size, bits, _ptr(out), _ptr(ws), wsb, _stream())
    _check(st, "moe_prefill")
    return out


def moe_combine(y, inv, scores, shared=None, out=None):
    """Fused unsort * score, sum over top_k, + shared (one pass)."""
    T, top_k = scores.shape
    H = y.shape[-1]
    _req_combine(y, inv, scores, shared, out)
    _dev(y, inv, scores, shared, out)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _ensure_selfcheck(y.device)
    st = lib().moegq_moe_combine(_ptr(y), _ptr(inv), _ptr(scores), _ptr(shared), T, top_k, H, _ptr(out),
                                 _stream())
    if st == ERR_SELFCHECK:          # the one-pass combine is off on this device: the unfused tail
        return moe_combine_unfused(y, inv, scores, shared, out=out)
    _check(st, "moe_combine")
    return out


def moe_combine_gated(y, inv, scores, shared, z, out=None):
    """moe_combine with the shared expert's sigmoid gate applied in the same pass."""
    T, top_k = scores.shape
    H = y.shape[-1]
    _req_combine(y, inv, scores, shared, out)
    if shared is None or z is None:
        raise ValueError("moe_combine_gated: shared and z are required")
    _req(z, "z", _BF)
    if z.numel() != T:
        raise ValueError(f"z: {z.numel()} values, expected {T}")
    _dev(y, inv, scores, shared, z, out)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _ensure_selfcheck(y.device)
    st = lib().moegq_moe_combine_gated(_ptr(y), _ptr(inv), _ptr(scores), _ptr(shared), _ptr(z), T, top_k, H,
                                       _ptr(out), _stream())
    if st == ERR_SELFCHECK:          # the one-pass combine is off on this device: gate, then the unfused tail
        return moe_combine_unfused(y, inv, scores, sigmoid_gate(shared, z), out=out)
    _check(st, "moe_combine_gated")
    return out


def moe_combine_unfused(y, inv, scores, shared=None, out=None, workspace=None):
    """The same tail as four kernels, each writing a bf16 tensor.  workspace:
    optional uint8 device tensor of workspace_bytes(OP_COMBINE_UNFUSED, ...) bytes."""
    T, top_k = scores.shape
    H = y.shape[-1]
    _req_combine(y, inv, scores, shared, out)
    _dev(y, inv, scores, shared, workspace, out)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    need = workspace_bytes(OP_COMBINE_UNFUSED, T * top_k, 0, H, 0)
    if workspace is not None and workspace.numel() >= need:
        ws, wsb = workspace, int(workspace.numel())
    else:
        ws, wsb = _workspace(need, y.device)
    st = lib().moegq_moe_combine_unfused(_ptr(y), _ptr(inv), _ptr(scores), _ptr(shared), T, top_k, H, _ptr(out),
                                         _ptr(ws), wsb, _stream())
    _check(st, "moe_combine_unfused")
    return out


def sort_pairs(idx, E: int):
    """(order, lhs, sorted_rhs, inv, counts, offsets), all int32 device tensors."""
    _req(idx, "idx", _IDX)
    _dev(idx)
    T, top_k = idx.shape
    P = T * top_k
    mk = lambda n: torch.empty(n, dtype=torch.int32, device=idx.device)
    order, lhs, srhs, inv, counts, offsets = mk(P), mk(P), mk(P), mk(P), mk(E), mk(E + 1)
    ws, wsb = _workspace(workspace_bytes(OP_SORT_PAIRS, P, E, 0, 0), idx.device)
    st = lib().moegq_sort_pairs(_ptr(idx), _dt(idx), T, top_k, E, _ptr(order), _ptr(lhs), _ptr(srhs), _ptr(inv),
                                _ptr(counts), _ptr(offsets), _ptr(ws), wsb, _stream())
    _check(st, "sort_pairs")
    return order, lhs, srhs, inv, counts, offsets


def schedule_tiles(offsets, E: int, P_max: int, bm: int, tile_mode=TILES_SCHEDULED):
    """(tiles [cap, 3], n_tiles [1]) device int32."""
    _req(offsets, "offsets", _IDX, (E + 1,))
    _dev(offsets)
    cap = (P_max + bm - 1) // bm + min(E, P_max)
    tiles = torch.full((max(cap, 1), 3), -7, dtype=torch.int32, device=offsets.device)
    n = torch.zeros(1, dtype=torch.int32, device=offsets.device)
    st = lib().moegq_schedule_tiles(_ptr(offsets), E, P_max, bm, tile_mode, _ptr(tiles), cap, _ptr(n), _stream())
    _check(st, "schedule_tiles")
    return tiles, n


def route(logits, top_k, idx=None, scores=None):
    """Router: fp32 logits [T, E] -> (idx int32 [T, top_k], scores bf16 [T, top_k]);
    top_k by logit (ties to the lower id) in ascending id, float64 softmax scores."""
    _dev(logits)
    if logits.dtype != torch.float32:
        raise MoegqError(-5, "route: logits must be float32")
    T, E = logits.shape
    logits = logits.contiguous()
    if idx is None:
        idx = torch.empty((T, top_k), dtype=torch.int32, device=logits.device)
    if scores is None:
        scores = torch.empty((T, top_k), dtype=torch.bfloat16, device=logits.device)
    _check(lib().moegq_route(_ptr(logits), T, E, top_k, _ptr(idx), _ptr(scores), _stream()), "route")
    return idx, scores


def rms_norm(x, w, eps=1e-6, out=None):
    M, K = x.shape
    _req(x, "x", _BF)
    _req(w, "w", _BF, (K,))
    _req(out, "out", _BF, (M, K))
    _dev(x, w, out)
    if out is None:
        out = torch.empty_like(x)
    _check(lib().moegq_rms_norm(_ptr(x), _ptr(w), M, K, eps, _ptr(out), _stream()), "rms_norm")
    return out


def sigmoid_gate(s, z, out=None):
    """bf16(sigmoid(z[t]) * s[t, :]); z [T, 1] or [T]."""
    T, H = s.shape
    _req(s, "s", _BF)
    _req(z, "z", _BF)
    if z.shape[0] != T:
        raise ValueError(f"z: {z.shape[0]} rows, expected {T}")
    _dev(s, out)
    zs = z.stride(0) if z.dim() >= 1 else 1
    if out is None:
        out = torch.empty_like(s)
    _check(lib().moegq_sigmoid_gate(_ptr(s), _ptr(z), zs, T, H, _ptr(out), _stream()), "sigmoid_gate")
    return out


def kv_feed(q, k, v, out=None):
    """bf16(q + bf16(k[:, :1] + v[:, :1]))."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _req(t, n, _BF)
    M, Nq = q.shape
    if k.shape[0] != M or v.shape[0] != M:
        raise ValueError("q, k and v must have the same rows")
    _dev(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    _check(lib().moegq_kv_feed(_ptr(q), _ptr(k), _ptr(v), M, Nq, k.shape[1], v.shape[1], _ptr(out), _stream()),
           "kv_feed")
    return out


def kv_feed_stacked(qkv, nq, nk, nv, out=None):
    """kv_feed on one stacked product qkv [M, nq + nk + nv] (q, k, v as its
    column ranges): bf16(q + bf16(k[:, :1] + v[:, :1]))."""
    _req(qkv, "qkv", _BF)
    _dev(qkv)
    M, L = qkv.shape
    if L != nq + nk + nv:
        raise ValueError("stacked width must be nq + nk + nv")
    if out is None:
        out = torch.empty((M, nq), dtype=qkv.dtype, device=qkv.device)
    base = qkv.data_ptr()
    es = qkv.element_size()
    _check(lib().moegq_kv_feed_ld(ctypes.c_void_p(base), L, ctypes.c_void_p(base + nq * es), L,
                                  ctypes.c_void_p(base + (nq + nk) * es), L, M, nq, _ptr(out), _stream()),
           "kv_feed_stacked")
    return out


def selfcheck(device="cuda") -> int:
    """Fused vs unfused combine, bit for bit (synchronizes).  Returns the status."""
    ws, wsb = _workspace(workspace_bytes(OP_SELFCHECK, 0, 0, 0, 0), device)
    return int(lib().moegq_selfcheck(_ptr(ws), wsb, _stream()))


def validate_indices(idx, E: int, sorted_=False) -> int:
    _dev(idx)
    flag = torch.zeros(1, dtype=torch.int32, device=idx.device)
    return int(lib().moegq_validate_indices(_ptr(idx), idx.numel(), E, int(sorted_), _ptr(flag), _stream()))
