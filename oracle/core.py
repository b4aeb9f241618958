"""Plain, slow, obviously-correct CPU definitions of the gathered affine-quantized
MoE expert path.  TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline
timing); never imported by the product path.

Conventions
-----------
* bf16 tensors travel as ``numpy.uint16`` bit patterns (numpy has no bf16).
* Floating-point arithmetic is float64 unless a step of the method fixes a
  narrower precision (the combine, which is defined on fp32 intermediates).
* Packed weights are ``numpy.uint32`` words.

Readings of points the pages leave open are marked ``READING:``; each is also
listed with its justification in the design notes of the repository.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "SUPPORTED_BITS", "SUPPORTED_GROUPS",
    "bf16_to_f64", "bf16_to_f32", "f64_to_bf16",
    "activations_f64", "promoted_type", "round_to",
    "MX_MODES", "MX_BLOCK", "e2m1_to_f64", "e4m3_to_f64", "e8m0_to_f64", "mx_dequant", "mx_matmul", "gather_qmm_mx",
    "unpack", "dequant", "quantized_matmul", "gather_qmm", "broadcast_gather_indices",
    "silu", "switch_glu", "sort_pairs", "schedule_tiles", "naive_tiles", "hybrid_tiles",
    "combine", "unsort", "shared_expert", "rms_norm", "moe_prefill_layer",
    "dense_forward", "validate_quant_args", "route", "gather_mm", "switch_glu_mm",
]

# [nuvec] "round_trip_error_is_about_half_a_step": bit widths 1..6 and 8, group
# sizes 32/64/128 are the supported grid of the format.
SUPPORTED_BITS = (1, 2, 3, 4, 5, 6, 8)
SUPPORTED_GROUPS = (32, 64, 128)


# ----------------------------------------------------------------------------
# bf16 helpers
# ----------------------------------------------------------------------------
def bf16_to_f64(u16) -> np.ndarray:
    """bf16 bit pattern -> value.  A bf16 is the upper half of an IEEE fp32."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_to_f32(u16) -> np.ndarray:
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def f64_to_bf16(x) -> np.ndarray:
    """Round a float64 (or float32) value to the nearest bf16, ties to even.

    Done directly on the value (no intermediate fp32 rounding): a bf16 has 8
    significant bits, so inside the binade [2^(e-1), 2^e) the representable
    values are the multiples of 2^(e-8); below the smallest normal (2^-126) the
    spacing stays at the smallest subnormal, 2^-133.  ``numpy.round`` rounds
    halves to even.  Magnitudes that round to 2^128 or more become infinity;
    NaN becomes the quiet NaN 0x7FC0.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    finite_nz = np.isfinite(x) & (ax > 0)
    _, e = np.frexp(np.where(finite_nz, ax, 1.0))
    quantum = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = np.where(finite_nz, np.round(ax / quantum) * quantum, ax)
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    signed = np.copysign(r, x).astype(np.float32)
    bits = (signed.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits).astype(np.uint16)
    return bits


# ----------------------------------------------------------------------------
# Argument checks: the error catalogue of the format
# ----------------------------------------------------------------------------
def validate_quant_args(K: int, gs: int, bits: int, packed_cols: int | None = None,
                        n_groups: int | None = None) -> None:
    """Raise ValueError for the arguments the format rejects.

    [nuvec] "invalid_arguments_are_rejected": group size 48 and bit width 7 are
    rejected, the quantized axis must be divisible by the group size, and a
    group size that disagrees with the packed shape is an error.
    """
    if gs not in SUPPORTED_GROUPS:
        raise ValueError(f"group size {gs} not in {SUPPORTED_GROUPS}")
    if bits not in SUPPORTED_BITS:
        raise ValueError(f"bits {bits} not in {SUPPORTED_BITS}")
    if K % gs:
        raise ValueError(f"quantized axis {K} not divisible by group size {gs}")
    if (K * bits) % 32:
        raise ValueError(f"quantized axis {K} x {bits} bits is not a whole number of words")
    if packed_cols is not None and packed_cols * 32 != K * bits:
        raise ValueError(f"packed width {packed_cols} words does not hold {K} codes of {bits} bits")
    if n_groups is not None and n_groups * gs != K:
        raise ValueError(f"{n_groups} groups of {gs} do not cover {K}")


# ----------------------------------------------------------------------------
# Unpack and dequantize
# ----------------------------------------------------------------------------
def unpack(words, K: int, bits: int) -> np.ndarray:
    """Codes of a packed row: code k occupies bits [k*bits, (k+1)*bits) of the
    row read as one little-endian bit stream of 32-bit words.

    READING: the pages fix the packed shape (cols*bits/32 words per row,
    [nuvec] round-trip test) but not the order inside a word; codes are taken
    LSB-first.  A code that straddles two words (3, 5, 6 bits) takes its high
    bits from the next word.
    """
    w = np.asarray(words, dtype=np.uint32)
    if w.shape[-1] * 32 < K * bits:
        raise ValueError("packed row too short")
    k = np.arange(K, dtype=np.int64)
    pos = k * bits
    lo = w[..., pos // 32].astype(np.uint64)
    nxt = np.minimum(pos // 32 + 1, w.shape[-1] - 1)
    hi = np.where((pos // 32 + 1) < w.shape[-1], w[..., nxt].astype(np.uint64), np.uint64(0))
    stream = lo | (hi << np.uint64(32))
    mask = np.uint64((1 << bits) - 1)
    return ((stream >> (pos % 32).astype(np.uint64)) & mask).astype(np.int64)


def dequant(words, scales, biases, gs: int, bits: int, length: int) -> np.ndarray:
    """Affine dequantization along the packed (last) axis: w = q*scale + bias,
    one scale and one bias per group of ``gs`` consecutive codes.

    [nuvec] "composed": codes times the group scale plus the group bias.
    Evaluated exactly in float64 (q*s has at most 16 significant bits and the
    sum with a bf16 bias is exact), so it equals fp32 fused multiply-add of the
    same operands before its final rounding.
    """
    validate_quant_args(length, gs, bits, np.asarray(words).shape[-1], np.asarray(scales).shape[-1])
    q = unpack(words, length, bits).astype(np.float64)
    s = bf16_to_f64(scales)
    b = bf16_to_f64(biases)
    g = np.arange(length) // gs
    return q * s[..., g] + b[..., g]


# ----------------------------------------------------------------------------
# quantized_matmul and gather_qmm
# ----------------------------------------------------------------------------
def activations_f64(x):
    """Activation values in float64 and their type: bf16 bit patterns
    (``numpy.uint16``), or ``numpy.float16`` / ``numpy.float32`` arrays.  Each
    conversion is exact."""
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return bf16_to_f64(a), "bf16"
    if a.dtype == np.float16:
        return a.astype(np.float64), "f16"
    if a.dtype == np.float32:
        return a.astype(np.float64), "f32"
    raise ValueError("activations must be bf16 bit patterns, float16 or float32")


def promoted_type(x_type: str) -> str:
    """Result type of a product of activations of ``x_type`` with bf16 scales.

    [nuvec] "reference": the product is computed in the type that the
    activation and scale types promote to; the batched case there checks that
    half precision promotes.  bf16 with bf16 stays bf16; float16 with bf16 has
    no common 16-bit type and becomes float32; float32 stays float32.
    """
    if x_type not in ("bf16", "f16", "f32"):
        raise ValueError(x_type)
    return "bf16" if x_type == "bf16" else "f32"


def round_to(y, t: str) -> np.ndarray:
    """Round float64 results once to type ``t`` (bf16 bit patterns or float32)."""
    return f64_to_bf16(y) if t == "bf16" else np.asarray(y, dtype=np.float64).astype(np.float32)


def quantized_matmul(x, words, scales, biases, transpose: bool = True, gs: int = 64,
                     bits: int = 4) -> np.ndarray:
    """out = x . dequant(W)^T  (transpose=True, W is [N, K*bits/32], groups run
    along K), or out = x . dequant(W) (transpose=False, W is [K, N*bits/32],
    groups run along N).  Leading batch axes broadcast.

    [nuvec] "reference" and "quantized_matmul_equals_the_dequantized_product":
    the product of x with the dequantized weights.  The sum over K is formed in
    float64 and rounded once to the promoted type (``promoted_type``): bf16 bit
    patterns for bf16 activations, float32 for float16 and float32 ones.
    """
    xf, xt = activations_f64(x)
    w = np.asarray(words)
    if transpose:
        K = xf.shape[-1]
        W = dequant(w, scales, biases, gs, bits, K)           # [..., N, K]
        y = np.matmul(xf, np.swapaxes(W, -1, -2))
    else:
        N = w.shape[-1] * 32 // bits
        W = dequant(w, scales, biases, gs, bits, N)           # [..., K, N]
        if W.shape[-2] != xf.shape[-1]:
            raise ValueError("inner sizes differ")
        y = np.matmul(xf, W)
    return round_to(y, promoted_type(xt))


# ----------------------------------------------------------------------------
# microscaling (mx) formats
# ----------------------------------------------------------------------------
# [MLX#4787] benchmark script: besides the affine modes, quantize() and
# quantized_matmul() take mode="mxfp8" and mode="mxfp4", and those modes
# return no biases.  READING: the pages name the modes but not their encoding;
# the encoding taken is the OCP Microscaling (MX) one: blocks of 32 elements
# along the packed axis share one E8M0 scale (a power of two, one byte), and
# the elements are E4M3 (mxfp8) or E2M1 (mxfp4) floats, packed LSB-first into
# 32-bit words like the affine codes (8 per word for mxfp4, 4 for mxfp8).
MX_MODES = {"mxfp4": 4, "mxfp8": 8}     # element bits
MX_BLOCK = 32


def e2m1_to_f64(codes) -> np.ndarray:
    """E2M1 element: sign bit 3, exponent bits 2-1 (bias 1), mantissa bit 0;
    exponent 0 is subnormal (mantissa * 0.5).  No infinities or NaN."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int32)))
    return sign * mag


def e4m3_to_f64(codes) -> np.ndarray:
    """E4M3 element: sign bit 7, exponent bits 6-3 (bias 7), mantissa bits
    2-0; exponent 0 is subnormal (mantissa/8 * 2^-6); exponent and mantissa
    all ones is NaN; no infinities."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32)))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e8m0_to_f64(e) -> np.ndarray:
    """E8M0 scale: 2^(e - 127); e = 255 is NaN."""
    e = np.asarray(e, dtype=np.int64)
    return np.where(e == 255, np.nan, np.ldexp(1.0, (e - 127).astype(np.int32)))


def mx_dequant(words, scales_u8, mode: str, length: int) -> np.ndarray:
    """Elements times their block's scale along the packed (last) axis."""
    if mode not in MX_MODES:
        raise ValueError("mode must be mxfp4 or mxfp8")
    if length % MX_BLOCK:
        raise ValueError("length must be a multiple of 32")
    bits = MX_MODES[mode]
    q = unpack(words, length, bits)
    v = e2m1_to_f64(q) if mode == "mxfp4" else e4m3_to_f64(q)
    sc = e8m0_to_f64(np.asarray(scales_u8, dtype=np.uint8))
    if sc.shape[-1] * MX_BLOCK != length:
        raise ValueError("scales do not match the packed length")
    return v * sc[..., np.arange(length) // MX_BLOCK]


def mx_matmul(x, words, scales_u8, mode: str, transpose: bool = True) -> np.ndarray:
    """x . dequant(W)^T (transpose=True, W [N, K*bits/32], blocks along K) or
    x . dequant(W) (W [K, N*bits/32], blocks along N) for an mx mode; float64
    sum rounded once to the promoted type (bf16 activations give bf16,
    float16/float32 give float32, as for the affine modes)."""
    xf, xt = activations_f64(x)
    w = np.asarray(words)
    if transpose:
        W = mx_dequant(w, scales_u8, mode, xf.shape[-1])
        y = np.matmul(xf, np.swapaxes(W, -1, -2))
    else:
        N = w.shape[-1] * 32 // MX_MODES[mode]
        W = mx_dequant(w, scales_u8, mode, N)
        if W.shape[-2] != xf.shape[-1]:
            raise ValueError("inner sizes differ")
        y = np.matmul(xf, W)
    return round_to(y, promoted_type(xt))


def gather_qmm_mx(x, words, scales_u8, lhs=None, rhs=None, transpose: bool = True, mode: str = "mxfp8"):
    """gather_qmm for an mx mode: out[j] = x[lhs[j]] . dequant(W[rhs[j]])^T."""
    x = np.asarray(x)
    _, xt = activations_f64(x[..., :0])
    w = np.asarray(words, dtype=np.uint32)
    sc = np.asarray(scales_u8, dtype=np.uint8)
    li, ri, shape = broadcast_gather_indices(x.shape[:-2], w.shape[:-2], lhs, rhs)
    M = x.shape[-2]
    xf = x.reshape((-1,) + x.shape[-2:])
    wf = w.reshape((-1,) + w.shape[-2:])
    sf = sc.reshape((-1,) + sc.shape[-2:])
    N = w.shape[-2] if transpose else w.shape[-1] * 32 // MX_MODES[mode]
    out = np.zeros((len(li), M, N), dtype=np.uint16 if promoted_type(xt) == "bf16" else np.float32)
    for j, (l, r) in enumerate(zip(li, ri)):
        out[j] = mx_matmul(xf[l], wf[r], sf[r], mode, transpose)
    return out.reshape(tuple(shape) + (M, N))


def broadcast_gather_indices(x_batch: tuple, w_batch: tuple, lhs=None, rhs=None):
    """Flattened (lhs, rhs) batch indices and the output batch shape.

    [nuvec] "gather_qmm_selects_batches": lhs indexes x's batch, rhs indexes the
    weights' batch; when absent they default to every batch in order, and the
    two broadcast together to the output batch shape.  Float indices and
    index shapes that do not broadcast are errors.
    """
    nx = int(np.prod(x_batch)) if len(x_batch) else 1
    nw = int(np.prod(w_batch)) if len(w_batch) else 1
    if lhs is None:
        lhs = np.arange(nx).reshape(x_batch)
    if rhs is None:
        rhs = np.arange(nw).reshape(w_batch)
    lhs = np.asarray(lhs)
    rhs = np.asarray(rhs)
    for a in (lhs, rhs):
        if not np.issubdtype(a.dtype, np.integer):
            raise ValueError("indices must be integers")
    try:
        shape = np.broadcast_shapes(lhs.shape, rhs.shape)
    except ValueError as exc:
        raise ValueError("index shapes do not broadcast") from exc
    return np.broadcast_to(lhs, shape).reshape(-1), np.broadcast_to(rhs, shape).reshape(-1), shape


def gather_qmm(x, words, scales, biases, lhs=None, rhs=None, transpose: bool = True,
               gs: int = 64, bits: int = 4) -> np.ndarray:
    """out[j] = x[lhs[j]] . dequant(W[rhs[j]])^T for every j of the broadcast
    index shape; output shape = index shape + [M, N].

    [MLX#4509] gq(): gather_qmm(x, w, s, b, rhs_indices=idx, transpose=True,
    group_size, bits).  [nuvec] "gather_qmm_selects_batches": each output batch
    equals quantized_matmul of the selected x batch and weight batch.
    """
    x = np.asarray(x)
    _, xt = activations_f64(x[..., :0])
    w = np.asarray(words, dtype=np.uint32)
    s = np.asarray(scales, dtype=np.uint16)
    b = np.asarray(biases, dtype=np.uint16)
    xb, wb = x.shape[:-2], w.shape[:-2]
    li, ri, shape = broadcast_gather_indices(xb, wb, lhs, rhs)
    M = x.shape[-2]
    xf = x.reshape((-1,) + x.shape[-2:])
    wf = w.reshape((-1,) + w.shape[-2:])
    sf = s.reshape((-1,) + s.shape[-2:])
    bf = b.reshape((-1,) + b.shape[-2:])
    if transpose:
        N = w.shape[-2]
    else:
        N = w.shape[-1] * 32 // bits
    out = np.zeros((len(li), M, N), dtype=np.uint16 if promoted_type(xt) == "bf16" else np.float32)
    for j, (l, r) in enumerate(zip(li, ri)):
        out[j] = quantized_matmul(xf[l], wf[r], sf[r], bf[r], transpose, gs, bits)
    return out.reshape(tuple(shape) + (M, N))


# ----------------------------------------------------------------------------
# SwitchGLU (decode and prefill expert chain)
# ----------------------------------------------------------------------------
def silu(g: np.ndarray) -> np.ndarray:
    """silu(g) = g * sigmoid(g) = g / (1 + exp(-g)), float64."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def switch_glu(x, idx, gate, up, down, gs: int = 64, bits: int = 4) -> np.ndarray:
    """y[t, k] = down_e( silu(gate_e(x_t)) * up_e(x_t) ), e = idx[t, k].

    [MLX#4509] moe(): the SwitchGLU order "up, gate, silu(gate)*up, down" over
    gathered experts.  Written as an expert loop: every active expert is
    dequantized once and applied to all the (token, slot) pairs routed to it.

    gate/up: (words [E, I, H*bits/32], scales [E, I, H/gs], biases [E, I, H/gs]);
    down: (words [E, H, I*bits/32], scales [E, H, I/gs], biases [E, H, I/gs]).
    x: [T, H] bf16, idx: [T, top_k] int.  Returns [T, top_k, H] bf16.

    READING: u and g are rounded to bf16 (each is a materialized bf16 tensor
    in the page's chain); h = bf16(g * sigmoid(g) * u) is formed in float64
    from those and rounded once.
    """
    x = np.asarray(x, dtype=np.uint16)
    idx = np.asarray(idx)
    T, H = x.shape
    top_k = idx.shape[1]
    y = np.zeros((T, top_k, H), dtype=np.uint16)
    xf = bf16_to_f64(x)
    for e in np.unique(idx):
        tt, kk = np.nonzero(idx == e)
        xe = xf[tt]
        Wg = dequant(gate[0][e], gate[1][e], gate[2][e], gs, bits, H)
        Wu = dequant(up[0][e], up[1][e], up[2][e], gs, bits, H)
        u = bf16_to_f64(f64_to_bf16(xe @ Wu.T))
        g = bf16_to_f64(f64_to_bf16(xe @ Wg.T))
        h = bf16_to_f64(f64_to_bf16(silu(g) * u))
        I = h.shape[1]
        Wd = dequant(down[0][e], down[1][e], down[2][e], gs, bits, I)
        y[tt, kk] = f64_to_bf16(h @ Wd.T)
    return y


# ----------------------------------------------------------------------------
# Expert sort, offsets, inverse permutation
# ----------------------------------------------------------------------------
def sort_pairs(idx, E: int):
    """Sort the flattened (token, slot) pairs by expert.

    [MTPLX#558] Change: the stock sorted chain sorts the pairs by expert, runs
    the experts on the sorted rows and un-sorts with the inverse permutation.
    [MLX#4567] Proposed changes: per-expert offsets precomputed from
    rhs_indices.

    Returns order[P] (sorted position -> flat pair p = t*top_k + k),
    lhs[P] = order // top_k (the token of each sorted row), sorted_rhs[P],
    inv[P] (pair -> sorted position), counts[E], offsets[E+1] (exclusive prefix).

    READING: ties (pairs of the same expert) keep flat pair order (stable sort).
    """
    idx = np.asarray(idx)
    top_k = idx.shape[1]
    f = idx.reshape(-1).astype(np.int64)
    if f.size and (f.min() < 0 or f.max() >= E):
        raise ValueError("expert index out of range")
    order = np.argsort(f, kind="stable")
    P = f.size
    inv = np.empty(P, dtype=np.int64)
    inv[order] = np.arange(P)
    counts = np.bincount(f, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    return (order.astype(np.int32), (order // top_k).astype(np.int32), f[order].astype(np.int32),
            inv.astype(np.int32), counts.astype(np.int32), offsets.astype(np.int32))


# ----------------------------------------------------------------------------
# Row-tile schedules
# ----------------------------------------------------------------------------
def schedule_tiles(offsets, bm: int) -> np.ndarray:
    """Expert-aware row tiles: no tile crosses an expert boundary.

    [MLX#4567] Proposed changes: each tile carries the row to start from, the
    expert to load and the number of valid rows, built from the per-expert
    offsets.  Every expert with c rows gets ceil(c/bm) tiles.

    READING: tiles are listed expert-major, then by row start; a tile is the
    triple (row_start, expert, valid_rows).
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    tiles = []
    for e in range(len(offsets) - 1):
        c = int(offsets[e + 1] - offsets[e])
        j = 0
        while j * bm < c:
            tiles.append((int(offsets[e]) + j * bm, e, min(bm, c - j * bm)))
            j += 1
    return np.array(tiles, dtype=np.int32).reshape(-1, 3)


def naive_tiles(offsets, bm: int):
    """Fixed row tiles over the sorted rows, blind to experts.

    [MLX#4567] Description: tile t covers sorted rows [t*bm, (t+1)*bm) and
    runs one K pass ("as many matmuls as necessary") for every expert present
    in it.  Returns (tiles [n, 2] = (row_start, valid_rows), passes per tile).
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    P = int(offsets[-1])
    tiles, passes = [], []
    for r0 in range(0, P, bm):
        r1 = min(P, r0 + bm)
        n = 0
        for e in range(len(offsets) - 1):
            lo, hi = offsets[e], offsets[e + 1]
            if hi > lo and lo < r1 and hi > r0:
                n += 1
        tiles.append((r0, r1 - r0))
        passes.append(n)
    return np.array(tiles, dtype=np.int32).reshape(-1, 2), np.array(passes, dtype=np.int32)


def hybrid_tiles(offsets, extra_rows: int = 0, big: int = 128, small: int = 32,
                 slots: int = 512, col_blocks: int = 4):
    """The two-size expert-aware schedule the whole-layer route runs.

    [MLX#4567] Proposed changes: a tile is (row to start from, expert, valid
    rows) and never spans two experts.  This library's rule for the tile
    height (its own design, stated here so that the GPU's tables can be
    checked entry by entry):
      * an expert with at least ``small`` rows gets ceil(c / big) tiles of
        ``big`` rows in the first table; an expert with fewer rows gets
        ceil(c / small) tiles of ``small`` rows in the second table;
      * except when the first table would hold so few tiles that, times the
        ``col_blocks`` column blocks of the first pass, they make at most
        slots // 8 work items: then every expert takes ``small``-row tiles;
      * an extra expert (index E, the shared expert) owns the rows
        [P, P + extra_rows) and is split by the same rule; its tiles follow
        the routed experts' tiles in each table.
    Each table lists its tiles expert-major, then by row start.
    Returns (big_table [n1, 3], small_table [n2, 3]) int32.
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    E = len(offsets) - 1
    P = int(offsets[-1])
    counts = [int(offsets[e + 1] - offsets[e]) for e in range(E)]
    firsts = [int(offsets[e]) for e in range(E)]
    if extra_rows > 0:
        counts.append(int(extra_rows))
        firsts.append(P)
    n_big = sum(-(-c // big) for c in counts if c >= small)
    threshold = small if n_big * col_blocks > slots // 8 else None   # None: no expert is big
    big_t, small_t = [], []
    for e, (c, r0) in enumerate(zip(counts, firsts)):
        if c == 0:
            continue
        if threshold is not None and c >= threshold:
            table, height = big_t, big
        else:
            table, height = small_t, small
        for j in range(0, c, height):
            table.append((r0 + j, e, min(height, c - j)))
    return (np.array(big_t, dtype=np.int32).reshape(-1, 3), np.array(small_t, dtype=np.int32).reshape(-1, 3))


# ----------------------------------------------------------------------------
# Combine tail
# ----------------------------------------------------------------------------
def unsort(y_sorted, inv, T: int, top_k: int) -> np.ndarray:
    """Token-order [T, top_k, H] view of expert-sorted rows: row (t, k) is
    sorted row inv[t*top_k + k].  [MTPLX#558] Motivation (the unsort step)."""
    y_sorted = np.asarray(y_sorted, dtype=np.uint16)
    return y_sorted[np.asarray(inv).reshape(T, top_k)]


def combine(y_sorted, inv, scores, shared=None) -> np.ndarray:
    """out[t] = bf16( bf16(sum_k bf16(y[t,k] * score[t,k])) + shared[t] ).

    [MTPLX#558] Motivation: the stock tail un-sorts the expert outputs,
    multiplies by the routing scores, sums over top_k (each step a bf16
    tensor) and adds the gated shared expert; the one-pass kernel keeps the
    same rounding.

    READING (fixed here, shared by the fused and unfused GPU kernels): each
    bf16 op is evaluated in fp32 and rounded to bf16 once; the product of two
    bf16 values is exact in fp32; the sum over top_k starts from slot 0 and
    adds slots 1..top_k-1 in order in fp32 before its single rounding.
    """
    scores = np.asarray(scores, dtype=np.uint16)
    T, top_k = scores.shape
    yt = bf16_to_f32(unsort(y_sorted, inv, T, top_k))           # [T, top_k, H] fp32
    sc = bf16_to_f32(scores)                                      # [T, top_k]
    acc = None
    for k in range(top_k):
        prod = (yt[:, k, :] * sc[:, k:k + 1]).astype(np.float32)  # exact in fp32
        p = bf16_to_f32(f64_to_bf16(prod))
        acc = p if acc is None else (acc + p).astype(np.float32)
    s = f64_to_bf16(acc)
    if shared is None:
        return s
    tot = (bf16_to_f32(s) + bf16_to_f32(shared)).astype(np.float32)
    return f64_to_bf16(tot)


# ----------------------------------------------------------------------------
# Shared expert, RMSNorm, whole layers
# ----------------------------------------------------------------------------
def rms_norm(x, w, eps: float = 1e-6) -> np.ndarray:
    """bf16( x / sqrt(mean(x^2) + eps) * w ), float64 inside.
    [MLX#4787] benchmark script: rms_norm between the projections, eps 1e-6."""
    xf = bf16_to_f64(x)
    wf = bf16_to_f64(w)
    r = 1.0 / np.sqrt(np.mean(xf * xf, axis=-1, keepdims=True) + eps)
    return f64_to_bf16(xf * r * wf)


def _dense_glu(x, gate, up, down, gs, bits):
    g = quantized_matmul(x, *gate, True, gs, bits)
    u = quantized_matmul(x, *up, True, gs, bits)
    h = f64_to_bf16(silu(bf16_to_f64(g)) * bf16_to_f64(u))
    return quantized_matmul(h, *down, True, gs, bits)


def shared_expert(x, gate, up, down, gate_row, gs: int = 64, bits: int = 4) -> np.ndarray:
    """Gated shared expert: bf16( sigmoid(z) * SwiGLU(x) ), z = x . w_gate^T.

    [MTPLX#558] Summary/Change: the shared expert and its sigmoid gate run
    before the combine, which receives the gated result.
    READING: the shared expert and its one-row gate are quantized like the
    routed experts; z and the SwiGLU output are bf16 tensors.
    """
    s = _dense_glu(x, gate, up, down, gs, bits)
    z = quantized_matmul(x, *gate_row, True, gs, bits)          # [T, 1]
    zf = bf16_to_f64(z)
    return f64_to_bf16(bf16_to_f64(s) / (1.0 + np.exp(-zf)))


def moe_prefill_layer(x, idx, scores, experts, shared_params=None, gs: int = 64, bits: int = 4):
    """One MoE layer on the expert-sorted route: sort, SwitchGLU on the sorted
    rows, gated shared expert, combine.  Returns (out [T, H], intermediates).

    [MTPLX#558] Summary/Change; [MLX#4509] SwitchGLU order.
    experts = (gate, up, down) triples as in switch_glu; shared_params =
    (gate, up, down, gate_row) or None.
    """
    idx = np.asarray(idx)
    T, top_k = idx.shape
    E = np.asarray(experts[0][0]).shape[0]
    order, lhs, srhs, inv, counts, offsets = sort_pairs(idx, E)
    y_tok = switch_glu(x, idx, *experts, gs=gs, bits=bits)           # [T, top_k, H]
    H = y_tok.shape[-1]
    y_sorted = y_tok.reshape(T * top_k, H)[order]
    shared = None if shared_params is None else shared_expert(x, *shared_params, gs=gs, bits=bits)
    out = combine(y_sorted, inv, scores, shared)
    return out, dict(order=order, lhs=lhs, sorted_rhs=srhs, inv=inv, counts=counts,
                     offsets=offsets, y_sorted=y_sorted, shared=shared)


def dense_forward(h0, sets, layers: int, norm_w, gs: int = 64, bits: int = 4) -> np.ndarray:
    """The chained decoder-shaped forward of few-row quantized_matmul.

    [MLX#4787] benchmark script, forward(): per layer rms_norm; q, k, v; o on
    q + (k[:, :1] + v[:, :1]) plus the residual; rms_norm; gate and up;
    silu(g)*u; down plus the residual.  Layer li uses weight set li % len(sets).
    Each set is a dict name -> (words, scales, biases) for q, k, v, o, g, u, dn.
    """
    h = np.asarray(h0, dtype=np.uint16)
    for li in range(layers):
        L = sets[li % len(sets)]
        x = rms_norm(h, norm_w, 1e-6)
        q = quantized_matmul(x, *L["q"], True, gs, bits)
        k = quantized_matmul(x, *L["k"], True, gs, bits)
        v = quantized_matmul(x, *L["v"], True, gs, bits)
        kv = f64_to_bf16(bf16_to_f64(k[:, :1]) + bf16_to_f64(v[:, :1]))
        o_in = f64_to_bf16(bf16_to_f64(q) + bf16_to_f64(kv))
        o = quantized_matmul(o_in, *L["o"], True, gs, bits)
        h = f64_to_bf16(bf16_to_f64(h) + bf16_to_f64(o))
        x = rms_norm(h, norm_w, 1e-6)
        g = quantized_matmul(x, *L["g"], True, gs, bits)
        u = quantized_matmul(x, *L["u"], True, gs, bits)
        a = f64_to_bf16(silu(bf16_to_f64(g)) * bf16_to_f64(u))
        d = quantized_matmul(a, *L["dn"], True, gs, bits)
        h = f64_to_bf16(bf16_to_f64(h) + bf16_to_f64(d))
    return h


# ----------------------------------------------------------------------------
# router
# ----------------------------------------------------------------------------
def route(logits, top_k: int):
    """The MoE block's routing from its router logits [T, E] (fp32).

    [MTPLX#558] Change: the one-kernel block routes tokens the same way as
    the unfused block it replaces, ahead of the sorted experts and the
    combine; the page does not define the routing itself.
    READING: the top_k experts with the largest logits (ties to the lower id),
    stored in ascending expert id; the score of a chosen expert is its softmax
    probability over all E logits, evaluated in float64 (max-subtracted), not
    renormalised over the chosen ones, rounded to fp32 and then to bf16.
    Returns (idx int32 [T, top_k], scores bf16 bits [T, top_k])."""
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    if not 0 < top_k <= E:
        raise ValueError("top_k must be in 1..E")
    idx = np.zeros((T, top_k), np.int32)
    scores = np.zeros((T, top_k), np.uint16)
    for t in range(T):
        row = [float(v) for v in lg[t]]
        chosen = sorted(sorted(range(E), key=lambda e: (-row[e], e))[:top_k])
        m = max(row)
        ex = [math.exp(v - m) for v in row]
        total = math.fsum(ex)
        for j, e in enumerate(chosen):
            idx[t, j] = e
            scores[t, j] = f64_to_bf16(np.float32(ex[e] / total))
    return idx, scores


# ----------------------------------------------------------------------------
# unquantized gather_mm
# ----------------------------------------------------------------------------
def gather_mm(x, w, lhs=None, rhs=None) -> np.ndarray:
    """out[j] = bf16( x[lhs[j]] . w[rhs[j]]^T ), float64 accumulation, for every
    j of the broadcast index shape; output shape = index shape + [M, N].

    [MLX#4567] (title, Proposed changes): gather_mm, the matrix product of the
    selected activation batch and the selected expert matrix, is the operation
    the expert-aware tile schedule speeds up.
    READING: the expert matrices are stored as a linear layer's weights, w [E, N, K]
    bf16 (the product takes their transpose), the layout of the quantized path.
    x [X, M, K] bf16; indices as in gather_qmm."""
    x = np.asarray(x, dtype=np.uint16)
    w = np.asarray(w, dtype=np.uint16)
    li, ri, shape = broadcast_gather_indices(x.shape[:-2], w.shape[:-2], lhs, rhs)
    M, N = x.shape[-2], w.shape[-2]
    xf = bf16_to_f64(x.reshape((-1,) + x.shape[-2:]))
    wf = w.reshape((-1,) + w.shape[-2:])
    out = np.zeros((len(li), M, N), dtype=np.uint16)
    cache = {}
    for j, (l, r) in enumerate(zip(li, ri)):
        if r not in cache:
            cache = {r: bf16_to_f64(wf[r])}
        out[j] = f64_to_bf16(xf[l] @ cache[r].T)
    return out.reshape(tuple(shape) + (M, N))


def switch_glu_mm(x, idx, gate, up, down) -> np.ndarray:
    """SwitchGLU on unquantized bf16 experts [E, N, K]: for every (token, slot)
    u = bf16(x w_up^T), g = bf16(x w_gate^T), h = bf16(silu(g) u),
    y = bf16(h w_down^T); returns y [T, top_k, H].
    [MLX#4509] SwitchGLU order (up, gate, silu(gate) * up, down)."""
    idx = np.asarray(idx)
    T, top_k = idx.shape
    x = np.asarray(x, dtype=np.uint16)
    H = np.asarray(down).shape[1]
    y = np.zeros((T, top_k, H), dtype=np.uint16)
    for e in np.unique(idx):
        toks, slots = np.nonzero(idx == e)
        xe = bf16_to_f64(x[toks])
        g = f64_to_bf16(xe @ bf16_to_f64(np.asarray(gate)[e]).T)
        u = f64_to_bf16(xe @ bf16_to_f64(np.asarray(up)[e]).T)
        gf = bf16_to_f64(g)
        h = f64_to_bf16(silu(gf) * bf16_to_f64(u))
        y[toks, slots] = f64_to_bf16(bf16_to_f64(h) @ bf16_to_f64(np.asarray(down)[e]).T)
    return y
