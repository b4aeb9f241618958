"""Seeded synthetic inputs shaped like the pages' workloads.

Shared by the tests, the smoke check and the benchmark.  It holds input
preparation only (random draws, bf16 encoding of drawn values, packing codes
into words, the host min-max quantizer, host-side routing); none of the
arithmetic of the gathered matmul, SwitchGLU, sort, schedule or combine.

Every draw comes from ``numpy.random.SeedSequence([config, stream, ...])``:
stream 0 = weights (one sub-stream per expert and matrix), 1 = activations,
2 = routing, 3 = shared expert, 4 = extra test streams.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

GATE, UP, DOWN = 0, 1, 2


def rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def to_bf16(x) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def from_bf16(u16) -> np.ndarray:
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def pack(codes, bits: int) -> np.ndarray:
    """Pack integer codes along the last axis into uint32 words, code k at bit
    offset k*bits of the little-endian word stream (LSB first)."""
    codes = np.asarray(codes, dtype=np.uint64)
    K = codes.shape[-1]
    assert (K * bits) % 32 == 0
    nw = K * bits // 32
    if 32 % bits == 0:
        per = 32 // bits
        c = codes.reshape(codes.shape[:-1] + (nw, per))
        shifts = (np.arange(per, dtype=np.uint64) * np.uint64(bits))
        return np.bitwise_or.reduce(c << shifts, axis=-1).astype(np.uint32)
    out = np.zeros(codes.shape[:-1] + (nw + 1,), dtype=np.uint64)
    for k in range(K):
        pos = k * bits
        v = codes[..., k] << np.uint64(pos % 32)
        out[..., pos // 32] |= v & np.uint64(0xFFFFFFFF)
        out[..., pos // 32 + 1] |= v >> np.uint64(32)
    return out[..., :nw].astype(np.uint32)


# ----------------------------------------------------------------------------
# weight generators
# ----------------------------------------------------------------------------
def drawn_matrix(g: np.random.Generator, N: int, K: int, gs: int, bits: int):
    """Codes uniform on [0, 2^bits), scales bf16 ~ U(0.005, 0.02) * 16 / 2^bits,
    biases bf16(-2^(bits-1) * scale + N(0, 0.001)): the tiny SwitchGLU recipe,
    generalised to 8-bit codes with the same dequantized spread."""
    levels = 1 << bits
    codes = g.integers(0, levels, size=(N, K), dtype=np.uint32)
    s = to_bf16(g.uniform(0.005, 0.02, size=(N, K // gs)).astype(np.float32) * np.float32(16.0 / levels))
    b = to_bf16(-np.float32(levels // 2) * from_bf16(s) + g.normal(0.0, 0.001, size=s.shape).astype(np.float32))
    return pack(codes, bits), s, b


def drawn_words(g: np.random.Generator, N: int, K: int, gs: int, bits: int):
    """Same distribution as drawn_matrix, drawn directly as random words (every
    code of a uniform word is uniform): fast for multi-GB benchmark weights."""
    levels = 1 << bits
    w = g.integers(0, 1 << 32, size=(N, K * bits // 32), dtype=np.uint64).astype(np.uint32)
    s = to_bf16(g.uniform(0.005, 0.02, size=(N, K // gs)).astype(np.float32) * np.float32(16.0 / levels))
    b = to_bf16(-np.float32(levels // 2) * from_bf16(s) + g.normal(0.0, 0.001, size=s.shape).astype(np.float32))
    return w, s, b


def minmax_quantize(w_f32, gs: int, bits: int):
    """Host min-max affine quantizer: per group scale = (max-min)/(2^bits-1) and
    bias = min, both rounded to bf16; q = clamp(rint((w-bias)/scale)) using the
    rounded scale and bias.  A constant group gets scale 0, bias = its value and
    codes 0.  Input values are rounded to bf16 first (weights are bf16)."""
    w = from_bf16(to_bf16(w_f32)).astype(np.float64)
    N, K = w.shape
    wg = w.reshape(N, K // gs, gs)
    mn = wg.min(-1)
    mx = wg.max(-1)
    levels = (1 << bits) - 1
    s_bits = to_bf16(((mx - mn) / levels).astype(np.float32))
    b_bits = to_bf16(mn.astype(np.float32))
    s = from_bf16(s_bits).astype(np.float64)[..., None]
    b = from_bf16(b_bits).astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint((wg - b) / np.where(s > 0, s, 1.0)), 0.0)
    q = np.clip(q, 0, levels).astype(np.uint32).reshape(N, K)
    return pack(q, bits), s_bits, b_bits


def normal_matrix(g: np.random.Generator, N: int, K: int, scale: float = 1.0) -> np.ndarray:
    return (g.standard_normal((N, K), dtype=np.float32) * np.float32(scale))


def minmax_matrix(g: np.random.Generator, N: int, K: int, gs: int, bits: int, scale: float = 1.0):
    return minmax_quantize(normal_matrix(g, N, K, scale), gs, bits)


def stack_experts(mats):
    return tuple(np.stack([m[i] for m in mats]) for i in range(3))


def expert_set(cfg: int, E: int, H: int, I: int, gs: int, bits: int, mode: str = "drawn",
               experts=None):
    """(gate, up, down) triples [E, ...].  Expert e / matrix j comes from its
    own seed stream [cfg, 0, e, j], so any subset can be regenerated alone.
    ``experts``: only these experts are drawn, the others stay zero."""
    shapes = {GATE: (I, H), UP: (I, H), DOWN: (H, I)}
    out = []
    for j in (GATE, UP, DOWN):
        N, K = shapes[j]
        W = np.zeros((E, N, K * bits // 32), dtype=np.uint32)
        S = np.zeros((E, N, K // gs), dtype=np.uint16)
        B = np.zeros((E, N, K // gs), dtype=np.uint16)
        for e in (range(E) if experts is None else sorted(set(int(v) for v in experts))):
            g = rng(cfg, 0, e, j)
            if mode == "drawn":
                W[e], S[e], B[e] = drawn_matrix(g, N, K, gs, bits)
            elif mode == "words":
                W[e], S[e], B[e] = drawn_words(g, N, K, gs, bits)
            elif mode == "minmax":
                W[e], S[e], B[e] = minmax_matrix(g, N, K, gs, bits)
            else:
                raise ValueError(mode)
        out.append((W, S, B))
    return tuple(out)


def activations(cfg: int, M: int, H: int, sub: int = 0) -> np.ndarray:
    return to_bf16(rng(cfg, 1, sub).standard_normal((M, H), dtype=np.float32))


def sorted_topk(cfg: int, M: int, E: int, top_k: int, sub: int = 0) -> np.ndarray:
    """Per-token expert lists: sorted samples without replacement."""
    g = rng(cfg, 2, sub)
    return np.stack([np.sort(g.choice(E, size=top_k, replace=False)) for _ in range(M)]).astype(np.int32)


def zipf_logits(cfg: int, T: int, E: int, zipf: float = 1.1, sub: int = 0) -> np.ndarray:
    """Router logits fp32 [T, E] = N(0,1) + bias_e with bias_e = -zipf * ln(r_e),
    r a seeded permutation of the ranks 1..E (so expert popularity ~ r^-zipf)."""
    g = rng(cfg, 2, sub)
    ranks = g.permutation(E) + 1
    bias = (-zipf * np.log(ranks.astype(np.float64))).astype(np.float32)
    return (g.standard_normal((T, E), dtype=np.float32) + bias[None, :]).astype(np.float32)


def zipf_routing(cfg: int, T: int, E: int, top_k: int, zipf: float = 1.1, sub: int = 0):
    """Routing inputs from zipf_logits: top-k by logit (ties to the lower id);
    scores = softmax over all E logits (float64) taken at the chosen experts,
    not renormalised, rounded to fp32 and then bf16.  Each token's slots are
    stored in ascending expert id."""
    logits = zipf_logits(cfg, T, E, zipf, sub)
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), -logits.astype(np.float64)), axis=-1)
    idx = np.sort(order[:, :top_k], axis=-1).astype(np.int32)
    l64 = logits.astype(np.float64)
    m = l64.max(-1, keepdims=True)
    p = np.exp(l64 - m)
    p /= p.sum(-1, keepdims=True)
    scores = to_bf16(np.take_along_axis(p, idx, axis=-1).astype(np.float32))
    return idx, scores


# ----------------------------------------------------------------------------
# workload descriptions (the five configurations)
# ----------------------------------------------------------------------------
@dataclass
class MoEShape:
    E: int
    top_k: int
    H: int
    I: int
    gs: int
    bits: int
    shared_I: int = 0


TINY = MoEShape(E=8, top_k=2, H=256, I=128, gs=64, bits=4)            # tiny SwitchGLU, M=4
DECODE = MoEShape(E=288, top_k=8, H=4096, I=2048, gs=64, bits=4)      # MoE decode, M=1/4
PREFILL = MoEShape(E=256, top_k=8, H=2048, I=512, gs=64, bits=4, shared_I=512)
LARGE4 = MoEShape(E=288, top_k=8, H=4096, I=2048, gs=64, bits=4)      # large prefill 4-bit
LARGE8 = MoEShape(E=288, top_k=8, H=4096, I=2048, gs=128, bits=8)     # large prefill 8-bit

# dense few-row chain: (hidden, q_out, kv_out, inter, layers), 8 weight sets
DENSE = dict(hidden=2560, q_out=4096, kv_out=1024, inter=9728, layers=36, sets=8)


def dense_dims(d=DENSE):
    h, qo, kvo, inter = d["hidden"], d["q_out"], d["kv_out"], d["inter"]
    return {"q": (qo, h), "k": (kvo, h), "v": (kvo, h), "o": (h, qo),
            "g": (inter, h), "u": (inter, h), "dn": (h, inter)}


def dense_sets(cfg: int, gs: int, bits: int, mode: str = "words", d=DENSE, n_sets=None):
    """8 weight sets of the dense chain; each matrix bf16(N(0,1)/sqrt(K))
    min-max quantized (mode 'minmax') or drawn codes (mode 'words')."""
    dims = dense_dims(d)
    sets = []
    for si in range(n_sets or d["sets"]):
        L = {}
        for j, (name, (N, K)) in enumerate(dims.items()):
            g = rng(cfg, 0, si, j)
            if mode == "minmax":
                L[name] = minmax_matrix(g, N, K, gs, bits, scale=1.0 / np.sqrt(K))
            else:
                # random words; scale chosen so the dequantized spread is about 1/sqrt(K)
                levels = 1 << bits
                w = g.integers(0, 1 << 32, size=(N, K * bits // 32), dtype=np.uint64).astype(np.uint32)
                s0 = np.float32(np.sqrt(12.0) / (levels * np.sqrt(K)))
                s = to_bf16(g.uniform(0.5, 1.5, size=(N, K // gs)).astype(np.float32) * s0)
                b = to_bf16(-np.float32(levels // 2) * from_bf16(s))
                L[name] = (w, s, b)
        sets.append(L)
    return sets


def shared_params(cfg: int, H: int, I: int, gs: int, bits: int):
    """Shared expert gate/up/down and its one-row sigmoid gate (stream 3)."""
    gate = drawn_matrix(rng(cfg, 3, 0), I, H, gs, bits)
    up = drawn_matrix(rng(cfg, 3, 1), I, H, gs, bits)
    down = drawn_matrix(rng(cfg, 3, 2), H, I, gs, bits)
    grow = drawn_matrix(rng(cfg, 3, 3), 1, H, gs, bits)
    return gate, up, down, grow


def integer_exact(g: np.random.Generator, N: int, K: int, gs: int, bits: int, j: int = 2):
    """Weights whose every product and partial sum is exact in fp32: scales
    2^-j, biases small integers times 2^-j."""
    levels = 1 << bits
    codes = g.integers(0, levels, size=(N, K), dtype=np.uint32)
    s = to_bf16(np.full((N, K // gs), 2.0 ** -j, dtype=np.float32))
    bi = g.integers(-levels // 2, 1, size=(N, K // gs)).astype(np.float32)
    b = to_bf16(bi * np.float32(2.0 ** -j))
    return pack(codes, bits), s, b


def integer_x(g: np.random.Generator, M: int, K: int, amp: int = 8) -> np.ndarray:
    return to_bf16(g.integers(-amp, amp + 1, size=(M, K)).astype(np.float32))


# ---- integer-exact SwitchGLU chain: every product and partial sum of gate,
#      up and down is exact in fp32, and the gate output is a power of two
#      >= 32 (so silu(g) rounds to g in fp32 and g * u is a bf16 value).
def group_unit_x(g: np.random.Generator, T: int, K: int, gs: int) -> np.ndarray:
    """Integer activations whose every group of gs consecutive elements sums
    to 1: entries uniform on {-1, 0, 1}, the last entry of each group set to
    make the sum."""
    x = g.integers(-1, 2, size=(T, K // gs, gs)).astype(np.float32)
    x[:, :, -1] = 1.0 - x[:, :, :-1].sum(axis=-1)
    return to_bf16(x.reshape(T, K))


def pow2_gate(g: np.random.Generator, N: int, K: int, gs: int, bits: int, targets=(32, 64)):
    """A gate matrix with random codes, zero scales and integer biases whose
    sum along each row is a value drawn from ``targets`` (powers of two)."""
    G = K // gs
    codes = g.integers(0, 1 << bits, size=(N, K), dtype=np.uint32)
    s = to_bf16(np.zeros((N, G), np.float32))
    b = g.integers(-4, 5, size=(N, G)).astype(np.float32)
    b[:, -1] = np.asarray(targets, np.float32)[g.integers(0, len(targets), size=N)] - b[:, :-1].sum(axis=1)
    return pack(codes, bits), s, to_bf16(b)


def dyadic_matrix(g: np.random.Generator, N: int, K: int, gs: int, bits: int, js=(4, 5), bias_den: int = 5):
    """Random codes, scales 2^-j (j drawn from js per group) and biases that
    are small integers times 2^-bias_den."""
    G = K // gs
    codes = g.integers(0, 1 << bits, size=(N, K), dtype=np.uint32)
    s = np.float32(2.0) ** -np.asarray(js, np.float32)[g.integers(0, len(js), size=(N, G))]
    b = g.integers(-8, 1, size=(N, G)).astype(np.float32) * np.float32(2.0 ** -bias_den)
    return pack(codes, bits), to_bf16(s), to_bf16(b)


def exact_glu_experts(cfg: int, E: int, H: int, I: int, gs: int, bits: int, experts=None):
    """Per-expert (gate, up, down) with the recipes above; experts outside
    ``experts`` (when given) get all-zero words and scales."""
    want = set(range(E)) if experts is None else set(int(e) for e in experts)
    mats = []
    for m, (N, K) in enumerate(((I, H), (I, H), (H, I))):
        ws = np.zeros((E, N, K * bits // 32), np.uint32)
        ss = np.zeros((E, N, K // gs), np.uint16)
        bs = np.zeros((E, N, K // gs), np.uint16)
        for e in sorted(want):
            gg = rng(cfg, 4, 100 + e, m)
            if m == 0:
                w, sc, bi = pow2_gate(gg, N, K, gs, bits)
            elif m == 1:
                w, sc, bi = dyadic_matrix(gg, N, K, gs, bits, js=(4, 5) if bits == 4 else (8, 9))
            else:
                w, sc, bi = dyadic_matrix(gg, N, K, gs, bits, js=(5, 6) if bits == 4 else (9, 10), bias_den=6)
            ws[e], ss[e], bs[e] = w, sc, bi
        mats.append((ws, ss, bs))
    return tuple(mats)


def exact_shared(cfg: int, H: int, I: int, gs: int, bits: int):
    """Shared expert (gate, up, down, gate_row) with the same recipes; the
    gate row's biases sum to 64, so its logit on group_unit_x rows is 64."""
    gate = pow2_gate(rng(cfg, 4, 7, 0), I, H, gs, bits)
    up = dyadic_matrix(rng(cfg, 4, 7, 1), I, H, gs, bits, js=(4, 5) if bits == 4 else (8, 9))
    down = dyadic_matrix(rng(cfg, 4, 7, 2), H, I, gs, bits, js=(5, 6) if bits == 4 else (9, 10), bias_den=6)
    grow = pow2_gate(rng(cfg, 4, 7, 3), 1, H, gs, bits, targets=(64,))
    return gate, up, down, grow


# ----------------------------------------------------------------------------
# device-side draws for benchmark-sized weights (GBs); same distributions as
# drawn_words / dense_sets(mode="words"), drawn with a seeded torch generator
# ----------------------------------------------------------------------------
def device_generator(device, *key):
    import torch
    seed = int(np.random.SeedSequence(list(key)).generate_state(1, dtype=np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def device_drawn_words(device, key, shape_rows, K: int, gs: int, bits: int, scale0=None):
    """(words int32 [*rows, K*bits/32], scales bf16 [*rows, K/gs], biases bf16)
    on the device.  scale0 None: scales U(0.005, 0.02) * 16 / 2^bits and biases
    -2^(bits-1) * s + N(0, 0.001); else scales U(0.5, 1.5) * scale0, biases
    -2^(bits-1) * s."""
    import torch
    g = device_generator(device, *key)
    levels = 1 << bits
    rows = tuple(shape_rows)
    w = torch.randint(-(1 << 31), (1 << 31) - 1, rows + (K * bits // 32,), dtype=torch.int32, device=device,
                      generator=g)
    u = torch.rand(rows + (K // gs,), device=device, generator=g, dtype=torch.float32)
    if scale0 is None:
        s = ((0.005 + 0.015 * u) * (16.0 / levels)).to(torch.bfloat16)
        n = torch.randn(rows + (K // gs,), device=device, generator=g, dtype=torch.float32) * 0.001
        b = (-(levels // 2) * s.float() + n).to(torch.bfloat16)
    else:
        s = ((0.5 + u) * scale0).to(torch.bfloat16)
        b = (-(levels // 2) * s.float()).to(torch.bfloat16)
    return w, s, b


def device_expert_set(device, cfg: int, E: int, H: int, I: int, gs: int, bits: int):
    return tuple(device_drawn_words(device, (cfg, 0, j), (E, N), K, gs, bits)
                 for j, (N, K) in ((GATE, (I, H)), (UP, (I, H)), (DOWN, (H, I))))


def device_dense_sets(device, cfg: int, gs: int, bits: int, d=DENSE, n_sets=None):
    out = []
    for si in range(n_sets or d["sets"]):
        L = {}
        for j, (name, (N, K)) in enumerate(dense_dims(d).items()):
            L[name] = device_drawn_words(device, (cfg, 0, si, j), (N,), K, gs, bits,
                                         scale0=float(np.sqrt(12.0) / ((1 << bits) * np.sqrt(K))))
        out.append(L)
    return out
