"""Pins for the CPU oracle: facts the pages and the mathematics fix, checked
without trusting the oracle's own formulas (worked examples, closed forms,
special cases, library routines, brute force on tiny inputs)."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def bf16_torch(x):
    """Library route: torch's fp32 -> bf16 conversion (round to nearest even)."""
    t = torch.from_numpy(np.asarray(x, dtype=np.float32).copy()).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------------------- bf16
def test_bf16_known_values():
    cases = [(1.0, 0x3F80), (1 + 2 ** -8, 0x3F80), (1 + 3 * 2 ** -8, 0x3F82), (-2.5, 0xC020),
             (float("inf"), 0x7F80), (-float("inf"), 0xFF80), (3.4e38, 0x7F80), (3.38e38, 0x7F7E),
             (2.0 ** -133, 0x0001), (2.0 ** -134, 0x0000), (3 * 2.0 ** -134, 0x0002), (0.0, 0x0000),
             (-0.0, 0x8000), (2.0 ** -126, 0x0080)]
    for v, want in cases:
        assert int(oracle.f64_to_bf16(v)) == want, (v, hex(int(oracle.f64_to_bf16(v))))
    assert int(oracle.f64_to_bf16(float("nan"))) == 0x7FC0


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(1)
    with np.errstate(over="ignore"):          # values past float32's range become inf and are dropped below
        x = (g.standard_normal(200000) * np.exp2(g.integers(-140, 128, 200000))).astype(np.float32)
    # exact ties, to exercise round-half-to-even
    ties = (np.arange(1, 20001, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    x = x[np.isfinite(x)]
    assert np.array_equal(oracle.f64_to_bf16(x), bf16_torch(x))
    assert np.array_equal(oracle.bf16_to_f32(bf16_torch(x)), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


# ----------------------------------------------------------------------------- unpack / dequant
def _golden_handpacked():
    rows = []
    for line in open(os.path.join(GOLD, "handpacked_codes.txt")):
        if line.startswith("#") or not line.strip():
            continue
        bits, words, codes, deq = [p.strip() for p in line.split("|")]
        rows.append((int(bits), [int(w, 16) for w in words.split()], [int(c) for c in codes.split()],
                     [float(d) for d in deq.split()]))
    return rows


@pytest.mark.parametrize("row", _golden_handpacked())
def test_handpacked_words(row):
    bits, words, codes, deq = row
    w = np.array([words], dtype=np.uint32)
    K = len(codes)
    assert oracle.unpack(w, K, bits)[0].tolist() == codes
    # one group covering the row needs K to be a valid group size; use 32 and repeat
    reps = 32 // K if K < 32 else 1
    ww = np.tile(w, (1, reps))
    s = oracle.f64_to_bf16(np.full((1, 1), 0.5))
    b = oracle.f64_to_bf16(np.full((1, 1), -4.0))
    got = oracle.dequant(ww, s, b, 32, bits, K * reps)[0]
    assert got.tolist() == deq * reps


def test_dequant_unit_scale_zero_bias_returns_codes():
    # nuvec "quantize_snaps_zero...": dequantize with ones/zeros yields the raw codes
    g = np.random.default_rng(2)
    for bits in (4, 8):
        for gs in (32, 64, 128):
            codes = g.integers(0, 1 << bits, size=(5, 256))
            w = synth.pack(codes, bits)
            one = oracle.f64_to_bf16(np.ones((5, 256 // gs)))
            zero = oracle.f64_to_bf16(np.zeros((5, 256 // gs)))
            assert np.array_equal(oracle.dequant(w, one, zero, gs, bits, 256), codes)


def test_dequant_constant_group_and_group_index():
    # constant group: scale 0, bias c gives c exactly (nuvec: constant groups are exact)
    w = synth.pack(np.full((2, 128), 7), 4)
    s = oracle.f64_to_bf16(np.zeros((2, 2)))
    b = oracle.f64_to_bf16(np.array([[0.75, -1.25], [3.0, 0.0]]))
    d = oracle.dequant(w, s, b, 64, 4, 128)
    assert (d[0, :64] == 0.75).all() and (d[0, 64:] == -1.25).all() and (d[1, :64] == 3).all()
    # element k uses group k // gs: distinct scales per group, code 1 everywhere
    w = synth.pack(np.ones((1, 256), dtype=np.int64), 4)
    s = oracle.f64_to_bf16(np.arange(1, 5)[None, :].astype(float))
    d = oracle.dequant(w, s, oracle.f64_to_bf16(np.zeros((1, 4))), 64, 4, 256)
    assert d[0].tolist() == [float(k // 64 + 1) for k in range(256)]


def test_straddling_widths_unpack():
    # 3-, 5- and 6-bit codes straddle words; a known bit stream pins them
    g = np.random.default_rng(3)
    for bits in (1, 2, 3, 5, 6):
        codes = g.integers(0, 1 << bits, size=(2, 64))
        w = synth.pack(codes, bits)
        stream = "".join(format(int(x), "032b")[::-1] for x in w[0])   # LSB-first bits
        want = [int(stream[k * bits:(k + 1) * bits][::-1], 2) for k in range(64)]
        assert oracle.unpack(w, 64, bits)[0].tolist() == want == codes[0].tolist()


# ----------------------------------------------------------------------------- quantized matmul
def _brute_qmm(x_u16, words, s_u16, b_u16, gs, bits, transpose=True):
    """Triple loop in exact rational arithmetic, codes read off the bit string.
    Activations are bf16 bit patterns (result bf16) or float16/float32 values
    (result float32)."""
    xa = np.asarray(x_u16)
    half_or_single = xa.dtype in (np.float16, np.float32)
    xvals = xa.astype(np.float64) if half_or_single else oracle.bf16_to_f64(xa)
    xv = [[Fraction(float(v)) for v in row] for row in xvals]
    sv = oracle.bf16_to_f64(s_u16)
    bv = oracle.bf16_to_f64(b_u16)
    rows = []
    for wr in words:
        stream = "".join(format(int(v), "032b")[::-1] for v in wr)
        rows.append(stream)
    if transpose:
        N, K = len(words), len(xv[0])
        W = [[Fraction(int(rows[n][k * bits:(k + 1) * bits][::-1], 2)) * Fraction(float(sv[n][k // gs]))
              + Fraction(float(bv[n][k // gs])) for k in range(K)] for n in range(N)]
        out = [[float(sum(xv[m][k] * W[n][k] for k in range(K))) for n in range(N)] for m in range(len(xv))]
    else:
        K = len(words)
        N = len(words[0]) * 32 // bits
        W = [[Fraction(int(rows[k][n * bits:(n + 1) * bits][::-1], 2)) * Fraction(float(sv[k][n // gs]))
              + Fraction(float(bv[k][n // gs])) for n in range(N)] for k in range(K)]
        out = [[float(sum(xv[m][k] * W[k][n] for k in range(K))) for n in range(N)] for m in range(len(xv))]
    if half_or_single:
        return np.array(out, dtype=np.float64).astype(np.float32)
    return oracle.f64_to_bf16(np.array(out))


@pytest.mark.parametrize("bits,gs,M,N,K", [(4, 32, 2, 5, 64), (4, 64, 3, 4, 128), (8, 32, 1, 3, 96),
                                           (8, 128, 2, 2, 128), (3, 32, 1, 3, 64)])
def test_qmm_brute_force(bits, gs, M, N, K):
    g = np.random.default_rng(bits * 100 + gs + K)
    x = synth.to_bf16(g.standard_normal((M, K)))
    w, s, b = synth.drawn_matrix(g, N, K, gs, bits)
    got = oracle.quantized_matmul(x, w, s, b, True, gs, bits)
    assert np.array_equal(got, _brute_qmm(x, w, s, b, gs, bits))
    # transpose=False: w is [K, N] with groups along N
    w2, s2, b2 = synth.drawn_matrix(g, K // 2, 64, 32, bits)       # K' = K//2 rows, N' = 64
    x2 = synth.to_bf16(g.standard_normal((M, K // 2)))
    got2 = oracle.quantized_matmul(x2, w2, s2, b2, False, 32, bits)
    assert got2.shape == (M, 64)
    assert np.array_equal(got2, _brute_qmm(x2, w2, s2, b2, 32, bits, transpose=False))


@pytest.mark.parametrize("xdt", [np.float16, np.float32])
@pytest.mark.parametrize("bits,gs", [(4, 32), (8, 64), (4, 128)])
def test_qmm_half_and_single_activations_brute_force(xdt, bits, gs):
    # float16 / float32 activations keep every bit (values off the bf16 grid:
    # a conversion to bf16 would change them) and the result is float32
    g = np.random.default_rng(bits * 7 + gs)
    M, N, K = 2, 3, 2 * gs
    x = (g.standard_normal((M, K)) * (1 + 2.0 ** -9)).astype(xdt)
    assert not np.array_equal(synth.from_bf16(synth.to_bf16(x.astype(np.float32))), x.astype(np.float32))
    w, s, b = synth.drawn_matrix(g, N, K, gs, bits)
    got = oracle.quantized_matmul(x, w, s, b, True, gs, bits)
    assert got.dtype == np.float32 and got.shape == (M, N)
    assert np.array_equal(got, _brute_qmm(x, w, s, b, gs, bits))
    w2, s2, b2 = synth.drawn_matrix(g, 24, gs, gs, bits)       # [K'=24, N'=gs], groups along N
    x2 = (g.standard_normal((M, 24)) * (1 + 2.0 ** -9)).astype(xdt)
    got2 = oracle.quantized_matmul(x2, w2, s2, b2, False, gs, bits)
    assert got2.dtype == np.float32 and got2.shape == (M, gs)
    assert np.array_equal(got2, _brute_qmm(x2, w2, s2, b2, gs, bits, transpose=False))


def test_promoted_type_matches_torch():
    # the result type is the promotion of the activation type with bf16 scales
    torch = pytest.importorskip("torch")
    names = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}
    for t, n in names.items():
        want = torch.promote_types(t, torch.bfloat16)
        assert oracle.promoted_type(n) == names[want]
    with pytest.raises(ValueError):
        oracle.activations_f64(np.zeros(3, dtype=np.int32))


def test_gather_qmm_batched_weights_promote_page_shape():
    # [nuvec] "quantized_matmul_equals_the_dequantized_product": weights with
    # batch [2, 1] (16 x 64, group 32, 4 bits) against float32 activations with
    # batch [3] (5 x 64) give a float32 result of shape [2, 3, 5, 16]
    g = np.random.default_rng(11)
    w, s, b = synth.drawn_matrix(g, 2 * 16, 64, 32, 4)
    w, s, b = w.reshape(2, 1, 16, 8), s.reshape(2, 1, 16, 2), b.reshape(2, 1, 16, 2)
    x = g.standard_normal((3, 5, 64)).astype(np.float32)
    got = oracle.gather_qmm(x, w, s, b, transpose=True, gs=32, bits=4)
    assert got.shape == (2, 3, 5, 16) and got.dtype == np.float32
    for i in range(2):
        for j in range(3):
            assert np.array_equal(got[i, j], _brute_qmm(x[j], w[i, 0], s[i, 0], b[i, 0], 32, 4))


def test_qmm_group_factored_identity():
    # sum_k x (q s + b) = sum_g ( s_g * sum_{k in g} x q + b_g * sum_{k in g} x )
    g = np.random.default_rng(5)
    for bits, gs in ((4, 64), (8, 128), (4, 32)):
        M, N, K = 3, 40, 512
        x = synth.to_bf16(g.standard_normal((M, K)))
        w, s, b = synth.drawn_matrix(g, N, K, gs, bits)
        codes = np.array([[int(format(int(v), "032b")[::-1][j * bits:(j + 1) * bits][::-1], 2)
                           for v in row for j in range(32 // bits)] for row in w], dtype=np.float64)
        xf = synth.from_bf16(x).astype(np.float64)
        sf = synth.from_bf16(s).astype(np.float64)
        bf = synth.from_bf16(b).astype(np.float64)
        G = K // gs
        xq = np.einsum("mgk,ngk->mng", xf.reshape(M, G, gs), codes.reshape(N, G, gs))
        sx = xf.reshape(M, G, gs).sum(-1)
        y = (xq * sf[None]).sum(-1) + sx @ bf.T
        assert np.array_equal(oracle.quantized_matmul(x, w, s, b, True, gs, bits), oracle.f64_to_bf16(y))


def test_qmm_integer_exact_closed_form():
    g = np.random.default_rng(6)
    for bits, gs in ((4, 64), (8, 128)):
        M, N, K = 2, 8, 256
        w, s, b = synth.integer_exact(g, N, K, gs, bits)
        x = synth.integer_x(g, M, K)
        codes = oracle.unpack(w, K, bits)                  # pinned above
        xi = synth.from_bf16(x).astype(np.int64)
        bi = (synth.from_bf16(b) * 4).astype(np.int64)     # biases are integers * 2^-2
        want4 = xi @ codes.T + (xi.reshape(M, K // gs, gs).sum(-1)) @ bi.T   # 4 * exact result
        want = oracle.f64_to_bf16(want4.astype(np.float64) / 4)
        assert np.array_equal(oracle.quantized_matmul(x, w, s, b, True, gs, bits), want)


def test_expert_routing_closed_form():
    # expert e has scale 0, bias e+1: y = (e+1) * sum(x), any wrong expert shows bitwise
    E, N, K, gs = 5, 4, 128, 64
    w = np.zeros((E, N, K // 8), dtype=np.uint32)
    s = oracle.f64_to_bf16(np.zeros((E, N, K // gs)))
    b = oracle.f64_to_bf16(np.broadcast_to(np.arange(1, E + 1)[:, None, None], (E, N, K // gs)).astype(float))
    g = np.random.default_rng(7)
    x = synth.integer_x(g, 3, K)
    rhs = np.array([4, 0, 2, 2, 1])
    lhs = np.array([0, 1, 2, 0, 1])
    out = oracle.gather_qmm(x[:, None, :], w, s, b, lhs=lhs, rhs=rhs, gs=gs, bits=4)
    xs = synth.from_bf16(x).astype(np.float64).sum(-1)
    for j in range(5):
        assert np.all(out[j, 0] == oracle.f64_to_bf16((rhs[j] + 1) * xs[lhs[j]]))


def test_gather_qmm_selects_batches_and_broadcasts():
    # nuvec "gather_qmm_selects_batches"
    g = np.random.default_rng(8)
    E, N, K = 3, 8, 64
    W = [synth.drawn_matrix(g, N, K, 32, 4) for _ in range(E)]
    w, s, b = (np.stack([m[i] for m in W]) for i in range(3))
    x = synth.to_bf16(g.standard_normal((4, 2, K)))
    got = oracle.gather_qmm(x, w, s, b, lhs=[3, 0, 2], rhs=[1, 2, 0], gs=32, bits=4)
    assert got.shape == (3, 2, N)
    for j, (l, r) in enumerate(zip([3, 0, 2], [1, 2, 0])):
        assert np.array_equal(got[j], oracle.quantized_matmul(x[l], w[r], s[r], b[r], True, 32, 4))
    x1 = synth.to_bf16(g.standard_normal((1, 1, K)))
    assert oracle.gather_qmm(x1, w, s, b, gs=32, bits=4).shape == (3, 1, N)
    x3 = synth.to_bf16(g.standard_normal((3, 1, K)))
    got = oracle.gather_qmm(x3, w[:, :, :], s, b, lhs=np.array([[2, 0], [1, 1]]), rhs=np.array([[2, 1]]),
                            gs=32, bits=4)
    assert got.shape == (2, 2, 1, N)
    assert np.array_equal(got[1, 0], oracle.quantized_matmul(x3[1], w[2], s[2], b[2], True, 32, 4))
    with pytest.raises(ValueError):
        oracle.gather_qmm(x, w, s, b, lhs=np.array([0.0]), gs=32, bits=4)
    with pytest.raises(ValueError):
        oracle.gather_qmm(x, w, s, b, lhs=[3, 0, 2], rhs=[0, 1], gs=32, bits=4)


def test_broadcast_gather_indices_cases():
    # defaults: every batch of x and of the weights in order, broadcast together
    li, ri, shape = oracle.broadcast_gather_indices((2, 1), (1, 3), None, None)
    assert tuple(shape) == (2, 3)
    assert li.tolist() == [0, 0, 0, 1, 1, 1] and ri.tolist() == [0, 1, 2, 0, 1, 2]
    # given indices of shapes [2, 1] and [1, 3]
    li, ri, shape = oracle.broadcast_gather_indices((4,), (3,), np.array([[3], [0]]), np.array([[2, 0, 1]]))
    assert tuple(shape) == (2, 3)
    assert li.tolist() == [3, 3, 3, 0, 0, 0] and ri.tolist() == [2, 0, 1, 2, 0, 1]
    with pytest.raises(ValueError):
        oracle.broadcast_gather_indices((4,), (3,), np.array([0.5]), None)
    with pytest.raises(ValueError):
        oracle.broadcast_gather_indices((4,), (3,), np.array([0, 1]), np.array([0, 1, 2]))


def test_invalid_arguments():
    # nuvec "invalid_arguments_are_rejected"
    for kw in (dict(K=64, gs=48, bits=4), dict(K=64, gs=64, bits=7), dict(K=96, gs=64, bits=4),
               dict(K=64, gs=64, bits=4, packed_cols=4), dict(K=64, gs=32, bits=4, n_groups=1)):
        with pytest.raises(ValueError):
            oracle.validate_quant_args(**kw)
    oracle.validate_quant_args(64, 64, 4, 8, 1)


def test_empty_product():
    # nuvec: an empty product keeps its shape [0, N]
    g = np.random.default_rng(9)
    w, s, b = synth.drawn_matrix(g, 16, 64, 64, 4)
    assert oracle.quantized_matmul(np.zeros((0, 64), np.uint16), w, s, b, True, 64, 4).shape == (0, 16)


def test_quantizer_round_trip_bounds():
    # nuvec "round_trip_error_is_about_half_a_step": single error <= 1.0001 step, mean <= step/2
    g = np.random.default_rng(10)
    for bits in (4, 8):
        for gs in (32, 64, 128):
            wf = (g.standard_normal((3, 2 * gs)) / 4).astype(np.float32)
            w, s, b = synth.minmax_quantize(wf, gs, bits)
            back = oracle.dequant(w, s, b, gs, bits, 2 * gs)
            orig = synth.from_bf16(synth.to_bf16(wf)).astype(np.float64)
            step = np.repeat(np.abs(oracle.bf16_to_f64(s)), gs, axis=-1)
            err = np.abs(back - orig)
            assert (err <= step * 1.0001).all()
            assert err.sum() <= step.sum() / 2


# ----------------------------------------------------------------------------- SwitchGLU
def _brute_switch_glu(x, idx, gate, up, down, gs, bits):
    """Per pair, per output, with math.fsum (correctly rounded sums) and the
    page's three steps written as scalar Python."""
    T, H = x.shape
    top_k = idx.shape[1]
    xf = oracle.bf16_to_f64(x)
    out = np.zeros((T, top_k, H), dtype=np.uint16)
    for t in range(T):
        for k in range(top_k):
            e = int(idx[t, k])
            Wg = oracle.dequant(gate[0][e], gate[1][e], gate[2][e], gs, bits, H)
            Wu = oracle.dequant(up[0][e], up[1][e], up[2][e], gs, bits, H)
            I = Wg.shape[0]
            hv = []
            for n in range(I):
                gv = float(oracle.bf16_to_f64(oracle.f64_to_bf16(math.fsum(xf[t] * Wg[n]))))
                uv = float(oracle.bf16_to_f64(oracle.f64_to_bf16(math.fsum(xf[t] * Wu[n]))))
                hv.append(float(oracle.bf16_to_f64(oracle.f64_to_bf16(gv / (1.0 + math.exp(-gv)) * uv))))
            Wd = oracle.dequant(down[0][e], down[1][e], down[2][e], gs, bits, I)
            out[t, k] = oracle.f64_to_bf16([math.fsum(np.array(hv) * Wd[j]) for j in range(H)])
    return out


def test_switch_glu_tiny_brute_force():
    sh = synth.TINY
    ex = synth.expert_set(0, sh.E, sh.H, sh.I, sh.gs, sh.bits, mode="drawn")
    x = synth.activations(0, 4, sh.H)
    idx = synth.sorted_topk(0, 4, sh.E, sh.top_k)
    got = oracle.switch_glu(x, idx, *ex, gs=sh.gs, bits=sh.bits)
    assert np.array_equal(got, _brute_switch_glu(x, idx, *ex, sh.gs, sh.bits))


def test_unsort_inverts_a_stable_expert_sort():
    """Rows put in expert order by an independent stable argsort come back to
    token order through the inverse permutation."""
    g = np.random.default_rng(31)
    T, top_k, E, H = 7, 3, 5, 4
    idx = np.sort(np.stack([g.choice(E, top_k, replace=False) for _ in range(T)]), axis=1)
    y_tok = g.integers(0, 1 << 16, size=(T, top_k, H)).astype(np.uint16)
    order = np.argsort(idx.reshape(-1), kind="stable")
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    assert np.array_equal(oracle.unsort(y_tok.reshape(T * top_k, H)[order], inv, T, top_k), y_tok)


def test_moe_prefill_layer_brute_force():
    """The sorted-route layer against token-order scalar code: each slot's
    brute-force SwitchGLU output times its score, summed in slot order in fp32
    with a bf16 rounding after each product and after the sum, plus the
    brute-force gated shared expert (sigmoid of its one-row gate logit), added
    in fp32 and rounded once.  A wrong permutation, gather row or slot order in
    the sort / unsort / combine composition changes the result."""
    sh = synth.TINY
    ex = synth.expert_set(0, sh.E, sh.H, sh.I, sh.gs, sh.bits, mode="drawn")
    g = np.random.default_rng(33)
    T = 5
    x = synth.activations(0, T, sh.H)
    idx = synth.sorted_topk(0, T, sh.E, sh.top_k)
    scores = synth.to_bf16(g.uniform(0.05, 0.6, size=(T, sh.top_k)))
    shp = (synth.drawn_matrix(g, sh.I, sh.H, sh.gs, sh.bits), synth.drawn_matrix(g, sh.I, sh.H, sh.gs, sh.bits),
           synth.drawn_matrix(g, sh.H, sh.I, sh.gs, sh.bits), synth.drawn_matrix(g, 1, sh.H, sh.gs, sh.bits))
    out, _ = oracle.moe_prefill_layer(x, idx, scores, ex, shp, gs=sh.gs, bits=sh.bits)
    y = _brute_switch_glu(x, idx, *ex, sh.gs, sh.bits)
    one = [tuple(a[None] for a in m) for m in shp[:3]]
    sw = _brute_switch_glu(x, np.zeros((T, 1), np.int64), *one, sh.gs, sh.bits)[:, 0]
    wz = oracle.dequant(*shp[3], sh.gs, sh.bits, sh.H)[0]
    xf = oracle.bf16_to_f64(x)
    f32 = np.float32
    r16 = lambda v: f32(oracle.bf16_to_f64(oracle.f64_to_bf16(float(v))))
    want = np.zeros((T, sh.H), np.uint16)
    for t in range(T):
        z = float(r16(math.fsum(xf[t] * wz)))
        for h in range(sh.H):
            acc = None
            for k in range(sh.top_k):
                p = r16(f32(oracle.bf16_to_f64(y[t, k, h])) * f32(oracle.bf16_to_f64(scores[t, k])))
                acc = p if acc is None else f32(acc + p)
            shared = r16(float(oracle.bf16_to_f64(sw[t, h])) / (1.0 + math.exp(-z)))
            want[t, h] = oracle.f64_to_bf16(float(f32(r16(acc) + shared)))
    assert np.array_equal(out, want)


def test_switch_glu_special_cases():
    sh = synth.TINY
    ex = list(synth.expert_set(0, sh.E, sh.H, sh.I, sh.gs, sh.bits, mode="drawn"))
    x = synth.activations(0, 4, sh.H)
    idx = synth.sorted_topk(0, 4, sh.E, sh.top_k)
    # gate = 0 -> silu(0) = 0 -> h = 0 -> y = 0
    zg = (ex[0][0], np.zeros_like(ex[0][1]), np.zeros_like(ex[0][2]))
    assert not oracle.switch_glu(x, idx, zg, ex[1], ex[2], gs=sh.gs, bits=sh.bits).any()
    # silu(g) = g for large g (1 + e^-40 == 1 in float64): constant gate 40 -> h = bf16(40 * u)
    cg = (ex[0][0], np.zeros_like(ex[0][1]), np.full_like(ex[0][2], oracle.f64_to_bf16(40.0 / sh.H)))
    xo = oracle.f64_to_bf16(np.ones((4, sh.H)))
    y1 = oracle.switch_glu(xo, idx, cg, ex[1], ex[2], gs=sh.gs, bits=sh.bits)
    for t in range(4):
        for k in range(sh.top_k):
            e = idx[t, k]
            Wu = oracle.dequant(ex[1][0][e], ex[1][1][e], ex[1][2][e], sh.gs, sh.bits, sh.H)
            u = oracle.bf16_to_f64(oracle.f64_to_bf16(Wu.sum(-1)))
            h = oracle.f64_to_bf16(40.0 * u)
            Wd = oracle.dequant(ex[2][0][e], ex[2][1][e], ex[2][2][e], sh.gs, sh.bits, sh.I)
            assert np.array_equal(y1[t, k], oracle.f64_to_bf16(Wd @ oracle.bf16_to_f64(h)))


# ----------------------------------------------------------------------------- sort and schedule
def test_sort_pairs_brute_force_and_invariants():
    g = np.random.default_rng(11)
    for T, top_k, E in ((1, 8, 288), (7, 2, 8), (64, 8, 16), (33, 4, 300)):
        idx = np.stack([np.sort(g.choice(E, top_k, replace=False)) for _ in range(T)])
        order, lhs, srhs, inv, counts, offsets = oracle.sort_pairs(idx, E)
        flat = idx.reshape(-1).tolist()
        want = sorted(range(len(flat)), key=lambda p: (flat[p], p))     # stable by pair index
        assert order.tolist() == want
        assert lhs.tolist() == [p // top_k for p in want]
        assert srhs.tolist() == [flat[p] for p in want]
        assert (order[inv] == np.arange(len(flat))).all() and (inv[order] == np.arange(len(flat))).all()
        assert counts.sum() == len(flat) and offsets[-1] == len(flat) and (np.diff(offsets) >= 0).all()
        assert all(counts[e] == flat.count(e) for e in range(E))


def test_schedule_worked_example():
    lines = {l.split()[0]: l for l in open(os.path.join(GOLD, "schedule_mlx4567.txt")) if not l.startswith("#")}
    bm = int(lines["bm"].split()[1])
    counts = [int(v) for v in lines["counts"].split()[1:]]
    offsets = np.concatenate([[0], np.cumsum(counts)])
    sched = oracle.schedule_tiles(offsets, bm)
    want = [tuple(int(v) for v in t.split(",")) for t in lines["scheduled"].split(")", 1)[1].split("|")]
    assert [tuple(t) for t in sched.tolist()] == want
    tiles, passes = oracle.naive_tiles(offsets, bm)
    assert passes.tolist() == [int(v) for v in lines["naive_passes"].split()[1:]]
    assert passes.sum() == 6 and len(sched) == 4
    per = [[int(v) for v in grp.split(",")] for grp in lines["naive_rows_per_expert"].split(None, 1)[1].split("|")]
    assert [sum(p) for p in per] == tiles[:, 1].tolist()


def test_schedule_random_invariants():
    g = np.random.default_rng(12)
    for _ in range(50):
        E = int(g.integers(1, 40))
        bm = int(g.choice([16, 32, 64, 128]))
        counts = g.integers(0, 300, E) * (g.random(E) < 0.7)
        offsets = np.concatenate([[0], np.cumsum(counts)])
        P = int(offsets[-1])
        sched = oracle.schedule_tiles(offsets, bm)
        assert sched[:, 2].sum() == P if len(sched) else P == 0
        assert (sched[:, 2] <= bm).all() and (sched[:, 2] > 0).all()
        for r0, e, v in sched:
            assert offsets[e] <= r0 and r0 + v <= offsets[e + 1]
        assert len(sched) == sum(-(-int(c) // bm) for c in counts)
        _, passes = oracle.naive_tiles(offsets, bm)
        assert len(sched) <= passes.sum()
        assert len(sched) <= P // bm + int((counts > 0).sum())


def test_hybrid_tiles_worked_example():
    """The two-size schedule on loads 200, 31, 0, 32, 5 (offsets 0 200 231 231
    263 268), 128- and 32-row tiles, 4 column blocks, worked by hand."""
    off = np.array([0, 200, 231, 231, 263, 268])
    # 8 slots: experts 0 and 3 reach 32 rows -> ceil(200/128) + ceil(32/128) = 3
    # tiles, x 4 column blocks = 12 items > 8 // 8 = 1, so two tile sizes
    big, small = oracle.hybrid_tiles(off, 0, 128, 32, 8, 4)
    assert big.tolist() == [[0, 0, 128], [128, 0, 72], [231, 3, 32]]
    assert small.tolist() == [[200, 1, 31], [263, 4, 5]]
    # 512 slots: 12 <= 512 // 8 = 64 items, so every expert takes 32-row tiles
    big, small = oracle.hybrid_tiles(off, 0, 128, 32, 512, 4)
    assert big.size == 0
    assert small.tolist() == [[0, 0, 32], [32, 0, 32], [64, 0, 32], [96, 0, 32], [128, 0, 32], [160, 0, 32],
                              [192, 0, 8], [200, 1, 31], [231, 3, 32], [263, 4, 5]]
    # an extra expert (index 5) of 40 rows at rows 268..307 joins each table last
    big, small = oracle.hybrid_tiles(off, 40, 128, 32, 8, 4)
    assert big.tolist() == [[0, 0, 128], [128, 0, 72], [231, 3, 32], [268, 5, 40]]
    assert small.tolist() == [[200, 1, 31], [263, 4, 5]]
    big, small = oracle.hybrid_tiles(off, 40, 128, 32, 512, 4)
    assert big.size == 0 and small.tolist()[-2:] == [[268, 5, 32], [300, 5, 8]]


def test_hybrid_tiles_reduce_to_one_size():
    """With every load at 32 rows or more and the fill rule off, the first
    table is the plain 128-row schedule; with the fill rule on, the second is
    the plain 32-row schedule."""
    g = np.random.default_rng(21)
    for _ in range(20):
        E = int(g.integers(1, 60))
        counts = g.integers(32, 700, E)
        off = np.concatenate([[0], np.cumsum(counts)])
        big, small = oracle.hybrid_tiles(off, 0, 128, 32, 0, 4)
        assert small.size == 0 and np.array_equal(big, oracle.schedule_tiles(off, 128))
        counts = g.integers(0, 700, E) * (g.random(E) < 0.7)
        off = np.concatenate([[0], np.cumsum(counts)])
        big, small = oracle.hybrid_tiles(off, 0, 128, 32, 1 << 40, 4)
        assert big.size == 0 and np.array_equal(small, oracle.schedule_tiles(off, 32))


def test_hybrid_tiles_random_invariants():
    """Random loads, both sides of the fill rule, with and without extra rows:
    every row of [0, P + extra) lies in exactly one tile; a tile stays inside
    its expert's rows and within its table's height; each table is
    expert-major with ascending row starts; with two sizes an expert's tiles
    sit in the first table exactly when it has at least 32 rows."""
    g = np.random.default_rng(22)
    for trial in range(60):
        E = int(g.integers(1, 300))
        counts = g.integers(0, 400, E) * (g.random(E) < 0.5)
        off = np.concatenate([[0], np.cumsum(counts)])
        P = int(off[-1])
        extra = int(g.integers(0, 300)) if trial % 2 else 0
        slots = int(g.choice([0, 512, 1 << 20]))
        big, small = oracle.hybrid_tiles(off, extra, 128, 32, slots, int(g.integers(1, 17)))
        ends = np.concatenate([off, [P + extra]])
        seen = np.zeros(P + extra, np.int64)
        for table, height in ((big, 128), (small, 32)):
            for r0, e, v in table:
                assert 0 < v <= height and ends[e] <= r0 and r0 + v <= ends[e + 1]
                seen[r0:r0 + v] += 1
            keys = [(int(e), int(r0)) for r0, e, _ in table]
            assert keys == sorted(keys)
        assert (seen == 1).all()
        if len(big):
            loads = np.concatenate([counts, [extra]])
            in_big = set(big[:, 1].tolist())
            assert in_big == {e for e in range(len(loads)) if loads[e] >= 32}


# ----------------------------------------------------------------------------- combine
def _torch_combine(y_sorted, inv, scores, shared):
    """Library route: torch bf16 arithmetic on the CPU (each op computes in fp32
    and rounds to bf16; the sum is an explicit fp32 loop)."""
    T, top_k = scores.shape
    ys = torch.from_numpy(y_sorted.astype(np.int16)).view(torch.bfloat16)
    sc = torch.from_numpy(scores.astype(np.int16)).view(torch.bfloat16)
    iv = torch.from_numpy(inv.astype(np.int64)).view(T, top_k)
    acc = None
    for k in range(top_k):
        p = ys[iv[:, k]] * sc[:, k:k + 1]
        acc = p.float() if acc is None else acc + p.float()
    out = acc.to(torch.bfloat16)
    if shared is not None:
        out = (out.float() + torch.from_numpy(shared.astype(np.int16)).view(torch.bfloat16).float()).to(torch.bfloat16)
    return out.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("T,top_k,H", [(5, 8, 64), (3, 1, 16), (17, 2, 40)])
def test_combine_matches_torch_bf16(T, top_k, H):
    g = np.random.default_rng(T * 7 + top_k)
    P = T * top_k
    y = synth.to_bf16(g.standard_normal((P, H)) * 3)
    inv = g.permutation(P).astype(np.int32)
    sc = synth.to_bf16(g.random((T, top_k)))
    sh = synth.to_bf16(g.standard_normal((T, H)))
    assert np.array_equal(oracle.combine(y, inv, sc, sh), _torch_combine(y, inv, sc, sh))
    assert np.array_equal(oracle.combine(y, inv, sc, None), _torch_combine(y, inv, sc, None))


def test_combine_special_cases():
    g = np.random.default_rng(13)
    T, top_k, H = 6, 4, 32
    P = T * top_k
    y = synth.to_bf16(g.standard_normal((P, H)))
    inv = g.permutation(P).astype(np.int32)
    # one-hot scores, no shared: the chosen slot's row comes back exactly
    sc = np.zeros((T, top_k), np.uint16)
    slot = g.integers(0, top_k, T)
    sc[np.arange(T), slot] = synth.to_bf16(np.float32(1.0))
    out = oracle.combine(y, inv, sc, None)
    for t in range(T):
        assert np.array_equal(out[t], y[inv[t * top_k + slot[t]]])
    # top_k = 1 with score 1 is a pure permutation
    inv1 = g.permutation(T).astype(np.int32)
    y1 = y[:T]
    out1 = oracle.combine(y1, inv1, synth.to_bf16(np.ones((T, 1), np.float32)), None)
    assert np.array_equal(out1, y1[inv1])


# ----------------------------------------------------------------------------- rms_norm, shared expert, chain
def test_rms_norm_against_torch():
    g = np.random.default_rng(14)
    x = synth.to_bf16(g.standard_normal((4, 256)) * 3)
    w = synth.to_bf16(g.standard_normal(256))
    xt = torch.from_numpy(synth.from_bf16(x).astype(np.float64))
    wt = torch.from_numpy(synth.from_bf16(w).astype(np.float64))
    ref = torch.nn.functional.rms_norm(xt, (256,), wt, eps=1e-6).numpy()
    assert np.array_equal(oracle.rms_norm(x, w, 1e-6), oracle.f64_to_bf16(ref))
    # constant row c: c / sqrt(c^2 + eps) * w
    c = oracle.f64_to_bf16(np.full((1, 256), 2.0))
    assert np.array_equal(oracle.rms_norm(c, w, 1e-6)[0], oracle.f64_to_bf16(2.0 / math.sqrt(4 + 1e-6) * synth.from_bf16(w)))


def test_shared_expert_gate_closed_form():
    # gate row with scale 0, bias 0 -> z = 0 -> sigmoid = 1/2 -> shared = bf16(s / 2) exactly
    sh = synth.PREFILL
    g = np.random.default_rng(15)
    H, I = 128, 64
    gate, up, down, grow = (synth.drawn_matrix(g, I, H, 64, 4), synth.drawn_matrix(g, I, H, 64, 4),
                            synth.drawn_matrix(g, H, I, 64, 4), synth.drawn_matrix(g, 1, H, 64, 4))
    grow0 = (grow[0], np.zeros_like(grow[1]), np.zeros_like(grow[2]))
    x = synth.to_bf16(g.standard_normal((3, H)))
    full = oracle.shared_expert(x, gate, up, down, grow0, 64, 4)
    swiglu = oracle.switch_glu(x, np.zeros((3, 1), np.int32), *[tuple(a[None] for a in m) for m in (gate, up, down)],
                               gs=64, bits=4)[:, 0]
    assert np.array_equal(full, oracle.f64_to_bf16(oracle.bf16_to_f64(swiglu) / 2))


def test_silu_against_torch():
    # SwitchGLU's activation (MLX issue 4509, moe(): silu(gate) * up) against torch's float64
    # silu over every bf16 value of magnitude up to 100, both signs
    import torch
    v = np.arange(0, 0x42C9, dtype=np.uint32).astype(np.uint16)
    g = np.concatenate([oracle.bf16_to_f64(v), -oracle.bf16_to_f64(v)])
    want = torch.nn.functional.silu(torch.from_numpy(g)).numpy()
    got = oracle.silu(g)
    assert np.all(np.abs(got - want) <= 4e-16 * np.abs(want) + 1e-300)
    assert oracle.silu(np.array([0.0]))[0] == 0.0 and oracle.silu(np.array([50.0]))[0] == 50.0


def test_shared_expert_gate_saturates_the_right_way():
    # gate row with scale 0 and bias 1 -> z = sum_k x_k; a constant row x = +-0.3125 over
    # H = 128 gives z = +-40 exactly.  sigmoid(40) = 1 - 4e-18, so the gated output is the
    # SwiGLU output itself; sigmoid(-40) = 4e-18, so it is below 1e-17 of it (a sign slip
    # in the exponent swaps the two)
    g = np.random.default_rng(16)
    H, I = 128, 64
    gate, up, down, grow = (synth.drawn_matrix(g, I, H, 64, 4), synth.drawn_matrix(g, I, H, 64, 4),
                            synth.drawn_matrix(g, H, I, 64, 4), synth.drawn_matrix(g, 1, H, 64, 4))
    one = synth.to_bf16(np.ones(1))[0]
    grow1 = (grow[0], np.zeros_like(grow[1]), np.full_like(grow[2], one))
    experts = [tuple(a[None] for a in m) for m in (gate, up, down)]
    for c in (0.3125, -0.3125):
        x = synth.to_bf16(np.full((2, H), c))
        assert np.array_equal(oracle.bf16_to_f64(oracle.quantized_matmul(x, *grow1, True, 64, 4)),
                              np.full((2, 1), 128 * c))
        full = oracle.bf16_to_f64(oracle.shared_expert(x, gate, up, down, grow1, 64, 4))
        swiglu = oracle.bf16_to_f64(oracle.switch_glu(x, np.zeros((2, 1), np.int32), *experts, gs=64, bits=4)[:, 0])
        assert np.abs(swiglu).max() > 0
        if c > 0:
            assert np.array_equal(full, swiglu)
        else:
            assert np.all(np.abs(full) <= 1e-17 * np.abs(swiglu))


def test_dense_forward_constant_weights_closed_form():
    """One layer with constant weights (scale 0, bias c): every projection is
    c * sum(input) broadcast along N, so the chain reduces to scalars per row."""
    d = dict(hidden=64, q_out=128, kv_out=64, inter=96, layers=1, sets=1)
    dims = synth.dense_dims(d)
    consts = {"q": 0.5, "k": 0.25, "v": -0.125, "o": 0.0625, "g": 0.03125, "u": -0.5, "dn": 0.25}
    L = {}
    for name, (N, K) in dims.items():
        L[name] = (np.zeros((N, K // 8), np.uint32), oracle.f64_to_bf16(np.zeros((N, K // 32))),
                   oracle.f64_to_bf16(np.full((N, K // 32), consts[name])))
    g = np.random.default_rng(16)
    h0 = synth.to_bf16(g.standard_normal((2, 64)))
    nw = oracle.f64_to_bf16(np.ones(64))
    got = oracle.dense_forward(h0, [L], 1, nw, gs=32, bits=4)
    r = lambda v: float(oracle.bf16_to_f64(oracle.f64_to_bf16(v)))
    for m in range(2):
        hrow = oracle.bf16_to_f64(h0[m])
        xs = oracle.bf16_to_f64(oracle.rms_norm(h0[m:m + 1], nw))[0].sum()
        q, k, v = r(0.5 * xs), r(0.25 * xs), r(-0.125 * xs)
        oin = r(q + r(k + v))
        o = r(0.0625 * oin * 128)
        h1 = oracle.bf16_to_f64(oracle.f64_to_bf16(hrow + o))
        x2 = oracle.bf16_to_f64(oracle.rms_norm(oracle.f64_to_bf16(h1)[None], nw))[0].sum()
        gg, uu = r(0.03125 * x2), r(-0.5 * x2)
        a = r(gg / (1 + math.exp(-gg)) * uu)
        dn = r(0.25 * a * 96)
        assert np.array_equal(got[m], oracle.f64_to_bf16(h1 + dn))


# ----------------------------------------------------------------------------- router
def test_route_selection_brute_force():
    """On tiny inputs the chosen set is the unique size-k subset whose every
    member beats every non-member (larger logit, or equal logit and lower id),
    found by enumerating all subsets."""
    import itertools
    g = np.random.default_rng(81)
    for E, k in ((5, 2), (6, 3), (7, 1), (4, 4)):
        for _ in range(20):
            lg = g.integers(-3, 4, size=(1, E)).astype(np.float32) * 0.5   # many equal logits
            beats = lambda a, b: lg[0, a] > lg[0, b] or (lg[0, a] == lg[0, b] and a < b)
            good = [S for S in itertools.combinations(range(E), k)
                    if all(beats(a, b) for a in S for b in range(E) if b not in S)]
            assert len(good) == 1
            idx, _ = oracle.route(lg, k)
            assert idx[0].tolist() == list(good[0])


def test_route_equal_logits_and_two_expert_closed_form():
    """All logits equal: the first k ids, each scored 1/E.  Two experts, k = 1:
    the larger one, scored 1 / (1 + e^-d) with d the logit gap (the logistic
    function), rounded to fp32 then bf16."""
    idx, sc = oracle.route(np.full((3, 10), 0.75, np.float32), 4)
    assert (idx == np.arange(4)).all()
    assert (sc == bf16_torch(np.float32(0.1))).all()
    for a, b in ((0.0, 1.0), (2.5, -1.25), (-3.0, -3.5), (7.0, 0.0)):
        idx, sc = oracle.route(np.array([[a, b]], np.float32), 1)
        d = abs(np.float64(np.float32(a)) - np.float64(np.float32(b)))
        assert idx[0, 0] == (0 if a >= b else 1)
        assert sc[0, 0] == bf16_torch(np.float32(1.0 / (1.0 + math.exp(-d))))[()]


def test_route_full_softmax_sums_to_one_and_matches_torch():
    """k = E: every score is the softmax probability; against torch's float64
    softmax (library route) after the same fp32 and bf16 roundings, and the
    unrounded probabilities sum to 1."""
    g = np.random.default_rng(82)
    lg = (g.standard_normal((6, 16)) * 3).astype(np.float32)
    idx, sc = oracle.route(lg, 16)
    assert (idx == np.arange(16)).all()
    p = torch.softmax(torch.from_numpy(lg.astype(np.float64)), dim=-1).numpy()
    assert np.array_equal(sc, bf16_torch(p.astype(np.float32)))
    assert np.allclose(p.sum(-1), 1.0, atol=1e-12)


def test_route_matches_the_input_recipe():
    """The routing recipe of the synthetic workloads (vectorised numpy) and the
    oracle's router (per-token loops, exactly summed softmax) agree bit for
    bit on the prefill shape."""
    for cfg, T, E, k in ((3, 96, 256, 8), (4, 40, 288, 8)):
        i1, s1 = synth.zipf_routing(cfg, T, E, k)
        i2, s2 = oracle.route(synth.zipf_logits(cfg, T, E), k)
        assert np.array_equal(i1, i2) and np.array_equal(s1, s2)


# ----------------------------------------------------------------------------- unquantized gather_mm
def test_gather_mm_brute_force_exact():
    """Tiny gather_mm against exact rational sums (Python loops, Fractions) of
    bf16 inputs, rounded once: every selected pair, every broadcast form."""
    g = np.random.default_rng(83)
    x = synth.to_bf16(g.standard_normal((3, 2, 5)).astype(np.float32))
    w = synth.to_bf16(g.standard_normal((4, 3, 5)).astype(np.float32))
    lhs = np.array([0, 2, 2, 1]); rhs = np.array([3, 0, 1, 3])
    got = oracle.gather_mm(x, w, lhs=lhs, rhs=rhs)
    xv, wv = oracle.bf16_to_f64(x), oracle.bf16_to_f64(w)
    for j in range(4):
        for m in range(2):
            for n in range(3):
                exact = sum(Fraction(float(xv[lhs[j], m, k])) * Fraction(float(wv[rhs[j], n, k])) for k in range(5))
                assert got[j, m, n] == oracle.f64_to_bf16(float(exact))
    # defaults: batch j of x against expert j when the batch shapes agree
    assert np.array_equal(oracle.gather_mm(x[:1], w[3:4])[0], got[0])


def test_gather_mm_rank_one_closed_form():
    """w_e = u_e v_e^T with small integers: out = (x . v_e) u_e, formed as a
    dot product first and a scaling second (all exact)."""
    g = np.random.default_rng(84)
    E, N, K, M = 3, 6, 16, 4
    u = g.integers(-3, 4, size=(E, N)).astype(np.float64)
    v = g.integers(-3, 4, size=(E, K)).astype(np.float64)
    w = oracle.f64_to_bf16(u[:, :, None] * v[:, None, :])
    x = oracle.f64_to_bf16(g.integers(-4, 5, size=(2, M, K)).astype(np.float64))
    rhs = np.array([2, 0, 1, 2, 1]); lhs = np.array([0, 1, 1, 0, 0])
    got = oracle.gather_mm(x, w, lhs=lhs, rhs=rhs)
    xv = oracle.bf16_to_f64(x)
    for j in range(len(rhs)):
        d = xv[lhs[j]] @ v[rhs[j]]
        want = oracle.f64_to_bf16(d[:, None] * u[rhs[j]][None, :])
        assert np.array_equal(oracle.bf16_to_f64(got[j]), oracle.bf16_to_f64(want))   # -0 == +0


def test_switch_glu_mm_matches_torch():
    """Unquantized SwitchGLU against torch's float64 matmul and SiLU (library
    route), with the same bf16 rounding points."""
    g = np.random.default_rng(85)
    E, H, I, T, k = 5, 32, 16, 6, 2
    mk = lambda *s: synth.to_bf16((g.standard_normal(s) * 0.3).astype(np.float32))
    gate, up, down = mk(E, I, H), mk(E, I, H), mk(E, H, I)
    x = mk(T, H)
    idx = np.stack([np.sort(g.choice(E, k, replace=False)) for _ in range(T)])
    got = oracle.switch_glu_mm(x, idx, gate, up, down)
    tb = lambda a: torch.from_numpy(oracle.bf16_to_f64(a))
    for t in range(T):
        for s_ in range(k):
            e = idx[t, s_]
            gg = tb(oracle.f64_to_bf16((tb(x[t]) @ tb(gate[e]).T).numpy()))
            uu = tb(oracle.f64_to_bf16((tb(x[t]) @ tb(up[e]).T).numpy()))
            hh = tb(oracle.f64_to_bf16((torch.nn.functional.silu(gg) * uu).numpy()))
            yy = oracle.f64_to_bf16((hh @ tb(down[e]).T).numpy())
            assert np.array_equal(got[t, s_], yy)


# ----------------------------------------------------------------------------- mx formats
def test_e4m3_and_e8m0_match_torch_decoders():
    # every E4M3 element code and every E8M0 scale code against torch's own
    # float8_e4m3fn / float8_e8m0fnu decoders
    torch = pytest.importorskip("torch")
    codes = np.arange(256)
    t = torch.arange(256, dtype=torch.uint8)
    want4 = t.view(torch.float8_e4m3fn).double().numpy()
    got4 = oracle.e4m3_to_f64(codes)
    assert np.array_equal(np.isnan(got4), np.isnan(want4))
    assert np.array_equal(got4[~np.isnan(got4)], want4[~np.isnan(want4)])
    assert np.array_equal(np.signbit(got4[~np.isnan(got4)]), np.signbit(want4[~np.isnan(want4)]))
    want8 = t.view(torch.float8_e8m0fnu).double().numpy()
    got8 = oracle.e8m0_to_f64(codes)
    assert np.array_equal(np.isnan(got8), np.isnan(want8))
    assert np.array_equal(got8[:255], want8[:255])


def test_e2m1_is_the_e4m3_subset():
    # an E2M1 element (exponent bias 1, one mantissa bit) has the value of the
    # E4M3 element with exponent e + 6 and mantissa 4 m (normal), or of the
    # E4M3 subnormal-free code for 0.5 (e = 0, m = 1) and zero; checked through
    # torch's E4M3 decoder
    torch = pytest.importorskip("torch")
    got = oracle.e2m1_to_f64(np.arange(16))
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        if e > 0:
            e4 = (s << 7) | ((e + 6) << 3) | (m << 2)
        else:
            e4 = (s << 7) | (6 << 3) if m else (s << 7)
        want = torch.tensor([e4], dtype=torch.uint8).view(torch.float8_e4m3fn).double().item()
        assert got[c] == want and np.signbit(got[c]) == np.signbit(want), c
    assert np.all(np.diff(got[:8]) > 0) and got[7] == 6.0


def _brute_mx(x, words, scales, mode, transpose):
    """Triple loop in exact rationals: element value (from the bit string) times
    2^(scale - 127)."""
    bits = oracle.MX_MODES[mode]
    xa = np.asarray(x)
    xvals = xa.astype(np.float64) if xa.dtype in (np.float16, np.float32) else oracle.bf16_to_f64(xa)
    xv = [[Fraction(float(v)) for v in row] for row in xvals]

    def elem(code):
        if mode == "mxfp4":
            s, e, m = code >> 3, (code >> 1) & 3, code & 1
            mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
        else:
            s, e, m = code >> 7, (code >> 3) & 15, code & 7
            mag = Fraction(m, 8) * Fraction(1, 64) if e == 0 else Fraction(2) ** (e - 7) * (1 + Fraction(m, 8))
        return -mag if s else mag

    rows = ["".join(format(int(v), "032b")[::-1] for v in wr) for wr in words]
    L = len(rows[0]) // bits

    def W(r, c):
        code = int(rows[r][c * bits:(c + 1) * bits][::-1], 2)
        return elem(code) * Fraction(2) ** (int(scales[r][c // 32]) - 127)

    if transpose:
        N, K = len(words), L
        out = [[float(sum(xv[mm][k] * W(n, k) for k in range(K))) for n in range(N)] for mm in range(len(xv))]
    else:
        K, N = len(words), L
        out = [[float(sum(xv[mm][k] * W(k, n) for k in range(K))) for n in range(N)] for mm in range(len(xv))]
    if xa.dtype in (np.float16, np.float32):
        return np.array(out).astype(np.float32)
    return oracle.f64_to_bf16(np.array(out))


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8"])
def test_mx_matmul_brute_force(mode):
    g = np.random.default_rng(21 if mode == "mxfp4" else 22)
    bits = oracle.MX_MODES[mode]
    M, N, K = 2, 3, 64
    # codes away from E4M3's NaN pattern; scales around 2^0
    codes = g.integers(0, 1 << bits, size=(N, K))
    if bits == 8:
        codes = np.where((codes & 0x7F) == 0x7F, 0x7E, codes)
    w = synth.pack(codes, bits)
    sc = g.integers(120, 134, size=(N, K // 32)).astype(np.uint8)
    x = synth.to_bf16(g.standard_normal((M, K)))
    got = oracle.mx_matmul(x, w, sc, mode, True)
    assert np.array_equal(got, _brute_mx(x, w, sc, mode, True))
    # without the transpose: [K'=5, N'=64] with blocks along N; float32 activations
    codes2 = g.integers(0, 1 << bits, size=(5, 64))
    if bits == 8:
        codes2 = np.where((codes2 & 0x7F) == 0x7F, 0x01, codes2)
    w2 = synth.pack(codes2, bits)
    sc2 = g.integers(110, 140, size=(5, 2)).astype(np.uint8)
    x2 = g.standard_normal((M, 5)).astype(np.float32)
    got2 = oracle.mx_matmul(x2, w2, sc2, mode, False)
    assert got2.dtype == np.float32
    assert np.array_equal(got2, _brute_mx(x2, w2, sc2, mode, False))


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8"])
def test_gather_qmm_mx_selects_pairs(mode):
    """gather_qmm_mx takes x[lhs] and expert rhs per pair over the broadcast
    index shape; each pair equals the exact-rational product of that pair."""
    g = np.random.default_rng(41 if mode == "mxfp4" else 42)
    bits = oracle.MX_MODES[mode]
    E, N, K, X, M = 3, 2, 64, 4, 1
    codes = g.integers(0, 1 << bits, size=(E, N, K))
    if bits == 8:
        codes = np.where((codes & 0x7F) == 0x7F, 0x7E, codes)
    w = np.stack([synth.pack(codes[e], bits) for e in range(E)])
    sc = g.integers(120, 134, size=(E, N, K // 32)).astype(np.uint8)
    x = synth.to_bf16(g.standard_normal((X, M, K)))
    lhs, rhs = np.array([[3], [0]]), np.array([[2, 0, 1]])
    got = oracle.gather_qmm_mx(x, w, sc, lhs=lhs, rhs=rhs, transpose=True, mode=mode)
    assert got.shape == (2, 3, M, N)
    for i in range(2):
        for j in range(3):
            assert np.array_equal(got[i, j], _brute_mx(x[lhs[i, 0]], w[rhs[0, j]], sc[rhs[0, j]], mode, True))


def test_mx_block_scale_applies_to_its_32_elements():
    # one element code (1.0 in both element types) everywhere, block scales
    # 2^0, 2^1, 2^-3: the dequantized row is 1, 2, 1/8 over the three blocks
    for mode, one in (("mxfp4", 0b0010), ("mxfp8", 0x38)):
        bits = oracle.MX_MODES[mode]
        w = synth.pack(np.full((1, 96), one), bits)
        d = oracle.mx_dequant(w, np.array([[127, 128, 124]], dtype=np.uint8), mode, 96)
        assert d[0].tolist() == [1.0] * 32 + [2.0] * 32 + [0.125] * 32
