"""GPU parity of the vector-unit route of gather_qmm against the oracle:
weights without the transpose ([E, K, N*bits/32], groups along N), float16
/ float32 activations (float32 result) in both layouts, and the bit widths
1, 2, 3, 5 and 6 (codes straddling words) in both layouts, with and without
the split of K, ragged column strips, row blocks and K tails.

Tolerances: bf16 results use the fixed bar |gpu - oracle| <= 1e-2 max|oracle|.
float32 results are held to the recursive-summation bound of the fp32
arithmetic: per output, |gpu - oracle| <= (K + 8) 2^-24 sum_k |x_k| (q_k |s| + |b|)
plus one ulp of the result (the kernel forms x s q and x b as separate
terms, so their magnitudes, not |x w|, set the bound)."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_parity, bf, host_bf, i32, words

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_gathered_amd as m
    m.lib()
    return m


def _experts(g, E, rows, cols, gs, bits):
    """E matrices [rows, cols] quantized along cols (the packed axis)."""
    ms = [synth.drawn_matrix(g, rows, cols, gs, bits) for _ in range(E)]
    return tuple(np.stack([m[i] for m in ms]) for i in range(3))


def _acts(g, shape, kind):
    v = g.standard_normal(shape).astype(np.float32)
    if kind == "bf16":
        return synth.to_bf16(v)
    if kind == "f16":
        return v.astype(np.float16)
    return (v * np.float32(1 + 2.0 ** -12)).astype(np.float32)     # off the bf16 grid


def _dev_acts(a):
    if a.dtype == np.uint16:
        return bf(a)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _abs_bound(x, w, s, b, lhs, rhs, transpose, gs, bits):
    """sum_k |x_k| (q_k |s| + |b|) per output, float64 (codes are >= 0)."""
    xf, _ = oracle.activations_f64(x)
    out = []
    for l, r in zip(lhs, rhs):
        s_abs = synth.to_bf16(np.abs(synth.from_bf16(s[r])))
        b_abs = synth.to_bf16(np.abs(synth.from_bf16(b[r])))
        if transpose:
            K = xf.shape[-1]
            W = oracle.dequant(w[r], s_abs, b_abs, gs, bits, K)          # [N, K]
            out.append(np.abs(xf[l]) @ W.T)
        else:
            N = w.shape[-1] * 32 // bits
            W = oracle.dequant(w[r], s_abs, b_abs, gs, bits, N)          # [K, N]
            out.append(np.abs(xf[l]) @ W)
    return np.stack(out)


def _check(got_t, want, x, w, s, b, lhs, rhs, transpose, gs, bits, name):
    if want.dtype == np.uint16:
        assert got_t.dtype == torch.bfloat16, name
        assert_parity(host_bf(got_t), want, name=name)
        return
    assert got_t.dtype == torch.float32, name
    got = got_t.cpu().numpy().astype(np.float64)
    w64 = want.astype(np.float64)
    assert np.isfinite(got).all(), name
    K = x.shape[-1]
    bound = (K + 8) * 2.0 ** -24 * _abs_bound(x, w, s, b, lhs, rhs, transpose, gs, bits).reshape(w64.shape)
    bound += np.spacing(np.abs(w64).astype(np.float32)).astype(np.float64)
    err = np.abs(got - w64)
    bad = err > bound
    assert not bad.any(), f"{name}: {bad.sum()} outputs off, worst {err[bad].max():.3g} vs {bound[bad].min():.3g}"


def _run(mg, g, *, kind, transpose, bits, gs, X, M, K, N, E, P, lhs_mode, name):
    x = _acts(g, (X, M, K), kind)
    rows, cols = (N, K) if transpose else (K, N)
    w, s, b = _experts(g, E, rows, cols, gs, bits)
    rhs = g.integers(0, E, size=P).astype(np.int32)
    if lhs_mode == "div":
        div = max(1, P // X)
        lhs = np.arange(P) // div
        lhs_t, kw = None, dict(lhs_div=div)
    else:
        lhs = g.integers(0, X, size=P)
        lhs_t, kw = i32(lhs), {}
    got = _gather(mg, _dev_acts(x), words(w), bf(s), bf(b), i32(rhs), lhs_t, transpose, gs, bits, **kw)
    want = oracle.gather_qmm(x, w, s, b, lhs=lhs, rhs=rhs, transpose=transpose, gs=gs, bits=bits)
    _check(got, want, x, w, s, b, lhs, rhs, transpose, gs, bits, name)


def _gather(mg, x, w, s, b, rhs, lhs, transpose, gs, bits, lhs_div=1):
    """gather_qmm through the C ABI with an explicit lhs_div (the binding's
    broadcast marshalling is exercised separately)."""
    import ctypes
    X, M, K = x.shape
    E = w.shape[0]
    N = w.shape[1] if transpose else w.shape[2] * 32 // bits
    P = rhs.numel()
    odt = torch.bfloat16 if x.dtype == torch.bfloat16 else torch.float32
    out = torch.empty((P, M, N), dtype=odt, device=x.device)
    need = mg.gather_qmm_workspace_bytes(P, E, M, N, K, mg._dt(x), transpose, bits, False)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    st = mg.lib().moegq_gather_qmm(mg._ptr(x), mg._dt(x), X, M, K, mg._ptr(w), mg.U32, mg._ptr(s), mg._ptr(b), E, N,
                                   mg._ptr(lhs), lhs_div, mg._ptr(rhs), mg.I32, P, 0, int(transpose), gs, bits,
                                   mg._ptr(out), ctypes.c_void_p(ws.data_ptr()), need, mg._stream())
    assert st == 0, mg.lib().moegq_status_string(st)
    torch.cuda.synchronize()
    return out


# without the transpose: one pair per row block; the column count leaves a
# ragged last strip (2112 columns = 264 words at 4 bits), K leaves a tail of
# 2 rows after the 4-row steps and of 10 after the 64-row activation chunks
NT_CASES = [
    # kind, bits, gs, X, M, K, N, E, P, lhs_mode
    ("bf16", 4, 64, 1, 1, 202, 2112, 3, 2, "div"),      # few items: K split
    ("bf16", 8, 32, 4, 3, 96, 160, 5, 9, "idx"),        # 8-bit, narrow strips (one word per lane)
    ("bf16", 4, 128, 2, 16, 256, 512, 4, 6, "div"),     # 16 rows: four row blocks
    ("f16", 4, 32, 3, 2, 130, 1024, 6, 5, "idx"),
    ("f32", 8, 128, 2, 5, 64, 2048, 2, 4, "div"),       # 8-bit, 4 words per lane
    ("f32", 4, 64, 64, 1, 320, 256, 16, 300, "idx"),    # many pairs: no split
]


@pytest.mark.parametrize("case", NT_CASES, ids=[f"{c[0]}-{c[1]}b-gs{c[2]}-M{c[4]}-K{c[5]}-N{c[6]}" for c in NT_CASES])
def test_without_transpose(mg, case):
    kind, bits, gs, X, M, K, N, E, P, lhs_mode = case
    g = np.random.default_rng(zlib.crc32(repr(case).encode()))
    _run(mg, g, kind=kind, transpose=False, bits=bits, gs=gs, X=X, M=M, K=K, N=N, E=E, P=P, lhs_mode=lhs_mode,
         name=f"nt {case}")


# with the transpose, float16 / float32 activations: N leaves a ragged row
# block (4 rows per wave), K spans several 128-word slices and a partial one
T_CASES = [
    ("f16", 4, 64, 1, 1, 4160, 37, 3, 2, "div"),        # K split over slices
    ("f32", 4, 32, 2, 2, 256, 130, 4, 6, "idx"),
    ("f32", 8, 128, 3, 4, 1152, 64, 2, 3, "div"),
    ("f16", 8, 32, 2, 7, 96, 45, 3, 4, "idx"),          # two row blocks
    ("f32", 4, 64, 8, 1, 2048, 256, 8, 64, "div"),      # decode-like
]


@pytest.mark.parametrize("case", T_CASES, ids=[f"{c[0]}-{c[1]}b-gs{c[2]}-M{c[4]}-K{c[5]}-N{c[6]}" for c in T_CASES])
def test_half_single_with_transpose(mg, case):
    kind, bits, gs, X, M, K, N, E, P, lhs_mode = case
    g = np.random.default_rng(zlib.crc32(repr(case).encode()))
    _run(mg, g, kind=kind, transpose=True, bits=bits, gs=gs, X=X, M=M, K=K, N=N, E=E, P=P, lhs_mode=lhs_mode,
         name=f"t {case}")


# every width of the format (nuvec "round_trip_error_is_about_half_a_step":
# 1-6 and 8 bits), both layouts, all three activation types
W_CASES = [
    # kind, transpose, bits, gs, X, M, K, N, E, P, lhs_mode
    ("bf16", True, 3, 32, 1, 1, 4128, 37, 3, 2, "div"),     # 3 bits: two 2048-code slices and a tail
    ("bf16", True, 5, 64, 2, 2, 320, 45, 4, 6, "idx"),
    ("f32", True, 6, 128, 3, 3, 256, 9, 2, 3, "div"),
    ("f16", True, 2, 64, 2, 1, 2112, 70, 3, 4, "idx"),
    ("bf16", True, 1, 32, 1, 1, 96, 130, 2, 2, "div"),
    ("bf16", False, 3, 32, 1, 1, 202, 2080, 3, 2, "div"),   # 65 chunks of 32 columns: a ragged strip
    ("f32", False, 5, 64, 2, 2, 130, 192, 4, 6, "idx"),
    ("f16", False, 6, 128, 3, 5, 64, 256, 2, 3, "div"),
    ("bf16", False, 2, 32, 2, 16, 96, 96, 3, 4, "idx"),
    ("f32", False, 1, 64, 1, 1, 300, 4096, 2, 2, "div"),
]


@pytest.mark.parametrize("case", W_CASES,
                         ids=[f"{c[0]}-{'t' if c[1] else 'nt'}-{c[2]}b-gs{c[3]}-M{c[5]}-K{c[6]}-N{c[7]}" for c in W_CASES])
def test_other_bit_widths(mg, case):
    kind, tr, bits, gs, X, M, K, N, E, P, lhs_mode = case
    g = np.random.default_rng(zlib.crc32(repr(case).encode()))
    _run(mg, g, kind=kind, transpose=tr, bits=bits, gs=gs, X=X, M=M, K=K, N=N, E=E, P=P, lhs_mode=lhs_mode,
         name=f"w {case}")


def test_split_and_unsplit_agree_with_oracle(mg):
    """The same product with one pair (split over K) and with the pair
    repeated 4096 times (enough waves: no split)."""
    g = np.random.default_rng(77)
    K, N, gs, bits = 1024, 512, 64, 4
    x = _acts(g, (1, 1, K), "bf16")
    w, s, b = _experts(g, 1, K, N, gs, bits)
    want = oracle.gather_qmm(x, w, s, b, lhs=[0], rhs=[0], transpose=False, gs=gs, bits=bits)
    assert mg.gather_qmm_workspace_bytes(1, 1, 1, N, K, mg.BF16, False, bits, False) > 0
    assert mg.gather_qmm_workspace_bytes(4096, 1, 1, N, K, mg.BF16, False, bits, False) == 0
    one = _gather(mg, bf(x), words(w), bf(s), bf(b), i32([0]), None, False, gs, bits)
    many = _gather(mg, bf(x), words(w), bf(s), bf(b), i32(np.zeros(4096)), None, False, gs, bits, lhs_div=4096)
    assert_parity(host_bf(one), want, name="split")
    for j in (0, 1, 4095):
        assert_parity(host_bf(many[j:j + 1]), want, name=f"unsplit {j}")


def test_quantized_matmul_batched_weights_promote(mg):
    """nuvec's batched case: weights [2, 1, 16, 64] (group 32, 4 bits) against
    float32 activations [3, 5, 64] give float32 [2, 3, 5, 16]."""
    g = np.random.default_rng(11)
    w, s, b = _experts(g, 2, 16, 64, 32, 4)
    w4, s4, b4 = w.reshape(2, 1, 16, 8), s.reshape(2, 1, 16, 2), b.reshape(2, 1, 16, 2)
    x = _acts(g, (3, 5, 64), "f32")
    got = mg.quantized_matmul(_dev_acts(x), words(w4), bf(s4), bf(b4), transpose=True, group_size=32, bits=4)
    assert tuple(got.shape) == (2, 3, 5, 16) and got.dtype == torch.float32
    want = oracle.gather_qmm(x, w4, s4, b4, transpose=True, gs=32, bits=4)
    lhs = np.tile(np.arange(3), 2)
    rhs = np.repeat(np.arange(2), 3)
    _check(got.reshape(6, 5, 16), want.reshape(6, 5, 16), x, w, s, b, lhs, rhs, True, 32, 4, "batched")


def test_quantized_matmul_dense_without_transpose(mg):
    """2-D weights [K, N/8] without the transpose, bf16 and float16 rows."""
    g = np.random.default_rng(12)
    K, N, gs, bits = 300, 384, 128, 4
    w, s, b = synth.drawn_matrix(g, K, N, gs, bits)
    for kind in ("bf16", "f16"):
        x = _acts(g, (7, K), kind)
        got = mg.quantized_matmul(_dev_acts(x), words(w), bf(s), bf(b), transpose=False, group_size=gs, bits=bits)
        assert tuple(got.shape) == (7, N)
        want = oracle.quantized_matmul(x, w, s, b, False, gs, bits)
        _check(got.reshape(1, 7, N), want.reshape(1, 7, N), x.reshape(1, 7, K), w[None], s[None], b[None],
               [0], [0], False, gs, bits, f"dense {kind}")


def test_decode_shape_without_transpose_sampled(mg):
    """The decode gate projection in the layout without the transpose: one
    token, 8 of 288 experts [4096, 2048] at 4 bits / group 64 (weights drawn
    for the 8 selected experts only); every output checked."""
    g = np.random.default_rng(13)
    K, N, gs, bits, P = 4096, 2048, 64, 4, 8
    w, s, b = _experts(g, P, K, N, gs, bits)
    x = _acts(g, (1, 1, K), "bf16")
    rhs = np.arange(P, dtype=np.int32)
    got = _gather(mg, bf(x), words(w), bf(s), bf(b), i32(rhs), None, False, gs, bits, lhs_div=P)
    want = oracle.gather_qmm(x, w, s, b, lhs=np.zeros(P, np.int64), rhs=rhs, transpose=False, gs=gs, bits=bits)
    assert_parity(host_bf(got), want, name="decode nt")


def test_empty_and_degenerate(mg):
    g = np.random.default_rng(14)
    w, s, b = _experts(g, 2, 64, 64, 32, 4)
    x = torch.zeros((1, 1, 64), dtype=torch.float32, device="cuda")
    out = _gather(mg, x, words(w), bf(s), bf(b), i32(np.zeros(0)), None, False, 32, 4)
    assert out.numel() == 0
    # zero activations give exactly zero
    z = _gather(mg, x, words(w), bf(s), bf(b), i32([1]), None, False, 32, 4)
    assert torch.count_nonzero(z).item() == 0


# ----------------------------------------------------------------------------- mx modes
def _mx_weights(g, E, rows, cols, mode, nan_free=True):
    """E matrices [rows, cols] of mx elements packed along cols, E8M0 scales
    around 2^0 (uint8 [E, rows, cols / 32])."""
    bits = oracle.MX_MODES[mode]
    codes = g.integers(0, 1 << bits, size=(E, rows, cols))
    if bits == 8 and nan_free:
        codes = np.where((codes & 0x7F) == 0x7F, 0x7E, codes)
    w = synth.pack(codes, bits)
    sc = g.integers(118, 136, size=(E, rows, cols // 32)).astype(np.uint8)
    return w, sc


def _mx_gather(mg, x, w, sc, rhs, lhs, transpose, mode, lhs_div=1):
    import ctypes
    X, M, K = x.shape
    E = w.shape[0]
    bits = oracle.MX_MODES[mode]
    code = mg.MX_MODES[mode][0]
    N = w.shape[1] if transpose else w.shape[2] * 32 // bits
    P = rhs.numel()
    odt = torch.bfloat16 if x.dtype == torch.bfloat16 else torch.float32
    out = torch.empty((P, M, N), dtype=odt, device=x.device)
    need = mg.lib().moegq_gather_qmm_mx_workspace_bytes(P, M, N, K, int(transpose), code)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    st = mg.lib().moegq_gather_qmm_mx(mg._ptr(x), mg._dt(x), X, M, K, mg._ptr(w), mg._ptr(sc), E, N, mg._ptr(lhs),
                                      lhs_div, mg._ptr(rhs), mg.I32, P, int(transpose), code, mg._ptr(out),
                                      ctypes.c_void_p(ws.data_ptr()), need, mg._stream())
    assert st == 0, mg.lib().moegq_status_string(st)
    torch.cuda.synchronize()
    return out


def _mx_check(got_t, want, x, w, sc, lhs, rhs, transpose, mode, name):
    if want.dtype == np.uint16:
        assert got_t.dtype == torch.bfloat16, name
        assert_parity(host_bf(got_t), want, name=name)
        return
    got = got_t.cpu().numpy().astype(np.float64)
    w64 = want.astype(np.float64)
    xf, _ = oracle.activations_f64(x)
    bits = oracle.MX_MODES[mode]
    bound = []
    for l, r in zip(lhs, rhs):
        L = xf.shape[-1] if transpose else w.shape[-1] * 32 // bits
        W = np.abs(oracle.mx_dequant(w[r], sc[r], mode, L))
        bound.append(np.abs(xf[l]) @ (W.T if transpose else W))
    K = x.shape[-1]
    bound = (K + 8) * 2.0 ** -24 * np.stack(bound).reshape(w64.shape)
    bound += np.spacing(np.abs(w64).astype(np.float32)).astype(np.float64)
    err = np.abs(got - w64)
    assert not (err > bound).any(), f"{name}: worst {err.max():.3g}"


MX_CASES = [
    # kind, transpose, mode, X, M, K, N, E, P, lhs_mode
    ("bf16", True, "mxfp8", 1, 1, 4160, 37, 3, 2, "div"),
    ("bf16", True, "mxfp4", 2, 2, 320, 45, 4, 6, "idx"),
    ("f32", True, "mxfp4", 3, 3, 2080, 9, 2, 3, "div"),
    ("f16", True, "mxfp8", 2, 1, 96, 70, 3, 4, "idx"),
    ("bf16", False, "mxfp4", 1, 1, 202, 2080, 3, 2, "div"),
    ("bf16", False, "mxfp8", 2, 5, 130, 192, 4, 6, "idx"),
    ("f32", False, "mxfp8", 3, 2, 64, 256, 2, 3, "div"),
    ("f16", False, "mxfp4", 2, 16, 96, 96, 3, 4, "idx"),
]


@pytest.mark.parametrize("case", MX_CASES,
                         ids=[f"{c[0]}-{'t' if c[1] else 'nt'}-{c[2]}-M{c[4]}-K{c[5]}-N{c[6]}" for c in MX_CASES])
def test_mx_modes(mg, case):
    kind, tr, mode, X, M, K, N, E, P, lhs_mode = case
    g = np.random.default_rng(zlib.crc32(repr(case).encode()))
    x = _acts(g, (X, M, K), kind)
    rows, cols = (N, K) if tr else (K, N)
    w, sc = _mx_weights(g, E, rows, cols, mode)
    rhs = g.integers(0, E, size=P).astype(np.int32)
    if lhs_mode == "div":
        div = max(1, P // X)
        lhs, lhs_t, kw = np.arange(P) // div, None, dict(lhs_div=div)
    else:
        lhs = g.integers(0, X, size=P)
        lhs_t, kw = i32(lhs), {}
    sc_t = torch.from_numpy(sc).cuda()
    got = _mx_gather(mg, _dev_acts(x), words(w), sc_t, i32(rhs), lhs_t, tr, mode, **kw)
    want = oracle.gather_qmm_mx(x, w, sc, lhs=lhs, rhs=rhs, transpose=tr, mode=mode)
    _mx_check(got, want, x, w, sc, lhs, rhs, tr, mode, f"mx {case}")


def test_mx_special_values(mg):
    """E8M0 byte 255 (NaN) poisons its block's outputs, byte 0 (2^-127) and
    E4M3 NaN elements follow the oracle; NaN positions must agree exactly."""
    g = np.random.default_rng(41)
    K, N = 128, 8
    x = _acts(g, (1, 1, K), "f32")
    codes = g.integers(0, 256, size=(1, N, K))
    codes = np.where((codes & 0x7F) == 0x7F, 0x7E, codes)
    codes[0, 5, 77] = 0xFF                            # one E4M3 NaN element in row 5
    w = synth.pack(codes, 8)
    sc = g.integers(118, 136, size=(1, N, K // 32)).astype(np.uint8)
    sc[0, 1, 2] = 255                                 # NaN scale: row 1
    sc[0, 2, 0] = 0                                   # 2^-127: row 2's first block vanishes
    got = _mx_gather(mg, _dev_acts(x), words(w), torch.from_numpy(sc).cuda(), i32([0]), None, True, "mxfp8")
    want = oracle.gather_qmm_mx(x, w, sc, lhs=[0], rhs=[0], transpose=True, mode="mxfp8")
    gv = got.cpu().numpy()
    assert np.array_equal(np.isnan(gv), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.allclose(gv[ok], want[ok], rtol=1e-5, atol=1e-30)


def test_quantized_matmul_mx_binding(mg):
    """The binding's quantized_matmul with mode="mxfp4": 2-D weights, bf16 rows."""
    g = np.random.default_rng(42)
    K, N = 256, 64
    w, sc = _mx_weights(g, 1, N, K, "mxfp4")
    x = _acts(g, (5, K), "bf16")
    got = mg.quantized_matmul(_dev_acts(x), words(w[0]), torch.from_numpy(sc[0]).cuda(), transpose=True,
                              mode="mxfp4")
    assert tuple(got.shape) == (5, N)
    want = oracle.mx_matmul(x, w[0], sc[0], "mxfp4", True)
    assert_parity(host_bf(got), want, name="qmm mx")


# ----------------------------------------------------------------------------- bitwise pins
EXACT_CASES = [
    # kind, transpose, bits, gs, M, K, N, P
    ("bf16", False, 4, 64, 1, 2048, 256, 1),     # split over K
    ("f32", False, 8, 32, 3, 512, 96, 2),
    ("f16", True, 4, 128, 2, 1024, 40, 3),
    ("f32", True, 3, 32, 1, 4096, 24, 1),        # split over slices
    ("bf16", False, 5, 64, 5, 320, 128, 2),
    ("bf16", True, 6, 64, 1, 640, 33, 2),
    ("bf16", True, 2, 32, 4, 256, 50, 2),
    ("f16", False, 1, 32, 2, 96, 2048, 1),
]


@pytest.mark.parametrize("case", EXACT_CASES, ids=[f"{c[0]}-{'t' if c[1] else 'nt'}-{c[2]}b-M{c[4]}" for c in EXACT_CASES])
def test_vector_route_integer_exact_bitwise(mg, case):
    """Scales 2^-2, integer biases times 2^-2 and small-integer activations:
    every product and partial sum (and the sum of the K split's partials) is
    exact in fp32, so the GPU equals the oracle bit for bit."""
    kind, tr, bits, gs, M, K, N, P = case
    g = np.random.default_rng(zlib.crc32(repr(case).encode()))
    rows, cols = (N, K) if tr else (K, N)
    ms = [synth.integer_exact(g, rows, cols, gs, bits) for _ in range(P)]
    w, s, b = (np.stack([m[i] for m in ms]) for i in range(3))
    xi = g.integers(-8, 9, size=(1, M, K)).astype(np.float32)
    x = synth.to_bf16(xi) if kind == "bf16" else xi.astype(np.float16 if kind == "f16" else np.float32)
    rhs = np.arange(P, dtype=np.int32)
    got = _gather(mg, _dev_acts(x), words(w), bf(s), bf(b), i32(rhs), None, tr, gs, bits, lhs_div=P)
    want = oracle.gather_qmm(x, w, s, b, lhs=np.zeros(P, np.int64), rhs=rhs, transpose=tr, gs=gs, bits=bits)
    if want.dtype == np.uint16:
        assert np.array_equal(host_bf(got), want)
    else:
        assert np.array_equal(got.cpu().numpy(), want)


@pytest.mark.parametrize("mode,tr", [("mxfp8", True), ("mxfp4", False), ("mxfp8", False), ("mxfp4", True)])
def test_mx_integer_exact_bitwise(mg, mode, tr):
    """mx elements with exponents near 2^0 (E4M3: exponent field 6..8), block
    scales 2^-1..2^1 and small-integer activations: exact in fp32, so bit for
    bit."""
    g = np.random.default_rng(zlib.crc32((mode + str(tr)).encode()))
    bits = oracle.MX_MODES[mode]
    M, K, N = 3, 1024, 64
    rows, cols = (N, K) if tr else (K, N)
    if bits == 8:
        codes = (g.integers(0, 2, size=(1, rows, cols)) << 7) | (g.integers(6, 9, size=(1, rows, cols)) << 3) \
            | g.integers(0, 8, size=(1, rows, cols))
    else:
        codes = g.integers(0, 16, size=(1, rows, cols))
    w = synth.pack(codes, bits)
    sc = g.integers(126, 129, size=(1, rows, cols // 32)).astype(np.uint8)
    x = g.integers(-8, 9, size=(1, M, K)).astype(np.float32)
    got = _mx_gather(mg, _dev_acts(x), words(w), torch.from_numpy(sc).cuda(), i32([0]), None, tr, mode)
    want = oracle.gather_qmm_mx(x, w, sc, lhs=[0], rhs=[0], transpose=tr, mode=mode)
    assert np.array_equal(got.cpu().numpy(), want)
