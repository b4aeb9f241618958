"""GPU parity: decode path (gathered qmv, SwitchGLU DECODE) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_parity, bf, host_bf, i32, triple, words

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_gathered_amd as m
    m.lib()
    return m


def _experts(ex):
    return [triple(m) for m in ex]


def test_tiny_switch_glu_decode_and_sorted(mg):
    """Tiny SwitchGLU: E=8, top-2, hidden 256, inter 128, 4-bit GS 64, M=4."""
    sh = synth.TINY
    ex = synth.expert_set(0, sh.E, sh.H, sh.I, sh.gs, sh.bits, mode="drawn")
    x = synth.activations(0, 4, sh.H)
    idx = synth.sorted_topk(0, 4, sh.E, sh.top_k)
    want = oracle.switch_glu(x, idx, *ex, gs=sh.gs, bits=sh.bits).reshape(-1, sh.H)
    g = _experts(ex)
    y, inv, mode = mg.switch_glu(bf(x), i32(idx), *g, group_size=sh.gs, bits=sh.bits, mode=mg.MODE_DECODE)
    assert mode == mg.MODE_DECODE
    assert_parity(host_bf(y), want, name="decode")
    y2, inv2, _ = mg.switch_glu(bf(x), i32(idx), *g, group_size=sh.gs, bits=sh.bits, mode=mg.MODE_SORTED)
    order = oracle.sort_pairs(idx, sh.E)[0]
    assert_parity(host_bf(y2), want[order], name="sorted")
    assert np.array_equal(inv2.cpu().numpy(), oracle.sort_pairs(idx, sh.E)[3])


@pytest.mark.parametrize("E,N,K,bits,gs,P", [
    (8, 64, 512, 4, 64, 6), (8, 36, 192, 4, 32, 5), (8, 13, 96, 8, 32, 3), (4, 40, 128, 8, 128, 4),
    (3, 300, 4096, 4, 128, 5), (2, 257, 2560, 8, 64, 3), (5, 64, 9728, 4, 64, 2), (1, 8, 32, 4, 32, 1),
    (4, 50, 2560, 4, 32, 3), (3, 33, 2048, 8, 128, 4), (2, 24, 6144, 4, 64, 2)])
def test_gather_qmv_shapes(mg, E, N, K, bits, gs, P):
    """M=1 rows per pair, ragged N, K off the 256-word slice, every group size."""
    g = np.random.default_rng(E * 1000 + N + K + bits)
    W = [synth.drawn_matrix(g, N, K, gs, bits) for _ in range(E)]
    w, s, b = (np.stack([m[i] for m in W]) for i in range(3))
    X = P + 2
    x = synth.to_bf16(g.standard_normal((X, 1, K)))
    lhs = g.integers(0, X, P)
    rhs = (np.arange(P) * 7 + 3) % E
    want = oracle.gather_qmm(x, w, s, b, lhs=lhs, rhs=rhs, gs=gs, bits=bits)
    out = mg.gather_qmm(bf(x), words(w), bf(s), bf(b), rhs_indices=i32(rhs), lhs_indices=i32(lhs),
                        group_size=gs, bits=bits)
    assert out.shape == (P, 1, N)
    assert_parity(host_bf(out), want, name=f"qmv {E},{N},{K},{bits},{gs}")


@pytest.mark.parametrize("bits,gs", [(4, 64), (4, 32), (8, 128), (8, 32)])
@pytest.mark.parametrize("M", [1, 3, 16, 40, 160])
def test_integer_exact_bitwise(mg, bits, gs, M):
    """Exact scales/biases and small-integer activations: every product and
    partial sum is exact, so GPU and oracle agree bit for bit on every route
    (M=1 qmv, 2..16 MFMA few-row, >16 MFMA tiles)."""
    g = np.random.default_rng(100 + M + bits + gs)
    N, K = 80, 512
    w, s, b = synth.integer_exact(g, N, K, gs, bits)
    x = synth.integer_x(g, M, K)
    want = oracle.quantized_matmul(x, w, s, b, True, gs, bits)
    got = host_bf(mg.affine_qmm(bf(x), words(w), bf(s), bf(b), group_size=gs, bits=bits))
    assert np.array_equal(got, want)


def test_expert_routing_bitwise(mg):
    """Expert e has scale 0, bias e+1: y = (e+1) * sum(x) exactly; a wrong
    expert or a wrong activation row shows bitwise."""
    E, N, K, gs = 6, 24, 256, 64
    w = np.zeros((E, N, K // 8), np.uint32)
    s = np.zeros((E, N, K // gs), np.uint16)
    b = np.broadcast_to(synth.to_bf16(np.arange(1, E + 1, dtype=np.float32))[:, None, None], (E, N, K // gs)).copy()
    g = np.random.default_rng(7)
    x = synth.integer_x(g, 5, K)[:, None, :]
    lhs = np.array([4, 0, 2, 2, 1, 3, 3])
    rhs = np.array([5, 0, 2, 3, 1, 4, 0])
    want = oracle.gather_qmm(x, w, s, b, lhs=lhs, rhs=rhs, gs=gs, bits=4)
    got = mg.gather_qmm(bf(x), words(w), bf(s), bf(b), rhs_indices=i32(rhs), lhs_indices=i32(lhs), group_size=gs)
    assert np.array_equal(host_bf(got), want)


@pytest.mark.parametrize("M,mode", [(1, "minmax"), (4, "drawn")])
def test_decode_full_shape(mg, M, mode):
    """MoE decode at hidden 4096, inter 2048, E=288, top-8, 4-bit GS 64; the
    selected experts are drawn (min-max of N(0,1), or drawn codes), the
    others stay zero on both sides."""
    sh = synth.DECODE
    idx = synth.sorted_topk(1, M, sh.E, sh.top_k)
    sel = np.unique(idx)
    x = synth.activations(1, M, sh.H)
    ex = synth.expert_set(1, sh.E, sh.H, sh.I, sh.gs, sh.bits, mode=mode, experts=sel)
    want = oracle.switch_glu(x, idx, *ex, gs=sh.gs, bits=sh.bits).reshape(-1, sh.H)
    y, _, _ = mg.switch_glu(bf(x), i32(idx), *_experts(ex), group_size=sh.gs, bits=sh.bits, mode=mg.MODE_DECODE)
    assert_parity(host_bf(y), want, name=f"decode M={M}")


def test_empty_inputs(mg):
    sh = synth.TINY
    ex = _experts(synth.expert_set(0, sh.E, sh.H, sh.I, sh.gs, sh.bits, mode="drawn"))
    x = torch.zeros((0, sh.H), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((0, 2), dtype=torch.int32, device="cuda")
    y, _, _ = mg.switch_glu(x, idx, *ex, group_size=sh.gs, bits=sh.bits, mode=mg.MODE_DECODE)
    assert y.shape == (0, sh.H)
    w0, s0, b0 = ex[2][0][0], ex[2][1][0], ex[2][2][0]        # down of expert 0: [H, I/8]
    out = mg.affine_qmm(torch.zeros((0, sh.I), dtype=torch.bfloat16, device="cuda"), w0, s0, b0, group_size=sh.gs)
    assert out.shape == (0, sh.H)


@pytest.mark.parametrize("M,K", [(1, 512), (3, 512), (20, 512), (1, 2560), (1, 4096), (1, 6144)])
def test_gather_qmm_glu(mg, M, K):
    """SwitchGLU's gate/up half over gathered experts (decode layout x[T, K],
    pair p on token p // top_k) against the oracle's SwitchGLU intermediate."""
    g = np.random.default_rng(90 + M)
    E, N, top_k, T = 6, 96, 2, 5
    gate = [synth.drawn_matrix(g, N, K, 64, 4) for _ in range(E)]
    up = [synth.drawn_matrix(g, N, K, 64, 4) for _ in range(E)]
    G = synth.stack_experts(gate)
    U = synth.stack_experts(up)
    x = synth.to_bf16(g.standard_normal((T, M, K)))
    rhs = g.integers(0, E, T * top_k)
    gg = oracle.gather_qmm(x, *G, lhs=np.arange(T * top_k) // top_k, rhs=rhs, gs=64, bits=4)
    uu = oracle.gather_qmm(x, *U, lhs=np.arange(T * top_k) // top_k, rhs=rhs, gs=64, bits=4)
    want = oracle.f64_to_bf16(oracle.silu(oracle.bf16_to_f64(gg)) * oracle.bf16_to_f64(uu))
    xd = bf(x) if M > 1 else bf(x[:, 0, :])
    got = mg.gather_qmm_glu(xd, triple(G), triple(U), i32(rhs), lhs_div=top_k, group_size=64, bits=4)
    assert_parity(host_bf(got), want, name=f"glu M={M}")


@pytest.mark.parametrize("N,K,bits,gs", [(97, 4096, 4, 64), (33, 512, 4, 32), (65, 2048, 8, 128), (1, 256, 8, 64),
                                         (129, 2560, 4, 128)])
def test_gather_qmm_glu_ragged(mg, N, K, bits, gs):
    """One-row GLU pairs with an odd number of output rows: the last two-row
    block of each expert has one row past N, whose loads must read zeros (the
    last expert of the stack included) and whose result is not written.  K
    covers rows of one and of two 256-word slices and a partial slice."""
    g = np.random.default_rng(N * 7 + K + bits)
    E, top_k, T = 4, 2, 5
    G = synth.stack_experts([synth.drawn_matrix(g, N, K, gs, bits) for _ in range(E)])
    U = synth.stack_experts([synth.drawn_matrix(g, N, K, gs, bits) for _ in range(E)])
    x = synth.to_bf16(g.standard_normal((T, 1, K)))
    rhs = (np.arange(T * top_k) * 3 + 1) % E
    rhs[-1] = E - 1
    lhs = np.arange(T * top_k) // top_k
    gg = oracle.gather_qmm(x, *G, lhs=lhs, rhs=rhs, gs=gs, bits=bits)
    uu = oracle.gather_qmm(x, *U, lhs=lhs, rhs=rhs, gs=gs, bits=bits)
    want = oracle.f64_to_bf16(oracle.silu(oracle.bf16_to_f64(gg)) * oracle.bf16_to_f64(uu))
    got = mg.gather_qmm_glu(bf(x[:, 0, :]), triple(G), triple(U), i32(rhs), lhs_div=top_k, group_size=gs, bits=bits)
    assert got.shape[-1] == N
    assert_parity(host_bf(got), want, name=f"glu ragged N={N} K={K} bits={bits}")


@pytest.mark.parametrize("M,H,I,E,top_k,bits,gs", [(1, 4096, 2048, 288, 8, 4, 64), (4, 4096, 2048, 288, 8, 4, 64),
                                                   (3, 256, 128, 8, 2, 4, 64), (2, 512, 384, 16, 4, 8, 128),
                                                   (5, 1024, 2560, 12, 8, 4, 32), (2, 256, 256, 20, 12, 4, 64)])
def test_moe_decode_fused_tail(mg, M, H, I, E, top_k, bits, gs):
    """Two-kernel decode layer (gate/up, then down fused with the combine) equals
    switch_glu DECODE followed by the separate combine, bit for bit, and the
    oracle within tolerance."""
    idx = synth.sorted_topk(11, M, E, top_k, sub=H + I)
    ex = synth.expert_set(11, E, H, I, gs, bits, mode="drawn", experts=np.unique(idx))
    x = synth.activations(11, M, H)
    g = np.random.default_rng(M + H)
    scores = synth.to_bf16(g.random((M, top_k)).astype(np.float32))
    shared = synth.to_bf16(g.standard_normal((M, H)).astype(np.float32))
    dev = [triple(m) for m in ex]
    xd, idd, scd, shd = bf(x), i32(idx), bf(scores), bf(shared)
    y = torch.empty((M * top_k, H), dtype=torch.bfloat16, device="cuda")
    out = mg.moe_decode(xd, idd, scd, *dev, shared=shd, group_size=gs, bits=bits, y=y)
    y_ref, _, _ = mg.switch_glu(xd, idd, *dev, group_size=gs, bits=bits, mode=mg.MODE_DECODE)
    out_ref = mg.moe_combine(y_ref, None, scd, shd)
    assert np.array_equal(host_bf(y), host_bf(y_ref))
    assert np.array_equal(host_bf(out), host_bf(out_ref))
    want_y = oracle.switch_glu(x, idx, *ex, gs=gs, bits=bits).reshape(-1, H)
    want = oracle.combine(want_y, np.arange(M * top_k, dtype=np.int32), scores, shared)
    assert_parity(host_bf(out), want, name="decode layer")
    out2 = mg.moe_decode(xd, idd, scd, *dev, shared=None, group_size=gs, bits=bits, y=y)
    assert np.array_equal(host_bf(out2), host_bf(mg.moe_combine(y_ref, None, scd, None)))


def test_gather_qmv_past_grid_limit(mg):
    """70,000 one-row pairs: the launch splits its pair axis into grids of
    65,535; pairs around each split (and the last) checked against the oracle."""
    g = np.random.default_rng(123)
    E, N, K, P = 5, 32, 128, 70000
    w, s, b = synth.stack_experts([synth.drawn_matrix(g, N, K, 64, 4) for _ in range(E)])
    x = synth.to_bf16(g.standard_normal((P, 1, K)))
    rhs = g.integers(0, E, P).astype(np.int32)
    got = host_bf(mg.gather_qmm(bf(x), words(w), bf(s), bf(b), rhs_indices=i32(rhs), group_size=64, bits=4))
    pick = np.array([0, 1, 65533, 65534, 65535, 65536, P - 2, P - 1])
    want = oracle.gather_qmm(x[pick], w, s, b, lhs=np.arange(len(pick)), rhs=rhs[pick], gs=64, bits=4)
    assert_parity(got[pick], want, name="past grid limit")


def test_moe_decode_past_grid_limit(mg):
    """65,600 tokens through the two-kernel decode layer (the fused down +
    combine launches its token axis in grids of 65,535); sampled tokens
    against the oracle's SwitchGLU and combine."""
    T, H, I, E, top_k, gs = 65600, 64, 64, 4, 2, 32
    g = np.random.default_rng(124)
    idx = np.sort(np.stack([g.choice(E, top_k, replace=False) for _ in range(T)]), axis=1).astype(np.int32)
    ex = synth.expert_set(12, E, H, I, gs, 4, mode="drawn")
    x = synth.to_bf16(g.standard_normal((T, H)))
    scores = synth.to_bf16(g.random((T, top_k)).astype(np.float32))
    dev = [triple(m) for m in ex]
    out = host_bf(mg.moe_decode(bf(x), i32(idx), bf(scores), *dev, group_size=gs, bits=4))
    pick = np.array([0, 65534, 65535, 65536, T - 1])
    want_y = oracle.switch_glu(x[pick], idx[pick], *ex, gs=gs, bits=4).reshape(-1, H)
    want = oracle.combine(want_y, np.arange(len(pick) * top_k, dtype=np.int32), scores[pick])
    assert_parity(out[pick], want, name="decode past grid limit")


@pytest.mark.parametrize("bits,gs", [(4, 128), (8, 64)])
def test_gather_qmv_longest_row(mg, bits, gs):
    """One-row pairs at the longest row the one-row kernels take (K 32768)."""
    g = np.random.default_rng(125 + bits)
    E, N, K, P = 3, 24, 32768, 4
    w, s, b = synth.stack_experts([synth.drawn_matrix(g, N, K, gs, bits) for _ in range(E)])
    x = synth.to_bf16(g.standard_normal((P, 1, K)))
    rhs = np.array([2, 0, 1, 2], np.int32)
    got = host_bf(mg.gather_qmm(bf(x), words(w), bf(s), bf(b), rhs_indices=i32(rhs), group_size=gs, bits=bits))
    want = oracle.gather_qmm(x, w, s, b, lhs=np.arange(P), rhs=rhs, gs=gs, bits=bits)
    assert_parity(got, want, name=f"K=32768 {bits}-bit")
    x1 = synth.to_bf16(g.standard_normal((1, K)))
    got1 = host_bf(mg.affine_qmm(bf(x1), words(w[1]), bf(s[1]), bf(b[1]), group_size=gs, bits=bits))
    assert_parity(got1, oracle.quantized_matmul(x1, w[1], s[1], b[1], True, gs, bits), name="dense K=32768")
