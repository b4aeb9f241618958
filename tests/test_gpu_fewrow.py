"""GPU parity of the few-row products (2..16 rows, MLX PR 4787's range) on the
exact-code matrix-core kernel, with K split over workgroups through a
workspace: against the oracle within tolerance, bit for bit on
integer-exact inputs, repeatable bit for bit, and leaving the workspace's
counters at zero; gathered pairs with several rows each."""
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


def _counters_zero(ws, N, glu=False):
    # one counter per column group: 16 columns for GLU pairs, 32 for the
    # plain products that split K; shapes that never split need no workspace
    if ws is None:
        return True
    items = -(-N // (16 if glu else 32))
    return not bool(ws[:4 * items].view(torch.int32).any())


@pytest.mark.parametrize("M", [2, 3, 4, 8, 16])
@pytest.mark.parametrize("bits,gs", [(4, 32), (4, 64), (4, 128), (8, 32), (8, 128)])
def test_split_k_parity(mg, M, bits, gs):
    g = np.random.default_rng(M * 11 + bits + gs)
    # 64 K chunks: two-block workgroups of plain products (3 column groups),
    # K split 4 ways; without a workspace one block per workgroup, no split
    N, K = 96, 8192
    w, s, b = synth.minmax_matrix(g, N, K, gs, bits, scale=1 / np.sqrt(K))
    x = synth.to_bf16(g.standard_normal((M, K)))
    want = oracle.quantized_matmul(x, w, s, b, True, gs, bits)
    ws = mg.affine_qmm_workspace(M, N, K)
    assert ws is not None
    args = (bf(x), words(w), bf(s), bf(b))
    got = mg.affine_qmm(*args, group_size=gs, bits=bits, workspace=ws)
    assert_parity(host_bf(got), want, name=f"split M={M} {bits}/{gs}")
    again = mg.affine_qmm(*args, group_size=gs, bits=bits, workspace=ws)
    assert np.array_equal(host_bf(again), host_bf(got))
    assert _counters_zero(ws, N)
    plain = mg.affine_qmm(*args, group_size=gs, bits=bits)       # no workspace: one split
    assert_parity(host_bf(plain), want, name="unsplit")
    r = synth.to_bf16(g.standard_normal((M, N)))
    got_r = mg.affine_qmm(*args, group_size=gs, bits=bits, residual=bf(r), workspace=ws)
    want_r = oracle.f64_to_bf16(oracle.bf16_to_f64(host_bf(got)) + oracle.bf16_to_f64(r))
    assert np.array_equal(host_bf(got_r), want_r)


@pytest.mark.parametrize("M", [2, 5, 16])
@pytest.mark.parametrize("bits,gs", [(4, 64), (8, 128)])
@pytest.mark.parametrize("K", [2048, 8192])
def test_split_k_integer_exact(mg, M, bits, gs, K):
    """Bit for bit on integer-exact inputs: K = 2048 on one-block 8-wave
    workgroups, K = 8192 split over two-block workgroups."""
    g = np.random.default_rng(300 + M + bits + K)
    N = 160
    w, s, b = synth.integer_exact(g, N, K, gs, bits)
    x = synth.integer_x(g, M, K, amp=3)
    want = oracle.quantized_matmul(x, w, s, b, True, gs, bits)
    ws = mg.affine_qmm_workspace(M, N, K)
    got = host_bf(mg.affine_qmm(bf(x), words(w), bf(s), bf(b), group_size=gs, bits=bits, workspace=ws))
    assert np.array_equal(got, want)
    assert _counters_zero(ws, N)


@pytest.mark.parametrize("M", [2, 4, 16])
@pytest.mark.parametrize("bits,gs", [(4, 64), (8, 32)])
def test_split_k_glu(mg, M, bits, gs):
    g = np.random.default_rng(500 + M + bits)
    N, K = 64, 2560
    gate = synth.minmax_matrix(g, N, K, gs, bits, scale=1 / np.sqrt(K))
    up = synth.minmax_matrix(g, N, K, gs, bits, scale=1 / np.sqrt(K))
    x = synth.to_bf16(g.standard_normal((M, K)))
    gg = oracle.quantized_matmul(x, *gate, True, gs, bits)
    uu = oracle.quantized_matmul(x, *up, True, gs, bits)
    want = oracle.f64_to_bf16(oracle.silu(oracle.bf16_to_f64(gg)) * oracle.bf16_to_f64(uu))
    ws = mg.affine_qmm_workspace(M, N, K, glu=True)
    tr = lambda m: (words(m[0]), bf(m[1]), bf(m[2]))
    got = mg.affine_qmm_glu(bf(x), tr(gate), tr(up), group_size=gs, bits=bits, workspace=ws)
    assert_parity(host_bf(got), want, name=f"glu split M={M}")
    assert _counters_zero(ws, N, glu=True)


def test_dense_shape_split(mg):
    """The chain's down projection shape (2560 x 9728, 4-bit GS 64) at 4 rows
    with the split, against the oracle on sampled columns."""
    g = np.random.default_rng(77)
    N, K, M = 2560, 9728, 4
    w, s, b = synth.minmax_matrix(g, N, K, 64, 4, scale=1 / np.sqrt(K))
    x = synth.to_bf16(g.standard_normal((M, K)))
    ws = mg.affine_qmm_workspace(M, N, K)
    got = host_bf(mg.affine_qmm(bf(x), words(w), bf(s), bf(b), group_size=64, bits=4, workspace=ws))
    cols = np.sort(g.choice(N, 96, replace=False))
    want = oracle.quantized_matmul(x, w[cols], s[cols], b[cols], True, 64, 4)
    assert_parity(got[:, cols], want, name="down shape")
    assert _counters_zero(ws, N)


def _expert_set(g, E, N, K, gs, bits):
    mats = [synth.drawn_matrix(g, N, K, gs, bits) for _ in range(E)]
    return tuple(np.stack([m[i] for m in mats]) for i in range(3))


@pytest.mark.parametrize("M", [3, 5, 16])
@pytest.mark.parametrize("bits,gs", [(4, 64), (8, 128), (4, 32)])
def test_gathered_few_rows(mg, M, bits, gs):
    """gather_qmm and gather_qmm_glu with M rows per pair, explicit lhs and rhs
    (one x batch used twice, one expert twice), ragged N: the matrix-core
    kernel gathering each pair's rows and expert (GLU pairs from 3 rows at 4
    bits, plain products from 5)."""
    g = np.random.default_rng(900 + M + bits + gs)
    E, N, K = 5, 72, 1024
    w, s, b = _expert_set(g, E, N, K, gs, bits)
    wu, su, bu = _expert_set(g, E, N, K, gs, bits)
    x = synth.to_bf16(g.standard_normal((6, M, K)))
    lhs, rhs = np.array([5, 0, 3, 3, 1]), np.array([4, 4, 0, 2, 1])
    got = mg.gather_qmm(bf(x), words(w), bf(s), bf(b), rhs_indices=i32(rhs), lhs_indices=i32(lhs),
                        group_size=gs, bits=bits)
    assert got.shape == (5, M, N)
    want = oracle.gather_qmm(x, w, s, b, lhs=lhs, rhs=rhs, gs=gs, bits=bits)
    assert_parity(host_bf(got), want, name=f"gather M={M} {bits}/{gs}")
    h = mg.gather_qmm_glu(bf(x), (words(w), bf(s), bf(b)), (words(wu), bf(su), bf(bu)), i32(rhs),
                          lhs_indices=i32(lhs), group_size=gs, bits=bits)
    gg = oracle.bf16_to_f64(want)
    uu = oracle.bf16_to_f64(oracle.gather_qmm(x, wu, su, bu, lhs=lhs, rhs=rhs, gs=gs, bits=bits))
    assert_parity(host_bf(h), oracle.f64_to_bf16(oracle.silu(gg) * uu), name=f"gather glu M={M} {bits}/{gs}")
