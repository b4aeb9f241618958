"""GPU parity of the few-row products (2..16 rows, MLX PR 4787's range) on the
exact-code matrix-core kernel, with K split over workgroups through a
workspace: against the oracle within tolerance, bit for bit on
integer-exact inputs, repeatable bit for bit, and leaving the workspace's
counters at zero."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_parity, bf, host_bf, words

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_gathered_amd as m
    m.lib()
    return m


def _counters_zero(ws, N):
    items = -(-N // 32)
    return not bool(ws[:4 * items].view(torch.int32).any())


@pytest.mark.parametrize("M", [2, 3, 4, 8, 16])
@pytest.mark.parametrize("bits,gs", [(4, 32), (4, 64), (4, 128), (8, 32), (8, 128)])
def test_split_k_parity(mg, M, bits, gs):
    g = np.random.default_rng(M * 11 + bits + gs)
    N, K = 96, 4096                       # 3 column groups, 32 K chunks: K split 8 ways
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
def test_split_k_integer_exact(mg, M, bits, gs):
    g = np.random.default_rng(300 + M + bits)
    N, K = 160, 2048
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
    assert _counters_zero(ws, N)


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
