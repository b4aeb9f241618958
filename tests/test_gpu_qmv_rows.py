"""GPU parity of the products with 2-4 activation rows per weight matrix
against the oracle: the vector kernel (every code it loads applied to all
the rows) for dense affine_qmm with and without the residual, GLU pairs of 2
rows and of 3-4 rows at 8 bits or with a K the matrix-core kernel does not
take, and gather_qmm with several rows per pair; the matrix-core kernel for
4-bit GLU pairs of 3-4 rows.  Both code widths, every group size, ragged
output rows, K of one partial and of several 256-word slices, 3 rows (one
padded row in the vector kernel)."""
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


@pytest.mark.parametrize("M", [2, 3, 4])
@pytest.mark.parametrize("bits,gs", [(4, 32), (4, 64), (4, 128), (8, 32), (8, 64), (8, 128)])
@pytest.mark.parametrize("N,K", [(203, 1280), (97, 8192)])
def test_affine_qmm_rows(mg, M, bits, gs, N, K):
    g = np.random.default_rng(M * 1000 + bits * 100 + gs + N)
    w, s, b = synth.drawn_words(g, N, K, gs, bits)
    x = synth.to_bf16(g.standard_normal((M, K)))
    want = oracle.quantized_matmul(x, w, s, b, True, gs, bits)
    got = mg.affine_qmm(bf(x), words(w), bf(s), bf(b), group_size=gs, bits=bits)
    assert_parity(host_bf(got), want, name=f"M={M} {bits}/{gs} N={N} K={K}")
    r = synth.to_bf16(g.standard_normal((M, N)))
    got_r = mg.affine_qmm(bf(x), words(w), bf(s), bf(b), group_size=gs, bits=bits, residual=bf(r))
    want_r = oracle.f64_to_bf16(oracle.bf16_to_f64(want) + oracle.bf16_to_f64(r))
    assert_parity(host_bf(got_r), want_r, name="residual")
    # in place: each output's residual is read by the lane that writes it
    rt = bf(r)
    mg.affine_qmm(bf(x), words(w), bf(s), bf(b), group_size=gs, bits=bits, residual=rt, out=rt)
    assert np.array_equal(host_bf(rt), host_bf(got_r))


# K = 2624 is a multiple of 32 and 64 but not of 128: only the smaller groups take it
@pytest.mark.parametrize("M", [2, 3, 4])
@pytest.mark.parametrize("bits,gs,K", [(4, 64, 2560), (8, 128, 2560), (4, 32, 2560), (4, 64, 2624), (4, 32, 2624), (8, 64, 2624)])
def test_affine_qmm_glu_rows(mg, M, bits, gs, K):
    """GLU pairs: at 4 bits K = 2560 sends 3 and 4 rows to the matrix-core
    kernel, K = 2624 (not a multiple of 128) keeps them on the vector kernel;
    8-bit pairs stay on the vector kernel."""
    g = np.random.default_rng(70 + M + bits + gs + K)
    N = 150
    gate = synth.drawn_matrix(g, N, K, gs, bits)
    up = synth.drawn_matrix(g, N, K, gs, bits)
    x = synth.to_bf16(g.standard_normal((M, K)))
    gg = oracle.quantized_matmul(x, *gate, True, gs, bits)
    uu = oracle.quantized_matmul(x, *up, True, gs, bits)
    want = oracle.f64_to_bf16(oracle.silu(oracle.bf16_to_f64(gg)) * oracle.bf16_to_f64(uu))
    got = mg.affine_qmm_glu(bf(x), triple(gate), triple(up), group_size=gs, bits=bits)
    assert_parity(host_bf(got), want, name=f"glu M={M} {bits}/{gs}")


@pytest.mark.parametrize("M", [2, 3, 4])
def test_gather_qmm_rows(mg, M):
    """Several rows per pair: explicit lhs and rhs, and rhs alone (x batch p)."""
    g = np.random.default_rng(90 + M)
    E, N, K = 5, 72, 512
    W = [synth.drawn_matrix(g, N, K, 64, 4) for _ in range(E)]
    w, s, b = (np.stack([m[i] for m in W]) for i in range(3))
    x = synth.to_bf16(g.standard_normal((6, M, K)))
    lhs, rhs = np.array([5, 0, 3, 3, 1]), np.array([4, 4, 0, 2, 1])
    got = mg.gather_qmm(bf(x), words(w), bf(s), bf(b), rhs_indices=i32(rhs), lhs_indices=i32(lhs), group_size=64)
    assert got.shape == (5, M, N)
    assert_parity(host_bf(got), oracle.gather_qmm(x, w, s, b, lhs=lhs, rhs=rhs, gs=64), name=f"lhs/rhs M={M}")
    rhs6 = np.array([1, 3, 0, 4, 2, 2])
    got = mg.gather_qmm(bf(x), words(w), bf(s), bf(b), rhs_indices=i32(rhs6), group_size=64)
    assert_parity(host_bf(got), oracle.gather_qmm(x, w, s, b, rhs=rhs6, gs=64), name=f"rhs M={M}")


def test_rows_outside_fp16_range(mg):
    """The vector kernel works in fp32 on bf16 inputs: rows of about 1e5 and
    1e-6 in one call, each held to the tolerance on its own scale."""
    g = np.random.default_rng(99)
    N, K = 64, 2048
    w, s, b = synth.drawn_words(g, N, K, 64, 4)
    x0 = g.standard_normal((4, K))
    x = synth.to_bf16((x0 * np.array([1e5, 1.0, 1e-6, 3.0])[:, None]).astype(np.float32))
    got = host_bf(mg.affine_qmm(bf(x), words(w), bf(s), bf(b), group_size=64, bits=4))
    want = oracle.quantized_matmul(x, w, s, b, True, 64, 4)
    for r in range(4):
        assert_parity(got[r:r + 1], want[r:r + 1], name=f"row {r}")
