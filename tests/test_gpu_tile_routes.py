"""GPU parity of the products that run on the bf16-operand matrix-core tiles
outside the SwitchGLU chain: sorted one-row gather_qmm without GLU (expert-
sorted pairs, x rows gathered through lhs indices; 32-row and 128-row tiles)
and dense affine_qmm from 128 rows.  Every output against the oracle, ragged
N and rows, both code widths and every group size, and activations far
outside fp16's range held to the tolerance on their own scale."""
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


def _sorted_pairs(idx):
    """Pairs (token, slot) ordered by expert, stable: lhs = token, rhs = expert."""
    flat = idx.reshape(-1)
    order = np.argsort(flat, kind="stable")
    return (order // idx.shape[1]).astype(np.int32), flat[order].astype(np.int32)


def _experts(g, E, N, K, gs, bits):
    mats = [synth.drawn_words(g, N, K, gs, bits) for _ in range(E)]
    return tuple(np.stack([m[i] for m in mats]) for i in range(3))


def _want_sorted(x, lhs, rhs, w, s, b, gs, bits):
    """oracle.quantized_matmul per expert on its gathered rows (gather_qmm is
    that product for each pair; the rows of one expert are independent)."""
    out = np.zeros((len(lhs), w.shape[1]), np.uint16)
    for e in np.unique(rhs):
        sel = np.nonzero(rhs == e)[0]
        out[sel] = oracle.quantized_matmul(x[lhs[sel]], w[e], s[e], b[e], True, gs, bits)
    return out


@pytest.mark.parametrize("T,E,top_k,N,K,gs,bits", [
    (150, 16, 4, 320, 1024, 64, 4),     # about 38 rows per expert: 32-row tiles, ragged N
    (150, 16, 4, 256, 1024, 32, 8),
    (97, 8, 2, 136, 512, 64, 8),        # one 256-column block, ragged
    (600, 4, 2, 384, 1024, 128, 4),     # 300 rows per expert: 128-row tiles
    (515, 6, 2, 264, 2048, 64, 4),
])
def test_sorted_gather_qmm_tiles(mg, T, E, top_k, N, K, gs, bits):
    g = np.random.default_rng(T + E + N + K + gs + bits)
    idx, _ = synth.zipf_routing(7, T, E, top_k, sub=N + bits)
    lhs, rhs = _sorted_pairs(idx)
    w, s, b = _experts(g, E, N, K, gs, bits)
    x = synth.to_bf16(g.standard_normal((T, K)))
    got = mg.gather_qmm(bf(x.reshape(T, 1, K)), words(w), bf(s), bf(b), rhs_indices=i32(rhs),
                        lhs_indices=i32(lhs), group_size=gs, bits=bits, sorted_indices=True)
    assert got.shape == (len(lhs), 1, N)
    want = _want_sorted(x, lhs, rhs, w, s, b, gs, bits)
    assert_parity(host_bf(got)[:, 0], want, name=f"sorted T={T} E={E} N={N} K={K} {bits}/{gs}")


@pytest.mark.parametrize("M,N,K,gs,bits", [
    (128, 256, 1024, 64, 4),
    (200, 300, 1024, 128, 8),
    (513, 520, 2048, 64, 4),    # ragged rows (4 full tiles and one row) and columns
    (1000, 264, 512, 32, 4),
])
def test_affine_qmm_tiles(mg, M, N, K, gs, bits):
    g = np.random.default_rng(M + N + K + gs + bits)
    w, s, b = synth.drawn_words(g, N, K, gs, bits)
    x = synth.to_bf16(g.standard_normal((M, K)))
    got = host_bf(mg.affine_qmm(bf(x), words(w), bf(s), bf(b), group_size=gs, bits=bits))
    want = oracle.quantized_matmul(x, w, s, b, True, gs, bits)
    assert_parity(got, want, name=f"dense M={M} N={N} K={K} {bits}/{gs}")


def _range_rows(g, T, K):
    """Rows scaled by 1e5 (every fifth row), 1e-6 (the next ones) and 1."""
    x0 = g.standard_normal((T, K))
    factor = np.ones(T)
    big, tiny = np.arange(0, T, 5), np.arange(1, T, 5)
    factor[big], factor[tiny] = 1e5, 1e-6
    rest = np.setdiff1d(np.arange(T), np.r_[big, tiny])
    return synth.to_bf16((x0 * factor[:, None]).astype(np.float32)), {"large": big, "tiny": tiny, "normal": rest}


def test_tile_routes_outside_fp16_range(mg):
    """Activations about 1e5 (outputs far above 65504) and about 1e-6 (products
    below fp16's normal range) through both routes."""
    g = np.random.default_rng(91)
    T, E, top_k, N, K, gs = 300, 8, 2, 264, 1024, 64
    x, groups = _range_rows(g, T, K)
    idx, _ = synth.zipf_routing(8, T, E, top_k, sub=3)
    lhs, rhs = _sorted_pairs(idx)
    w, s, b = _experts(g, E, N, K, gs, 4)
    got = host_bf(mg.gather_qmm(bf(x.reshape(T, 1, K)), words(w), bf(s), bf(b), rhs_indices=i32(rhs),
                                lhs_indices=i32(lhs), group_size=gs, bits=4, sorted_indices=True))[:, 0]
    want = _want_sorted(x, lhs, rhs, w, s, b, gs, 4)
    for name, rows in groups.items():
        pairs = np.nonzero(np.isin(lhs, rows))[0]
        assert_parity(got[pairs], want[pairs], name=f"sorted {name} rows")
    assert np.abs(oracle.bf16_to_f64(want[np.isin(lhs, groups["large"])])).max() > 65504
    got = host_bf(mg.affine_qmm(bf(x), words(w[0]), bf(s[0]), bf(b[0]), group_size=gs, bits=4))
    want = oracle.quantized_matmul(x, w[0], s[0], b[0], True, gs, 4)
    for name, rows in groups.items():
        assert_parity(got[rows], want[rows], name=f"dense {name} rows")
