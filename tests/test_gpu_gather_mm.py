"""GPU parity of unquantized gather_mm (bf16 expert matrices) against the
oracle: the expert-sorted route on the matrix cores (64-row scheduled tiles),
one-row pairs in any order, and several rows per pair."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_parity, bf, host_bf, i32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_gathered_amd as m
    m.lib()
    return m


def _w(g, E, N, K, scale=0.05):
    return synth.to_bf16((g.standard_normal((E, N, K)) * scale).astype(np.float32))


@pytest.mark.parametrize("T,E,N,K", [(256, 64, 256, 512), (331, 32, 200, 384), (40, 8, 96, 128)])
def test_gather_mm_sorted_route(mg, T, E, N, K):
    """Pairs sorted by expert (the sorted chain's layout), x rows gathered
    through lhs: scheduled 64-row tiles, ragged per-expert counts."""
    g = np.random.default_rng(T + E)
    idx, _ = synth.zipf_routing(5, T, E, 8 if E >= 8 else 2, sub=T)
    order, lhs, srhs, _, _, _ = oracle.sort_pairs(idx, E)
    x = synth.to_bf16(g.standard_normal((T, K)).astype(np.float32))
    w = _w(g, E, N, K)
    got = host_bf(mg.gather_mm(bf(x), bf(w), i32(srhs), lhs_indices=i32(lhs), sorted_indices=True))
    want = oracle.gather_mm(x[:, None, :], w, lhs=lhs, rhs=srhs)[:, 0]
    assert_parity(got, want, name=f"sorted T={T}")


@pytest.mark.parametrize("P,N,K,div", [(37, 300, 264, 1), (16, 2048, 4096, 8), (5, 7, 8, 5)])
def test_gather_mm_one_row_any_order(mg, P, N, K, div):
    """One activation row per pair, experts in any order (x row = p // div)."""
    g = np.random.default_rng(P + N)
    E = 11
    x = synth.to_bf16(g.standard_normal(((P + div - 1) // div, K)).astype(np.float32))
    w = _w(g, E, N, K)
    rhs = g.integers(0, E, size=P).astype(np.int32)
    got = host_bf(mg.gather_mm(bf(x), bf(w), i32(rhs), lhs_div=div))
    want = oracle.gather_mm(x[:, None, :], w, lhs=np.arange(P) // div, rhs=rhs)[:, 0]
    assert_parity(got, want, name=f"one-row P={P}")


def test_gather_mm_many_rows_per_pair(mg):
    """M > 1 rows per pair (70: two row tiles per pair), lhs chosen freely."""
    g = np.random.default_rng(93)
    X, M, K, E, N, P = 4, 70, 256, 5, 200, 6
    x = synth.to_bf16(g.standard_normal((X, M, K)).astype(np.float32))
    w = _w(g, E, N, K)
    lhs = np.array([3, 0, 0, 2, 1, 3], np.int32)
    rhs = np.array([4, 4, 1, 0, 2, 1], np.int32)
    got = host_bf(mg.gather_mm(bf(x), bf(w), i32(rhs), lhs_indices=i32(lhs)))
    want = oracle.gather_mm(x, w, lhs=lhs, rhs=rhs)
    assert_parity(got, want, name="many rows")


def test_gather_mm_prefill_shape_sampled(mg):
    """The benchmark shape: 2048 tokens, top-8 of 256 experts, N 512, K 2048,
    sorted pairs on the GPU; sampled pairs through the oracle."""
    g = np.random.default_rng(94)
    T, E, N, K = 2048, 256, 512, 2048
    idx, _ = synth.zipf_routing(3, T, E, 8)
    order, lhs, srhs, _, _, _ = oracle.sort_pairs(idx, E)
    x = synth.to_bf16(g.standard_normal((T, K)).astype(np.float32))
    w = _w(g, E, N, K, 0.02)
    got = host_bf(mg.gather_mm(bf(x), bf(w), i32(srhs), lhs_indices=i32(lhs), sorted_indices=True))
    sub = np.sort(g.choice(len(srhs), 64, replace=False))
    want = oracle.gather_mm(x[:, None, :], w, lhs=lhs[sub], rhs=srhs[sub])[:, 0]
    assert_parity(got[sub], want, name="prefill shape sampled")
