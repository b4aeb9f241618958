"""GPU parity: combine tail (fused vs unfused vs oracle, bit for bit), the
self-check, and dense few-row quantized matmul with the decoder chain glue."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_parity, bf, host_bf, host_i32, i32, triple, words

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_gathered_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("T,top_k,H", [(128, 8, 2048), (331, 8, 2048), (2048, 8, 2048), (4096, 8, 2048),
                                       (3, 1, 16), (17, 2, 40), (5, 8, 4096), (11, 4, 32), (13, 6, 48),
                                       (9, 3, 64), (7, 5, 24)])
def test_combine_bitwise(mg, T, top_k, H):
    g = np.random.default_rng(T + top_k + H)
    P = T * top_k
    y = synth.to_bf16(g.standard_normal((P, H)) * 3)
    inv = g.permutation(P).astype(np.int32)
    sc = synth.to_bf16(g.random((T, top_k)))
    sh = synth.to_bf16(g.standard_normal((T, H)))
    for shared in (sh, None):
        want = oracle.combine(y, inv, sc, shared)
        sd = None if shared is None else bf(shared)
        fused = host_bf(mg.moe_combine(bf(y), i32(inv), bf(sc), sd))
        unfused = host_bf(mg.moe_combine_unfused(bf(y), i32(inv), bf(sc), sd))
        assert np.array_equal(fused, unfused)
        assert np.array_equal(fused, want)
    # inv = None means token order
    want = oracle.combine(y, np.arange(P, dtype=np.int32), sc, sh)
    assert np.array_equal(host_bf(mg.moe_combine(bf(y), None, bf(sc), bf(sh))), want)


def test_selfcheck_and_forced_failure(mg, monkeypatch):
    assert mg.selfcheck() == 0
    monkeypatch.setenv("MOEGQ_FORCE_SELFCHECK_FAIL", "1")
    assert mg.selfcheck() == -9


def test_validate_indices(mg):
    assert mg.validate_indices(i32(np.array([0, 3, 3, 7])), 8, sorted_=True) == 0
    assert mg.validate_indices(i32(np.array([0, 3, 2, 7])), 8, sorted_=True) == -10
    assert mg.validate_indices(i32(np.array([0, 8])), 8) == -10


@pytest.mark.parametrize("M", [1, 2, 3, 4, 6, 8, 12, 16, 33, 200])
@pytest.mark.parametrize("bits,gs", [(4, 32), (4, 64), (4, 128), (8, 32), (8, 64), (8, 128)])
def test_affine_qmm_rows(mg, M, bits, gs):
    g = np.random.default_rng(M * 7 + bits * 3 + gs)
    N, K = 200, 1280
    w, s, b = synth.minmax_matrix(g, N, K, gs, bits, scale=1 / np.sqrt(K))
    x = synth.to_bf16(g.standard_normal((M, K)))
    want = oracle.quantized_matmul(x, w, s, b, True, gs, bits)
    got = mg.affine_qmm(bf(x), words(w), bf(s), bf(b), group_size=gs, bits=bits)
    assert_parity(host_bf(got), want, name=f"M={M} {bits}/{gs}")
    if M <= 16:
        r = synth.to_bf16(g.standard_normal((M, N)))
        got_r = mg.affine_qmm(bf(x), words(w), bf(s), bf(b), group_size=gs, bits=bits, residual=bf(r))
        want_r = oracle.f64_to_bf16(oracle.bf16_to_f64(want) + oracle.bf16_to_f64(r))
        assert_parity(host_bf(got_r), want_r, name="residual")
        # in place (out is the residual buffer): each output's residual is read
        # by the lane that writes it, so the result is the same bit for bit
        rt = bf(r)
        mg.affine_qmm(bf(x), words(w), bf(s), bf(b), group_size=gs, bits=bits, residual=rt, out=rt)
        assert np.array_equal(host_bf(rt), host_bf(got_r))


@pytest.mark.parametrize("M", [1, 4, 16])
def test_affine_qmm_full_shape_sampled(mg, M):
    """Dense gate projection at its real size (N 9728, K 2560) and the down
    projection (N 2560, K 9728): GPU on all outputs, oracle on sampled columns."""
    g = np.random.default_rng(40 + M)
    for N, K in ((9728, 2560), (2560, 9728)):
        w, s, b = synth.drawn_words(g, N, K, 64, 4)
        x = synth.to_bf16(g.standard_normal((M, K)))
        got = host_bf(mg.affine_qmm(bf(x), words(w), bf(s), bf(b), group_size=64, bits=4))
        cols = np.sort(g.choice(N, 128, replace=False))
        want = oracle.quantized_matmul(x, w[cols], s[cols], b[cols], True, 64, 4)
        assert_parity(got[:, cols], want, name=f"sampled {N}x{K} M={M}")


@pytest.mark.parametrize("M,N", [(3, 8200), (16, 8200), (6, 2600), (16, 2600), (4, 1040)])
def test_affine_qmm_wide_ragged(mg, M, N):
    """Few-row products on wide matrices whose last 16-column block is ragged
    (N 8200, 2600, 1040), with a K split over several waves; plain and gate/up."""
    g = np.random.default_rng(60 + M + N)
    K = 1024
    w, s, b = synth.drawn_words(g, N, K, 64, 4)
    x = synth.to_bf16(g.standard_normal((M, K)))
    got = host_bf(mg.affine_qmm(bf(x), words(w), bf(s), bf(b), group_size=64, bits=4))
    cols = np.unique(np.concatenate([g.choice(N, 96, replace=False), np.arange(N - 40, N)]))
    want = oracle.quantized_matmul(x, w[cols], s[cols], b[cols], True, 64, 4)
    assert_parity(got[:, cols], want, name=f"blocks M={M} N={N}")
    w2, s2, b2 = synth.drawn_words(g, N, K, 64, 4)
    got2 = host_bf(mg.affine_qmm_glu(bf(x), (words(w), bf(s), bf(b)), (words(w2), bf(s2), bf(b2)),
                                     group_size=64, bits=4))
    gg = oracle.quantized_matmul(x, w[cols], s[cols], b[cols], True, 64, 4)
    uu = oracle.quantized_matmul(x, w2[cols], s2[cols], b2[cols], True, 64, 4)
    want2 = oracle.f64_to_bf16(oracle.silu(oracle.bf16_to_f64(gg)) * oracle.bf16_to_f64(uu))
    assert_parity(got2[:, cols], want2, name=f"blocks glu M={M} N={N}")


@pytest.mark.parametrize("M", [1, 5, 16, 40, 300])
def test_affine_qmm_glu(mg, M):
    g = np.random.default_rng(50 + M)
    N, K = 96, 512
    gate = synth.drawn_matrix(g, N, K, 64, 4)
    up = synth.drawn_matrix(g, N, K, 64, 4)
    x = synth.to_bf16(g.standard_normal((M, K)))
    gg = oracle.quantized_matmul(x, *gate, True, 64, 4)
    uu = oracle.quantized_matmul(x, *up, True, 64, 4)
    want = oracle.f64_to_bf16(oracle.silu(oracle.bf16_to_f64(gg)) * oracle.bf16_to_f64(uu))
    got = mg.affine_qmm_glu(bf(x), triple(gate), triple(up), group_size=64, bits=4)
    assert_parity(host_bf(got), want, name=f"glu M={M}")


@pytest.mark.parametrize("M,K", [(1, 2560), (4, 4096), (16, 9728), (3, 100), (2, 2048), (5, 8192)])
def test_rms_norm_paths(mg, M, K):
    """RMSNorm on the GPU (16-byte path with the row in registers for K a
    multiple of 8 up to 8192, element path otherwise) against the oracle."""
    g = np.random.default_rng(70 + K)
    x = synth.to_bf16(g.standard_normal((M, K)) * 2)
    w = synth.to_bf16(1 + 0.1 * g.standard_normal(K))
    want = oracle.rms_norm(x, w, 1e-6)
    got = host_bf(mg.rms_norm(bf(x), bf(w)))
    assert_parity(got, want, name=f"rms_norm M={M} K={K}")


def test_dense_chain_small(mg):
    """Two layers of the decoder chain (rms_norm, q/k/v, kv feed, o + residual,
    rms_norm, SwiGLU, down + residual) at reduced width, 2 weight sets."""
    d = dict(hidden=256, q_out=512, kv_out=128, inter=768, layers=2, sets=2)
    sets = synth.dense_sets(2, 64, 4, mode="minmax", d=d)
    g = np.random.default_rng(60)
    for M in (1, 4, 16):
        h0 = synth.to_bf16(g.standard_normal((M, 256)))
        nw = synth.to_bf16(np.ones(256, np.float32))
        want = oracle.dense_forward(h0, sets, 2, nw, gs=64, bits=4)
        dsets = [{k: triple(v) for k, v in L.items()} for L in sets]
        h = bf(h0)
        nwd = bf(nw)
        for li in range(2):
            L = dsets[li % 2]
            x = mg.rms_norm(h, nwd)
            q = mg.affine_qmm(x, *L["q"], group_size=64)
            k = mg.affine_qmm(x, *L["k"], group_size=64)
            v = mg.affine_qmm(x, *L["v"], group_size=64)
            o_in = mg.kv_feed(q, k, v)
            h = mg.affine_qmm(o_in, *L["o"], group_size=64, residual=h)
            x = mg.rms_norm(h, nwd)
            a = mg.affine_qmm_glu(x, L["g"], L["u"], group_size=64)
            h = mg.affine_qmm(a, *L["dn"], group_size=64, residual=h)
        assert_parity(host_bf(h), want, name=f"chain M={M}")


def test_dense_chain_stacked_qkv(mg):
    """The chain with q, k and v as one stacked product [q_out + 2 kv_out,
    hidden] and the kv feed reading its column ranges (the benchmark's form)."""
    import torch
    d = dict(hidden=256, q_out=512, kv_out=128, inter=768, layers=2, sets=2)
    sets = synth.dense_sets(2, 64, 4, mode="minmax", d=d)
    g = np.random.default_rng(61)
    for M in (1, 4, 16):
        h0 = synth.to_bf16(g.standard_normal((M, 256)))
        nw = synth.to_bf16(np.ones(256, np.float32))
        want = oracle.dense_forward(h0, sets, 2, nw, gs=64, bits=4)
        dsets = []
        for L in sets:
            t = {k: triple(v) for k, v in L.items()}
            t["qkv"] = tuple(torch.cat([t["q"][i], t["k"][i], t["v"][i]], 0).contiguous() for i in range(3))
            dsets.append(t)
        h = bf(h0)
        nwd = bf(nw)
        for li in range(2):
            L = dsets[li % 2]
            x = mg.rms_norm(h, nwd)
            qkv = mg.affine_qmm(x, *L["qkv"], group_size=64)
            h = mg.affine_qmm(mg.kv_feed_stacked(qkv, 512, 128, 128), *L["o"], group_size=64, residual=h)
            x = mg.rms_norm(h, nwd)
            a = mg.affine_qmm_glu(x, L["g"], L["u"], group_size=64)
            h = mg.affine_qmm(a, *L["dn"], group_size=64, residual=h)
        assert_parity(host_bf(h), want, name=f"stacked chain M={M}")


def test_gather_qmm_page_cases(mg):
    """nuvec "gather_qmm_selects_batches" / gather kernels: explicit lhs/rhs,
    default indices, broadcast index shapes, rows M > 1, sorted grouped rows."""
    g = np.random.default_rng(70)
    E, N, K = 3, 8, 64
    W = [synth.drawn_matrix(g, N, K, 32, 4) for _ in range(E)]
    w, s, b = (np.stack([m[i] for m in W]) for i in range(3))
    dw = (words(w), bf(s), bf(b))
    x = synth.to_bf16(g.standard_normal((4, 2, K)))
    got = mg.gather_qmm(bf(x), *dw, rhs_indices=i32([1, 2, 0]), lhs_indices=i32([3, 0, 2]), group_size=32)
    assert_parity(host_bf(got), oracle.gather_qmm(x, w, s, b, lhs=[3, 0, 2], rhs=[1, 2, 0], gs=32), name="lhs/rhs")
    x1 = synth.to_bf16(g.standard_normal((1, 1, K)))
    got = mg.gather_qmm(bf(x1), *dw, group_size=32)
    assert got.shape == (3, 1, N)
    assert_parity(host_bf(got), oracle.gather_qmm(x1, w, s, b, gs=32), name="defaults")
    x3 = synth.to_bf16(g.standard_normal((3, 1, K)))
    li, ri = np.array([[2, 0], [1, 1]]), np.array([[2, 1]])
    got = mg.gather_qmm(bf(x3), *dw, rhs_indices=i32(ri), lhs_indices=i32(li), group_size=32)
    assert got.shape == (2, 2, 1, N)
    assert_parity(host_bf(got), oracle.gather_qmm(x3, w, s, b, lhs=li, rhs=ri, gs=32), name="broadcast")
    # rows per batch 33..40 (tile route), unaligned N
    for (e, n, k, m, nb) in ((4, 64, 256, 40, 3), (4, 40, 128, 33, 2)):
        Wb = [synth.drawn_matrix(g, n, k, 64, 4) for _ in range(e)]
        wb, sb, bb = (np.stack([q[i] for q in Wb]) for i in range(3))
        xb = synth.to_bf16(g.standard_normal((nb, m, k)))
        ids = (np.arange(nb) * 7 + 3) % e
        got = mg.gather_qmm(bf(xb), words(wb), bf(sb), bf(bb), rhs_indices=i32(ids), group_size=64)
        assert_parity(host_bf(got), oracle.gather_qmm(xb, wb, sb, bb, rhs=ids, gs=64), name=f"tiles M={m}")
    # sorted single rows: grouped route (100 and 70 batches), and too few rows per expert (20)
    for (e, n, k, nb) in ((8, 64, 256, 100), (16, 48, 192, 70), (8, 64, 256, 20)):
        Wb = [synth.drawn_matrix(g, n, k, 64, 4) for _ in range(e)]
        wb, sb, bb = (np.stack([q[i] for q in Wb]) for i in range(3))
        xb = synth.to_bf16(g.standard_normal((nb, 1, k)))
        ids = np.sort((np.arange(nb) * 7 + 3) % e)
        got = mg.gather_qmm(bf(xb), words(wb), bf(sb), bf(bb), rhs_indices=i32(ids), group_size=64,
                            sorted_indices=True)
        assert_parity(host_bf(got), oracle.gather_qmm(xb, wb, sb, bb, rhs=ids, gs=64), name=f"sorted {nb}")
