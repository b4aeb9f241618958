"""GPU parity: expert sort, tile schedules, sorted SwitchGLU (prefill) and the
whole MoE layer with combine, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_parity, bf, host_bf, host_i32, i32, triple

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_gathered_amd as m
    m.lib()
    return m


# up to 4096 pairs one workgroup sorts; (512, 8) is that limit, (513, 8) and
# more take the three-launch block sort
SORT_CASES = [(1, 8, 288), (4, 8, 288), (7, 2, 8), (128, 8, 256), (331, 8, 256), (512, 8, 256),
              (513, 8, 256), (2048, 8, 256), (4096, 8, 256), (4123, 8, 288), (3, 4, 1024), (4096, 1, 3),
              (5000, 1, 3), (1, 1, 1)]


@pytest.mark.parametrize("T,top_k,E", SORT_CASES)
def test_sort_pairs_bitwise(mg, T, top_k, E):
    if T >= 128:
        idx, _ = synth.zipf_routing(3, T, E, top_k, sub=T)
    else:
        idx = synth.sorted_topk(5, T, E, top_k, sub=T)
    got = mg.sort_pairs(i32(idx), E)
    want = oracle.sort_pairs(idx, E)
    for name, g, w in zip(("order", "lhs", "sorted_rhs", "inv", "counts", "offsets"), got, want):
        assert np.array_equal(host_i32(g), w), name


def test_sort_pairs_unsorted_slots_and_duplicates(mg):
    # slots not in ascending order and repeated experts inside a token: stability by pair index
    g = np.random.default_rng(3)
    idx = g.integers(0, 5, size=(300, 6)).astype(np.int32)
    got = mg.sort_pairs(i32(idx), 5)
    want = oracle.sort_pairs(idx, 5)
    for a, b in zip(got, want):
        assert np.array_equal(host_i32(a), b)


@pytest.mark.parametrize("bm", [16, 32, 64, 128])
@pytest.mark.parametrize("mode", [0, 1])
def test_schedule_tiles_bitwise(mg, bm, mode):
    g = np.random.default_rng(bm + mode)
    for trial in range(4):
        E = int(g.integers(1, 300))
        counts = (g.integers(0, 200, E) * (g.random(E) < 0.6)).astype(np.int64)
        if trial == 0:
            E, counts = 4, np.array([13, 8, 2, 10])   # MLX PR 4567 example
        offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        P = int(offsets[-1])
        tiles, n = mg.schedule_tiles(i32(offsets), E, P, bm, mode)
        n = int(n.item())
        if mode == 0:
            want = oracle.schedule_tiles(offsets, bm)
            assert n == len(want)
            assert np.array_equal(host_i32(tiles[:n]), want)
        else:
            want, _ = oracle.naive_tiles(offsets, bm)
            assert n == len(want)
            t = host_i32(tiles[:n])
            assert np.array_equal(t[:, [0, 2]], want) and (t[:, 1] == -1).all()


def _prefill_case(T, cfg=3, shape=synth.PREFILL, mode="drawn", sub=0):
    sh = shape
    idx, scores = synth.zipf_routing(cfg, T, sh.E, sh.top_k, sub=sub)
    x = synth.activations(cfg, T, sh.H, sub=sub)
    ex = synth.expert_set(cfg, sh.E, sh.H, sh.I, sh.gs, sh.bits, mode=mode, experts=np.unique(idx))
    return sh, idx, scores, x, ex


@pytest.mark.parametrize("T", [128, 331])
@pytest.mark.parametrize("tile_mode,bm", [(0, 0), (0, 16), (0, 32), (0, 64), (0, 128), (1, 16), (1, 64), (1, 128)])
def test_sorted_switch_glu(mg, T, tile_mode, bm):
    """MoE prefill shape (hidden 2048, E=256, top-8, inter 512, 4-bit GS 64):
    expert-sorted gate/up + SiLU and down over scheduled or naive tiles."""
    sh, idx, scores, x, ex = _prefill_case(T)
    want_tok = oracle.switch_glu(x, idx, *ex, gs=sh.gs, bits=sh.bits).reshape(-1, sh.H)
    order, *_, inv_w, _, _ = oracle.sort_pairs(idx, sh.E)
    y, inv, mode = mg.switch_glu(bf(x), i32(idx), *[triple(m) for m in ex], group_size=sh.gs, bits=sh.bits,
                                 mode=mg.MODE_SORTED, tile_mode=tile_mode, bm=bm)
    assert np.array_equal(host_i32(inv), inv_w)
    assert_parity(host_bf(y), want_tok[order], name=f"sorted T={T} bm={bm} mode={tile_mode}")


@pytest.mark.parametrize("T", [128, 331])
def test_moe_layer_with_combine(mg, T):
    """Whole layer: sorted SwitchGLU, gated shared expert, fused combine."""
    sh, idx, scores, x, ex = _prefill_case(T, sub=1)
    shp = synth.shared_params(3, sh.H, sh.shared_I, sh.gs, sh.bits)
    want, inter = oracle.moe_prefill_layer(x, idx, scores, ex, shp, gs=sh.gs, bits=sh.bits)
    xd = bf(x)
    y, inv, _ = mg.switch_glu(xd, i32(idx), *[triple(m) for m in ex], group_size=sh.gs, bits=sh.bits,
                              mode=mg.MODE_SORTED)
    g_, u_, d_, r_ = (triple(m) for m in shp)
    h = mg.affine_qmm_glu(xd, g_, u_, group_size=sh.gs, bits=sh.bits)
    s_ = mg.affine_qmm(h, *d_, group_size=sh.gs, bits=sh.bits)
    z = mg.affine_qmm(xd, *r_, group_size=sh.gs, bits=sh.bits)
    shared = mg.sigmoid_gate(s_, z)
    assert_parity(host_bf(shared), inter["shared"], name="shared expert")
    out = mg.moe_combine(y, inv, bf(scores), shared)
    assert_parity(host_bf(out), want, name=f"layer T={T}")
    # the fused combine equals the unfused tail bit for bit, and the oracle's
    # combine on the GPU's own expert outputs
    out2 = mg.moe_combine_unfused(y, inv, bf(scores), shared)
    assert np.array_equal(host_bf(out), host_bf(out2))
    assert np.array_equal(host_bf(out), oracle.combine(host_bf(y), host_i32(inv), scores, host_bf(shared)))


@pytest.mark.parametrize("bits,gs", [(4, 64), (8, 128)])
def test_large_prefill_sampled(mg, bits, gs):
    """Large MoE prefill (hidden 4096, E=288, top-8, inter 2048) at 713 rows:
    the GPU runs the whole problem; sampled experts are checked against the
    oracle row by row (all their sorted rows, every column)."""
    sh = synth.LARGE4 if bits == 4 else synth.LARGE8
    T = 713
    idx, _ = synth.zipf_routing(4, T, sh.E, sh.top_k)
    x = synth.activations(4, T, sh.H)
    ex = synth.expert_set(4 + bits, sh.E, sh.H, sh.I, sh.gs, sh.bits, mode="words")
    for tile_mode, bm in ((0, 0), (0, 32), (1, 16)):
        y, inv, _ = mg.switch_glu(bf(x), i32(idx), *[triple(m) for m in ex], group_size=sh.gs, bits=sh.bits,
                                  mode=mg.MODE_SORTED, tile_mode=tile_mode, bm=bm)
        yh = host_bf(y)
        order, lhs, srhs, inv_w, counts, offsets = oracle.sort_pairs(idx, sh.E)
        assert np.array_equal(host_i32(inv), inv_w)
        hot = int(np.argmax(counts))
        rare = int(np.flatnonzero(counts == counts[counts > 0].min())[0])
        for e in (hot, rare):
            rows = np.arange(offsets[e], offsets[e + 1])
            toks = lhs[rows]
            sub_idx = np.full((len(rows), 1), e, np.int32)
            want = oracle.switch_glu(x[toks], sub_idx, *ex, gs=sh.gs, bits=sh.bits)[:, 0]
            assert_parity(yh[rows], want, name=f"expert {e} bits {bits} mode {tile_mode}")


def test_auto_mode_and_identity_inv(mg):
    sh = synth.TINY
    ex = [triple(m) for m in synth.expert_set(0, sh.E, sh.H, sh.I, sh.gs, sh.bits, mode="drawn")]
    x = synth.activations(0, 4, sh.H)
    idx = synth.sorted_topk(0, 4, sh.E, sh.top_k)
    inv = torch.full((8,), -1, dtype=torch.int32, device="cuda")
    y, inv, mode = mg.switch_glu(bf(x), i32(idx), *ex, group_size=sh.gs, bits=sh.bits, inv=inv)
    assert mode == mg.MODE_DECODE
    assert host_i32(inv).tolist() == list(range(8))


@pytest.mark.parametrize("T", [128, 331])
@pytest.mark.parametrize("with_shared", [True, False])
def test_moe_prefill_layer(mg, T, with_shared):
    """Whole layer in one entry point (sort, routed and shared experts in the
    same tile launches, gated one-pass combine) against the oracle's layer."""
    sh, idx, scores, x, ex = _prefill_case(T, sub=2)
    shp = synth.shared_params(3, sh.H, sh.shared_I, sh.gs, sh.bits) if with_shared else None
    want, _ = oracle.moe_prefill_layer(x, idx, scores, ex, shp, gs=sh.gs, bits=sh.bits)
    got = mg.moe_prefill(bf(x), i32(idx), bf(scores), *[triple(m) for m in ex],
                         shared=None if shp is None else tuple(triple(m) for m in shp),
                         group_size=sh.gs, bits=sh.bits)
    assert_parity(host_bf(got), want, name=f"layer T={T} shared={with_shared}")


@pytest.mark.parametrize("T", [512, 1024, 2048, 4096])
def test_moe_prefill_layer_2048_sampled(mg, T):
    """The 512-, 1024-, 2048- and 4096-row layers (hidden 2048, 256 experts, top-8,
    inter 512, shared expert) on the GPU; the oracle recomputes 48 sampled
    tokens (a token's output depends only on its own row, experts and scores).
    Above 512 rows the activation prep rides in the block sort's count
    launch."""
    sh = synth.PREFILL
    idx, scores = synth.zipf_routing(3, T, sh.E, sh.top_k)
    x = synth.activations(3, T, sh.H)
    ex = synth.expert_set(3, sh.E, sh.H, sh.I, sh.gs, sh.bits, mode="words", experts=np.unique(idx))
    shp = synth.shared_params(3, sh.H, sh.shared_I, sh.gs, sh.bits)
    got = host_bf(mg.moe_prefill(bf(x), i32(idx), bf(scores), *[triple(m) for m in ex],
                                 shared=tuple(triple(m) for m in shp), group_size=sh.gs, bits=sh.bits))
    sub = np.sort(np.random.default_rng(11).choice(T, 48, replace=False))
    want, _ = oracle.moe_prefill_layer(x[sub], idx[sub], scores[sub], ex, shp, gs=sh.gs, bits=sh.bits)
    assert_parity(got[sub], want, name=f"layer {T} sampled")


def test_combine_gated_bitwise(mg):
    """The gate inside the combine equals sigmoid_gate + combine bit for bit."""
    g = np.random.default_rng(12)
    T, top_k, H = 331, 8, 2048
    P = T * top_k
    y = synth.to_bf16(g.standard_normal((P, H)) * 3)
    inv = g.permutation(P).astype(np.int32)
    sc = synth.to_bf16(g.random((T, top_k)))
    s = synth.to_bf16(g.standard_normal((T, H)))
    z = synth.to_bf16(g.standard_normal(T) * 3)
    ref = mg.moe_combine(bf(y), i32(inv), bf(sc), mg.sigmoid_gate(bf(s), bf(z)))
    got = mg.moe_combine_gated(bf(y), i32(inv), bf(sc), bf(s), bf(z))
    assert np.array_equal(host_bf(got), host_bf(ref))


def test_moe_prefill_repeatable(mg):
    """Five calls of the 512-row layer give the same bits (no race in the
    asynchronous loads into LDS, the tile schedule or the combine)."""
    sh = synth.PREFILL
    T = 512
    idx, scores = synth.zipf_routing(3, T, sh.E, sh.top_k, sub=5)
    x = synth.activations(3, T, sh.H, sub=5)
    ex = [triple(m) for m in synth.expert_set(3, sh.E, sh.H, sh.I, sh.gs, sh.bits, mode="words",
                                              experts=np.unique(idx))]
    shp = tuple(triple(m) for m in synth.shared_params(3, sh.H, sh.shared_I, sh.gs, sh.bits))
    outs = [host_bf(mg.moe_prefill(bf(x), i32(idx), bf(scores), *ex, shared=shp, group_size=sh.gs, bits=sh.bits))
            for _ in range(5)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_large_hybrid_repeatable(mg):
    """The sorted SwitchGLU at the large shape (713 rows: hot experts in
    128-row tiles, partly filled tiles in the 64- and 32-row bodies, tail
    experts in 32-row tiles) gives the same bits on every call, eager and
    replayed as a HIP graph.  Regression: in the last steps of the short
    tiles fewer loads follow a step's own, and a step wait that did not
    shrink with them let a wave reach the barrier with its rows still in
    flight into LDS, where the other waves read them."""
    sh = synth.LARGE4
    dev = torch.device("cuda")
    gate, up, down = synth.device_expert_set(dev, 4, sh.E, sh.H, sh.I, sh.gs, sh.bits)
    T = 713
    idx_np, _ = synth.zipf_routing(4, T, sh.E, sh.top_k)
    idx = torch.from_numpy(idx_np).to(dev)
    x = bf(synth.activations(4, T, sh.H))
    y = torch.empty((T * sh.top_k, sh.H), dtype=torch.bfloat16, device=dev)
    inv = torch.empty(T * sh.top_k, dtype=torch.int32, device=dev)

    def run():
        mg.switch_glu(x, idx, gate, up, down, group_size=sh.gs, bits=sh.bits, mode=mg.MODE_SORTED,
                      tile_mode=0, bm=0, y=y, inv=inv)

    run()
    torch.cuda.synchronize()
    ref = y.clone()
    for _ in range(6):
        y.zero_()
        run()
        torch.cuda.synchronize()
        assert torch.equal(y, ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for _ in range(6):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref)


@pytest.mark.parametrize("T", [1, 4, 37])
def test_moe_prefill_few_tokens(mg, T):
    """The whole-layer entry point with fewer tokens than one tile (every
    routed expert and the shared expert in 32-row tiles)."""
    sh, idx, scores, x, ex = _prefill_case(T, sub=7)
    shp = synth.shared_params(3, sh.H, sh.shared_I, sh.gs, sh.bits)
    want, _ = oracle.moe_prefill_layer(x, idx, scores, ex, shp, gs=sh.gs, bits=sh.bits)
    got = mg.moe_prefill(bf(x), i32(idx), bf(scores), *[triple(m) for m in ex],
                         shared=tuple(triple(m) for m in shp), group_size=sh.gs, bits=sh.bits)
    assert_parity(host_bf(got), want, name=f"layer T={T}")


def test_moe_prefill_8bit_large_sampled(mg):
    """Whole layer at the large shape with 8-bit GS 128 codes (hidden 4096,
    288 experts, inter 2048), no shared expert: 713 rows on the GPU, 3
    sampled tokens (up to 24 experts) through the oracle."""
    sh = synth.LARGE8
    T = 713
    idx, scores = synth.zipf_routing(4, T, sh.E, sh.top_k, sub=3)
    x = synth.activations(4, T, sh.H, sub=3)
    ex = synth.expert_set(12, sh.E, sh.H, sh.I, sh.gs, sh.bits, mode="words", experts=np.unique(idx))
    got = host_bf(mg.moe_prefill(bf(x), i32(idx), bf(scores), *[triple(m) for m in ex], shared=None,
                                 group_size=sh.gs, bits=sh.bits))
    sub = np.sort(np.random.default_rng(13).choice(T, 3, replace=False))
    want, _ = oracle.moe_prefill_layer(x[sub], idx[sub], scores[sub], ex, None, gs=sh.gs, bits=sh.bits)
    assert_parity(got[sub], want, name="layer 8-bit sampled")


def _host_experts(trips, uniq):
    """Host copies (uint32 words, bf16 bits) of the experts `uniq` of device weight triples."""
    out = []
    for w, sc, bi in trips:
        u = torch.from_numpy(uniq.astype(np.int64)).to(w.device)
        out.append((w.index_select(0, u).cpu().numpy().view(np.uint32),
                    host_bf(sc.index_select(0, u)), host_bf(bi.index_select(0, u))))
    return out


@pytest.mark.parametrize("T,bits,nsub", [(4123, 4, 3), (8192, 4, 2), (16384, 4, 2), (4123, 8, 2)])
def test_large_layer_timed_sizes_sampled(mg, T, bits, nsub):
    """The large layer (hidden 4096, 288 experts, top-8, inter 2048, no shared
    expert) at the sizes the benchmark times, with the benchmark's weights
    (drawn on the device): the GPU runs all T rows; the oracle recomputes a few
    sampled tokens from host copies of the experts they use."""
    sh = synth.LARGE4 if bits == 4 else synth.LARGE8
    dev = torch.device("cuda")
    ex = synth.device_expert_set(dev, 4, sh.E, sh.H, sh.I, sh.gs, sh.bits)
    idx, scores = synth.zipf_routing(4, T, sh.E, sh.top_k)
    x = synth.activations(4, T, sh.H)
    got = host_bf(mg.moe_prefill(bf(x), i32(idx), bf(scores), *ex, shared=None, group_size=sh.gs, bits=sh.bits))
    sub = np.sort(np.random.default_rng(T + bits).choice(T, nsub, replace=False))
    uniq = np.unique(idx[sub])
    local = np.searchsorted(uniq, idx[sub]).astype(np.int32)       # ascending ids stay ascending
    want, _ = oracle.moe_prefill_layer(x[sub], local, scores[sub], _host_experts(ex, uniq), None,
                                       gs=sh.gs, bits=sh.bits)
    del ex
    torch.cuda.empty_cache()
    assert_parity(got[sub], want, name=f"large layer T={T} bits={bits}")
