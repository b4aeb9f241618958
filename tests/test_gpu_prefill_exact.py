"""GPU parity of the production prefill route (the whole-layer entry point and
the sorted SwitchGLU on the matrix cores) against the oracle:

* integer-exact inputs, compared bit for bit: every product and partial sum
  of gate, up and down is exact in fp32 and the gate outputs are powers of two
  >= 32, so silu(g) * u is a bf16 value on both sides and any correct
  summation order gives the oracle's bits;
* the sort results and both tile tables the layer writes, read back from its
  workspace, against the oracle's sort and two-size schedule;
* the 2048-row layer on every token;
* the large layer at the benchmark's sizes, sampled by tile class (first and
  last rows of 128-row tiles, 32-row tail tiles, the last active expert);
* activations and intermediates outside fp16's range.
"""
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


# ----------------------------------------------------------------------------- preconditions
def _frac_bits(a) -> int:
    """Smallest m with every a * 2^m an integer (a holds dyadic values)."""
    a = np.abs(np.asarray(a, np.float64))
    for m in range(0, 64):
        v = a * 2.0 ** m
        if np.all(v == np.floor(v)):
            return m
    raise AssertionError("not dyadic")


def _assert_fp32_exact(a, b, what):
    """Every partial sum of a @ b.T is exact in fp32 in any order: all terms
    are multiples of 2^-m and the sum of their magnitudes stays below 2^(24-m)."""
    m = _frac_bits(a) + _frac_bits(b)
    bound = (np.abs(a) @ np.abs(b).T).max() if a.size and b.size else 0.0
    assert bound * 2.0 ** m < 2.0 ** 24, f"{what}: inputs are not integer-exact ({bound} at 2^-{m})"


def _check_chain(x_u16, rows_per_expert, experts, gs, bits):
    """Preconditions of the integer-exact chain for each expert's rows."""
    for e, toks in rows_per_expert.items():
        xf = oracle.bf16_to_f64(x_u16[toks])
        gate, up, down = ((m[0][e], m[1][e], m[2][e]) for m in experts)
        H = xf.shape[1]
        Wg = oracle.dequant(*gate, gs, bits, H)
        Wu = oracle.dequant(*up, gs, bits, H)
        _assert_fp32_exact(xf, Wg, f"gate e={e}")
        _assert_fp32_exact(xf, Wu, f"up e={e}")
        g = xf @ Wg.T
        assert set(np.unique(g)) <= {32.0, 64.0, 128.0}, f"gate e={e}: not a power of two >= 32"
        ur = oracle.bf16_to_f64(oracle.f64_to_bf16(xf @ Wu.T))
        h = g * ur
        assert np.abs(h).max() < 65504, f"e={e}: intermediate beyond fp16's range"
        Wd = oracle.dequant(*down, gs, bits, Wg.shape[0])
        _assert_fp32_exact(h, Wd, f"down e={e}")


def _exact_case(T, bits=4, gs=64, sub=0):
    sh = synth.PREFILL
    idx, scores = synth.zipf_routing(3, T, sh.E, sh.top_k, sub=sub)
    x = synth.group_unit_x(synth.rng(3, 4, 1, sub), T, sh.H, gs)
    ex = synth.exact_glu_experts(3 + sub, sh.E, sh.H, sh.I, gs, bits, experts=np.unique(idx))
    rows = {int(e): np.nonzero((idx == e).any(axis=1))[0] for e in np.unique(idx)}
    _check_chain(x, rows, ex, gs, bits)
    return sh, idx, scores, x, ex


@pytest.mark.parametrize("T", [37, 331, 2048])
@pytest.mark.parametrize("with_shared", [True, False])
def test_moe_prefill_integer_exact_bitwise(mg, T, with_shared):
    """The whole-layer entry point (both tile sizes, the shared expert as one
    more expert of the tile launches, the gated combine) equals the oracle's
    layer bit for bit on integer-exact inputs."""
    sh, idx, scores, x, ex = _exact_case(T, sub=T % 7)
    shp = synth.exact_shared(3, sh.H, sh.I, sh.gs, sh.bits) if with_shared else None
    if shp is not None:
        xf = oracle.bf16_to_f64(x)
        Wr = oracle.dequant(*shp[3], sh.gs, sh.bits, sh.H)
        assert set(np.unique(xf @ Wr.T)) == {64.0}
        _check_chain(x, {0: np.arange(T)}, tuple((m[0][None], m[1][None], m[2][None]) for m in shp[:3]),
                     sh.gs, sh.bits)
    want, _ = oracle.moe_prefill_layer(x, idx, scores, ex, shp, gs=sh.gs, bits=sh.bits)
    got = host_bf(mg.moe_prefill(bf(x), i32(idx), bf(scores), *[triple(m) for m in ex],
                                 shared=None if shp is None else tuple(triple(m) for m in shp),
                                 group_size=sh.gs, bits=sh.bits))
    bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
    assert bad.size == 0, f"{bad.size} elements differ, first at {np.unravel_index(bad[0], got.shape)}"


@pytest.mark.parametrize("T,bm", [(331, 0), (2048, 0), (331, 128), (2048, 128)])
def test_sorted_switch_glu_integer_exact_bitwise(mg, T, bm):
    """Sorted SwitchGLU on the matrix cores: bm 0 runs the two-size schedule in
    one launch per pass, bm 128 the 128-row tiles alone; expert-sorted y
    equals the oracle's bit for bit."""
    sh, idx, scores, x, ex = _exact_case(T, sub=1)
    want_tok = oracle.switch_glu(x, idx, *ex, gs=sh.gs, bits=sh.bits).reshape(-1, sh.H)
    order = oracle.sort_pairs(idx, sh.E)[0]
    y, inv, _ = mg.switch_glu(bf(x), i32(idx), *[triple(m) for m in ex], group_size=sh.gs, bits=sh.bits,
                              mode=mg.MODE_SORTED, tile_mode=mg.TILES_SCHEDULED, bm=bm)
    got = host_bf(y)
    assert np.array_equal(got, want_tok[order])


# ----------------------------------------------------------------------------- tile tables
def _zero_experts(E, H, I, gs, bits, dev="cuda"):
    def mat(N, K):
        return (torch.zeros((E, N, K * bits // 32), dtype=torch.int32, device=dev),
                torch.zeros((E, N, K // gs), dtype=torch.bfloat16, device=dev),
                torch.zeros((E, N, K // gs), dtype=torch.bfloat16, device=dev))
    return mat(I, H), mat(I, H), mat(H, I)


def _zero_shared(H, I, gs, bits, dev="cuda"):
    def mat(N, K):
        return (torch.zeros((N, K * bits // 32), dtype=torch.int32, device=dev),
                torch.zeros((N, K // gs), dtype=torch.bfloat16, device=dev),
                torch.zeros((N, K // gs), dtype=torch.bfloat16, device=dev))
    return mat(I, H), mat(I, H), mat(H, I), mat(1, H)


TABLE_CASES = [(T, s) for T in (1, 4, 37, 128, 331, 512, 513, 2048, 4096) for s in (True, False)]
_theta_sides = set()


@pytest.mark.parametrize("T,with_shared", TABLE_CASES)
def test_moe_prefill_tables_bitwise(mg, T, with_shared):
    """The sort results and the two tile tables the whole-layer entry point
    writes (one-workgroup sort up to 4096 pairs, block sort above) equal the
    oracle's sort and two-size schedule entry for entry."""
    sh = synth.PREFILL
    idx, scores = synth.zipf_routing(3, T, sh.E, sh.top_k, sub=T)
    dev = torch.device("cuda")
    ex = _zero_experts(sh.E, sh.H, sh.I, sh.gs, sh.bits)
    shp = _zero_shared(sh.H, sh.I, sh.gs, sh.bits) if with_shared else None
    ws = torch.full((mg.moe_prefill_workspace_bytes(T, sh.top_k, sh.E, sh.H, sh.I, with_shared),), 0xA5,
                    dtype=torch.uint8, device=dev)
    x = torch.zeros((T, sh.H), dtype=torch.bfloat16, device=dev)
    mg.moe_prefill(x, i32(idx), bf(scores), *ex, shared=shp, group_size=sh.gs, bits=sh.bits, workspace=ws)
    tb = mg.moe_prefill_tables(ws, T, sh.top_k, sh.E, sh.H, sh.I, with_shared)
    L = tb["layout"]
    order, lhs, srhs, inv, counts, offsets = oracle.sort_pairs(idx, sh.E)
    P = T * sh.top_k
    extra = T if with_shared else 0
    assert np.array_equal(host_i32(tb["inv"]), inv)
    assert np.array_equal(host_i32(tb["lhs"]), np.concatenate([lhs, np.arange(extra)]))
    assert np.array_equal(host_i32(tb["sorted_rhs"]), srhs)
    assert np.array_equal(host_i32(tb["counts"]), counts)
    assert np.array_equal(host_i32(tb["offsets"]), offsets)
    big, small = oracle.hybrid_tiles(offsets, extra, L["big"], L["small"], L["slots"], L["col_blocks"])
    assert np.array_equal(host_i32(tb["tiles"]).reshape(-1, 3), big)
    assert np.array_equal(host_i32(tb["small_tiles"]).reshape(-1, 3), small)
    assert P + extra == int(big[:, 2].sum() + small[:, 2].sum())
    _theta_sides.add(len(big) > 0)


def test_tables_cover_both_schedules():
    """The cases above include layers with and without 128-row tiles."""
    if len(_theta_sides) == 0:
        pytest.skip("table cases did not run")
    assert _theta_sides == {True, False}


# ----------------------------------------------------------------------------- full and sampled layers
def test_moe_prefill_layer_2048_every_token(mg):
    """The 2048-row layer (hidden 2048, 256 experts, top-8, inter 512, shared
    expert) checked against the oracle on all 2048 tokens."""
    sh = synth.PREFILL
    T = 2048
    idx, scores = synth.zipf_routing(3, T, sh.E, sh.top_k)
    x = synth.activations(3, T, sh.H)
    ex = synth.expert_set(3, sh.E, sh.H, sh.I, sh.gs, sh.bits, mode="words", experts=np.unique(idx))
    shp = synth.shared_params(3, sh.H, sh.shared_I, sh.gs, sh.bits)
    got = host_bf(mg.moe_prefill(bf(x), i32(idx), bf(scores), *[triple(m) for m in ex],
                                 shared=tuple(triple(m) for m in shp), group_size=sh.gs, bits=sh.bits))
    want, _ = oracle.moe_prefill_layer(x, idx, scores, ex, shp, gs=sh.gs, bits=sh.bits)
    assert_parity(got, want, name="layer 2048 every token")


def _host_expert(trips, e):
    out = []
    for w, sc, bi in trips:
        out.append((w[e:e + 1].cpu().numpy().view(np.uint32), host_bf(sc[e:e + 1]), host_bf(bi[e:e + 1])))
    return out


def _tile_class_rows(big, small, offsets, rng_):
    """Sorted rows chosen by tile class, grouped by expert: the first and last
    rows of up to 6 of the hottest expert's 128-row tiles, the last 128-row
    tile's rows, every row of two 32-row tail tiles, and every row of the
    last active expert."""
    pick = {}

    def add(e, rows):
        pick.setdefault(int(e), set()).update(int(r) for r in rows)

    if len(big):
        counts = np.diff(offsets)
        hot = int(np.argmax(counts))
        ht = big[big[:, 1] == hot]
        for t in ht[np.linspace(0, len(ht) - 1, min(6, len(ht))).astype(int)]:
            add(hot, (t[0], t[0] + t[2] - 1))
        last = big[-1]
        add(last[1], range(last[0], last[0] + last[2]))
    if len(small):
        for t in small[rng_.choice(len(small), min(2, len(small)), replace=False)]:
            add(t[1], range(t[0], t[0] + t[2]))
    e_last = int(np.flatnonzero(np.diff(offsets))[-1])
    add(e_last, range(offsets[e_last], offsets[e_last + 1]))
    return {e: np.array(sorted(r)) for e, r in pick.items()}


@pytest.mark.parametrize("T,bits", [(4123, 4), (8192, 4), (16384, 4), (4123, 8)])
def test_large_layer_tile_classes(mg, T, bits):
    """The large layer's sorted SwitchGLU (hidden 4096, 288 experts, top-8,
    inter 2048) at the benchmark's sizes and weights: the GPU runs all rows;
    the oracle recomputes the rows of every tile class (see
    _tile_class_rows), each as its own tensor for the tolerance."""
    sh = synth.LARGE4 if bits == 4 else synth.LARGE8
    dev = torch.device("cuda")
    ex = synth.device_expert_set(dev, 4, sh.E, sh.H, sh.I, sh.gs, sh.bits)
    idx, _ = synth.zipf_routing(4, T, sh.E, sh.top_k)
    x = synth.activations(4, T, sh.H)
    y, inv, _ = mg.switch_glu(bf(x), i32(idx), *ex, group_size=sh.gs, bits=sh.bits, mode=mg.MODE_SORTED)
    yh = host_bf(y)
    order, lhs, srhs, inv_w, counts, offsets = oracle.sort_pairs(idx, sh.E)
    assert np.array_equal(host_i32(inv), inv_w)
    L = mg.moe_prefill_layout(T, sh.top_k, sh.E, sh.H, sh.I, False)
    big, small = oracle.hybrid_tiles(offsets, 0, L["big"], L["small"], L["slots"], L["col_blocks"])
    picks = _tile_class_rows(big, small, offsets, np.random.default_rng(T + bits))
    for e, rows in picks.items():
        gate, up, down = _host_expert(ex, e)
        want = oracle.switch_glu(x[lhs[rows]], np.zeros((len(rows), 1), np.int32), gate, up, down,
                                 gs=sh.gs, bits=sh.bits)[:, 0]
        assert_parity(yh[rows], want, name=f"T={T} bits={bits} expert {e} ({len(rows)} rows)")
    del ex, y
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- range
@pytest.mark.parametrize("entry", ["moe_prefill", "switch_glu"])
def test_prefill_outside_fp16_range(mg, entry):
    """bf16 activations far outside fp16's range (|x| about 1e5 on some tokens,
    about 1e-6 on others) and intermediates above 65504: each group of tokens
    is held to the tolerance on its own scale."""
    sh = synth.PREFILL
    T = 331
    idx, scores = synth.zipf_routing(3, T, sh.E, sh.top_k, sub=9)
    x0 = oracle.bf16_to_f64(synth.activations(3, T, sh.H, sub=9))
    factor = np.ones(T)
    big_t, tiny_t = np.arange(0, T, 5), np.arange(1, T, 5)
    factor[big_t], factor[tiny_t] = 1e5, 1e-6
    x = synth.to_bf16((x0 * factor[:, None]).astype(np.float32))
    ex = synth.expert_set(3, sh.E, sh.H, sh.I, sh.gs, sh.bits, mode="words", experts=np.unique(idx))
    if entry == "moe_prefill":
        shp = synth.shared_params(3, sh.H, sh.shared_I, sh.gs, sh.bits)
        want, inter = oracle.moe_prefill_layer(x, idx, scores, ex, shp, gs=sh.gs, bits=sh.bits)
        got = host_bf(mg.moe_prefill(bf(x), i32(idx), bf(scores), *[triple(m) for m in ex],
                                     shared=tuple(triple(m) for m in shp), group_size=sh.gs, bits=sh.bits))
        groups = {"large": big_t, "tiny": tiny_t, "normal": np.setdiff1d(np.arange(T), np.r_[big_t, tiny_t])}
        for name, toks in groups.items():
            assert_parity(got[toks], want[toks], name=f"{entry} {name} tokens")
    else:
        want = oracle.switch_glu(x, idx, *ex, gs=sh.gs, bits=sh.bits)
        y, inv, _ = mg.switch_glu(bf(x), i32(idx), *[triple(m) for m in ex], group_size=sh.gs, bits=sh.bits,
                                  mode=mg.MODE_SORTED)
        yt = host_bf(y)[host_i32(inv)].reshape(T, sh.top_k, sh.H)
        for name, toks in (("large", big_t), ("tiny", tiny_t)):
            assert_parity(yt[toks], want[toks], name=f"{entry} {name} tokens")
    # the large tokens' intermediates exceed fp16's largest finite value
    xf = oracle.bf16_to_f64(x[big_t[:1]])
    e = int(idx[big_t[0], 0])
    Wg = oracle.dequant(ex[0][0][e], ex[0][1][e], ex[0][2][e], sh.gs, sh.bits, sh.H)
    Wu = oracle.dequant(ex[1][0][e], ex[1][1][e], ex[1][2][e], sh.gs, sh.bits, sh.H)
    h = oracle.silu(xf @ Wg.T) * (xf @ Wu.T)
    assert np.abs(h).max() > 65504
