"""GPU parity of the router: expert ids bit for bit and bf16 scores bit for bit
against the oracle's router, and the whole prefill layer fed by the GPU
router equals the layer fed by the host routing."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import bf, host_bf, i32, triple

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_gathered_amd as m
    m.lib()
    return m


def _check(mg, logits, k):
    idx, sc = mg.route(torch.from_numpy(logits).cuda(), k)
    want_i, want_s = oracle.route(logits, k)
    assert np.array_equal(idx.cpu().numpy(), want_i)
    assert np.array_equal(host_bf(sc), want_s)


@pytest.mark.parametrize("cfg,T,E,k", [(3, 2048, 256, 8), (4, 37, 288, 8), (5, 9, 1024, 64), (6, 13, 64, 64),
                                       (7, 11, 100, 3), (8, 5, 1, 1), (9, 21, 65, 5)])
def test_route_bitwise(mg, cfg, T, E, k):
    _check(mg, synth.zipf_logits(cfg, T, E), k)


def test_route_ties_and_spread(mg):
    """Many equal logits (ties go to the lower id), and logits far apart
    (scores that underflow bf16 to zero)."""
    g = np.random.default_rng(91)
    _check(mg, g.integers(-2, 3, size=(50, 40)).astype(np.float32), 6)
    _check(mg, np.full((4, 300), -1.5, np.float32), 8)
    _check(mg, (g.standard_normal((16, 256)) * 40).astype(np.float32), 8)


def test_prefill_layer_from_router(mg):
    """route + moe_prefill on the GPU equals moe_prefill with the host routing
    of the same logits, bit for bit."""
    sh = synth.PREFILL
    T = 331
    logits = synth.zipf_logits(3, T, sh.E, sub=4)
    x = synth.activations(3, T, sh.H, sub=4)
    ex = [triple(m) for m in synth.expert_set(3, sh.E, sh.H, sh.I, sh.gs, sh.bits, mode="words")]
    shp = tuple(triple(m) for m in synth.shared_params(3, sh.H, sh.shared_I, sh.gs, sh.bits))
    idx, sc = mg.route(torch.from_numpy(logits).cuda(), sh.top_k)
    got = mg.moe_prefill(bf(x), idx, sc, *ex, shared=shp, group_size=sh.gs, bits=sh.bits)
    hi, hs = oracle.route(logits, sh.top_k)
    want = mg.moe_prefill(bf(x), i32(hi), bf(hs), *ex, shared=shp, group_size=sh.gs, bits=sh.bits)
    assert np.array_equal(host_bf(got), host_bf(want))
