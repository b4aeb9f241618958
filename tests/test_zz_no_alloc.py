"""The allocation-free decode entry point (the intermediate in the library's
static per-GPU scratch) against the workspace entry point, bit for bit: the
same kernels on the same inputs, on two calls in a row (the second smaller),
called through the C ABI with raw device pointers."""
import ctypes

import numpy as np
import pytest
import torch

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


def _case(M, E, H, I, top_k, gs, bits, sub, mode="drawn"):
    idx = synth.sorted_topk(21, M, E, top_k, sub=sub)
    ex = synth.expert_set(21, E, H, I, gs, bits, mode=mode, experts=np.unique(idx))
    x = synth.activations(21, M, H, sub=sub)
    g = np.random.default_rng(M + H + sub)
    scores = synth.to_bf16(g.random((M, top_k)).astype(np.float32))
    shared = synth.to_bf16(g.standard_normal((M, H)).astype(np.float32))
    return bf(x), i32(idx), bf(scores), bf(shared), [triple(m) for m in ex]


def _static(mg, x, idx, scores, shared, ex, gs, bits, out):
    T, H = x.shape
    top_k = idx.shape[1]
    E, I = ex[0][0].shape[0], ex[0][0].shape[1]
    p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    return mg.lib().moegq_moe_decode_static(p(x), T, H, I, E, p(idx), top_k, p(scores), p(shared),
                                            *[p(t) for m in ex for t in m], gs, bits, p(out), None,
                                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_static_decode_matches_workspace_entry(mg):
    assert mg.static_scratch_bytes() == 8 << 20
    runs = [(4, 64, 1024, 512, 8, 64, 4, 0), (1, 64, 1024, 512, 8, 64, 4, 1)]   # the second call is smaller
    for M, E, H, I, top_k, gs, bits, sub in runs:
        x, idx, scores, shared, ex = _case(M, E, H, I, top_k, gs, bits, sub)
        want = mg.moe_decode(x, idx, scores, *ex, shared=shared, group_size=gs, bits=bits)
        out = torch.full((M, H), 7.0, dtype=torch.bfloat16, device="cuda")
        assert _static(mg, x, idx, scores, shared, ex, gs, bits, out) == 0
        torch.cuda.synchronize()
        assert np.array_equal(host_bf(out), host_bf(want)), f"M={M}"


def test_static_decode_headline_shape_and_limit(mg):
    """The decode shape (hidden 4096, inter 2048, top-8) at 16 tokens, then 1;
    and a size beyond the scratch is refused with nothing launched."""
    sh = synth.DECODE
    E = 12
    for M, sub in ((16, 3), (1, 4)):
        x, idx, scores, shared, ex = _case(M, E, sh.H, sh.I, sh.top_k, sh.gs, sh.bits, sub, mode="words")
        want = mg.moe_decode(x, idx, scores, *ex, shared=None, group_size=sh.gs, bits=sh.bits)
        got = mg.moe_decode_static(x, idx, scores, *ex, shared=None, group_size=sh.gs, bits=sh.bits)
        assert np.array_equal(host_bf(got), host_bf(want)), f"M={M}"
    # 257 tokens x 8 x 2048 x 2 bytes > 8 MiB
    idx = i32(synth.sorted_topk(21, 257, E, sh.top_k, sub=5))
    x = bf(synth.activations(21, 257, sh.H, sub=5))
    scores = torch.ones((257, sh.top_k), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((257, sh.H), dtype=torch.bfloat16, device="cuda")
    assert _static(mg, x, idx, scores, None, ex, sh.gs, sh.bits, out) == -7
    torch.cuda.synchronize()
    assert not bool(out.view(torch.int16).any())
