"""The fused-combine self-check and its fallback (MTPLX PR 558 Change and
Tests: a bitwise self-check of the one-kernel combine at 128 rows, top-8,
hidden 2048; a difference or failure turns the one-kernel route off for the
process).  A forced failure must route the whole-layer entry point through
the unfused tail, which gives the same bits, and make the standalone fused
combines refuse so that the binding runs the unfused tail."""
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


def test_selfcheck_passes(mg):
    assert mg.selfcheck() == 0
    assert mg.selfcheck_state() == 1


def test_forced_failure_takes_unfused_tail(mg, monkeypatch):
    sh = synth.PREFILL
    T = 331
    idx, scores = synth.zipf_routing(3, T, sh.E, sh.top_k, sub=4)
    x = synth.activations(3, T, sh.H, sub=4)
    ex = [triple(m) for m in synth.expert_set(3, sh.E, sh.H, sh.I, sh.gs, sh.bits, mode="words",
                                                experts=np.unique(idx))]
    shp = tuple(triple(m) for m in synth.shared_params(3, sh.H, sh.shared_I, sh.gs, sh.bits))
    nbytes = mg.moe_prefill_workspace_bytes(T, sh.top_k, sh.E, sh.H, sh.I, True)
    lay = mg.moe_prefill_layout(T, sh.top_k, sh.E, sh.H, sh.I, True)
    tail0 = lay["offsets"]["tail"]
    P = T * sh.top_k
    try:
        assert mg.selfcheck() == 0
        ws = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda")
        fused = host_bf(mg.moe_prefill(bf(x), i32(idx), bf(scores), *ex, shared=shp, group_size=sh.gs,
                                       bits=sh.bits, workspace=ws))
        tail = ws[tail0:tail0 + 2 * (P + 2 * T) * sh.H]
        assert bool((tail == 0x5A).all()), "the one-pass combine does not touch the tail scratch"
        # y and inv of the sorted route, for the standalone combines
        y, inv, _ = mg.switch_glu(bf(x), i32(idx), *ex, group_size=sh.gs, bits=sh.bits, mode=mg.MODE_SORTED)
        shared = torch.randn((T, sh.H), device="cuda").to(torch.bfloat16)
        z = torch.randn((T,), device="cuda").to(torch.bfloat16)
        c_fused = host_bf(mg.moe_combine(y, inv, bf(scores), shared))
        g_fused = host_bf(mg.moe_combine_gated(y, inv, bf(scores), shared, z))

        monkeypatch.setenv("MOEGQ_FORCE_SELFCHECK_FAIL", "1")
        assert mg.selfcheck() == mg.ERR_SELFCHECK
        assert mg.selfcheck_state() == 2
        ws.fill_(0x5A)
        fb = host_bf(mg.moe_prefill(bf(x), i32(idx), bf(scores), *ex, shared=shp, group_size=sh.gs,
                                    bits=sh.bits, workspace=ws))
        assert not bool((tail == 0x5A).all()), "the fallback writes the unfused tail's scratch"
        assert np.array_equal(fb, fused)
        out = torch.empty((T, sh.H), dtype=torch.bfloat16, device="cuda")
        st = mg.lib().moegq_moe_combine(mg._ptr(y), mg._ptr(inv), mg._ptr(bf(scores)), mg._ptr(shared), T,
                                        sh.top_k, sh.H, mg._ptr(out), mg._stream())
        assert st == mg.ERR_SELFCHECK
        assert np.array_equal(host_bf(mg.moe_combine(y, inv, bf(scores), shared)), c_fused)
        assert np.array_equal(host_bf(mg.moe_combine_gated(y, inv, bf(scores), shared, z)), g_fused)
    finally:
        monkeypatch.delenv("MOEGQ_FORCE_SELFCHECK_FAIL", raising=False)
        assert mg.selfcheck() == 0
    assert mg.selfcheck_state() == 1
