"""Benchmark of the gathered affine-quantized MoE path on one MI355X.

Headline (``value``): MoE decode at hidden 4096, inter 2048, 288 experts,
top-8, 4-bit weights with group size 64, one token: effective weight GB/s
(tokens * top_k * bytes per expert / time, duplicates counted) over a chain of
42 layers with distinct index sets, so the experts come from HBM.  One layer
is gate/up gather + SiLU (one kernel), then the down gather fused with the
combine over top_k.  A step is one pass over the 42-layer chain, captured as
one HIP graph; --steps sets how many replays are timed (each between its own
HIP events; the median is reported with the min and max), --warmup how many
untimed replays come first.

Further legs reported in the same JSON line (not ``value``): the same decode
at 4 tokens, isolated (one index set, cache-resident) and isolated with cold
caches; measured ceilings (streaming read, bf16 MFMA loop); the MoE-layer
prefill at 128-4096 rows (hidden 2048, 256 experts, inter 512, gated shared
expert, combine); the expert-aware vs naive tile schedules and the whole
layer on the large prefill (hidden 4096, 288 experts, inter 2048) at
713-16384 rows; the fused against the unfused combine; unquantized
gather_mm; the vector-unit route; the dense few-row chain (36 decoder
layers, 8 weight sets) and its sweep over rows 1-16, 4/8-bit codes and group
sizes 32/64/128; and the oracle timed on the host (cpu_baseline).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs a,b,...]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # a step is one replay of the 42-layer decode chain (about 1 ms); each of
    # the `steps` timed replays sits between its own events (median reported)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--legs", default="decode,ceilings,prefill,large,combine,gather_mm,vec,dense,fewrow,cpu")
    ap.add_argument("--prefill-rows", default="2048,128,512,4096", help="row counts of the prefill leg")
    ap.add_argument("--large-rows", default="713,4123,8192,16384", help="row counts of the large-prefill leg")
    ap.add_argument("--quiet", action="store_true")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Timer:
    """HIP events on torch's current stream (the stream the kernels run on)."""

    def __init__(self, torch):
        self.t = torch
        self.ev = []

    def mark(self, tag):
        e = self.t.cuda.Event(enable_timing=True)
        e.record()
        self.ev.append((tag, e))

    def spans(self):
        self.t.cuda.synchronize()
        out = {}
        for (tag, a), (_, b) in zip(self.ev[:-1], self.ev[1:]):
            if tag is None:
                continue
            out.setdefault(tag, []).append(a.elapsed_time(b) * 1e3)   # us
        return out


# ----------------------------------------------------------------------------- decode
class GraphStats:
    """Per-call microseconds of a captured graph over its timed replays: each
    replay is bracketed by its own HIP events on the replaying stream."""

    def __init__(self, per_replay_us, calls):
        v = np.asarray(per_replay_us, dtype=np.float64) / calls
        self.replays = len(v)
        self.median = float(np.median(v))
        self.mean = float(v.mean())
        self.min = float(v.min())
        self.max = float(v.max())

    def as_dict(self, scale=1.0, unit="us"):
        return {f"median_{unit}": round(self.median * scale, 4), f"min_{unit}": round(self.min * scale, 4),
                f"max_{unit}": round(self.max * scale, 4), "replays": self.replays}


def capture(torch, fn, n, check=None):
    """Capture fn(0..n-1) into one HIP graph and verify three replays against
    an eager run (check() -> tensor)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    if check is not None:
        for i in range(n):
            fn(i)
        ref = check().clone()
        for _ in range(3):
            check().zero_()
            g.replay()
            torch.cuda.synchronize()
            if not torch.equal(check(), ref):
                raise RuntimeError("graph replay differs from eager execution")
    return g


def time_replays(torch, g, reps, warm=2, between=None):
    """Event-timed replays of graph g: `warm` untimed replays, then `reps`
    replays each between two events (between(): optional work enqueued before
    each timed replay, outside its events).  Returns microseconds per replay."""
    for _ in range(warm):
        g.replay()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
    torch.cuda.synchronize()
    for i in range(reps):
        if between is not None:
            between()
        ev[2 * i].record()
        g.replay()
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    return [ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e3 for i in range(reps)]


def graph_stats(torch, fn, n, reps=10, check=None, warm=2):
    """Capture fn(0..n-1) as one graph and time `reps` replays; per-call stats."""
    g = capture(torch, fn, n, check)
    return GraphStats(time_replays(torch, g, reps, warm), n)


def graph_time_us(torch, fn, n, reps=10, check=None):
    """Median microseconds per call of fn over `reps` replays of a graph of n calls."""
    return graph_stats(torch, fn, n, reps, check).median


def decode_leg(torch, m, synth, M, steps, warmup, n_sets=42, isolated=False, cfg=1):
    """One MoE decode layer: gather gate/up + SiLU, then gather down fused with
    the combine (scores 1/8, no shared expert).  A step is one pass over the
    chain of n_sets layers with distinct index sets (MLX issue 4509's chained
    x42 protocol), captured as one HIP graph; `steps` replays are timed one by
    one with HIP events (median, min, max)."""
    sh = synth.DECODE
    dev = torch.device("cuda")
    gate, up, down = synth.device_expert_set(dev, cfg, sh.E, sh.H, sh.I, sh.gs, sh.bits)
    idx_sets = [torch.from_numpy(synth.sorted_topk(cfg, M, sh.E, sh.top_k, sub=i)).to(dev) for i in range(n_sets)]
    x = torch.from_numpy(synth.activations(cfg, M, sh.H).view(np.int16)).view(torch.bfloat16).to(dev)
    scores = torch.full((M, sh.top_k), 0.125, dtype=torch.bfloat16, device=dev)
    P = M * sh.top_k
    h = torch.empty((P, sh.I), dtype=torch.bfloat16, device=dev)
    out = torch.empty((M, sh.H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(m.workspace_bytes(m.OP_MOE_DECODE, P, sh.E, sh.I), dtype=torch.uint8, device=dev)

    def idx_of(i):
        return idx_sets[0 if isolated else i % n_sets]

    def layer(i):
        m.moe_decode(x, idx_of(i), scores, gate, up, down, group_size=sh.gs, bits=sh.bits, out=out, workspace=ws)

    def k1(i):
        m.gather_qmm_glu(x, gate, up, idx_of(i).view(-1), lhs_div=sh.top_k, group_size=sh.gs, bits=sh.bits, out=h)

    for i in range(n_sets):
        layer(i)
    torch.cuda.synchronize()
    # the page's own protocol: host-timed eager calls, one synchronize at the end
    t0 = time.perf_counter()
    for i in range(steps * n_sets):
        layer(i)
    torch.cuda.synchronize()
    el_eager = (time.perf_counter() - t0) / (steps * n_sets)
    chain = GraphStats(time_replays(torch, capture(torch, layer, n_sets, check=lambda: out), steps, warmup),
                       n_sets)
    kst = GraphStats(time_replays(torch, capture(torch, k1, n_sets, check=lambda: h), steps, warmup), n_sets)
    bpe = 3 * (sh.I * sh.H * sh.bits // 8 + 2 * sh.I * (sh.H // sh.gs) * 2)
    eff = M * sh.top_k * bpe
    k1_bytes = P * 2 * sh.I * (sh.H * sh.bits // 8 + 2 * (sh.H // sh.gs) * 2) + M * sh.H * 2 + P * sh.I * 2
    res = {
        "tokens": M, "isolated": isolated, "layers_per_step": n_sets,
        "timing": f"hip graph of the {n_sets}-layer chain, {chain.replays} replays, each between its own events",
        "ms_per_step": chain.median * n_sets * 1e-3,
        "us_per_layer": chain.as_dict(),
        "effective_gbs": eff / (chain.median * 1e-6) / 1e9,
        "effective_gbs_range": [eff / (chain.max * 1e-6) / 1e9, eff / (chain.min * 1e-6) / 1e9],
        "eager_us_per_layer": el_eager * 1e6, "eager_effective_gbs": eff / el_eager / 1e9,
        "gate_up_us": kst.as_dict(), "down_combine_us_approx": chain.median - kst.median,
        "gate_up_bytes": k1_bytes, "gate_up_gbs": k1_bytes / (kst.median * 1e-6) / 1e9, "bytes_per_expert": bpe,
        "_layer_us": chain.median, "_k1_us": kst.median,
    }
    del gate, up, down
    torch.cuda.empty_cache()
    return res


def decode_cold_leg(torch, m, synth, reps=20, M=1, cfg=1, flush_bytes=1 << 30):
    """One isolated decode layer with cold caches: before each timed layer a
    streaming read of a 1 GiB buffer (four times the 256 MB memory-side cache)
    evicts its weights; the layer (one HIP graph) is timed between its own
    events, the flush outside them."""
    sh = synth.DECODE
    dev = torch.device("cuda")
    gate, up, down = synth.device_expert_set(dev, cfg, sh.E, sh.H, sh.I, sh.gs, sh.bits)
    idx = torch.from_numpy(synth.sorted_topk(cfg, M, sh.E, sh.top_k, sub=0)).to(dev)
    x = torch.from_numpy(synth.activations(cfg, M, sh.H).view(np.int16)).view(torch.bfloat16).to(dev)
    scores = torch.full((M, sh.top_k), 0.125, dtype=torch.bfloat16, device=dev)
    P = M * sh.top_k
    out = torch.empty((M, sh.H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(m.workspace_bytes(m.OP_MOE_DECODE, P, sh.E, sh.I), dtype=torch.uint8, device=dev)
    flush = torch.empty(flush_bytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    layer = lambda i=0: m.moe_decode(x, idx, scores, gate, up, down, group_size=sh.gs, bits=sh.bits, out=out,
                                     workspace=ws)
    g = capture(torch, layer, 1, check=lambda: out)
    us = time_replays(torch, g, reps, warm=1, between=lambda: m.probe_stream_read(flush, 2048, sink))
    st = GraphStats(us, 1)
    bpe = 3 * (sh.I * sh.H * sh.bits // 8 + 2 * sh.I * (sh.H // sh.gs) * 2)
    eff = M * sh.top_k * bpe
    del gate, up, down, flush
    torch.cuda.empty_cache()
    return {"tokens": M, "us_per_layer": st.as_dict(), "effective_gbs": eff / (st.median * 1e-6) / 1e9,
            "timing": "one layer per replay after a 1 GiB streaming read outside the events"}


def ceilings_leg(torch, m, reps=10):
    """Measured ceilings: a plain streaming read of 2 GiB (128-bit loads, 4, 8
    and 16 workgroups of 256 threads per compute unit), the same read at the
    byte counts of single products, and a plain bf16 MFMA loop (8 independent
    v_mfma_f32_16x16x32_bf16 chains per wave, 1 and 2 workgroups of 4 waves
    per compute unit)."""
    dev = torch.device("cuda")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    res = {"compute_units": cus}
    for per_cu in (4, 8, 16):
        st = graph_stats(torch, lambda i: m.probe_stream_read(buf, per_cu * cus, sink), 1, reps=reps)
        res[f"stream_read_{per_cu}wg_per_cu"] = {"us": st.as_dict(), "tb_s": nbytes / (st.median * 1e-6) / 1e12}
    # the same read at the byte counts of single products, one launch per
    # product-sized slice of the 2 GiB buffer in one graph (the slices cycle
    # through 8x the 256 MB memory-side cache, so each launch reads HBM), with
    # one 4-load pass per thread or 8 grid-stride workgroups per compute unit
    sizes = {"dense_o_2560x4096": 5898240, "dense_qkv_6144x2560": 8847360, "dense_down_2560x9728": 14008320,
             "dense_gate_up_2x9728x2560": 28016640, "decode_down_8x4096x2048": 37748736,
             "decode_gate_up_16x2048x4096": 75497472}
    by_size = {}
    for name, size in sizes.items():
        stride = (size + 4095) // 4096 * 4096
        n = min(64, nbytes // stride)
        one_pass = -(-size // (16 * 4 * 256))
        row = {"bytes": size, "launches_per_graph": n}
        for label, blocks in (("one_pass", one_pass), ("8wg_per_cu", 8 * cus)):
            st = graph_stats(torch, lambda i: m.probe_stream_read(buf[i * stride:i * stride + size], blocks, sink), n,
                             reps=reps)
            row[label] = {"blocks": blocks, "us": st.as_dict(), "tb_s": size / (st.median * 1e-6) / 1e12}
        by_size[name] = row
    res["stream_read_by_size"] = by_size
    del buf
    out = torch.zeros(1, dtype=torch.float32, device=dev)
    iters = 4096
    for per_cu in (1, 2):
        flops = m.probe_mfma_bf16(iters, per_cu * cus, out)
        st = graph_stats(torch, lambda i: m.probe_mfma_bf16(iters, per_cu * cus, out), 1, reps=reps)
        res[f"mfma_bf16_{per_cu}wg_per_cu"] = {"us": st.as_dict(), "tflops": flops / (st.median * 1e-6) / 1e12,
                                              "frac_of_2500": flops / (st.median * 1e-6) / 2.5e15}
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- prefill
def layer_bytes_flops(sh, T, counts, shared):
    """Algorithmic flops and bytes of one MoE prefill layer (weights of the
    active experts once, activations once per materialized tensor)."""
    P = T * sh.top_k
    active = int((counts > 0).sum())
    H, I = sh.H, sh.I
    SI = sh.shared_I if shared else 0
    flops = P * 6 * H * I + (T * 6 * H * SI + T * 2 * H if shared else 0)
    B = lambda n, k: n * (k * sh.bits // 8 + 2 * (k // sh.gs) * 2)
    wbytes = active * (2 * B(I, H) + B(H, I)) + ((2 * B(SI, H) + B(H, SI) + B(1, H)) if shared else 0)
    act = (T * H * 2 + P * I * 2 * 2 + P * H * 2          # x, h_sorted write+read, y_sorted write
           + (T * SI * 2 * 2 + T * H * 2 if shared else 0)   # shared h write+read, shared y write
           + P * H * 2 + (T * H * 2 if shared else 0) + T * H * 2)   # combine: y, shared, out
    return flops, wbytes + act


def prefill_leg(torch, m, synth, rows=(2048, 128, 512, 4096), steps=100, warmup=5, cfg=3):
    """The MoE layer of hidden 2048, 256 experts, top-8, inter 512, 4-bit GS 64
    with a gated shared expert: one moe_prefill call per step (sort, routed +
    shared experts, gated combine), timed as HIP-graph replays of 10 layers."""
    sh = synth.PREFILL
    dev = torch.device("cuda")
    gate, up, down = synth.device_expert_set(dev, cfg, sh.E, sh.H, sh.I, sh.gs, sh.bits)
    sg, su, sd = synth.device_expert_set(dev, cfg + 100, 1, sh.H, sh.shared_I, sh.gs, sh.bits)
    sg, su, sd = [tuple(t[0] for t in trip) for trip in (sg, su, sd)]
    grow = tuple(t[0] for t in synth.device_drawn_words(dev, (cfg, 3, 3), (1, 1), sh.H, sh.gs, sh.bits))
    res = {}
    for T in rows:
        idx_np, scores_np = synth.zipf_routing(cfg, T, sh.E, sh.top_k)
        idx = torch.from_numpy(idx_np).to(dev)
        scores = torch.from_numpy(scores_np.view(np.int16)).view(torch.bfloat16).to(dev)
        x = torch.from_numpy(synth.activations(cfg, T, sh.H).view(np.int16)).view(torch.bfloat16).to(dev)
        out = torch.empty((T, sh.H), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(m.moe_prefill_workspace_bytes(T, sh.top_k, sh.E, sh.H, sh.I, True), dtype=torch.uint8,
                         device=dev)
        counts = np.bincount(idx_np.reshape(-1), minlength=sh.E)

        def step(i=0):
            m.moe_prefill(x, idx, scores, gate, up, down, shared=(sg, su, sd, grow), group_size=sh.gs,
                          bits=sh.bits, out=out, workspace=ws)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        el_eager = (time.perf_counter() - t0) / steps
        lst = graph_stats(torch, step, 10, reps=max(10, steps // 10), check=lambda: out)
        el = lst.median * 1e-6
        # the router on the GPU (fp32 logits of the same routing), alone and in front of the layer
        logits = torch.from_numpy(synth.zipf_logits(cfg, T, sh.E)).to(dev)
        ridx = torch.empty((T, sh.top_k), dtype=torch.int32, device=dev)
        rsc = torch.empty((T, sh.top_k), dtype=torch.bfloat16, device=dev)
        route = lambda i=0: m.route(logits, sh.top_k, idx=ridx, scores=rsc)
        route_us = graph_time_us(torch, route, 10, reps=max(10, steps // 10), check=lambda: ridx)

        def step_logits(i=0):
            route()
            m.moe_prefill(x, ridx, rsc, gate, up, down, shared=(sg, su, sd, grow), group_size=sh.gs,
                          bits=sh.bits, out=out, workspace=ws)

        el_logits = graph_time_us(torch, step_logits, 10, reps=max(10, steps // 10), check=lambda: out) * 1e-6
        flops, nbytes = layer_bytes_flops(sh, T, counts, True)
        r = {"rows": T, "active_experts": int((counts > 0).sum()), "max_load": int(counts.max()),
             "ms_per_layer": el * 1e3, "ms_per_layer_stats": lst.as_dict(1e-3, "ms"),
             "eager_ms_per_layer": el_eager * 1e3, "timing": "hip graph of 10 layers, replays timed one by one",
             "router_us": route_us, "ms_per_layer_from_logits": el_logits * 1e3,
             "gflop": flops / 1e9, "bytes": nbytes,
             "mfma_util": flops / el / (MFMA_BF16_PEAK_TFLOPS * 1e12),
             "hbm_frac": nbytes / el / (HBM_PEAK_GBS * 1e9)}
        r["roofline_frac"] = max(r["mfma_util"], r["hbm_frac"])
        res[f"rows{T}"] = r
        del ws
    del gate, up, down
    torch.cuda.empty_cache()
    return res


def hybrid_tile_count(counts, inter, small_max=32, big=128, slots=512):
    """Tiles of the library's hybrid schedule for these per-expert counts (a
    host-side restatement for the report): 128-row tiles for experts with at
    least 32 rows and 32-row tiles for the others, or 32-row tiles for every
    expert when the 128-row tiles would give the gate/up pass at most
    slots / 8 work items."""
    nbig = sum(-(-int(c) // big) for c in counts if c >= small_max)
    if nbig * -(-inter // 128) <= slots // 8:
        return int(sum(-(-int(c) // small_max) for c in counts if c > 0))
    return int(nbig + sum(1 for c in counts if 0 < c < small_max))


def tile_counts(counts, bm, mode, inter):
    """(tiles, K passes) of one pass of the sorted route for per-expert loads
    `counts` (host arithmetic for the report): expert-aware tiles of bm rows,
    naive fixed bm-row tiles (one K pass per expert present in a tile), or the
    two-size schedule (bm 0)."""
    if mode == "naive":
        offs = np.concatenate([[0], np.cumsum(counts)])
        P = int(offs[-1])
        passes = 0
        for r0 in range(0, P, bm):
            r1 = min(P, r0 + bm)
            passes += int(((offs[1:] > r0) & (offs[:-1] < r1) & (counts > 0)).sum())
        return -(-P // bm), passes
    if bm == 0:
        n = hybrid_tile_count(counts, inter)
        return n, n
    n = int(sum(-(-int(c) // bm) for c in counts))
    return n, n


def large_leg(torch, m, synth, rows=(713, 4123, 8192, 16384), reps=10, cfg=4):
    """Large MoE prefill (hidden 4096, 288 experts, top-8, inter 2048): at each
    size the sorted SwitchGLU under the expert-aware schedule against naive
    row tiling, both at BM 16 (MLX PR 4567's comparison: tile and K-pass
    counts, ms), the expert-aware schedule at BM 64 and the two-size schedule
    the library runs; and the whole layer (moe_prefill, no shared expert),
    4-bit GS 64 and, at 4123 rows, 8-bit GS 128.  HIP-graph replays."""
    res = {}
    for bits in (4, 8):
        sh = synth.LARGE4 if bits == 4 else synth.LARGE8
        dev = torch.device("cuda")
        gate, up, down = synth.device_expert_set(dev, cfg, sh.E, sh.H, sh.I, sh.gs, sh.bits)
        for T in (rows if bits == 4 else (4123,)):
            idx_np, scores_np = synth.zipf_routing(cfg, T, sh.E, sh.top_k)
            idx = torch.from_numpy(idx_np).to(dev)
            scores = torch.from_numpy(scores_np.view(np.int16)).view(torch.bfloat16).to(dev)
            x = torch.from_numpy(synth.activations(cfg, T, sh.H).view(np.int16)).view(torch.bfloat16).to(dev)
            P = T * sh.top_k
            counts = np.bincount(idx_np.reshape(-1), minlength=sh.E)
            r = {"rows": T, "bits": bits, "active_experts": int((counts > 0).sum()), "max_load": int(counts.max()),
                 "experts_under_16_rows": int(((counts > 0) & (counts < 16)).sum())}
            flops = P * 6 * sh.H * sh.I
            if bits == 4:
                y = torch.empty((P, sh.H), dtype=torch.bfloat16, device=dev)
                inv = torch.empty(P, dtype=torch.int32, device=dev)
                for name, tmode, bm in (("scheduled_bm16", 0, 16), ("naive_bm16", 1, 16), ("scheduled_bm64", 0, 64),
                                        ("two_size", 0, 0)):
                    run = lambda i=0: m.switch_glu(x, idx, gate, up, down, group_size=sh.gs, bits=sh.bits,
                                                   mode=m.MODE_SORTED, tile_mode=tmode, bm=bm, y=y, inv=inv)
                    st = graph_stats(torch, run, 1, reps=reps if T <= 4123 else max(3, reps // 3), check=lambda: y)
                    tiles, passes = tile_counts(counts, bm, "naive" if tmode else "scheduled", sh.I)
                    r[name] = {"ms": st.median * 1e-3, "ms_stats": st.as_dict(1e-3, "ms"), "tiles": tiles,
                               "k_passes": passes,
                               "mfma_util": flops / (st.median * 1e-6) / (MFMA_BF16_PEAK_TFLOPS * 1e12)}
                del y, inv
            out = torch.empty((T, sh.H), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(m.moe_prefill_workspace_bytes(T, sh.top_k, sh.E, sh.H, sh.I, False),
                             dtype=torch.uint8, device=dev)
            layer = lambda i=0: m.moe_prefill(x, idx, scores, gate, up, down, shared=None, group_size=sh.gs,
                                              bits=sh.bits, out=out, workspace=ws)
            st = graph_stats(torch, layer, 3, reps=reps, check=lambda: out)
            el = st.median * 1e-6
            flops_l, nbytes = layer_bytes_flops(sh, T, counts, False)
            r["layer"] = {"ms": el * 1e3, "ms_stats": st.as_dict(1e-3, "ms"), "timing": "hip graph of 3 layers",
                          "gflop": flops_l / 1e9, "bytes": nbytes,
                          "mfma_util": flops_l / el / (MFMA_BF16_PEAK_TFLOPS * 1e12),
                          "hbm_frac": nbytes / el / (HBM_PEAK_GBS * 1e9)}
            res[f"rows{T}_bits{bits}"] = r
            del ws, out
        del gate, up, down
        torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- unquantized gather_mm
def gather_mm_leg(torch, m, synth, steps=20):
    """Unquantized bf16 gather_mm on the expert-sorted route (the operation
    the expert-aware schedule was designed for): 2048 tokens, top-8 of 256
    experts, N 512, K 2048 (the prefill shape's gate projection), pairs sorted
    by expert, 64-row scheduled tiles on the matrix cores; and one decode token
    (8 pairs, N 2048, K 4096) on the one-row path.  HIP-graph replays."""
    dev = torch.device("cuda")
    res = {}
    T, E, N, K, top_k = 2048, 256, 512, 2048, 8
    g = synth.device_generator(dev, 6, 0)
    w = (torch.randn((E, N, K), device=dev, generator=g) * 0.02).to(torch.bfloat16)
    idx_np, _ = synth.zipf_routing(3, T, E, top_k)
    flat = idx_np.reshape(-1)
    order = np.argsort(flat, kind="stable")
    srhs = torch.from_numpy(flat[order].astype(np.int32)).to(dev)
    lhs = torch.from_numpy((order // top_k).astype(np.int32)).to(dev)
    x = torch.randn((T, K), device=dev, generator=g).to(torch.bfloat16)
    P = T * top_k
    out = torch.empty((P, N), dtype=torch.bfloat16, device=dev)
    fn = lambda i=0: m.gather_mm(x, w, srhs, lhs_indices=lhs, sorted_indices=True, out=out)
    us = graph_time_us(torch, fn, 10, reps=10, check=lambda: out)
    active = int(np.unique(flat).size)
    flops = 2.0 * P * N * K
    nbytes = active * N * K * 2 + T * K * 2 + P * N * 2
    res["sorted_2048x8_e256_n512_k2048"] = {
        "us": us, "tflops": flops / us / 1e6, "mfma_util": flops / (us * 1e-6) / (MFMA_BF16_PEAK_TFLOPS * 1e12),
        "hbm_frac": nbytes / (us * 1e-6) / (HBM_PEAK_GBS * 1e9), "active_experts": active, "pairs": P}
    del w
    # one decode token: 8 pairs over [288, 2048, 4096] bf16 experts
    E2, N2, K2 = 288, 2048, 4096
    w2 = (torch.randn((E2, N2, K2), device=dev, generator=g) * 0.02).to(torch.bfloat16)
    sets = [torch.from_numpy(synth.sorted_topk(1, 1, E2, 8, sub=i).reshape(-1)).to(dev) for i in range(42)]
    x2 = torch.randn((1, K2), device=dev, generator=g).to(torch.bfloat16)
    out2 = torch.empty((8, N2), dtype=torch.bfloat16, device=dev)
    fn2 = lambda i=0: m.gather_mm(x2, w2, sets[i % 42], lhs_div=8, out=out2)
    us2 = graph_time_us(torch, fn2, 42, reps=10, check=lambda: out2)
    b2 = 8 * N2 * K2 * 2
    res["decode_1tok_8pairs_n2048_k4096"] = {"us": us2, "gbs": b2 / us2 / 1e3,
                                             "hbm_frac": b2 / (us2 * 1e-6) / (HBM_PEAK_GBS * 1e9)}
    del w2
    torch.cuda.empty_cache()
    return res


def vec_leg(torch, m, synth, steps=42, cfg=1):
    """The vector-unit route of gather_qmm at the decode shape (one token,
    8 of 288 experts, 4-bit, group 64): the gate projection stored without
    the transpose ([288, 4096, 2048/8] words, groups along N) with bf16
    activations, and the transposed gate projection with float32 activations
    (float32 result), the transposed gate projection at 3 bits (codes
    straddle words), and in the mxfp8 and mxfp4 modes.  42 index sets chained in one HIP graph, as the decode
    leg does, so that weights come from HBM."""
    sh = synth.DECODE
    dev = torch.device("cuda")
    gate = synth.device_drawn_words(dev, (cfg, 0, synth.GATE), (sh.E, sh.I), sh.H, sh.gs, sh.bits)
    E, H, I = sh.E, sh.H, sh.I
    sets = [torch.from_numpy(synth.sorted_topk(cfg, 1, E, sh.top_k, sub=i).reshape(-1)).to(dev) for i in range(42)]
    P = sh.top_k
    res = {}
    # without the transpose: the same bytes read as [E, K = H, N = I] with groups along N
    w_nt = gate[0].view(E, H, I * sh.bits // 32)
    s_nt = gate[1].view(E, H, I // sh.gs)
    b_nt = gate[2].view(E, H, I // sh.gs)
    gate3 = synth.device_drawn_words(dev, (cfg, 0, synth.GATE, 3), (sh.E, sh.I), sh.H, sh.gs, 3)
    for name, x, w, s, b, tr, N, bits in (
            ("no_transpose_bf16_1tok_8pairs_k4096_n2048",
             torch.randn((1, 1, H), device=dev).to(torch.bfloat16), w_nt, s_nt, b_nt, False, I, sh.bits),
            ("transpose_f32_act_1tok_8pairs_n2048_k4096",
             torch.randn((1, 1, H), device=dev, dtype=torch.float32), *gate, True, I, sh.bits),
            ("transpose_bf16_3bit_1tok_8pairs_n2048_k4096",
             torch.randn((1, 1, H), device=dev).to(torch.bfloat16), *gate3, True, I, 3)):
        per_pair = I * H * bits // 8 + 2 * I * (H // sh.gs) * 2
        odt = torch.bfloat16 if x.dtype == torch.bfloat16 else torch.float32
        out = torch.empty((P, 1, N), dtype=odt, device=dev)
        need = m.gather_qmm_workspace_bytes(P, E, 1, N, H, m._dt(x), tr, bits, False)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        fn = lambda i, x=x, w=w, s=s, b=b, tr=tr, out=out, ws=ws, bits=bits: m.gather_qmm(
            x, w, s, b, rhs_indices=sets[i % 42], transpose=tr, group_size=sh.gs, bits=bits, out=out,
            workspace=ws)
        us = graph_time_us(torch, fn, 42, reps=10, check=lambda out=out: out)
        nbytes = P * per_pair + H * x.element_size() + P * N * out.element_size()
        plan_ks = need // (P * N * 4)
        res[name] = {"us": us, "gbs": nbytes / us / 1e3, "hbm_frac": nbytes / (us * 1e-6) / (HBM_PEAK_GBS * 1e9),
                     "bytes": nbytes, "k_splits": int(plan_ks) if plan_ks else 1}
    del gate, gate3
    # mx modes, transposed gate projection, bf16 activations: E8M0 scale bytes
    # around 2^0; E4M3 bytes with bit 3 cleared (no NaN pattern)
    g = synth.device_generator(dev, cfg, 7)
    x = torch.randn((1, 1, H), device=dev).to(torch.bfloat16)
    for mode, bits in (("mxfp8", 8), ("mxfp4", 4)):
        w = torch.randint(-(1 << 31), (1 << 31) - 1, (E, I, H * bits // 32), dtype=torch.int32, device=dev,
                          generator=g)
        if bits == 8:
            w &= 0xF7F7F7F7 - (1 << 32)
        sc = torch.randint(118, 136, (E, I, H // 32), dtype=torch.uint8, device=dev, generator=g)
        out = torch.empty((P, 1, I), dtype=torch.bfloat16, device=dev)
        need = int(m.lib().moegq_gather_qmm_mx_workspace_bytes(P, 1, I, H, 1, m.MX_MODES[mode][0]))
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        fn = lambda i, w=w, sc=sc, out=out, ws=ws, mode=mode: m.gather_qmm_mx(
            x, w, sc, rhs_indices=sets[i % 42], transpose=True, mode=mode, out=out, workspace=ws)
        us = graph_time_us(torch, fn, 42, reps=10, check=lambda out=out: out)
        nbytes = P * (I * H * bits // 8 + I * (H // 32)) + H * 2 + P * I * 2
        res[f"{mode}_transpose_bf16_1tok_8pairs_n2048_k4096"] = {
            "us": us, "gbs": nbytes / us / 1e3, "hbm_frac": nbytes / (us * 1e-6) / (HBM_PEAK_GBS * 1e9),
            "bytes": nbytes, "k_splits": need // (P * I * 4) if need else 1}
        del w, sc
    torch.cuda.empty_cache()
    return res


def combine_leg(torch, m, synth, reps=20, cfg=3):
    """The layer's tail at the 2048-row prefill shape (top-8, hidden 2048,
    shared expert): the fused combine (one pass) against the unfused tail
    (unsort, x score, sum over top_k, + shared: four kernels, each writing a
    bf16 tensor), HIP-graph replays of 10 calls each.  The two outputs are
    checked bit for bit."""
    dev = torch.device("cuda")
    T, top_k, H = 2048, 8, 2048
    P = T * top_k
    g = synth.device_generator(dev, cfg, 8)
    y = torch.randn((P, H), device=dev, generator=g).to(torch.bfloat16)
    inv = torch.randperm(P, device=dev, generator=g).to(torch.int32)
    scores = torch.rand((T, top_k), device=dev, generator=g).to(torch.bfloat16)
    shared = torch.randn((T, H), device=dev, generator=g).to(torch.bfloat16)
    out_f = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    out_u = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(m.workspace_bytes(m.OP_COMBINE_UNFUSED, P, 0, H, 0), dtype=torch.uint8, device=dev)
    fused = lambda i: m.moe_combine(y, inv, scores, shared, out=out_f)
    unfused = lambda i: m.moe_combine_unfused(y, inv, scores, shared, out=out_u, workspace=ws)
    us_f = graph_time_us(torch, fused, 10, reps=max(10, reps // 10), check=lambda: out_f)
    us_u = graph_time_us(torch, unfused, 10, reps=max(10, reps // 10), check=lambda: out_u)
    torch.cuda.synchronize()
    if not torch.equal(out_f.view(torch.int16), out_u.view(torch.int16)):
        raise RuntimeError("fused combine differs from the unfused tail")
    # bytes each form moves: fused reads y, inv, scores, shared and writes out;
    # unfused writes and re-reads [T, top_k, H] twice, then [T, H]
    b_f = P * H * 2 + P * 4 + P * 2 + T * H * 2 + T * H * 2
    b_u = (P * H * 2 + P * 4 + P * H * 2) + (P * H * 2 + P * 2 + P * H * 2) + (P * H * 2 + T * H * 2) \
        + (T * H * 2 * 3)
    return {"rows": T, "top_k": top_k, "hidden": H,
            "fused_us": us_f, "fused_bytes": b_f, "fused_hbm_frac": b_f / (us_f * 1e-6) / (HBM_PEAK_GBS * 1e9),
            "unfused_us": us_u, "unfused_bytes": b_u,
            "unfused_hbm_frac": b_u / (us_u * 1e-6) / (HBM_PEAK_GBS * 1e9),
            "speedup": us_u / us_f, "bitwise_equal": True}


# ----------------------------------------------------------------------------- dense chain
def dense_leg(torch, m, synth, rows=(1, 4, 16), bits=4, gs=64, reps=10, warmup=2, cfg=2, eager=True):
    dev = torch.device("cuda")
    d = synth.DENSE
    sets = synth.device_dense_sets(dev, cfg, gs, bits, d)
    # q, k and v read the same normalized rows: their weights are stacked into
    # one [q_out + 2 kv_out, hidden] matrix (the same bytes) and run as one product
    nq, nk = d["q_out"], d["kv_out"]
    for L in sets:
        L["qkv"] = tuple(torch.cat([L["q"][i], L["k"][i], L["v"][i]], 0).contiguous() for i in range(3))
        del L["q"], L["k"], L["v"]
    torch.cuda.empty_cache()
    nw = torch.ones(d["hidden"], dtype=torch.bfloat16, device=dev)
    hid, nqkv, qo, inter = d["hidden"], nq + 2 * nk, d["q_out"], d["inter"]
    per_fwd = 0
    for name, (N, K) in synth.dense_dims(d).items():
        per_fwd += N * (K * bits // 8 + 2 * (K // gs) * 2)
    per_fwd *= d["layers"]
    res = {"bits": bits, "group_size": gs, "forward_weight_bytes": per_fwd}
    # one zero-filled K-split workspace per product shape (its layout follows N, K)
    ws = {k: m.affine_qmm_workspace(max(rows), n_, k_, glu, device=dev)
          for k, (n_, k_, glu) in {"qkv": (nqkv, hid, False), "o": (hid, qo, False),
                                   "gu": (inter, hid, True), "dn": (hid, inter, False)}.items()}
    for M in rows:
        h0 = torch.randn((M, d["hidden"]), device=dev).to(torch.bfloat16)
        # the last layer writes into a fixed buffer, so that graph replays can
        # be checked against an eager forward
        h_out = torch.empty((M, d["hidden"]), dtype=torch.bfloat16, device=dev)

        def fwd():
            h = h0.clone()
            for li in range(d["layers"]):
                L = sets[li % d["sets"]]
                x = m.rms_norm(h, nw)
                qkv = m.affine_qmm(x, *L["qkv"], group_size=gs, bits=bits, workspace=ws["qkv"])
                h = m.affine_qmm(m.kv_feed_stacked(qkv, nq, nk, nk), *L["o"], group_size=gs, bits=bits, residual=h,
                                 workspace=ws["o"])
                x = m.rms_norm(h, nw)
                a = m.affine_qmm_glu(x, L["g"], L["u"], group_size=gs, bits=bits, workspace=ws["gu"])
                h = m.affine_qmm(a, *L["dn"], group_size=gs, bits=bits, residual=h, workspace=ws["dn"],
                                 out=h_out if li == d["layers"] - 1 else None)
            return h

        for _ in range(warmup):
            fwd()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps if eager else 0):
            t0 = time.perf_counter()
            fwd()
            torch.cuda.synchronize()
            ts.append(time.perf_counter() - t0)
        # the same forward captured once as a HIP graph: kernel time without the
        # per-call host work of ~300 launches from Python
        fst = graph_stats(torch, lambda i: fwd(), 1, reps=reps, check=lambda: h_out)
        g_s = fst.median * 1e-6
        res[f"rows{M}"] = {"ms_per_forward": g_s * 1e3, "ms_stats": fst.as_dict(1e-3, "ms"), "gbs": per_fwd / g_s / 1e9,
                           "hbm_frac": per_fwd / g_s / (HBM_PEAK_GBS * 1e9), "timing": "hip graph of one forward"}
        if eager:
            med = float(np.median(ts))
            res[f"rows{M}"].update({"eager_ms_per_forward": med * 1e3, "eager_gbs": per_fwd / med / 1e9})
    del sets
    torch.cuda.empty_cache()
    return res


def fewrow_sweep_leg(torch, m, synth, rows=(1, 2, 3, 4, 6, 8, 12, 16), reps=5):
    """The dense 36-layer chain (MLX #4787's few-row regime) at every row count
    1..16 of the sweep, for 4- and 8-bit codes and group sizes 32, 64, 128:
    ms per forward (HIP graph, median of `reps` replays) and the fraction of
    HBM peak that the forward's weight bytes would take."""
    out = {}
    for bits in (4, 8):
        for gs in (32, 64, 128):
            r = dense_leg(torch, m, synth, rows=rows, bits=bits, gs=gs, reps=reps, warmup=1, eager=False)
            out[f"w{bits}g{gs}"] = {"forward_weight_bytes": r["forward_weight_bytes"],
                                    "ms_per_forward": {M: round(r[f"rows{M}"]["ms_per_forward"], 4) for M in rows},
                                    "hbm_frac": {M: round(r[f"rows{M}"]["hbm_frac"], 4) for M in rows}}
    return out


# ----------------------------------------------------------------------------- counter calibration
CALIB_BYTES = 256 << 20


def calib_leg(torch, reps=3):
    """A plain device copy of CALIB_BYTES (fp32 tensors): its FETCH_SIZE and
    WRITE_SIZE counter readings against the known bytes give the scale that
    turns those counters into HBM bytes."""
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_bytes": CALIB_BYTES, "reps": reps}


# counter-derived HBM traffic of the headline kernel, measured on the source
# files listed in the summary; reported only while those files are unchanged
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "qmv_glu_decode_m1_chain42_traffic.txt")


def source_digest(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counted_traffic():
    """Bytes per launch from the committed counter summary, or None when it is
    missing or the kernel's sources changed since it was taken."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    kv = {}
    for line in open(TRAFFIC_SUMMARY):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    try:
        files = kv["sources"].split()
        if source_digest(files) != kv["sources_sha256"]:
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError, OSError):
        return None


# ----------------------------------------------------------------------------- CPU baseline
def cpu_baseline(torch, synth, n_layers=5, cfg=1):
    """The oracle (numpy) on a bounded sample of the headline workload: n_layers
    MoE decode layers at one token, dequantizing only the selected experts,
    on the same device-drawn weights (copied back for the selected experts)."""
    import oracle
    sh = synth.DECODE
    dev = torch.device("cuda")
    gate, up, down = synth.device_expert_set(dev, cfg, sh.E, sh.H, sh.I, sh.gs, sh.bits)
    x = synth.activations(cfg, 1, sh.H)
    tot = 0.0
    host = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16) if t.dtype == torch.bfloat16 \
        else t.contiguous().cpu().numpy().view(np.uint32)
    for i in range(n_layers):
        idx = synth.sorted_topk(cfg, 1, sh.E, sh.top_k, sub=i)
        sel = np.unique(idx)
        pos = {int(e): j for j, e in enumerate(sel)}
        rid = np.vectorize(lambda e: pos[int(e)])(idx)
        sub = [tuple(host(t[torch.from_numpy(sel).to(dev)]) for t in trip) for trip in (gate, up, down)]
        t0 = time.perf_counter()
        oracle.switch_glu(x, rid, *sub, gs=sh.gs, bits=sh.bits)
        tot += time.perf_counter() - t0
    bpe = 3 * (sh.I * sh.H * sh.bits // 8 + 2 * sh.I * (sh.H // sh.gs) * 2)
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas_threads = None
    del gate, up, down
    torch.cuda.empty_cache()
    return {"value": n_layers * sh.top_k * bpe / tot / 1e9, "unit": "GB/s", "cores": os.cpu_count(),
            "blas_threads": blas_threads, "kind": "oracle",
            "sample": f"{n_layers} MoE decode layers (1 token, top-8 of 288 experts, hidden 4096, inter 2048, "
                      f"4-bit GS 64), {tot:.1f} s of CPU time", "seconds": tot}


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus N > 1 is not supported "
                                   "(the library has no multi-GPU path)"}))
        sys.exit(2)
    import torch
    import moe_expert_gathered_amd as m
    import synth
    m.lib()
    legs = set(a.legs.split(","))
    torch.cuda.set_device(0)
    log(f"decode M=1 chained: {a.steps} timed replays of the 42-layer chain")
    head = decode_leg(torch, m, synth, 1, a.steps, a.warmup)
    extra = {"decode_m1_chained": head}
    if "decode" in legs:
        log("decode M=1 isolated, M=1 isolated cold, M=4 chained")
        reps = max(a.steps, 10)
        extra["decode_m1_isolated"] = decode_leg(torch, m, synth, 1, reps, a.warmup, isolated=True)
        extra["decode_m1_isolated_cold"] = decode_cold_leg(torch, m, synth, reps=max(reps, 20))
        extra["decode_m4_chained"] = decode_leg(torch, m, synth, 4, reps, a.warmup)
    if "ceilings" in legs:
        log("measured ceilings")
        extra["ceilings"] = ceilings_leg(torch, m)
    if "prefill" in legs:
        rows = tuple(int(v) for v in a.prefill_rows.split(","))
        log(f"prefill rows {rows}")
        extra["prefill"] = prefill_leg(torch, m, synth, rows=rows)
    if "large" in legs:
        rows = tuple(int(v) for v in a.large_rows.split(","))
        log(f"large prefill rows {rows}")
        extra["large_prefill"] = large_leg(torch, m, synth, rows=rows)
    if "gather_mm" in legs:
        log("unquantized gather_mm")
        extra["gather_mm"] = gather_mm_leg(torch, m, synth)
    if "combine" in legs:
        log("== combine leg")
        extra["combine"] = combine_leg(torch, m, synth)
    if "vec" in legs:
        log("== vec leg")
        extra["vec"] = vec_leg(torch, m, synth)
    if "dense" in legs:
        log("dense chain")
        extra["dense_chain"] = dense_leg(torch, m, synth)
    if "fewrow" in legs:
        log("few-row sweep: rows 1..16, bits 4/8, group sizes 32/64/128")
        extra["fewrow_sweep"] = fewrow_sweep_leg(torch, m, synth)
    if "calib" in legs:
        log("counter calibration copy")
        extra["calib"] = calib_leg(torch)
    cpu = None
    if "cpu" in legs:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(torch, synth)
    k1_us = head.pop("_k1_us")
    head.pop("_layer_us")
    for leg in ("decode_m1_isolated", "decode_m4_chained"):
        if leg in extra:
            extra[leg].pop("_k1_us")
            extra[leg].pop("_layer_us")
    ach = head["gate_up_bytes"] / (k1_us * 1e-6) / 1e9
    line = {
        "metric": "effective weight GB/s (M=1/4 MoE decode) + MoE-layer ms at 2048-row prefill",
        "value": round(head["effective_gbs"], 2), "unit": "GB/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(head["ms_per_step"], 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "moe_decode_h4096_i2048_e288_top8_w4g64_m1_chain42", "hidden": 4096,
                   "inter": 2048, "experts": 288, "top_k": 8, "bits": 4, "group_size": 64, "tokens": 1,
                   "index_sets": 42, "step": "one pass over the 42-layer chain (42 MoE decode layers)"},
        "roofline": {"bound": "hbm", "kernel": "qmv_kernel<4,64,glu,2,2> (gathered gate+up, SiLU)", "achieved": round(ach, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": counted_traffic(),
                     "bytes_per_launch": head["gate_up_bytes"], "avg_launch_us": round(k1_us, 3)},
        "cpu_baseline": cpu,
        "legs": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
