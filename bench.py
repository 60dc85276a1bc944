#!/usr/bin/env python3
"""MoE-layer benchmark on one MI355X.

Headline workload (one step = one token through the whole hot path of 40
distinct seeded MoE layers -- router, top-8, permutation, expert FFNs with
in-kernel 4-bit dequantisation, combine -- with a residual add between
layers and a fresh N(0,1) input per step): decode, T = 1.  The 40-layer
chain is captured once in a HIP graph and replayed per step.

Also measured in the same run and reported in the same JSON line:
  - the unit the decode step repeats (one layer launch: router, top-8 and
    both expert GEMVs with combine) timed with HIP events on the stream it
    runs on, against HBM peak;
  - the measured sustained HBM read rate (a streaming read probe);
  - prefill, T = 4096 tokens through one layer (rotating over the 40 layers
    so the weights are not cache resident), with MFMA utilisation;
  - the CPU oracle on a bounded sample of the decode workload.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

H, I, E, TOPK = 2048, 512, 256, 8
EXPERT_BYTES = 3 * I * H // 2 + 3 * (I * H // 64) * 2 * 2      # 1,769,472 B
EXPERT_FLOP_PER_TOKEN = 2 * 3 * I * H                           # 6,291,456
# algorithmic bytes of one decode layer at T = 1: 8 routed + 1 shared expert,
# the router matrix and the shared-expert gate vector
LAYER_DECODE_BYTES = 9 * EXPERT_BYTES + E * H * 2 + H * 2       # 16,977,920
HBM_PEAK_GBS = 8000.0
BF16_DENSE_PEAK_TFLOPS = 2516.6     # 256 CU x 2.4 GHz x 4096 flop/clk/CU (fp16 = bf16 rate)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gen_layers(n, skewed=False, threads=16):
    from gemv_router_softmax_amd import synth
    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(lambda l: synth.make_layer(synth.PROD, seed=0, layer=l,
                                                      skewed_bias=skewed), range(n)))


def event_pairs(n):
    import torch
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n)]


def decode_chain(D, args):
    """The 40-layer T = 1 chain (moe_chain_forward: every layer after the
    first is two kernels) captured once in a HIP graph and replayed per
    step with a fresh input token."""
    import torch
    import gemv_router_softmax_amd as moe
    from gemv_router_softmax_amd import synth

    K, W = args.steps, args.warmup
    xs = torch.from_numpy(np.stack([synth.make_x(1, seed=0, step=s) for s in range(W + K)])
                          .view(np.int16)).cuda()                       # [W+K, 1, H]
    x0 = torch.empty((1, H), dtype=torch.int16, device="cuda")
    xo = torch.empty((1, H), dtype=torch.int16, device="cuda")
    ws = moe.workspace(1)
    chain = moe.LayerChain(D)

    def run():
        moe.moe_chain_forward(x0, chain, xo, ws)

    x0.copy_(xs[0])
    run()
    torch.cuda.synchronize()
    g = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        torch.cuda.synchronize()

    def step(s):
        x0.copy_(xs[s])
        if g is not None:
            g.replay()
        else:
            run()

    for s in range(W):
        step(s)
    torch.cuda.synchronize()
    e0, e1 = event_pairs(1)[0]
    e0.record()
    for s in range(K):
        step(W + s)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    return ms, xs


def decode_layer_timing(D, xs, reps):
    """HIP events on the launch stream around eager 40-layer chain calls at
    T = 1 -- the same call, kernels and arguments that the graph replays.
    Each call is queued behind a ~0.5 ms streaming read, so its kernels run
    back to back on the GPU instead of waiting for the host; the per-layer
    time is the call's time over the layer count (the first layer's router
    kernel included)."""
    import torch
    import gemv_router_softmax_amd as moe

    ws = moe.workspace(1)
    xo = torch.empty((1, H), dtype=torch.int16, device="cuda")
    pad = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    pad.fill_(1)
    sink = torch.zeros(4096, dtype=torch.float32, device="cuda")
    chain = moe.LayerChain(D)
    pairs = event_pairs(reps)
    for r in range(reps + 1):
        cur = xs[r % xs.shape[0]]
        moe.moe_probe_read(pad, sink)
        if r == 0:                      # warm-up
            moe.moe_chain_forward(cur, chain, xo, ws)
        else:
            a, b = pairs[r - 1]
            a.record()
            moe.moe_chain_forward(cur, chain, xo, ws)
            b.record()
        torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in pairs]) / len(D)
    del pad
    return float(ms.mean()), float(np.median(ms))


def read_ceiling(gib=4, reps=5):
    import torch
    import gemv_router_softmax_amd as moe
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(4096, dtype=torch.float32, device="cuda")
    moe.moe_probe_read(buf, sink)
    pairs = event_pairs(reps)
    for a, b in pairs:
        a.record()
        moe.moe_probe_read(buf, sink)
        b.record()
    torch.cuda.synchronize()
    best = min(a.elapsed_time(b) for a, b in pairs)
    del buf
    return buf_gbs(gib << 30, best)


def copy_calibration(mib=256, reps=5):
    """A plain copy of known size for scaling the HBM byte counters
    (FETCH_SIZE / WRITE_SIZE) of a profiled run: the counters of
    probe_copy_kernel read against mib MiB read and mib MiB written."""
    import torch
    import gemv_router_softmax_amd as moe
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(3)
    for _ in range(reps):
        moe.moe_probe_copy(dst, src)
    torch.cuda.synchronize()
    del src, dst


# the kernel sources a profile's figures depend on (the host file only
# orchestrates launches)
DECODE_SOURCES = ("decode.hip", "block_util.hpp", "common.hpp")


def decode_source_hash():
    """Hash of the sources of the decode layer kernels: a traffic figure
    measured on other code is not reported."""
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, "gemv_router_softmax_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


EXPERT_SOURCES = ("expert.hip", "block_util.hpp", "common.hpp")


def expert_source_hash():
    """Hash of the sources of the prefill grouped GEMM."""
    h = hashlib.sha256()
    for f in EXPERT_SOURCES:
        with open(os.path.join(ROOT, "gemv_router_softmax_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profile_json(name, source_hash):
    """The JSON block of a committed rocprofv3 summary under profiles/, or
    None if it is missing or was taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", name)
    try:
        with open(path) as fh:
            m = re.search(r"```json\n(.*?)\n```", fh.read(), re.S)
        d = json.loads(m.group(1))
    except (OSError, AttributeError, ValueError):
        return None
    if d.get("source_hash") != source_hash:
        return None
    return d


def measured_traffic():
    """HBM bytes per chained decode layer (decode_gateup_dec +
    decode_down_dec) from the rocprofv3 PMC summary."""
    d = profile_json("decode_layer_t1_traffic.md", decode_source_hash())
    return None if d is None else d.get("bytes_per_launch")


def kernel_level_decode():
    """SURVEY's kernel-level decode figure: the active-expert bytes of a
    layer (9 x 1,769,472 B) over the summed average rocprofv3 durations of
    the two expert kernels of a chained layer, from the kernel-trace
    summary of the 40-layer chain."""
    d = profile_json("decode_t1_chain40_kernel_stats.md", decode_source_hash())
    if d is None:
        return None
    us = d["decode_gateup_dec_avg_us"] + d["decode_down_dec_avg_us"]
    gbs = 9 * EXPERT_BYTES / (us * 1e-6) / 1e9
    return {"expert_bytes": 9 * EXPERT_BYTES, "kernels_us": us, "gbs": gbs,
            "frac_of_hbm_peak": gbs / HBM_PEAK_GBS, "source": "profiles/decode_t1_chain40_kernel_stats.md"}


def gemm_clock():
    """Shader clock inside the prefill GEMM kernels (GRBM_GUI_ACTIVE cycles
    over the dispatch duration, from the rocprofv3 counter summary)."""
    d = profile_json("prefill_t4096_gemm_clock.md", expert_source_hash())
    return None if d is None else {"per_kernel_ghz": d["ghz"], "time_weighted_ghz": d["ghz_weighted"]}


def buf_gbs(nbytes, ms):
    return nbytes / (ms * 1e-3) / 1e9


def prefill(D, T, iters):
    """One layer at T tokens, rotating over the layers so the weights are not
    cache resident.  Each timed call is captured once in its own HIP graph
    and replayed with HIP events around each replay, so the host's launch
    rate never shows in the GPU time."""
    import torch
    import gemv_router_softmax_amd as moe
    from gemv_router_softmax_amd import synth

    x = moe.to_device_bits(synth.make_x(T, seed=0))
    y = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ws = moe.workspace(T)
    ids = torch.empty((T, 8), dtype=torch.int32, device="cuda")
    w = torch.empty((T, 8), dtype=torch.float32, device="cuda")
    sg = torch.empty((T,), dtype=torch.float32, device="cuda")
    counts = torch.empty(256, dtype=torch.int32, device="cuda")
    offs = torch.empty(257, dtype=torch.int32, device="cuda")
    perm = torch.empty(8 * T, dtype=torch.int32, device="cuda")
    inv = torch.empty(8 * T, dtype=torch.int32, device="cuda")
    out = torch.empty((9 * T, H), dtype=torch.float32, device="cuda")
    nl = min(iters, len(D))

    def capture(fn):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def timed(graphs):
        for g in graphs:          # warm-up
            g.replay()
        torch.cuda.synchronize()
        pairs = event_pairs(iters)
        for i, (a, b) in enumerate(pairs):
            a.record()
            graphs[i % len(graphs)].replay()
            b.record()
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in pairs])

    layer_graphs = [capture(lambda Dl=D[(i + 3) % len(D)]: moe.moe_layer_forward(x, Dl, y, ws))
                    for i in range(nl)]
    ms = timed(layer_graphs)
    del layer_graphs
    # the expert FFN (grouped GEMM) alone, on routing computed beforehand
    ffn_graphs = []
    for i in range(nl):
        Dl = D[(i + 7) % len(D)]
        moe.moe_route(x, Dl.w_router, Dl.router_bias, Dl.w_shared_gate, ids, w, sg, ws)
        moe.moe_permute(ids, counts, offs, perm, inv, ws)
        ffn_graphs.append(capture(lambda Dl=Dl: moe.moe_expert_ffn(
            x, Dl, offs, perm, out, ws, path=moe.MOE_PATH_PREFILL)))
    # the routing of the last captured layer is what every FFN replay reads
    fms = timed(ffn_graphs)
    del ffn_graphs
    flops = EXPERT_FLOP_PER_TOKEN * 9 * T
    clk = gemm_clock()
    return {
        "T": T,
        "timing": "HIP events around graph replays, one layer per replay",
        "gemm_clock_ghz": clk,
        "expert_ffn_mfma_util_at_measured_clock": (
            None if clk is None else flops / (fms.mean() * 1e-3)
            / (BF16_DENSE_PEAK_TFLOPS * 1e12 * clk["time_weighted_ghz"] / 2.4)),
        "layer_ms": float(ms.mean()),
        "tokens_per_s": T / (ms.mean() * 1e-3),
        "layer_mfma_util": flops / (ms.mean() * 1e-3) / (BF16_DENSE_PEAK_TFLOPS * 1e12),
        "expert_ffn_ms": float(fms.mean()),
        "expert_ffn_tflops": flops / (fms.mean() * 1e-3) / 1e12,
        "expert_ffn_mfma_util": flops / (fms.mean() * 1e-3) / (BF16_DENSE_PEAK_TFLOPS * 1e12),
    }


def _graphs_timed(fns, iters):
    """Capture each callable once in its own HIP graph, then replay them in
    turn with HIP events around every replay; returns the per-replay ms."""
    import torch
    graphs = []
    for fn in fns:
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        graphs.append(g)
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    pairs = event_pairs(iters)
    for i, (a, b) in enumerate(pairs):
        a.record()
        graphs[i % len(graphs)].replay()
        b.record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in pairs])


def prefill_sweep(D, Ts, iters):
    """One layer at each T (rotating over the layers), graph-replayed: tokens/s,
    MFMA utilisation of the expert flops and the algorithmic HBM rate (all 257
    experts' weights are touched from T of a few hundred up)."""
    import torch
    import gemv_router_softmax_amd as moe
    from gemv_router_softmax_amd import synth
    out = []
    for T in Ts:
        x = moe.to_device_bits(synth.make_x(T, seed=0))
        y = torch.empty((T, H), dtype=torch.int16, device="cuda")
        ws = moe.workspace(T)
        nl = min(iters, len(D))
        ms = _graphs_timed([lambda Dl=D[(i + 11) % len(D)]: moe.moe_layer_forward(x, Dl, y, ws)
                            for i in range(nl)], iters)
        t = float(ms.mean()) * 1e-3
        flops = EXPERT_FLOP_PER_TOKEN * 9 * T
        wbytes = 257 * EXPERT_BYTES + E * H * 2 + H * 2 + 2 * T * H * 2
        out.append({"T": T, "layer_ms": t * 1e3, "tokens_per_s": T / t,
                    "mfma_util": flops / t / (BF16_DENSE_PEAK_TFLOPS * 1e12),
                    "tflops": flops / t / 1e12, "weight_gbs": wbytes / t / 1e9,
                    "bound": "mfma" if flops / wbytes > BF16_DENSE_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3
                             else "hbm"})
        del x, y, ws
    return out


def prefill_chain(D, T, iters):
    """T tokens through the whole layer chain with residual adds (one
    moe_chain_forward call captured as a HIP graph): tokens/s and per-layer
    time."""
    import torch
    import gemv_router_softmax_amd as moe
    from gemv_router_softmax_amd import synth
    x0 = moe.to_device_bits(synth.make_x(T, seed=0))
    xo = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ws = moe.workspace(T)
    chain = moe.LayerChain(D)
    ms = _graphs_timed([lambda: moe.moe_chain_forward(x0, chain, xo, ws)], iters)
    t = float(ms.mean()) * 1e-3
    return {"T": T, "layers": len(D), "chain_ms": t * 1e3, "tokens_per_s": T / t,
            "layer_us": t / len(D) * 1e6,
            "weight_gbs": len(D) * (257 * EXPERT_BYTES + E * H * 2) / t / 1e9}


def skewed_chunked(T_total, chunk, iters, layers=4):
    """The Zipf-biased router: T_total tokens in chunks of `chunk` through one
    layer, rotating over a few skewed layers, each call one HIP graph:
    pipelined (moe_layer_forward_chunked: the next chunk's routing and
    permutation on a second stream under the current chunk's GEMMs) and, for
    comparison, the chunks back to back on one stream."""
    import torch
    import gemv_router_softmax_amd as moe
    from gemv_router_softmax_amd import synth
    Ds = [moe.DeviceLayer(L) for L in gen_layers(layers, skewed=True)]
    x = moe.to_device_bits(synth.make_x(T_total, seed=0))
    y = torch.empty((T_total, H), dtype=torch.int16, device="cuda")
    ws = moe.workspace(chunk)
    ws1 = moe.workspace(chunk)

    def run_seq(Dl):
        for c0 in range(0, T_total, chunk):
            moe.moe_layer_forward(x[c0:c0 + chunk], Dl, y[c0:c0 + chunk], ws)

    def run_pipe(Dl):
        moe.moe_layer_forward_chunked(x, Dl, y, chunk, ws, ws1)
    seq = float(_graphs_timed([lambda Dl=Dl: run_seq(Dl) for Dl in Ds], iters).mean()) * 1e-3
    t = float(_graphs_timed([lambda Dl=Dl: run_pipe(Dl) for Dl in Ds], iters).mean()) * 1e-3
    flops = EXPERT_FLOP_PER_TOKEN * 9 * T_total
    nch = (T_total + chunk - 1) // chunk
    return {"T": T_total, "chunk": chunk, "ms": t * 1e3, "tokens_per_s": T_total / t,
            "mfma_util": flops / t / (BF16_DENSE_PEAK_TFLOPS * 1e12),
            "ms_back_to_back": seq * 1e3, "us_per_chunk": t / nch * 1e6,
            "us_per_chunk_back_to_back": seq / nch * 1e6}


GREEDY_V = 151936     # synthetic vocabulary (the pages give none): a Qwen-family size


def greedy_decode(D, steps, V=GREEDY_V, reps=10):
    """The greedy decode step kept on the GPU: embedding lookup of the
    previous token -> the whole layer chain -> output-head GEMV + argmax ->
    the next token, in device memory for the next step; one HIP graph per
    step.  Also the head kernel alone (HIP events around eager calls):
    V x 4 KB of bf16 head per call."""
    import torch
    import gemv_router_softmax_amd as moe
    from gemv_router_softmax_amd import synth
    head, emb = synth.make_head(V, seed=0)
    hd, ed = moe.to_device_bits(head), moe.to_device_bits(emb)
    del head, emb
    chain = moe.LayerChain(D)
    tok = torch.tensor([1], dtype=torch.int32, device="cuda")
    x = torch.empty((1, H), dtype=torch.int16, device="cuda")
    xo = torch.empty_like(x)
    ws = moe.workspace(1)

    def step():
        moe.moe_embed(tok, ed, x)
        moe.moe_chain_forward(x, chain, xo, ws)
        moe.moe_lm_head_argmax(xo, hd, tok, ws)
    ms = _graphs_timed([step], steps)
    pairs = event_pairs(reps)
    for a, b in pairs:
        a.record()
        moe.moe_lm_head_argmax(xo, hd, tok, ws)
        b.record()
    torch.cuda.synchronize()
    hms = np.array([a.elapsed_time(b) for a, b in pairs])
    hbytes = V * H * 2 + H * 2
    t = float(ms.mean()) * 1e-3
    return {"vocab": V, "layers": len(D), "step_ms": t * 1e3, "tokens_per_s": 1.0 / t,
            "head_ms": float(hms.mean()), "head_gbs": hbytes / (hms.mean() * 1e-3) / 1e9,
            "head_frac_of_hbm_peak": hbytes / (hms.mean() * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "timing": "graph replays of the whole step; head: HIP events around eager calls"}


def gdn_scan_leg(T=2048, hk=None, hv=None, iters=50):
    """The gated delta rule scan of one recurrent layer over T tokens
    (moe_gdn_scan: gdn_prep + gdn_scan), HIP events around graph replays of
    the call.  Algorithmic work: the chunked form's matrix products as the
    kernels issue them (fp16 MFMA), per 64-token chunk and value head
    11.5 MFLOP; bytes: q, k, v, g, beta in, o out, the state in and out."""
    import torch
    import gemv_router_softmax_amd as moe
    from gemv_router_softmax_amd import synth
    hk = hk or synth.GDN_HK
    hv = hv or synth.GDN_HV
    x = synth.make_gdn(T, hk, hv, seed=0)
    q, k, v = (moe.to_device_bits(a) for a in (x.q, x.k, x.v))
    g, beta, s0 = (torch.from_numpy(a).cuda() for a in (x.g, x.beta, x.s0))
    o = torch.empty((T, hv, 128), dtype=torch.int16, device="cuda")
    s_out = torch.empty((hv, 128, 128), dtype=torch.float32, device="cuda")
    ws = moe.gdn_workspace(T, hv)
    ms = _graphs_timed([lambda: moe.moe_gdn_scan(q, k, v, g, beta, o, ws, s0=s0, s_out=s_out)],
                       iters)
    t = float(ms.mean()) * 1e-3
    nch = (T + 63) // 64
    flops = nch * hv * 11534336
    nbytes = T * hk * 128 * 2 * 2 + T * hv * 128 * 2 * 2 + T * hv * 4 * 2 + hv * 128 * 128 * 4 * 2
    return {"T": T, "key_heads": hk, "value_heads": hv, "dim": 128, "chunk": 64,
            "us": t * 1e6, "tokens_per_s": T / t, "mfma_gflop": flops / 1e9,
            "tflops": flops / t / 1e12, "mfma_util": flops / t / (BF16_DENSE_PEAK_TFLOPS * 1e12),
            "io_bytes": nbytes, "io_gbs": nbytes / t / 1e9,
            "workspace_bytes": moe.moe_gdn_workspace_bytes(T, hv),
            "timing": "HIP events around graph replays of one moe_gdn_scan call"}


def gdn_step_leg(layers=40, hk=None, hv=None, iters=50, T=1):
    """One decode token (or T tokens) through `layers` recurrent layers
    (moe_gdn_scan; T = 1 takes the token-by-token kernel), each layer with
    its own state updated in place, captured as one HIP graph; per-layer
    time from HIP events.  Bytes per layer: the state read and written
    (fp32 [hv][128][128] each way) plus q, k, v, g, beta and o."""
    import torch
    import gemv_router_softmax_amd as moe
    from gemv_router_softmax_amd import synth
    hk = hk or synth.GDN_HK
    hv = hv or synth.GDN_HV
    xs = [synth.make_gdn(T, hk, hv, seed=100 + i) for i in range(layers)]
    dev = [tuple(moe.to_device_bits(a) for a in (x.q, x.k, x.v)) +
           tuple(torch.from_numpy(a).cuda() for a in (x.g, x.beta, x.s0)) for x in xs]
    o = torch.empty((T, hv, 128), dtype=torch.int16, device="cuda")
    ws = moe.gdn_workspace(T, hv)

    def step():
        for q, k, v, g, beta, st in dev:
            moe.moe_gdn_scan(q, k, v, g, beta, o, ws, s0=st, s_out=st)

    ms = _graphs_timed([step], iters)
    t = float(ms.mean()) * 1e-3 / layers
    nbytes = hv * 128 * 128 * 4 * 2 + T * (hk * 128 * 2 * 2 + hv * 128 * 2 * 2 + hv * 4 * 2)
    return {"T": T, "layers": layers, "key_heads": hk, "value_heads": hv, "dim": 128,
            "us_per_layer": t * 1e6, "bytes_per_layer": nbytes, "gbs": nbytes / t / 1e9,
            "frac_of_hbm_peak": nbytes / t / 1e9 / HBM_PEAK_GBS,
            "timing": "HIP events around graph replays of the layers' calls, one after another"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(layers, budget_s):
    """The oracle (plain fp64 C, OpenMP) timed on this host on bounded
    samples: decode T = 1 through the whole chain on all threads (the line's
    value) and on one thread, and the first 512 tokens of the T = 4096
    prefill input through one layer."""
    import oracle
    from gemv_router_softmax_amd import synth
    o = oracle.load()
    nthreads = o.threads()

    def decode(budget, max_steps):
        t0 = time.perf_counter()
        n = 0
        while True:
            x = synth.make_x(1, seed=0, step=n)
            for L in layers:
                y = o.layer_forward(L, x).y
                x = o.round_bf16(o.bf16_decode(x) + o.bf16_decode(y))
            n += 1
            el = time.perf_counter() - t0
            if el >= budget or n >= max_steps:
                return n, el

    n, el = decode(budget_s * 0.6, 64)
    o.set_threads(1)
    n1, el1 = decode(budget_s * 0.25, 64)
    o.set_threads(nthreads)
    xp = synth.make_x(4096, seed=0)[:512]
    t0 = time.perf_counter()
    o.layer_forward(layers[3 % len(layers)], xp)
    elp = time.perf_counter() - t0
    try:
        affinity = len(os.sched_getaffinity(0))
    except OSError:
        affinity = None
    return {"value": n / el, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{n} decode steps (T=1) through the same {len(layers)}-layer chain, "
                      f"{el:.1f} s of CPU work on {nthreads} threads",
            "single_thread": {"value": n1 / el1, "unit": "tokens/s",
                              "sample": f"{n1} decode steps through the {len(layers)}-layer "
                                        f"chain, {el1:.1f} s"},
            "prefill_t4096_sample": {"value": 512 / elp, "unit": "tokens/s",
                                     "sample": f"the first 512 of the 4096 prefill tokens "
                                               f"through one layer, {elp:.1f} s on {nthreads} "
                                               f"threads"},
            "cpu_model": cpu_model(), "host_logical_cpus": os.cpu_count(),
            "affinity_cpus": affinity}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=40)
    ap.add_argument("--kernel-reps", type=int, default=5)
    ap.add_argument("--prefill-iters", type=int, default=20)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the prefill T sweep, the T=512 chain, the skewed chunked run and "
                         "the greedy step")
    ap.add_argument("--legs", default="t4096,sweep,chain512,skewed,greedy,gdn",
                    help="which of the extra measurements to run (comma list; for profiling "
                         "one of them alone)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 256 MiB device copy (scales profiled HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the MoE layer here runs on a single MI355X "
              "(no collectives are built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import gemv_router_softmax_amd as moe
    moe.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    t = time.time()
    host = gen_layers(args.layers)
    log(f"generated {args.layers} layers in {time.time() - t:.1f}s")
    t = time.time()
    D = [moe.DeviceLayer(L) for L in host]
    torch.cuda.synchronize()
    log(f"uploaded {sum(d.nbytes for d in D) / 1e9:.2f} GB in {time.time() - t:.1f}s")
    if args.no_cpu_baseline:
        del host

    ms, xs = decode_chain(D, args)
    ms_per_step = ms / args.steps
    tok_s = args.steps / (ms * 1e-3)
    log(f"decode chain: {ms_per_step * 1e3:.1f} us/token, {tok_s:.1f} tokens/s")

    k_mean, k_med = decode_layer_timing(D, xs, args.kernel_reps)
    per_launch_bytes = LAYER_DECODE_BYTES
    achieved = per_launch_bytes / (k_mean * 1e-3) / 1e9
    log(f"decode layer (eager chain): {k_mean * 1e3:.2f} us/layer (median {k_med * 1e3:.2f}), "
        f"{achieved:.0f} GB/s; graph chain {ms_per_step * 1e3 / args.layers:.2f} us/layer")
    ceiling = read_ceiling()
    log(f"read ceiling: {ceiling:.0f} GB/s")
    if args.copy_calibration:
        copy_calibration()
    traffic = measured_traffic()

    legs = set(args.legs.split(",")) if not args.no_extra else {"t4096"}
    pre = None
    if not args.no_prefill and "t4096" in legs:
        pre = prefill(D, 4096, args.prefill_iters)
        log(f"prefill T=4096: {pre}")
    sweep = chain512 = skewed = None
    if not args.no_prefill and "sweep" in legs:
        sweep = prefill_sweep(D, (256, 1024, 2048, 4096), args.prefill_iters)
        log(f"prefill sweep: {sweep}")
    if not args.no_prefill and "chain512" in legs:
        chain512 = prefill_chain(D, 512, 5)
        log(f"prefill chain T=512: {chain512}")
    if not args.no_prefill and "skewed" in legs:
        skewed = skewed_chunked(16384, 4096, 8)
        log(f"skewed chunked prefill: {skewed}")

    greedy = None
    if "greedy" in legs:
        greedy = greedy_decode(D, 200)
        log(f"greedy decode step: {greedy}")
    gdn = None
    gdn_step = None
    if "gdn" in legs:
        gdn = gdn_scan_leg()
        log(f"gated delta rule scan: {gdn}")
        gdn_step = gdn_step_leg()
        log(f"gated delta rule decode step: {gdn_step}")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(host, args.cpu_seconds)
        log(f"cpu baseline: {cpu}")

    chain_bytes = args.layers * 9 * EXPERT_BYTES
    out = {
        "metric": "MoE-layer tokens/s; HBM GB/s at T=1 decode; MFMA util at T=4096 prefill",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded layers and inputs, random-init weights)",
        "config": {"workload": f"decode T=1 through a {args.layers}-layer MoE chain with "
                               "residual adds, fresh N(0,1) input per step",
                   "layers": args.layers, "T": 1, "hidden": H, "experts": E, "topk": TOPK,
                   "expert_width": I, "group": 64, "weights": "uint4 + fp16 scale/bias",
                   "arithmetic": "fp16 (bf16 router) products, fp32 accumulation",
                   "hip_graph": not args.no_graph},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "decode layer at T=1 inside the chain (decode_gateup_dec + "
                               "decode_down_dec), eager chain behind a long read",
                     "bytes_per_launch": per_launch_bytes, "launch_us": k_mean * 1e3,
                     "frac_of_read_ceiling": achieved / ceiling,
                     "kernel_level": kernel_level_decode()},
        "active_expert_bytes_per_token": chain_bytes,
        "wallclock_gbs": chain_bytes / (ms_per_step * 1e-3) / 1e9,
        "hbm_read_ceiling_gbs": ceiling,
        "prefill_t4096": pre,
        "prefill_sweep": sweep,
        "prefill_chain_t512": chain512,
        "prefill_skewed_t16384_chunks4096": skewed,
        "greedy_decode_step": greedy,
        "gdn_scan_t2048": gdn,
        "gdn_step_t1": gdn_step,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
