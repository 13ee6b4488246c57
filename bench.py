#!/usr/bin/env python3
"""Benchmark: HSTU jagged causal pointwise attention on one MI355X.

Workload: the long-sequence bf16 attention batch -- 16 users with lognormal
lengths (median 2048) clipped to [256, 8192], H = 8 heads, d_qk = d_v = 64,
alpha = 1/8192, relative bias from 256 position buckets and 32 log2 time-delta
buckets, Q, K, V ~ N(0, 1) (seed 1002).  One step = the jagged scheduler plus
the attention kernel over the whole batch, inputs resident in device memory.

Prints one JSON line: causal TFLOP/s (FLOPs = sum_b H n_b (n_b + 1) / 2 * 2 (d_qk + d_v)),
tokens/s, the attention kernel's roofline figures (HIP events around its launches)
and the fp64 CPU oracle timed on a bounded sample of the same rows.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
METRIC = "HSTU jagged causal attn TFLOP/s + tokens/s on 1 MI355X; % of bf16 MFMA peak"
COUNTERS = os.path.join(ROOT, "profiles", "attn_long_hbm_counters.json")
KERNEL_SRC = os.path.join(ROOT, "hstu_sequential_transduction_jagged_amd", "csrc", "attention.hip")


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def causal_flops(lengths, H, dqk, dv):
    return float(sum(H * int(n) * (int(n) + 1) // 2 * 2 * (dqk + dv) for n in lengths))


def traffic_from_profile(launch_bytes_alg):
    """HBM bytes per attention launch from committed rocprofv3 counter runs, or None when
    none were taken or the kernel source changed since."""
    if not os.path.exists(COUNTERS):
        return None
    with open(COUNTERS) as f:
        c = json.load(f)
    if c.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return c.get("hbm_bytes_per_launch")


def cpu_baseline(inp, seconds=15.0, seed=7):
    """The fp64 oracle (as it stands) on a random sample of (token, head) rows of the
    same workload, sized to about `seconds` of CPU time; rate in causal TFLOP/s."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(seed)
    offs = inp.offsets.astype(np.int64)
    b = oracle.Bias(oracle.BIAS_RAB_PT, inp.ts, inp.bias.w_pos, inp.bias.w_time)

    def run(R):
        toks = rng.integers(0, inp.T, size=R)
        heads = rng.integers(0, inp.H, size=R)
        bi = np.searchsorted(offs, toks, side="right") - 1
        fl = float(((toks - offs[bi] + 1) * 2 * (inp.dqk + inp.dv)).sum())
        t0 = time.perf_counter()
        oracle.attention_rows(inp.offsets, inp.q, inp.k, inp.v, b, inp.alpha, toks, heads)
        return fl, time.perf_counter() - t0

    # grow the sample until one run takes at least a second, then scale it to `seconds`
    R = 500
    fl, dt = run(R)
    while dt < 1.0 and R < inp.T * inp.H:
        R = min(inp.T * inp.H, R * 4)
        fl, dt = run(R)
    if dt < seconds and R < inp.T * inp.H:
        R = int(min(inp.T * inp.H, R * seconds / max(dt, 1e-3)))
        fl, dt = run(R)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "%d random (token, head) rows of the attn_long batch (%.3g causal FLOP), "
                      "fp64, %.1f s" % (R, fl, dt),
            "tokens_per_s_equiv": None}


def bench_stack8(args, dev):
    """The 8-layer stack forward (D=512, H=8, d=64, B=128 power-law users, stochastic length
    cap 1024, residual): one step = all 8 layers, each f1 GEMM + SiLU + split, the jagged
    attention with the position / time bias, and the LayerNorm-gate-f2 GEMM with the residual."""
    import numpy as np
    import torch
    from hstu_sequential_transduction_jagged_amd import binding, synth
    inp = synth.stack8()
    bf = torch.bfloat16
    t = lambda a, d=None: torch.from_numpy(np.ascontiguousarray(a)).to(dev, d) if d else \
        torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x0 = t(inp.x, bf)
    offs = t(inp.offsets.astype(np.int32))
    ts = t(inp.ts)
    layers = []
    for L in inp.layers:
        layers.append(dict(w1=t(L.w1, bf), b1=t(L.b1), gamma=t(L.gamma), beta=t(L.beta),
                           w2=t(L.w2, bf), b2=t(L.b2),
                           bias=binding.make_bias(binding.BIAS_RAB_PT, ts, t(L.bias.w_pos),
                                                  t(L.bias.w_time))))
    D = x0.shape[1]
    ws = torch.empty(binding.stack_workspace_bytes(inp.B, inp.T, D, inp.H, inp.dqk, inp.dv,
                                                   inp.max_seqlen), dtype=torch.uint8, device=dev)
    y = torch.empty_like(x0)

    def step():
        # all 8 layers in one call; with --fuse-boundaries each layer's LN-gate-f2 and the next
        # layer's f1 run as one kernel
        return binding.hstu_stack_fwd(x0, offs, inp.max_seqlen, layers, inp.H, inp.dqk, inp.dv,
                                      inp.alpha, True, inp.ln_eps,
                                      fuse_boundaries=args.fuse_boundaries, out=y, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps
    lengths = np.diff(inp.offsets.astype(np.int64))
    T = int(inp.T)
    N1 = 2 * inp.H * (inp.dqk + inp.dv)
    gemm = 2.0 * T * D * N1 + 2.0 * T * inp.H * inp.dv * D
    flops = len(layers) * (causal_flops(lengths, inp.H, inp.dqk, inp.dv) + gemm)
    print(json.dumps({
        "metric": "HSTU 8-layer stack forward TFLOP/s (attention causal FLOPs + f1/f2 GEMM FLOPs)",
        "value": round(flops / step_s / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "stack8", "fused_boundaries": bool(args.fuse_boundaries),
                   "B": inp.B, "layers": len(layers), "D": D, "H": inp.H,
                   "d_qk": inp.dqk, "d_v": inp.dv, "T": T, "max_len": int(lengths.max()),
                   "bias": "rab_pt P=256 NT=32", "alpha": inp.alpha, "seed": inp.seed},
        "tokens_per_s": round(T / step_s, 1),
        "pct_of_bf16_peak": round(100.0 * flops / step_s / 1e12 / PEAK_BF16_TFLOPS, 2)}),
        flush=True)


def bench_genrank(args, dev):
    """The GenRank action-oriented layer at its full size: tokens = item_emb[id] + action_emb[a]
    (10^6 items, Zipf(1.1) ids, 4 action types, rows of 512 bf16), then one HSTU layer with the
    ALiBi bias (D = 512, H = 8, d = 64, B = 64 users of 512..4096 events).  One step = the
    token gather-sum + the layer (f1 GEMM + SiLU + split, attention, LayerNorm-gate-f2)."""
    import numpy as np
    import torch
    from hstu_sequential_transduction_jagged_amd import binding, synth
    g = synth.genrank()
    L = g.layers[0]
    bf = torch.bfloat16
    t = lambda a, d=None: torch.from_numpy(np.ascontiguousarray(a)).to(dev, d) if d else \
        torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    item_table = t(g.item_table, bf)
    action_table = t(g.action_table, bf)
    ids = t(g.item_ids.astype(np.int32))
    aids = t(g.action_ids.astype(np.int32))
    offs = t(g.offsets.astype(np.int32))
    w1, w2 = t(L.w1, bf), t(L.w2, bf)
    b1, b2, gamma, beta = t(L.b1), t(L.b2), t(L.gamma), t(L.beta)
    bias = binding.make_bias(binding.BIAS_ALIBI)
    D, T = g.D, int(g.T)
    x = torch.empty((T, D), dtype=bf, device=dev)
    y = torch.empty((T, D), dtype=bf, device=dev)
    ws = torch.empty(binding.layer_workspace_bytes(g.B, T, D, g.H, g.dqk, g.dv, g.max_seqlen),
                     dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        binding.hstu_embed_sum_fwd(item_table, action_table, ids, aids, out=x)
        if ev is not None:
            ev[1].record()
        binding.hstu_layer_fwd(x, offs, g.max_seqlen, w1, b1, gamma, beta, w2, b2, g.H, g.dqk,
                               g.dv, bias, g.alpha, False, g.ln_eps, out=y, workspace=ws)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps
    emb_s = float(np.mean([a.elapsed_time(b) for a, b, _ in evs])) / 1e3
    layer_s = float(np.mean([b.elapsed_time(c) for _, b, c in evs])) / 1e3
    lengths = np.diff(g.offsets.astype(np.int64))
    N1 = 2 * g.H * (g.dqk + g.dv)
    attn = causal_flops(lengths, g.H, g.dqk, g.dv)
    gemm = 2.0 * T * D * N1 + 2.0 * T * g.H * g.dv * D
    flops = attn + gemm
    # token construction: the item row read, the output row written, two int32 ids per token
    # (the four action rows stay in cache)
    emb_bytes = T * (D * 2 + D * 2 + 8)
    print(json.dumps({
        "metric": "GenRank layer forward TFLOP/s (attention causal FLOPs + f1/f2 GEMM FLOPs)",
        "value": round(flops / step_s / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "genrank", "B": g.B, "D": D, "H": g.H, "d_qk": g.dqk,
                   "d_v": g.dv, "T": T, "max_len": int(lengths.max()), "n_items": 1000000,
                   "n_actions": 4, "bias": "alibi slopes 2^(-8(h+1)/H)", "alpha": g.alpha,
                   "seed": g.seed},
        "tokens_per_s": round(T / step_s, 1),
        "pct_of_bf16_peak": round(100.0 * flops / step_s / 1e12 / PEAK_BF16_TFLOPS, 2),
        "layer_ms": round(layer_s * 1e3, 4),
        "embed_sum": {"ms": round(emb_s * 1e3, 4), "bytes": emb_bytes,
                      "GB_per_s": round(emb_bytes / emb_s / 1e9, 1),
                      "frac_of_hbm_peak": round(emb_bytes / emb_s / 8e12, 4)},
        "attention_causal_flop": attn, "gemm_flop": gemm}), flush=True)


def bench_attn_bwd(args, dev):
    """Gradients of the attention on the attn_long batch (dq, dk, dv and the position / time
    table gradients for a random upstream gradient); one step = one hstu_attn_bwd call."""
    import numpy as np
    import torch
    from hstu_sequential_transduction_jagged_amd import binding, synth
    inp = synth.attn_long()
    bf = torch.bfloat16
    t = lambda a, d=None: torch.from_numpy(np.ascontiguousarray(a)).to(dev, d) if d else \
        torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    q, k, v = t(inp.q, bf), t(inp.k, bf), t(inp.v, bf)
    rng = np.random.default_rng(9)
    d_o = t(synth.round_bf16(rng.standard_normal(inp.q.shape).astype(np.float32)), bf)
    offs = t(inp.offsets.astype(np.int32))
    bias = binding.make_bias(binding.BIAS_RAB_PT, t(inp.ts), t(inp.bias.w_pos), t(inp.bias.w_time))
    ws = torch.empty(binding.attn_workspace_bytes(inp.B, inp.H, inp.max_seqlen, inp.T),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        binding.hstu_attn_bwd(q, k, v, d_o, offs, inp.max_seqlen, bias, inp.alpha, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps
    kms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    k_avg = sum(kms) / len(kms) * 1e-3
    lengths = np.diff(inp.offsets.astype(np.int64))
    # algorithmic FLOPs: four products per causal pair (dA = dO V^T, dV, dQ, dK), 2 d each
    flops = 2.0 * causal_flops(lengths, inp.H, inp.dqk, inp.dv)
    tf = flops / k_avg / 1e12
    print(json.dumps({
        "metric": "HSTU jagged causal attention backward TFLOP/s (4 products per causal pair)",
        "value": round(flops / step_s / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "attn_long backward", "B": inp.B, "H": inp.H, "d_qk": inp.dqk,
                   "d_v": inp.dv, "T": int(inp.T), "bias": "rab_pt P=256 NT=32",
                   "alpha": inp.alpha, "seed": inp.seed},
        "tokens_per_s": round(inp.T / step_s, 1),
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "attn_bwd_dq_kernel + attn_bwd_dkv_kernel (whole call)",
                     "call_ms_p10_p50_p90": [round(kms[int(f * (len(kms) - 1))], 4)
                                             for f in (0.1, 0.5, 0.9)]}}), flush=True)


def bench_layer_bwd(args, dev):
    """Gradients of one layer of the 8-layer stack (D=512, H=8, d=64, B=128 power-law users
    after stochastic length, residual): one step = hstu_layer_bwd after a forward on the same
    inputs (the forward is not timed)."""
    import numpy as np
    import torch
    from hstu_sequential_transduction_jagged_amd import binding, synth
    inp = synth.stack8(n_layers=1)
    L = inp.layers[0]
    bf = torch.bfloat16
    t = lambda a, d=None: torch.from_numpy(np.ascontiguousarray(a)).to(dev, d) if d else \
        torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x = t(inp.x, bf)
    offs = t(inp.offsets.astype(np.int32))
    w1, b1, g, be, w2, b2 = t(L.w1, bf), t(L.b1), t(L.gamma), t(L.beta), t(L.w2, bf), t(L.b2)
    bias = binding.make_bias(binding.BIAS_RAB_PT, t(inp.ts), t(L.bias.w_pos), t(L.bias.w_time))
    D, H, T = inp.D, inp.H, inp.T
    fws = torch.empty(binding.layer_workspace_bytes(inp.B, T, D, H, 64, 64, inp.max_seqlen),
                      dtype=torch.uint8, device=dev)
    binding.hstu_layer_fwd(x, offs, inp.max_seqlen, w1, b1, g, be, w2, b2, H, 64, 64, bias,
                           inp.alpha, True, inp.ln_eps, workspace=fws)
    rng = np.random.default_rng(11)
    dy = t(synth.round_bf16(rng.standard_normal((T, D)).astype(np.float32)), bf)
    bws = torch.empty(int(binding.lib().hstu_layer_bwd_workspace_bytes(inp.B, T, H, 64, 64,
                                                                      inp.max_seqlen)),
                      dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        binding.hstu_layer_bwd(x, offs, inp.max_seqlen, w1, b1, g, be, w2, H, 64, 64, bias,
                               inp.alpha, True, inp.ln_eps, fws, dy, workspace=bws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps
    kms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    k_avg = sum(kms) / len(kms) * 1e-3
    lengths = np.diff(inp.offsets.astype(np.int64))
    N1, HV = 2 * H * 128, H * 64
    # algorithmic FLOPs: twice the forward's (input and weight gradients of both GEMMs, four
    # products per causal pair in the attention)
    flops = 2.0 * (2.0 * T * D * N1 + 2.0 * T * HV * D) + 2.0 * causal_flops(lengths, H, 64, 64)
    tf = flops / k_avg / 1e12
    print(json.dumps({
        "metric": "HSTU layer backward TFLOP/s (2x the forward's GEMM and attention FLOPs)",
        "value": round(flops / step_s / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "stack8 layer backward", "B": inp.B, "D": D, "H": H, "d_qk": 64,
                   "d_v": 64, "T": int(T), "bias": "rab_pt P=256 NT=32", "alpha": inp.alpha,
                   "seed": inp.seed},
        "tokens_per_s": round(T / step_s, 1),
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "hstu_layer_bwd (whole call)",
                     "call_ms_p10_p50_p90": [round(kms[int(f * (len(kms) - 1))], 4)
                                             for f in (0.1, 0.5, 0.9)]}}), flush=True)


def bench_sl(args, dev):
    """Stochastic Length on the device: the 8-layer stack's batch before subsampling (B=128,
    lengths clip(Zipf(1.2), 1, 4096), token rows of 512 bf16 + int64 timestamps), N_c = 4096,
    alpha = 1.6 (target 776 events); one step = select + offsets + gather.  Also reports the
    share of events removed for alpha in 1.6 .. 2.0 on this batch."""
    import numpy as np
    import torch
    from hstu_sequential_transduction_jagged_amd import binding, synth
    rng = np.random.default_rng(1004)
    lengths = synth.zipf_lengths(rng, 128, 1.2, 1, 4096)
    offs_np = synth.offsets_from_lengths(lengths)
    T = int(offs_np[-1])
    D = 512
    x = torch.from_numpy(synth.round_bf16(rng.standard_normal((T, D)).astype(np.float32))).to(dev, torch.bfloat16)
    ts = torch.from_numpy(np.arange(T, dtype=np.int64)).to(dev)
    offs = torch.from_numpy(offs_np.astype(np.int32)).to(dev)
    u = torch.from_numpy(rng.random(128).astype(np.float32)).to(dev)
    keys = torch.from_numpy(rng.random(T).astype(np.float32)).to(dev)
    N_c, alpha = 4096, 1.6
    max_len = int(lengths.max())
    out_o = torch.empty(129, dtype=torch.int32, device=dev)
    src = torch.empty(T, dtype=torch.int32, device=dev)
    x_out, ts_out = torch.empty_like(x), torch.empty_like(ts)
    ws = torch.empty(binding.lib().hstu_stochastic_length_workspace_bytes(128, T), dtype=torch.uint8,
                     device=dev)
    L = binding.lib()
    stream = torch.cuda.current_stream(dev)
    P = binding._ptr

    def step(a=alpha):
        st = L.hstu_stochastic_length(128, P(offs), max_len, T, N_c, a, P(u), P(keys), P(x), D * 2,
                                      P(ts), P(out_o), P(src), P(x_out), P(ts_out), P(ws),
                                      ws.numel(), binding._stream(dev))
        binding._check("hstu_stochastic_length", st)

    sweep = {}
    for a in (1.6, 1.7, 1.8, 1.9, 2.0):
        step(a)
        torch.cuda.synchronize()
        sweep[str(a)] = round(1.0 - int(out_o[-1].item()) / T, 4)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps
    kms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    k_avg = sum(kms) / len(kms) * 1e-3
    T_out = int(out_o[-1].item())
    # algorithmic bytes: keys and draws read once, each kept row + timestamp read and written,
    # one source index written per kept event
    alg = 4 * T + 4 * 128 + T_out * (2 * D * 2 + 16 + 4) + 8 * 129
    gbs = alg / k_avg / 1e9
    print(json.dumps({
        "metric": "Stochastic Length on device: input tokens/s (select + offsets + row gather)",
        "value": round(T / step_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u32/bf16 rows", "data": "synthetic",
        "config": {"workload": "stack8 batch before SL", "B": 128, "T_in": T, "T_out": T_out,
                   "N_c": N_c, "alpha": alpha, "target_len": int(np.floor(N_c ** (alpha / 2))),
                   "row_bytes": D * 2},
        "removed_share_by_alpha": sweep,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(gbs / 8000.0, 4), "traffic": None,
                     "kernel": "sl_select + sl_offsets + sl_gather (whole call)",
                     "call_ms_p10_p50_p90": [round(kms[int(f * (len(kms) - 1))], 4)
                                             for f in (0.1, 0.5, 0.9)]}}), flush=True)


def bench_mfalcon(args, dev):
    """Candidate scoring over cached histories (M-FALCON): 16 users with the attention
    benchmark's history lengths, 1024 candidates each, H=8, d=64, position / time bias; one
    step = one call scoring every candidate of every user against its history K / V."""
    import numpy as np
    import torch
    from hstu_sequential_transduction_jagged_amd import binding, synth
    inp = synth.mfalcon()
    bf = torch.bfloat16
    t = lambda a, d=None: torch.from_numpy(np.ascontiguousarray(a)).to(dev, d) if d else \
        torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    qc, kc, vc, kh, vh = (t(a, bf) for a in (inp.qc, inp.kc, inp.vc, inp.kh, inp.vh))
    ho, co = t(inp.hist_offsets.astype(np.int32)), t(inp.cand_offsets.astype(np.int32))
    ts_h, ts_c = t(inp.ts_h), t(inp.ts_c)
    bias = binding.make_bias(binding.BIAS_RAB_PT, ts_h, t(inp.bias.w_pos), t(inp.bias.w_time))
    out = torch.empty_like(qc)
    ws = torch.empty(binding.candidates_workspace_bytes(inp.B, inp.H, inp.max_hist, inp.Th, inp.Tc),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        binding.hstu_attn_candidates_fwd(qc, kc, vc, co, inp.max_cand, kh, vh, ho, inp.max_hist,
                                         bias, ts_c, inp.alpha, out=out, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps
    kms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    k_avg = sum(kms) / len(kms) * 1e-3
    hist = np.diff(inp.hist_offsets.astype(np.int64))
    cand = np.diff(inp.cand_offsets.astype(np.int64))
    flops = float(sum(int(m) * inp.H * (int(n) + 1) * 2 * 2 * inp.d for n, m in zip(hist, cand)))
    tf = flops / k_avg / 1e12
    print(json.dumps({
        "metric": "M-FALCON candidate scoring TFLOP/s + candidates/s on 1 MI355X",
        "value": round(flops / step_s / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mfalcon", "B": inp.B, "H": inp.H, "d": inp.d,
                   "candidates_per_user": int(cand.max()), "hist_tokens": int(inp.Th),
                   "max_hist": int(inp.max_hist), "bias": "rab_pt P=256 NT=32",
                   "alpha": inp.alpha, "seed": inp.seed},
        "candidates_per_s": round(inp.Tc / step_s, 1),
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel": "attn_cand_bf16_kernel",
                     "kernel_ms_p10_p50_p90": [round(kms[int(f * (len(kms) - 1))], 4)
                                               for f in (0.1, 0.5, 0.9)]}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="attn_long", choices=["attn_long", "stack8", "mfalcon", "attn_bwd", "sl", "layer_bwd", "genrank"],
                    help="attn_long (the headline attention batch), stack8 (the 8-layer HSTU "
                         "stack forward: f1 GEMM + SiLU, attention, LayerNorm-gate-f2, residual) "
                         "mfalcon (1024 candidates per user scored over cached histories) or "
                         "attn_bwd (the attention's gradients on the attn_long batch), sl "
                         "(Stochastic Length on the stack's batch), layer_bwd (one stack "
                         "layer's gradients) or genrank (item + action tokens and one ALiBi "
                         "layer at the GenRank size)")
    ap.add_argument("--regime", default="workload", choices=["workload", "nonlinear"],
                    help="attn_long: the workload's alpha = 1/8192 and tables N(0, 0.02), or "
                         "alpha = 1/8 with tables N(0, 1) (SiLU far from linear)")
    ap.add_argument("--fuse-boundaries", action="store_true",
                    help="stack8: run each layer's LayerNorm-gate-f2 and the next layer's f1 as one "
                         "kernel (the single-operator form between attentions)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB five times "
                         "(calibrates the HBM byte counters against a known traffic)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the attention shards by user with no communication between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from hstu_sequential_transduction_jagged_amd import binding, synth
    if not os.path.exists(binding.LIB_PATH):
        from hstu_sequential_transduction_jagged_amd import build as _b
        _b.build()

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe_mib:
        nbytes = args.copy_probe_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": nbytes, "copy_probe_bytes_written": nbytes,
                          "launches": 5}), flush=True)
        return
    if args.workload == "stack8":
        bench_stack8(args, dev)
        return
    if args.workload == "mfalcon":
        bench_mfalcon(args, dev)
        return
    if args.workload == "attn_bwd":
        bench_attn_bwd(args, dev)
        return
    if args.workload == "sl":
        bench_sl(args, dev)
        return
    if args.workload == "layer_bwd":
        bench_layer_bwd(args, dev)
        return
    if args.workload == "genrank":
        bench_genrank(args, dev)
        return
    if args.regime == "nonlinear":
        # the same batch with alpha = 1/8 and bias tables of std 1: most tiles leave the
        # two-fma Taylor path for the polynomial or exact SiLU
        inp = synth.attn_long(alpha=1.0 / 8.0, table_std=1.0)
    else:
        inp = synth.attn_long()
    lengths = np.diff(inp.offsets.astype(np.int64))
    bf = torch.bfloat16
    q = torch.from_numpy(inp.q).to(dev, bf)
    k = torch.from_numpy(inp.k).to(dev, bf)
    v = torch.from_numpy(inp.v).to(dev, bf)
    offs = torch.from_numpy(inp.offsets.astype(np.int32)).to(dev)
    ts = torch.from_numpy(inp.ts).to(dev)
    wp = torch.from_numpy(inp.bias.w_pos).to(dev)
    wt = torch.from_numpy(inp.bias.w_time).to(dev)
    bias = binding.make_bias(binding.BIAS_RAB_PT, ts, wp, wt)
    out = torch.empty((inp.T, inp.H, inp.dv), dtype=bf, device=dev)
    ws = torch.empty(binding.attn_workspace_bytes(inp.B, inp.H, inp.max_seqlen, inp.T),
                     dtype=torch.uint8, device=dev)

    def step(ev=None):
        # plan (work list), prepare (key norm bounds, timestamp statistics, tile classes), then
        # the attention kernel alone between the events
        binding.hstu_attn_plan(binding.DTYPE_BF16, inp.B, inp.H, inp.dqk, offs, inp.max_seqlen, ws)
        binding.hstu_attn_prepare(k, offs, inp.max_seqlen, ws, bias)
        if ev is not None:
            ev[0].record()
        binding.hstu_attn_fwd_prepared(q, k, v, offs, inp.max_seqlen, ws, bias, inp.alpha, 1.0,
                                       out=out)
        if ev is not None:
            ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / args.steps
    kern_ms = [a.elapsed_time(b) for a, b in evs]
    kern_s = float(np.mean(kern_ms)) / 1e3

    flops = causal_flops(lengths, inp.H, inp.dqk, inp.dv)
    T = int(inp.T)
    value = flops / step_s / 1e12
    achieved = flops / kern_s / 1e12
    # algorithmic bytes per launch: q, k, v read once, o written once, timestamps, tables
    alg_bytes = T * inp.H * (inp.dqk * 2 + inp.dv * 2) * 2 + T * 8 + (256 + 32) * 4
    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "attn_long", "B": inp.B, "H": inp.H, "d_qk": inp.dqk,
                   "d_v": inp.dv, "N_max": 8192, "max_len": int(lengths.max()), "T": T,
                   "causal_pairs": int(sum(int(n) * (int(n) + 1) // 2 for n in lengths)),
                   "bias": "rab_pt P=256 NT=32", "alpha": inp.alpha, "seed": inp.seed,
                   "regime": args.regime},
        "tokens_per_s": round(T / step_s, 1),
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_profile(alg_bytes) if args.regime == "workload" else None,
                     "kernel": "attn_bf16_kernel<1, false, 64>", "kernel_ms": round(kern_s * 1e3, 4),
                     "kernel_ms_p10_p50_p90": [round(float(np.percentile(kern_ms, q)), 4)
                                               for q in (10, 50, 90)],
                     "flop_per_launch": flops, "algorithmic_bytes_per_launch": alg_bytes},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp)
        res["cpu_baseline"].pop("tokens_per_s_equiv", None)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
