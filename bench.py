"""Benchmark of the fused MoE layer forward on one MI355X.

Default workload: the largest layer that fits one GPU, the DeepSeek-V3-shape
MoE block of the SGLang page "srt/models/deepseek_v2.py" (DeepseekV2MoE:
E=256 routed experts, top_k=8, hidden=7168, moe_intermediate_size=2048,
sigmoid scoring with e_score_correction_bias, grouped top-k 8/4,
routed_scaling_factor 2.5) with bf16 weights at prefill size T=8192 tokens,
and its decode size T=64 beside it.  A step is one pass of the whole layer
(routing, permutation, w13 + SiLU-and-mul, w2 + weighted combine) over one
batch of synthetic inputs already resident in HBM.  Every other
configuration (tiny, Mixtral-shape, Qwen-style, DeepSeek-V3 fp8 with its
shared expert) is timed beside it under "configs".  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--config dsv3] [--cpu-sample N]
    python bench.py --profile-config NAME   # only NAME's forward, for counter runs
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FusedMoE fwd tokens/s + TFLOP/s (prefill) / HBM GB/s (decode), 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector/matrix
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def _weight_bytes(cfg):
    return {"f32": 4, "bf16": 2, "fp8": 1}[cfg.w_dtype]


def algorithmic_bytes(cfg, T, active_experts):
    """Weights of the experts that received rows (+ fp8 scales, + shared
    expert), hidden in, out, router logits, routing ids and weights."""
    wb = _weight_bytes(cfg)

    def mlp_bytes(I):
        b = 3 * cfg.H * I * wb
        if cfg.fp8:
            b += (2 * I // 128) * (cfg.H // 128) * 4 + (cfg.H // 128) * (I // 128) * 4
        return b

    act_b = 4 if cfg.act_dtype == "f32" else 2
    return (mlp_bytes(cfg.I) * active_experts + mlp_bytes(cfg.Is) * cfg.shared
            + 2 * T * cfg.H * act_b + T * cfg.E * 4 + T * cfg.K * 8)


def w13_flops(cfg, T):
    return 4.0 * T * cfg.H * (cfg.K * cfg.I + cfg.shared * cfg.Is)


def w13_bytes(cfg, T, active_experts):
    """Algorithmic bytes of one w13 launch: the gate/up weights of the experts
    that received rows (+ block scales), each token's hidden row once, and the
    activation rows written."""
    wb = _weight_bytes(cfg)

    def w13_of(I):
        b = 2 * I * cfg.H * wb
        if cfg.fp8:
            b += (2 * I // 128) * (cfg.H // 128) * 4
        return b

    act_b = 1 if cfg.fp8 else (4 if cfg.act_dtype == "f32" else 2)
    x_b = 4 if cfg.act_dtype == "f32" else 2
    return (w13_of(cfg.I) * active_experts + w13_of(cfg.Is) * cfg.shared + T * cfg.H * x_b
            + T * (cfg.K * cfg.I + cfg.shared * cfg.Is) * act_b)


def _stats(ms):
    ms = np.asarray(ms, np.float64)
    return {"median": float(np.median(ms)), "min": float(np.min(ms)), "mean": float(np.mean(ms))}


def kernel_roofline(flops, byts, seconds, peak_tflops):
    """Roofline of one kernel from its algorithmic FLOPs and bytes: the bound
    is whichever takes longer at the published peaks; `frac` is the achieved
    rate of that resource over its peak (= the attainable-roofline fraction
    max(F/P, B/BW) / t), and both fractions are reported."""
    t_f = flops / (peak_tflops * 1e12)
    t_b = byts / (PEAK_HBM_GBS * 1e9)
    tflops = flops / seconds / 1e12
    gbs = byts / seconds / 1e9
    if t_b >= t_f:
        r = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        r = {"bound": "mfma", "achieved": tflops, "peak": peak_tflops, "unit": "TFLOP/s"}
    r["frac"] = r["achieved"] / r["peak"]
    r.update({"mfma_frac": tflops / peak_tflops, "hbm_frac": gbs / PEAK_HBM_GBS,
              "attainable_frac": max(t_f, t_b) / seconds, "algorithmic_flops": flops,
              "algorithmic_bytes": byts})
    return r


def time_layer(cfg, inp, steps, warmup):
    """Time `steps` passes of the whole layer through the library's entry
    points (wall clock around exactly `steps` steps, synchronised on both
    sides), with HIP events on the launch stream around every step and
    around the w13 GEMM; then the product entry point moe_forward alone."""
    import torch

    from mixture_experts_layer_14_amd.layer import FusedMoE, Stages, params_for

    T = cfg.T
    layer = FusedMoE(params_for(cfg, T), inp)
    st = Stages(layer, T)
    hidden, logits = inp["hidden"], inp["router_logits"]
    bias = inp.get("e_score_correction_bias")
    stream = torch.cuda.current_stream()

    def events(n):
        return [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    s0, s1, w0, w1 = events(steps), events(steps), events(steps), events(steps)

    def step(i=None):
        if i is not None:
            s0[i].record(stream)
        st.topk(logits, bias)
        st.align()
        if st.xq is not None:
            st.quant(hidden)
        if i is not None:
            w0[i].record(stream)
        st.w13(hidden)
        if i is not None:
            w1[i].record(stream)
        st.w2()
        if i is not None:
            s1[i].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = [a.elapsed_time(b) for a, b in zip(s0, s1)]
    w13_ms = [a.elapsed_time(b) for a, b in zip(w0, w1)]
    active = int((st.offsets[1:] - st.offsets[:-1] > 0).sum().item())
    # the product entry point (one call for the whole layer), timed alone
    out = torch.empty_like(st.out)
    f0, f1 = events(steps), events(steps)
    for _ in range(max(1, warmup)):
        layer.forward(hidden, logits, bias, out=out)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(steps):
        f0[i].record(stream)
        layer.forward(hidden, logits, bias, out=out)
        f1[i].record(stream)
    torch.cuda.synchronize()
    fwd_wall = (time.perf_counter() - t1) / steps * 1e3
    fwd_ms = [a.elapsed_time(b) for a, b in zip(f0, f1)]
    del layer, st, out
    torch.cuda.empty_cache()
    return {"ms_per_step": elapsed / steps * 1e3, "step_ms": _stats(step_ms),
            "w13_ms": _stats(w13_ms), "active_experts": active,
            "forward_ms_per_step": fwd_wall, "forward_ms": _stats(fwd_ms)}


def time_router(cfg, T, gate_dtype, steps, warmup):
    """moe_router_gemm (the router gate GEMM ahead of moe_topk) alone, and
    moe_router_topk (gate GEMM and top-k, no logits kept), HIP events on their
    stream; algorithmic bytes = hidden + gate + logits (GEMM) or + ids and
    weights (fused), FLOPs = 2 T E H; the roofline is the larger of the two
    times at the MI355X peaks."""
    import torch

    from mixture_experts_layer_14_amd import binding, synth
    from mixture_experts_layer_14_amd.layer import params_for

    x = synth.make_hidden(cfg, T, device="cuda")
    g = synth.make_gate(cfg, gate_dtype, device="cuda")
    p = params_for(cfg, T)
    ws = torch.empty(max(binding.moe_workspace_size(p), 256), dtype=torch.uint8, device="cuda")
    out = torch.empty(T, cfg.E, dtype=torch.float32, device="cuda")
    ids = torch.empty(T, cfg.K, dtype=torch.int32, device="cuda")
    wts = torch.empty(T, cfg.K, dtype=torch.float32, device="cuda")
    b_ = synth.make_correction_bias(cfg)
    bias = None if b_ is None else torch.from_numpy(b_).cuda()
    p.scoring_func = binding.SIGMOID if cfg.scoring == "sigmoid" else binding.SOFTMAX
    p.num_expert_group, p.topk_group, p.routed_scaling_factor = cfg.n_group, cfg.topk_group, cfg.rsf
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(warmup):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    ms = timed(lambda: binding.moe_router_gemm(p, x, g, out, ws))
    ms_f = timed(lambda: binding.moe_router_topk(p, x, g, bias, ids, wts, None, ws))
    x_b = 4 if cfg.act_dtype == "f32" else 2
    base = T * cfg.H * x_b + cfg.E * cfg.H * (4 if gate_dtype == "f32" else 2)
    byts, byts_f = base + T * cfg.E * 4, base + T * cfg.K * 8
    flops = 2.0 * T * cfg.E * cfg.H
    t_f = flops / (PEAK_BF16_TFLOPS * 1e12)
    t_roof = max(byts / (PEAK_HBM_GBS * 1e9), t_f)
    t_roof_f = max(byts_f / (PEAK_HBM_GBS * 1e9), t_f)
    del x, g, ws, out
    return {"workload": "%s router T=%d E=%d H=%d gate %s" % (cfg.name, T, cfg.E, cfg.H, gate_dtype),
            "us": ms * 1e3, "GBps": byts / (ms * 1e-3) / 1e9,
            "tflops": flops / (ms * 1e-3) / 1e12, "roofline_frac": t_roof / (ms * 1e-3),
            "bound": "hbm" if byts / (PEAK_HBM_GBS * 1e9) >= t_f else "mfma",
            "router_topk_us": ms_f * 1e3, "router_topk_roofline_frac": t_roof_f / (ms_f * 1e-3)}


def shared_streams(cfg_name, Ts, iters=50, warmup=5):
    """The shared expert as a slot of the grouped GEMMs (moe_forward with
    num_shared_experts = 1) against the pages' alternative: the routed layer
    and the shared MLP (a one-expert layer whose only weight is 1) on two
    streams of default priority, joined and added.  Times per forward with
    HIP events; also the difference of the two outputs."""
    import dataclasses

    import torch

    from mixture_experts_layer_14_amd import synth
    from mixture_experts_layer_14_amd.layer import FusedMoE, params_for

    base = synth.CONFIGS[cfg_name]
    full = synth.make_inputs(base, max(Ts), device="cuda")
    res = []
    for T in Ts:
        cfg = base.with_T(T)
        inp = dict(full, hidden=full["hidden"][:T].contiguous(),
                   router_logits=full["router_logits"][:T].contiguous())
        fused = FusedMoE(params_for(cfg, T), inp)
        rcfg = dataclasses.replace(cfg, shared=0)
        routed = FusedMoE(params_for(rcfg, T), {k: v for k, v in inp.items()
                                               if not k.startswith("shared")})
        scfg = dataclasses.replace(cfg, E=1, K=1, shared=0, scoring="softmax", n_group=0,
                                   topk_group=0, rsf=1.0, correction_bias=False)
        sw = {"w13": inp["shared_w13"][None], "w2": inp["shared_w2"][None],
              "w13_scale": None if inp.get("shared_w13_scale") is None else inp["shared_w13_scale"][None],
              "w2_scale": None if inp.get("shared_w2_scale") is None else inp["shared_w2_scale"][None]}
        shared = FusedMoE(params_for(scfg, T), sw)
        zero_logits = torch.zeros(T, 1, dtype=torch.float32, device="cuda")
        x, lg, b = inp["hidden"], inp["router_logits"], inp.get("e_score_correction_bias")
        out_f = torch.empty(T, cfg.H, dtype=torch.bfloat16, device="cuda")
        out_r = torch.empty_like(out_f)
        out_s = torch.empty_like(out_f)
        main = torch.cuda.current_stream()
        side = torch.cuda.Stream()  # default priority

        def two_streams():
            side.wait_stream(main)
            routed.forward(x, lg, b, out=out_r)
            with torch.cuda.stream(side):
                shared.forward(x, zero_logits, None, out=out_s)
            main.wait_stream(side)
            out_r.add_(out_s)

        def timed(fn):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(main)
            for _ in range(iters):
                fn()
            e.record(main)
            torch.cuda.synchronize()
            return a.elapsed_time(e) / iters * 1e3

        t_f = timed(lambda: fused.forward(x, lg, b, out=out_f))
        t_2 = timed(two_streams)
        diff = (out_r.float() - out_f.float()).abs().max().item() / max(out_f.float().abs().max().item(), 1e-30)
        res.append({"T": T, "fused_slot_us": t_f, "two_streams_us": t_2, "rel_diff": diff})
        print(json.dumps(res[-1]), flush=True)
        del fused, routed, shared, inp
        torch.cuda.empty_cache()
    print(json.dumps({"shared_expert": cfg_name, "results": res}), flush=True)


def measured_peaks():
    """What this GPU reaches: the library's bf16 MFMA loop and HBM read
    stream (moe_peak_mfma_bf16 / moe_peak_read), best of 3 timed runs."""
    import torch

    from mixture_experts_layer_14_amd import binding

    blocks, iters = 1024, 20000
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    binding.moe_peak_mfma_bf16(100, blocks, sink)
    best = None
    for _ in range(3):
        a.record()
        binding.moe_peak_mfma_bf16(iters, blocks, sink)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    mfma = blocks * 4 * iters * 8 * 32768.0 / (best * 1e-3) / 1e12
    buf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    rblocks = 16384
    rsink = torch.empty(rblocks * 256, dtype=torch.int32, device="cuda")
    binding.moe_peak_read(buf, rblocks, rsink)
    best = None
    for _ in range(3):
        a.record()
        binding.moe_peak_read(buf, rblocks, rsink)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    read = buf.numel() / (best * 1e-3) / 1e9
    del buf, sink, rsink
    torch.cuda.empty_cache()
    return {"bf16_mfma_tflops": mfma, "hbm_read_GBps": read,
            "spec": {"bf16_mfma_tflops": PEAK_BF16_TFLOPS, "hbm_GBps": PEAK_HBM_GBS}}


def cpu_sample(cfg, inp, tokens, threads=None):
    """The oracle as it stands on `tokens` of the workload (only the experts
    they use are copied to the host), and its routing + permutation over all
    T tokens; host threads (<= 16, or `threads`)."""
    from mixture_experts_layer_14_amd import synth
    from oracle import oracle as O

    if threads is None:
        threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
        threads = max(1, min(threads, 16))
    bits = synth.tensor_bits
    logits = bits(inp["router_logits"])
    bias = bits(inp.get("e_score_correction_bias"))
    scoring = O.SIGMOID if cfg.scoring == "sigmoid" else O.SOFTMAX
    t0 = time.perf_counter()
    ids, _ = O.route(logits, cfg.K, bias=bias, scoring=scoring, renormalize=cfg.renormalize,
                     n_group=cfg.n_group, topk_group=cfg.topk_group,
                     routed_scaling_factor=cfg.rsf)
    O.permute(ids, cfg.E)
    t_route = time.perf_counter() - t0
    tok = list(range(min(tokens, cfg.T)))
    used = sorted(set(int(e) for e in ids[tok].reshape(-1)))

    def per_expert(key):
        t = inp.get(key)
        return None if t is None else {e: bits(t[e]) for e in used}

    L = dict(T=cfg.T, E=cfg.E, K=cfg.K, H=cfg.H, I=cfg.I, scoring=scoring,
             renormalize=cfg.renormalize, n_group=cfg.n_group, topk_group=cfg.topk_group,
             routed_scaling_factor=cfg.rsf, x_dtype=O.F32 if cfg.act_dtype == "f32" else O.BF16,
             w_dtype={"f32": O.F32, "bf16": O.BF16, "fp8": O.E4M3}[cfg.w_dtype], act_fp8=cfg.fp8,
             hidden=bits(inp["hidden"]), logits=logits, bias=bias,
             w13=per_expert("w13"), w2=per_expert("w2"), w13_scale=per_expert("w13_scale"),
             w2_scale=per_expert("w2_scale"), shared_I=cfg.shared_I if cfg.shared else 0)
    if cfg.shared:
        for k in ("shared_w13", "shared_w2", "shared_w13_scale", "shared_w2_scale"):
            L[k] = bits(inp.get(k))
    t0 = time.perf_counter()
    O.moe_forward_tokens(L, tok, nthreads=threads)
    dt = time.perf_counter() - t0
    return {"value": len(tok) / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d tokens, full layer in float64, %.2f s; routing + permutation of "
                      "all %d tokens %.3f s" % (len(tok), cfg.T, dt, cfg.T, t_route)}


# (config, CPU sample tokens): the five configurations at their sizes
PER_CONFIG = [("tiny", 64), ("mixtral_decode", 8), ("mixtral", 8), ("qwen", 32),
              ("dsv3_decode", 4), ("dsv3", 4), ("dsv3_fp8", 4)]


def per_config(steps, warmup, peaks, with_cpu, names=None):
    """Every configuration through moe_forward: median and min of the
    per-forward HIP-event times, tokens/s, TFLOP/s, GB/s of algorithmic
    bytes, their fractions of the published and the measured peaks, and the
    attainable-roofline fraction max(F/P, B/BW) / t."""
    import torch

    from mixture_experts_layer_14_amd import synth
    from mixture_experts_layer_14_amd.layer import FusedMoE, Stages, params_for

    rows = []
    for name, sample in PER_CONFIG:
        if names is not None and name not in names:
            continue
        cfg = synth.CONFIGS[name]
        T = cfg.T
        inp = synth.make_inputs(cfg, T, device="cuda")
        layer = FusedMoE(params_for(cfg, T), inp)
        x, lg, b = inp["hidden"], inp["router_logits"], inp.get("e_score_correction_bias")
        out = torch.empty(T, cfg.H, dtype=torch.float32 if cfg.act_dtype == "f32" else torch.bfloat16,
                          device="cuda")
        n = steps if T >= 1024 else max(steps, 50)
        for _ in range(warmup):
            layer.forward(x, lg, b, out=out)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        stream = torch.cuda.current_stream()
        for e0, e1 in ev:
            e0.record(stream)
            layer.forward(x, lg, b, out=out)
            e1.record(stream)
        torch.cuda.synchronize()
        ms = _stats([e0.elapsed_time(e1) for e0, e1 in ev])
        t = ms["median"] * 1e-3
        st = Stages(layer, T)
        st.topk(lg, b)
        st.align()
        active = int((st.offsets[1:] - st.offsets[:-1] > 0).sum().item())
        flops = cfg.flops()
        byts = algorithmic_bytes(cfg, T, active)
        peak = {"bf16": PEAK_BF16_TFLOPS, "fp8": PEAK_FP8_TFLOPS, "f32": PEAK_F32_TFLOPS}[cfg.w_dtype]
        t_f, t_b = flops / (peak * 1e12), byts / (PEAK_HBM_GBS * 1e9)
        row = {"config": name, "T": T, "dtype": cfg.w_dtype, "iters": n, "ms": ms["median"],
               "ms_min": ms["min"], "ms_mean": ms["mean"], "tokens_per_s": T / t,
               "tflops": flops / t / 1e12, "GBps": byts / t / 1e9, "active_experts": active,
               "mfma_frac": flops / t / 1e12 / peak, "hbm_frac": byts / t / 1e9 / PEAK_HBM_GBS,
               "bound": "mfma" if t_f >= t_b else "hbm", "roofline_frac": max(t_f, t_b) / t}
        if peaks and cfg.w_dtype == "bf16":
            m_f = flops / (peaks["bf16_mfma_tflops"] * 1e12)
            m_b = byts / (peaks["hbm_read_GBps"] * 1e9)
            row["roofline_frac_measured_peaks"] = max(m_f, m_b) / t
        if with_cpu:
            row["cpu_baseline"] = cpu_sample(cfg, inp, sample)
            if name == "tiny":  # the tiny layer also on one host thread
                row["cpu_baseline_1thread"] = cpu_sample(cfg, inp, sample, threads=1)
        rows.append(row)
        print("config %s: median %.3f ms, min %.3f ms" % (name, ms["median"], ms["min"]),
              file=sys.stderr, flush=True)
        del layer, st, inp, out
        torch.cuda.empty_cache()
    return rows


def profile_config(name, steps, warmup):
    """Only `name`'s forward through moe_forward (warmup + steps calls): the
    program a counter run (rocprofv3 --pmc) profiles, so each dispatch of a
    moe kernel in its output belongs to this one configuration."""
    import torch

    from mixture_experts_layer_14_amd import synth
    from mixture_experts_layer_14_amd.layer import FusedMoE, params_for

    cfg = synth.CONFIGS[name]
    inp = synth.make_inputs(cfg, cfg.T, device="cuda")
    layer = FusedMoE(params_for(cfg, cfg.T), inp)
    x, lg, b = inp["hidden"], inp["router_logits"], inp.get("e_score_correction_bias")
    torch.cuda.synchronize()
    print("profile %s: inputs ready" % name, flush=True)
    for i in range(warmup + steps):
        layer.forward(x, lg, b)
        torch.cuda.synchronize()
        print("profile %s: forward %d done" % (name, i), flush=True)


def source_digest():
    """sha256 over the sources of the grouped GEMM kernels (and the headers
    they share): identifies the kernels a stored counter measurement belongs
    to."""
    import glob
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_layer_14_amd", "csrc")
    names = ("moe_gemm*", "moe_device.h", "moe_internal.h")
    for path in sorted(p for n in names for p in glob.glob(os.path.join(csrc, n))):
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode())
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(kernel_key):
    """HBM bytes per launch of `kernel_key` from profiles/hbm_traffic.md, if
    that file was measured on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        line = line.strip().lstrip("-").strip()
        if ":" in line and line.split(":", 1)[0].strip().replace("_", "").isalnum():
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha256") != source_digest():
        return None
    v = fields.get("%s_bytes_per_launch" % kernel_key)
    return float(v) if v else None


def calibrate_copy(nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters (FETCH_SIZE / WRITE_SIZE) of a profiler run."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}))


WORKLOAD = {
    "dsv3": "DeepSeek-V3-shape MoE layer forward (E=256, top_k=8, hidden=7168, "
            "intermediate=2048, bf16 weights; sigmoid + correction bias, grouped top-k 8 groups / 4, "
            "routed_scaling_factor 2.5), prefill T=8192",
    "dsv3_decode": "DeepSeek-V3-shape MoE layer forward, bf16, decode T=64",
    "dsv3_fp8": "DeepSeek-V3-shape MoE layer forward, fp8 e4m3 experts (128x128 block scales, "
                "group-128 activation quant) + 1 shared expert, T=8192",
    "mixtral": "Mixtral-shape MoE layer forward (E=8, top_k=2, hidden=4096, intermediate=14336, "
               "bf16; softmax + renormalize), prefill T=4096",
    "mixtral_decode": "Mixtral-shape MoE layer forward, bf16, decode T=32",
    "qwen": "Qwen-style MoE layer forward (E=128, top_k=8, hidden=2048, intermediate=768, bf16; "
            "Zipf-skewed softmax routing), T=16384",
}


def _peak(cfg):
    return {"bf16": PEAK_BF16_TFLOPS, "fp8": PEAK_FP8_TFLOPS, "f32": PEAK_F32_TFLOPS}[cfg.w_dtype]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="dsv3")
    ap.add_argument("--decode-config", default="dsv3_decode")
    ap.add_argument("--cpu-sample", type=int, default=256,
                    help="tokens of the headline workload the CPU oracle computes")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration table and the measured peaks")
    ap.add_argument("--configs", default="",
                    help="comma-separated subset of the per-configuration table")
    ap.add_argument("--profile-config", default="",
                    help="only run this configuration's forward (for counter runs)")
    ap.add_argument("--shared-streams", action="store_true",
                    help="only compare the shared expert as a GEMM slot with a second stream")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build runs the whole expert set on a single "
              "MI355X (no expert/tensor parallelism); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from mixture_experts_layer_14_amd import binding, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.shared_streams:
        shared_streams("dsv3_fp8", [1, 16, 64, 256, 8192])
        return
    binding.load()
    if args.profile_config:
        profile_config(args.profile_config, args.steps, args.warmup)
        return
    cfg = synth.CONFIGS[args.config]
    T = cfg.T
    inp = synth.make_inputs(cfg, T, device="cuda")
    r = time_layer(cfg, inp, args.steps, args.warmup)
    flops = cfg.flops()
    peak = _peak(cfg)
    w13_s = r["w13_ms"]["mean"] * 1e-3
    roof = kernel_roofline(w13_flops(cfg, T), w13_bytes(cfg, T, r["active_experts"]), w13_s, peak)
    roof.update({"kernel": "w13 grouped GEMM + SiLU-and-mul",
                 "traffic": stored_traffic("%s_w13" % cfg.name),
                 "avg_kernel_ms": r["w13_ms"]["mean"], "median_kernel_ms": r["w13_ms"]["median"],
                 "min_kernel_ms": r["w13_ms"]["min"]})
    t_step = r["ms_per_step"] * 1e-3
    layer_bytes = algorithmic_bytes(cfg, T, r["active_experts"])
    line = {
        "metric": METRIC,
        "value": T / t_step,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8-e4m3", "f32": "f32"}[cfg.w_dtype],
        "data": "synthetic (seeded N(0,1) hidden and logits, N(0,0.02) weights)",
        "config": {"workload": WORKLOAD.get(cfg.name, cfg.name), "E": cfg.E, "top_k": cfg.K,
                   "hidden": cfg.H, "intermediate": cfg.I, "T": T, "weights": cfg.w_dtype,
                   "routing": "%s%s%s" % (cfg.scoring, "+renormalize" if cfg.renormalize else "",
                                          " grouped %d/%d" % (cfg.n_group, cfg.topk_group)
                                          if cfg.n_group > 1 else "")},
        "step_ms": r["step_ms"],
        "tflops": flops / t_step / 1e12,
        "mfma_frac": flops / t_step / 1e12 / peak,
        "hbm_GBps": layer_bytes / t_step / 1e9,
        "layer_attainable_frac": max(flops / (peak * 1e12), layer_bytes / (PEAK_HBM_GBS * 1e9)) / t_step,
        "forward_ms_per_step": r["forward_ms_per_step"],
        "forward_ms": r["forward_ms"],
        "active_experts": r["active_experts"],
        "roofline": roof,
    }
    if not args.no_cpu and args.cpu_sample > 0:
        line["cpu_baseline"] = cpu_sample(cfg, inp, args.cpu_sample)
    del inp
    torch.cuda.empty_cache()
    if args.decode_config:
        dcfg = synth.CONFIGS[args.decode_config]
        dinp = synth.make_inputs(dcfg, dcfg.T, device="cuda")
        d = time_layer(dcfg, dinp, max(args.steps, 50), args.warmup)
        del dinp
        torch.cuda.empty_cache()
        byts = algorithmic_bytes(dcfg, dcfg.T, d["active_experts"])
        gbs = byts / (d["ms_per_step"] * 1e-3) / 1e9
        line["decode"] = {"workload": WORKLOAD.get(dcfg.name, dcfg.name), "T": dcfg.T,
                          "ms_per_step": d["ms_per_step"], "step_ms": d["step_ms"],
                          "tokens_per_s": dcfg.T / (d["ms_per_step"] * 1e-3),
                          "hbm_GBps": gbs, "hbm_frac": gbs / PEAK_HBM_GBS,
                          "algorithmic_bytes": byts, "active_experts": d["active_experts"],
                          "forward_ms_per_step": d["forward_ms_per_step"],
                          "forward_ms": d["forward_ms"]}
        droof = kernel_roofline(w13_flops(dcfg, dcfg.T), w13_bytes(dcfg, dcfg.T, d["active_experts"]),
                                d["w13_ms"]["mean"] * 1e-3, _peak(dcfg))
        droof.update({"kernel": "w13 weight-streaming GEMM + SiLU-and-mul",
                      "traffic": stored_traffic("%s_w13" % dcfg.name),
                      "avg_kernel_ms": d["w13_ms"]["mean"], "median_kernel_ms": d["w13_ms"]["median"],
                      "min_kernel_ms": d["w13_ms"]["min"]})
        line["decode"]["roofline"] = droof
    # the router gate GEMM (a separate entry point, not part of the step)
    dsv3, mix = synth.CONFIGS["dsv3"], synth.CONFIGS["mixtral"]
    line["router"] = [time_router(dsv3, dsv3.T, "f32", 20, 3),
                      time_router(dsv3, 64, "f32", 50, 3),
                      time_router(mix, mix.T, "bf16", 20, 3),
                      time_router(mix, 32, "bf16", 50, 3)]
    if not args.no_configs:
        peaks = measured_peaks()
        line["measured_peaks"] = peaks
        names = [n for n in args.configs.split(",") if n] or None
        line["configs"] = per_config(10, 3, peaks, not args.no_cpu, names)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
