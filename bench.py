"""Throughput of the dual-stream MMDiT block core on one MI355X.

A step is one mmdit_block_fwd over the 480p workload: 32760 visual tokens (81 frames at
480x832 -> 21x30x52 latent grid) + 512 conditioning tokens, width 3072, 24 heads x 128,
FFN 12288 (GELU), 1536-d timestep bottleneck, bf16 weights and activations (seeded
synthetic inputs, resident in HBM before the timed region).

Prints one JSON line: block tokens/s (value), the joint-attention TFLOP/s and its fraction
of the bf16 MFMA peak (roofline; the attention kernel's duration is read from hipEvents the
library records around it on the stream it runs on), the per-stage breakdown, and the
float64 oracle timed on this host on a bounded sample (cpu_baseline).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "joint-attn TFLOP/s + % bf16 MFMA peak; block tokens/s at 32760+512 tokens"
PEAK_BF16_TFLOPS = 2500.0      # MI355X published dense bf16 MFMA peak
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5000.0       # MI355X published dense fp8 MFMA peak

# HBM bytes per attention stage of the block at this workload (joint_attn_mfma_kernel plus the
# merge kernel of its split tail, the two launches the stage's events bracket), from two
# rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the
# same counter reads for a 1 GiB device copy (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0).  Valid only
# for the kernel source they were taken on: a different joint_attention.hip reports null.
ATTN_COUNTERS = {"source_sha256": "39024d9182be8c82",
                 "fetch_kib": 1104356.0 + 15815.9, "write_kib": 227870.6 + 3056.0,
                 "fetch_scale": 2.0, "write_scale": 1.0}


def attention_traffic_bytes():
    import hashlib
    src = os.path.join(ROOT, "video_diffusion_transformer_mmdit_amd", "csrc", "joint_attention.hip")
    with open(src, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    c = ATTN_COUNTERS
    if not digest.startswith(c["source_sha256"]):
        return None
    return (c["fetch_kib"] * c["fetch_scale"] + c["write_kib"] * c["write_scale"]) * 1024.0


class Hip:
    """hipEvent plumbing through ctypes (the library records the events on its stream)."""

    def __init__(self):
        self.L = ctypes.CDLL("libamdhip64.so")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self) -> int:
        e = ctypes.c_void_p()
        if self.L.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        if self.L.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, e: int):
        self.L.hipEventDestroy(ctypes.c_void_p(e))


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def cpu_baseline(cfg, raw):
    """The float64 oracle on this host, on a bounded sample of the same workload.

    The oracle computes K and V of every token (a fixed cost of a few seconds) and then the
    per-query work of the sampled rows (attention over all keys, out-projection, FFN).  A tiny
    and a large row sample give the fixed and the per-row cost; the full-job time is
    extrapolated linearly (rows are independent given K and V).  The large sample is sized so
    that its per-row work clearly exceeds the run-to-run noise of the fixed part."""
    import oracle
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    x_vis = wl.to_f64(raw["x_vis"], wl.BF16)
    x_cond = wl.to_f64(raw["x_cond"], wl.BF16)
    tvec = wl.to_f64(raw["tvec"], wl.BF16)
    w = {s: {k: wl.to_f64(raw[f"{s}.{k}"], wl.BF16) for k in wl.STREAM_WEIGHTS} for s in ("vis", "cond")}
    times = []
    sizes = [(16, 8), (1536, 256)]
    for nv, nc in sizes:
        rv = wl.sample_rows(cfg.n_vis, nv, seed=900 + nv)
        rc = wl.sample_rows(cfg.n_cond, nc, seed=901 + nc)
        t0 = time.perf_counter()
        oracle.block_forward(x_vis, x_cond, tvec, w["vis"], w["cond"], cfg.grid, cfg.heads, cfg.ln_eps,
                             cfg.qk_eps, vis_rows=rv, cond_rows=rc, keep=False)
        times.append(time.perf_counter() - t0)
        log(f"oracle sample {nv}+{nc} rows: {times[-1]:.2f} s")
    (n1, t1), (n2, t2) = (sum(sizes[0]), times[0]), (sum(sizes[1]), times[1])
    if not t2 > t1:
        raise RuntimeError(f"cpu baseline: the large sample ({t2:.2f} s) was not slower than the small one ({t1:.2f} s)")
    per_row = (t2 - t1) / (n2 - n1)
    fixed = max(t1 - n1 * per_row, 0.0)
    t_full = fixed + cfg.n_tokens * per_row
    return {"value": cfg.n_tokens / t_full, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"float64 numpy oracle block forward, K/V of all {cfg.n_tokens} tokens plus "
                       f"{sizes[0][0]}+{sizes[0][1]} and {sizes[1][0]}+{sizes[1][1]} sampled query rows "
                       f"({t1:.1f} s, {t2:.1f} s); full job extrapolated as fixed {fixed:.1f} s + "
                       f"{per_row * 1e3:.1f} ms/row x {cfg.n_tokens} rows = {t_full:.0f} s")}


def time_calls(fn, reps: int = 20, warm: int = 3) -> float:
    """Average ms of fn() over reps calls on torch's current stream (the library launches on
    it), from one pair of events around the loop."""
    import torch
    for _ in range(warm):
        fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    b.synchronize()
    return a.elapsed_time(b) / reps


def attention_configs(dev):
    """The four attention workloads on their own: seeded Q, K, V in the workload's dtype ->
    prologue (qk_norm_rope: Q^/K^ in f16 for the 16-bit workloads, f32 for the fp32 one; the
    16-bit workloads' bf16 V cast to f16, the type the QKV GEMM hands the block's attention)
    -> joint attention (with the split-tail workspace), each timed with events over repeated
    calls.  The fp32 workload (40 tokens, 2 heads) is launch-bound; it is reported for
    completeness."""
    import torch
    import video_diffusion_transformer_mmdit_amd as mm
    import workloads as wl
    res = {}
    ws = torch.empty(mm.ATTN_SPLIT_BYTES, dtype=torch.uint8, device=dev)
    for cfg, reps in ((wl.ATTN_TINY, 50), (wl.ATTN_LAYER, 50), (wl.ATTN_480P, 10), (wl.ATTN_720P, 5)):
        raw = wl.attention_inputs(cfg)
        if cfg.dtype == wl.F32:
            t = {k: torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(dev) for k, v in raw.items()}
            qk_dt = torch.float32
        else:
            t = {k: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to(dev) for k, v in raw.items()}
            qk_dt = torch.float16
        rope = mm.Rope3D.make(cfg.grid, cfg.rope_split, cfg.rope_base)
        qv, kv = mm.qk_norm_rope(t["q_vis"], t["k_vis"], t["gq_vis"], t["gk_vis"], rope=rope, eps=cfg.qk_eps,
                                 out_dtype=qk_dt)
        qc, kc = mm.qk_norm_rope(t["q_cond"], t["k_cond"], t["gq_cond"], t["gk_cond"], eps=cfg.qk_eps, out_dtype=qk_dt)
        ov = torch.empty((cfg.batch, cfg.n_vis, cfg.heads, 128), dtype=torch.float32, device=dev)
        oc = torch.empty((cfg.batch, cfg.n_cond, cfg.heads, 128), dtype=torch.float32, device=dev)
        if cfg.dtype == wl.F32:
            vv, vc = t["v_vis"], t["v_cond"]
        else:
            vv, vc = mm.cast(t["v_vis"], torch.float16), mm.cast(t["v_cond"], torch.float16)

        def prologue():
            mm.qk_norm_rope(t["q_vis"], t["k_vis"], t["gq_vis"], t["gk_vis"], rope=rope, eps=cfg.qk_eps,
                            q_out=qv, k_out=kv)
            mm.qk_norm_rope(t["q_cond"], t["k_cond"], t["gq_cond"], t["gk_cond"], eps=cfg.qk_eps, q_out=qc, k_out=kc)
            if cfg.dtype != wl.F32:
                mm.cast(t["v_vis"], torch.float16, out=vv)
                mm.cast(t["v_cond"], torch.float16, out=vc)

        ms_n = time_calls(prologue, reps=reps)
        ms_a = time_calls(lambda: mm.joint_attention(qv, kv, vv, qc, kc, vc, o_vis=ov, o_cond=oc,
                                                     workspace=ws), reps=reps)
        el_in = 4 if cfg.dtype == wl.F32 else 2
        el_out = 4 if cfg.dtype == wl.F32 else 2
        n_ops = 2 if cfg.dtype == wl.F32 else 3   # Q, K (and V) read once and written once
        nbytes = n_ops * cfg.n_tokens * cfg.batch * cfg.heads * 128 * (el_in + el_out)
        fl = cfg.attn_flops
        res[cfg.name] = {
            "tokens": cfg.n_tokens, "dtype": cfg.dtype, "attention_ms": round(ms_a, 4),
            "attention_tflops": round(fl / ms_a / 1e9, 3 if fl < 1e10 else 1),
            "attention_frac_bf16_peak": round(fl / ms_a / 1e9 / PEAK_BF16_TFLOPS, 5),
            "prologue_ms": round(ms_n, 4), "prologue_GB_per_s": round(nbytes / ms_n / 1e6, 1),
            "prologue_frac_hbm": round(nbytes / ms_n / 1e6 / PEAK_HBM_GBS, 4),
            "prologue": "qk_norm_rope" + ("" if cfg.dtype == wl.F32 else " + V cast to f16")}
        if cfg.dtype == wl.F32:
            res[cfg.name]["note"] = "launch-bound (40 tokens, 2 heads; fp32 VALU kernel)"
        del t, qv, kv, qc, kc, vv, vc, ov, oc
    del ws
    return res


def memory_bound_kernels(dev):
    """The block's memory-bound kernels at the 480p visual stream's shapes, alone: the
    modulation GEMV (one stream's W_mod 18432 x 1536 bf16), LN-modulate before attention (x
    bf16 -> h f16) and before the FFN (x1 f32 -> h2 f16), and QK-RMSNorm + 3D RoPE in place on
    the packed q|k|v rows (f16).  Algorithmic bytes: each tensor read or written once.  A
    device-to-device copy of the LN's x (201 MB read, 201 MB written) is timed beside them as
    the rate a plain stream reaches on this machine (`frac_copy`)."""
    import torch
    import video_diffusion_transformer_mmdit_amd as mm
    import workloads as wl
    cfg = wl.BLOCK_480P
    C, N = cfg.width, cfg.n_vis
    g = torch.Generator(device=dev).manual_seed(7)
    out = {}
    w = (torch.randn((6 * C, cfg.t_dim), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    bm = (torch.randn((6 * C,), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    tv = torch.randn((1, cfg.t_dim), generator=g, device=dev).to(torch.bfloat16)
    mod = torch.empty((1, 6 * C), dtype=torch.float32, device=dev)
    ms = time_calls(lambda: mm.modulation(w, bm, tv, out=mod), reps=50)
    nb = w.numel() * 2
    out["modulation_gemv"] = {"ms": round(ms, 4), "bytes": nb, "GB_per_s": round(nb / ms / 1e6, 1),
                              "frac_hbm": round(nb / ms / 1e6 / PEAK_HBM_GBS, 4)}
    x = torch.randn((1, N, C), generator=g, device=dev).to(torch.bfloat16)
    x1 = torch.randn((1, N, C), generator=g, device=dev)
    h = torch.empty((1, N, C), dtype=torch.float16, device=dev)
    shift, scale = mod[:, :C], mod[:, C:2 * C]
    for name, src, el in (("modulate_ln_attention", x, 2), ("modulate_ln_ffn", x1, 4)):
        ms = time_calls(lambda: mm.modulate_ln(src, shift, scale, y=h), reps=20)
        nb = N * C * (el + 2)
        out[name] = {"ms": round(ms, 4), "bytes": nb, "GB_per_s": round(nb / ms / 1e6, 1),
                     "frac_hbm": round(nb / ms / 1e6 / PEAK_HBM_GBS, 4)}
    xc = torch.empty_like(x)
    ms = time_calls(lambda: xc.copy_(x), reps=20)
    nb = 2 * x.numel() * 2
    copy_gbs = nb / ms / 1e6
    out["device_copy"] = {"ms": round(ms, 4), "bytes": nb, "GB_per_s": round(copy_gbs, 1),
                          "frac_hbm": round(copy_gbs / PEAK_HBM_GBS, 4)}
    del x, x1, h, xc
    qkv = torch.randn((1, N, 3, cfg.heads, 128), generator=g, device=dev).to(torch.float16)
    gq = (1 + 0.1 * torch.randn((128,), generator=g, device=dev)).to(torch.bfloat16)
    gk = (1 + 0.1 * torch.randn((128,), generator=g, device=dev)).to(torch.bfloat16)
    rope = mm.Rope3D.make(cfg.grid)
    q, k = qkv[:, :, 0], qkv[:, :, 1]
    ms = time_calls(lambda: mm.qk_norm_rope(q, k, gq, gk, rope=rope, q_out=q, k_out=k), reps=20)
    nb = 4 * N * C * 2
    out["qk_norm_rope"] = {"ms": round(ms, 4), "bytes": nb, "GB_per_s": round(nb / ms / 1e6, 1),
                           "frac_hbm": round(nb / ms / 1e6 / PEAK_HBM_GBS, 4)}
    for k, v in out.items():
        if k != "device_copy":
            v["frac_copy"] = round(v["GB_per_s"] / copy_gbs, 4)
    return out


def next_rows(dev):
    """The conditioning path that produces tvec (full 1536-d and Lite 16-d bottleneck) and the
    Lite 2x2 merge / unpatchify at 480p, timed on their own (not part of the block step)."""
    import torch
    import video_diffusion_transformer_mmdit_amd as mm
    import workloads as wl
    out = {}
    for cfg in (wl.TIMESTEP_FULL, wl.TIMESTEP_LITE):
        raw = wl.timestep_inputs(cfg)
        t = torch.from_numpy(raw["t"]).to(dev)
        ws = [torch.from_numpy(raw[k].view(np.int16)).view(torch.bfloat16).to(dev) for k in wl.TIMESTEP_WEIGHTS]
        bufs = mm.timestep_embed(t, *ws)
        ms = time_calls(lambda: mm.timestep_embed(t, *ws, hidden=bufs[0], temb=bufs[1], tvec=bufs[2]), reps=50)
        wbytes = sum(w.numel() * 2 for w in ws)
        out[f"timestep_path_dt{cfg.t_dim}"] = {
            "us": round(ms * 1e3, 2), "batch": cfg.batch, "weight_bytes": wbytes,
            "GB_per_s": round(wbytes / (ms * 1e-3) / 1e9, 1), "launches": 3}
    cfg = wl.LITE_480P
    raw = wl.lite_inputs(cfg)
    t = {k: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to(dev) for k, v in raw.items()}
    ym = torch.empty((1, cfg.n_merged, cfg.width), dtype=torch.bfloat16, device=dev)
    yu = torch.empty((1, cfg.n_full, cfg.width), dtype=torch.bfloat16, device=dev)
    half = cfg.flops / 2
    ms_m = time_calls(lambda: mm.lite_merge(t["x"], t["w_merge"], t["b_merge"], cfg.grid, y=ym))
    ms_u = time_calls(lambda: mm.lite_unpatchify(t["y"], t["w_unpatch"], t["b_unpatch"], cfg.grid, y=yu))
    out["lite_merge_480p"] = {"ms": round(ms_m, 4), "tflops": round(half / (ms_m * 1e-3) / 1e12, 1),
                              "shape": f"M={cfg.n_merged} N={cfg.width} K={4 * cfg.width}, bf16 in/out"}
    out["lite_unpatchify_480p"] = {"ms": round(ms_u, 4), "tflops": round(half / (ms_u * 1e-3) / 1e12, 1),
                                   "shape": f"M={cfg.n_merged} N={4 * cfg.width} K={cfg.width}, bf16 in/out"}
    del t, ym, yu
    out["lite_block_480p"] = lite_block(dev)
    out["fp8_gemm_480p"] = fp8_gemms(dev)
    out["attention_8bit"] = attention_8bit(dev)
    return out


def attention_8bit(dev):
    """The 8-bit joint attention at 480p and 720p (seeded N(0,1) Q^, K^, V in bf16, 24 heads):
    operand quantization and the attention kernel timed separately, beside the 16-bit kernel
    on the same inputs (Q^/K^ in f16 as the block feeds it)."""
    import torch
    import video_diffusion_transformer_mmdit_amd as mm
    import workloads as wl
    res = {}
    # key-range results of the kernels' split tails (allocated once, outside the timing)
    ws = torch.empty(mm.ATTN_SPLIT_BYTES, dtype=torch.uint8, device=dev)
    for cfg in (wl.ATTN_480P, wl.ATTN_720P):
        raw = wl.attention_inputs(cfg)
        t = {k: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to(dev) for k, v in raw.items()}
        ops = mm.attn8_quantize(t["q_vis"], t["k_vis"], t["v_vis"], t["q_cond"], t["k_cond"], t["v_cond"])
        ov = torch.empty((1, cfg.n_vis, cfg.heads, 128), dtype=torch.float32, device=dev)
        oc = torch.empty((1, cfg.n_cond, cfg.heads, 128), dtype=torch.float32, device=dev)
        ms_q = time_calls(lambda: mm.attn8_quantize(t["q_vis"], t["k_vis"], t["v_vis"], t["q_cond"], t["k_cond"],
                                                    t["v_cond"], out=ops), reps=5, warm=1)
        ms_a = time_calls(lambda: mm.joint_attention_8bit(ops, o_vis=ov, o_cond=oc, workspace=ws), reps=5, warm=1)
        h16 = {k: t[k].to(torch.float16) for k in ("q_vis", "k_vis", "v_vis", "q_cond", "k_cond", "v_cond")}
        ms_16 = time_calls(lambda: mm.joint_attention(h16["q_vis"], h16["k_vis"], h16["v_vis"], h16["q_cond"],
                                                      h16["k_cond"], h16["v_cond"], o_vis=ov, o_cond=oc,
                                                      workspace=ws),
                           reps=5, warm=1)
        fl = cfg.attn_flops
        res[cfg.name.split("_")[0]] = {
            "tokens": cfg.n_tokens, "attention_ms": round(ms_a, 4), "tflops": round(fl / ms_a / 1e9, 1),
            "frac_8bit_peak": round(fl / ms_a / 1e9 / PEAK_FP8_TFLOPS, 4),
            "quantize_ms": round(ms_q, 4), "f16_attention_ms": round(ms_16, 4),
            "f16_tflops": round(fl / ms_16 / 1e9, 1)}
        del t, ops, ov, oc, h16
    del ws
    return res


def block_8bit(cfg, wv, wc, t, rope, hip):
    """The 480p block in the Wan report's 8-bit inference setup (section 4.4.3): the four GEMM
    matrices quantized to E4M3 per tensor once, at load; every GEMM on FP8 operands (its f16
    input quantized per token inside the step) and the 8-bit joint attention (its operands
    quantized inside the step).  Same inputs as the 16-bit step; stages from hipEvents."""
    import torch
    import video_diffusion_transformer_mmdit_amd as mm
    dev = t["x_vis"].device
    w8v, w8c = mm.fp8_block_weights(wv), mm.fp8_block_weights(wc)
    dims = mm.BlockDims.make(cfg.width, cfg.heads, cfg.ffn, cfg.t_dim, cfg.ln_eps, cfg.qk_eps,
                             act_dtype=torch.float16, matrix_dtype=torch.float8_e4m3fn)
    ws = torch.empty(mm.block_workspace_bytes(dims, 1, cfg.n_vis, cfg.n_cond), dtype=torch.uint8, device=dev)
    ov = torch.empty((1, cfg.n_vis, cfg.width), dtype=torch.float32, device=dev)
    oc = torch.empty((1, cfg.n_cond, cfg.width), dtype=torch.float32, device=dev)
    steps = 10
    events = [[hip.event() for _ in range(2 * mm.STAGE_COUNT)] for _ in range(steps)]

    def step(evs=None):
        mm.block_fwd(dims, w8v, w8c, t["x_vis"], t["x_cond"], t["tvec"], rope, workspace=ws, out_vis=ov,
                     out_cond=oc, stage_events=evs)
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    stage = {name: float(np.mean([hip.elapsed_ms(e[2 * i], e[2 * i + 1]) for e in events]))
             for i, name in enumerate(mm.STAGES)}
    for e in events:
        for x in e:
            hip.destroy(x)
    att = stage["attention"]
    return {"ms_per_step": round(ms, 4), "tokens": cfg.n_tokens, "tokens_per_s": round(cfg.n_tokens / (ms * 1e-3), 1),
            "stages_ms": {k: round(v, 4) for k, v in stage.items()},
            "attention_tflops": round(cfg.attn_flops / (att * 1e-3) / 1e12, 1),
            "attention_frac_8bit_peak": round(cfg.attn_flops / (att * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
            "note": "GEMM stages include the per-token FP8 quantization of their input, the attention stage "
                    "the quantization of its operands; weights quantized once at load"}


def lite_block(dev):
    """One block of the Lite backbone at 480p: the 2x2-merged 21x15x26 = 8190 visual tokens +
    512 conditioning tokens, the 16-wide timestep bottleneck, otherwise the block above."""
    import torch
    import video_diffusion_transformer_mmdit_amd as mm
    import workloads as wl
    cfg = wl.BlockConfig("lite_block480p", 3072, 24, 128, 12288, 16, (21, 15, 26), 512, seed=6)
    raw = wl.block_inputs(cfg)
    t = {k: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to(dev) for k, v in raw.items()}
    wv = {k: t[f"vis.{k}"] for k in wl.STREAM_WEIGHTS}
    wc = {k: t[f"cond.{k}"] for k in wl.STREAM_WEIGHTS}
    dims = mm.BlockDims.make(cfg.width, cfg.heads, cfg.ffn, cfg.t_dim, act_dtype=torch.float16)
    rope = mm.Rope3D.make(cfg.grid)
    ws = torch.empty(mm.block_workspace_bytes(dims, 1, cfg.n_vis, cfg.n_cond), dtype=torch.uint8, device=dev)
    ov = torch.empty((1, cfg.n_vis, cfg.width), dtype=torch.float32, device=dev)
    oc = torch.empty((1, cfg.n_cond, cfg.width), dtype=torch.float32, device=dev)
    ms = time_calls(lambda: mm.block_fwd(dims, wv, wc, t["x_vis"], t["x_cond"], t["tvec"], rope, workspace=ws,
                                         out_vis=ov, out_cond=oc), reps=10, warm=2)
    return {"ms": round(ms, 4), "tokens": cfg.n_tokens, "tokens_per_s": round(cfg.n_tokens / (ms * 1e-3), 1),
            "tflops": round(cfg.total_flops / (ms * 1e-3) / 1e12, 1)}


def fp8_gemms(dev):
    """The visual stream's four GEMM shapes at 480p (M = 32760) with FP8 operands (per-token
    x scales, per-tensor W scale) beside the same shapes with f16 operands, and the
    per-token quantization of the two activation widths."""
    import torch
    import video_diffusion_transformer_mmdit_amd as mm
    M = 32760
    g = torch.Generator(device=dev).manual_seed(0)
    res = {}
    for name, N, K, epi in (("qkv", 9216, 3072, mm.EPI_NONE), ("out_proj", 3072, 3072, mm.EPI_NONE),
                            ("ffn_up", 12288, 3072, mm.EPI_GELU), ("ffn_down", 3072, 12288, mm.EPI_NONE)):
        x = torch.randn((M, K), generator=g, device=dev, dtype=torch.float16)
        w = (torch.randn((N, K), generator=g, device=dev, dtype=torch.float16) * 0.02)
        xq, xs = mm.quantize_fp8(x)
        wq, ws = mm.quantize_fp8(w, per_row=False)
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
        fl = 2.0 * M * N * K
        ms8 = time_calls(lambda: mm.linear_fp8(xq, xs, wq, ws, None, epilogue=epi, y=y), reps=10)
        ms16 = time_calls(lambda: mm.linear(x, w, None, epilogue=epi, y=y), reps=10)
        msq = time_calls(lambda: mm.quantize_fp8(x, q=xq, scales=xs), reps=10)
        res[name] = {"M": M, "N": N, "K": K, "fp8_ms": round(ms8, 4), "fp8_tflops": round(fl / ms8 / 1e9, 1),
                     "fp8_frac_peak": round(fl / ms8 / 1e9 / PEAK_FP8_TFLOPS, 4),
                     "f16_ms": round(ms16, 4), "f16_tflops": round(fl / ms16 / 1e9, 1),
                     "quantize_x_ms": round(msq, 4), "quantize_x_GB_per_s": round(M * K * 3 / msq / 1e6, 1)}
        del x, w, xq, wq, y
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--act-dtype", choices=("f16", "bf16"), default="f16",
                    help="type of the 16-bit intermediates and MFMA operands")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true", help="skip the timing of the timestep path and Lite merge")
    ap.add_argument("--next", choices=("all", "block_8bit"), default="all",
                    help="which next rows to time (block_8bit: only the 8-bit block, e.g. for a profile)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload attention records and the memory-bound kernels alone")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (5 times): the reference "
                         "kernel for scaling FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the block core runs on a single MI355X (no sharding, no "
              "collectives); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import video_diffusion_transformer_mmdit_amd as mm
    import workloads as wl

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": n * 4, "launches": 5}), flush=True)
        return

    cfg = wl.BLOCK_480P
    dev = torch.device("cuda:0")
    log(f"generating inputs {cfg.name}")
    raw = wl.block_inputs(cfg)
    t = {k: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to(dev) for k, v in raw.items()}
    wv = {k: t[f"vis.{k}"] for k in wl.STREAM_WEIGHTS}
    wc = {k: t[f"cond.{k}"] for k in wl.STREAM_WEIGHTS}
    act_dt = torch.float16 if args.act_dtype == "f16" else torch.bfloat16
    # With f16 operands the four GEMM matrices are converted to f16 once, at load, as a
    # deployment stores them (the block then reads them as given); `per_call_conversion`
    # below times the same step with the bf16 matrices converted inside every call.
    dims_bf = mm.BlockDims.make(cfg.width, cfg.heads, cfg.ffn, cfg.t_dim, cfg.ln_eps, cfg.qk_eps, act_dtype=act_dt)
    if act_dt == torch.float16:
        conv = lambda w: {k: (mm.cast(v, torch.float16) if k in mm.MATRIX_KEYS else v) for k, v in w.items()}  # noqa: E731
        wv_bf, wc_bf = wv, wc
        wv, wc = conv(wv), conv(wc)
        dims = mm.BlockDims.make(cfg.width, cfg.heads, cfg.ffn, cfg.t_dim, cfg.ln_eps, cfg.qk_eps,
                                 act_dtype=act_dt, matrix_dtype=torch.float16)
    else:
        wv_bf, wc_bf, dims = wv, wc, dims_bf
    rope = mm.Rope3D.make(cfg.grid, cfg.rope_split, cfg.rope_base)
    ws = torch.empty(mm.block_workspace_bytes(dims_bf, 1, cfg.n_vis, cfg.n_cond), dtype=torch.uint8, device=dev)
    out_v = torch.empty((1, cfg.n_vis, cfg.width), dtype=torch.float32, device=dev)
    out_c = torch.empty((1, cfg.n_cond, cfg.width), dtype=torch.float32, device=dev)

    hip = Hip()
    nst = mm.STAGE_COUNT
    events = [[hip.event() for _ in range(2 * nst)] for _ in range(args.steps)]

    def step(evs=None):
        mm.block_fwd(dims, wv, wc, t["x_vis"], t["x_cond"], t["tvec"], rope, workspace=ws,
                     out_vis=out_v, out_cond=out_c, stage_events=evs)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_ms = {name: [] for name in mm.STAGES}
    for evs in events:
        for si, name in enumerate(mm.STAGES):
            stage_ms[name].append(hip.elapsed_ms(evs[2 * si], evs[2 * si + 1]))
    step_gpu_ms = [hip.elapsed_ms(evs[0], evs[-1]) for evs in events]
    for evs in events:
        for e in evs:
            hip.destroy(e)
    ms_per_step = wall * 1e3 / args.steps
    stage_avg = {k: float(np.mean(v)) for k, v in stage_ms.items()}
    attn_ms = stage_avg["attention"]
    attn_tflops = cfg.attn_flops / (attn_ms * 1e-3) / 1e12
    tokens_s = cfg.n_tokens / (ms_per_step * 1e-3)
    log(f"{ms_per_step:.3f} ms/step, attention {attn_ms:.3f} ms = {attn_tflops:.1f} TFLOP/s")

    res = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.act_dtype,
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights; no checkpoint)",
        "config": {"workload": "480p MMDiT block forward: 32760 visual (21x30x52) + 512 conditioning tokens, "
                               "C=3072, 24x128 heads, FFN 12288 GELU, Dt=1536",
                   "global_batch": 1, "seq_len": cfg.n_tokens, "parallelism": "none (1 GPU)",
                   "inputs_and_weights": "bf16" + ("; the four GEMM matrices converted once to f16 at load"
                                                    if act_dt == torch.float16 else ""),
                   "mfma_operands": args.act_dtype,
                   "accumulate": "f32", "output_dtype": "f32"},
        "roofline": {"bound": "mfma", "kernel": "joint_attn_mfma_kernel (+ joint_attn_merge_kernel of its split tail)",
                     "achieved": round(attn_tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": attention_traffic_bytes(),
                     "flops_per_launch": cfg.attn_flops, "avg_launch_ms": round(attn_ms, 4)},
        "joint_attention": {"tflops": round(attn_tflops, 1), "frac_bf16_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                            "ms": round(attn_ms, 4), "tokens": cfg.n_tokens},
        "block_tflops": round(cfg.total_flops / (ms_per_step * 1e-3) / 1e12, 1),
        "stages_ms": {k: round(v, 4) for k, v in stage_avg.items()},
        "step_gpu_ms": round(float(np.mean(step_gpu_ms)), 4),
    }
    # the same step with bf16 matrices converted to f16 inside every call
    def step_bf():
        mm.block_fwd(dims_bf, wv_bf, wc_bf, t["x_vis"], t["x_cond"], t["tvec"], rope, workspace=ws,
                     out_vis=out_v, out_cond=out_c)
    step_bf()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(5):
        step_bf()
    torch.cuda.synchronize()
    res["per_call_conversion"] = {"ms_per_step": round((time.perf_counter() - t1) * 1e3 / 5, 4),
                                  "note": "bf16 GEMM matrices converted to f16 inside every call (5 steps)"}
    # memory-bound stages of the step, from the same events (algorithmic bytes of both streams)
    n_tok = cfg.n_tokens
    stage_bytes = {"qk_norm_rope": 4 * n_tok * cfg.width * 2,                    # q, k read + written (f16)
                   "ln2": n_tok * cfg.width * (4 + 2)}                             # x1 f32 -> h2 f16
    res["memory_bound_stages"] = {
        k: {"ms": round(stage_avg[k], 4), "bytes": b, "GB_per_s": round(b / stage_avg[k] / 1e6, 1),
            "frac_hbm": round(b / stage_avg[k] / 1e6 / PEAK_HBM_GBS, 4)} for k, b in stage_bytes.items()}
    if not args.no_configs:
        log("attention workloads (40 to 76112 tokens) and memory-bound kernels alone")
        res["attention_configs"] = attention_configs(dev)
        res["memory_bound_kernels"] = memory_bound_kernels(dev)
    if not args.no_next:
        log("timestep path and Lite merge / unpatchify")
        res["next_rows"] = next_rows(dev) if args.next == "all" else {}
        log("8-bit block at 480p")
        del ws
        res["next_rows"]["block_8bit_480p"] = block_8bit(cfg, wv_bf, wc_bf, t, rope, hip)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on this host)")
        res["cpu_baseline"] = cpu_baseline(cfg, raw)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
