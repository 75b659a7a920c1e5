#!/usr/bin/env python3
"""Benchmark of the gfx950 decoder-layer library on one MI355X.

Headline: LLaMA-7B-shape single-layer prefill (B=1, T=2048, d=4096, 32 heads
x 128, f=11008, bf16 with fp32 accumulation), tokens/s of the whole layer.
One step = one full layer call (RMSNorm, QKV + RoPE + cache append, causal
attention, o_proj + residual, RMSNorm, gate/up + SwiGLU, down + residual)
over the batch; inputs and weights are resident in HBM before timing starts.

Also reported on the same line:
  roofline      the dominant kernel (gate/up projection + SwiGLU, 43% of the
                layer's flops): algorithmic flops / its average duration,
                timed live with HIP events on the library's stream during the
                timed steps, against the 2.5 PFLOP/s dense bf16 MFMA peak;
                layer_mfma_frac is the whole layer call's fraction;
  layer.step_roofline, decode.step_roofline
                every step of the per-step breakdown against its own
                roofline (flops against the bf16 peak for the projections
                and the prefill attention, HBM bytes against 8 TB/s for the
                norms, the decode attention and the decode projections);
  decode        LLaMA-7B-shape decode step (32 sequences at position 4095):
                algorithmic bytes / step time against 8 TB/s HBM, with the
                oracle's rate on a sample of it (decode.cpu_baseline);
  decode_paged  the same step over a paged KV cache (pages of 64 slots in
                shuffled order);
  decode_int8   the same step over the int8 KV cache (codes and one fp32
                scale per row; its own algorithmic bytes);
  decode_paged_int8
                the same over int8 page pools;
  prefill_int8  the headline prefill writing and reading the int8 KV cache
                (the chunk's rows quantized into their slots; attention over
                code * scale);
  other_configs the 7B shape with bidirectional attention, the 13B-shape
                prefill, the 70B-shape GQA prefill and its 64 decode steps,
                the same two at one GPU's share of the 70B layer under 8-way
                tensor parallelism, the 7B shape over chunks of 128 and 512
                tokens, and greedy generation with a 32-layer 7B-shape stack;
  cpu_baseline  the CPU oracle on a bounded prefix of the same prefill
                workload, on this host's cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--headline-only]
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

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_flops(wl, T, B, bidirectional=False):
    """2 N P_lin + causal attention 4 dh H sum_t (t + 1) (positions 0..T-1);
    bidirectional: every token sees all T slots, 4 dh H T^2 per sequence."""
    d, H, Hkv, dh, f = wl.d_model, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.d_ff
    p_lin = d * (H + 2 * Hkv) * dh + H * dh * d + 3 * d * f
    attn = 4 * dh * H * B * (T * T if bidirectional else T * (T + 1) // 2)
    return 2 * B * T * p_lin + attn


def decode_bytes(wl, B, pos):
    """Weights and gains once, every sequence's prior K/V, the appended K/V,
    x in and y out (bf16)."""
    d, H, Hkv, dh, f = wl.d_model, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.d_ff
    es = 2
    p_lin = d * (H + 2 * Hkv) * dh + H * dh * d + 3 * d * f
    return es * (p_lin + 2 * d) + es * B * 2 * Hkv * dh * pos + es * B * 2 * Hkv * dh + 2 * es * B * d


def step_rooflines(wl, B, T, step_ms, pos=None):
    """Each step of the per-step breakdown against its own roofline: the
    projections and the prefill attention in algorithmic flops against the
    bf16 peak, the RMSNorms and the decode attention in algorithmic HBM
    bytes against 8 TB/s; weight-streaming (decode) projections in weight
    bytes.  Times are the event-timed steps, each with its launch gap.
    Prefill: T tokens at positions 0..T-1 per sequence; decode (pos given):
    one token per sequence at position pos."""
    d, H, Hkv, dh, f = wl.d_model, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.d_ff
    M, es = B * T, 2
    nqkv = (H + 2 * Hkv) * dh
    if pos is None:
        work = {
            "rmsnorm_attn": ("GB/s", es * (2 * M * d + d)),
            "qkv_rope_cache": ("TFLOP/s", 2 * M * nqkv * d),
            "attention": ("TFLOP/s", 4 * dh * H * B * (T * (T + 1) // 2)),
            "o_proj_residual": ("TFLOP/s", 2 * M * d * H * dh),
            "rmsnorm_mlp": ("GB/s", 4 * M * d + es * (M * d + d)),
            "gate_up_swiglu": ("TFLOP/s", 2 * M * 2 * f * d),
            "down_residual": ("TFLOP/s", 2 * M * d * f),
        }
    else:
        work = {
            "rmsnorm_attn": ("GB/s", es * (2 * M * d + d)),
            "qkv_rope_cache": ("GB/s", es * nqkv * d),
            "attention": ("GB/s", es * B * 2 * Hkv * dh * (pos + 1)),
            "o_proj_residual": ("GB/s", es * d * H * dh),
            "rmsnorm_mlp": ("GB/s", 4 * M * d + es * (M * d + d)),
            "gate_up_swiglu": ("GB/s", es * 2 * f * d),
            "down_residual": ("GB/s", es * d * f),
        }
    out = {}
    for k, (unit, amount) in work.items():
        if k not in step_ms:
            continue
        t = step_ms[k] * 1e-3
        rate = amount / t / (1e12 if unit == "TFLOP/s" else 1e9)
        peak = PEAK_BF16_TFLOPS if unit == "TFLOP/s" else PEAK_HBM_GBPS
        out[k] = {"unit": unit, "achieved": rate, "frac": rate / peak}
    return out


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(kernel_src):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    p = os.path.join(PROFILES, "gate_up_swiglu_llama7b_prefill_pmc.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        prof = json.load(f)
    if prof.get("source_sha") != source_sha(kernel_src):
        return None
    return prof.get("traffic_bytes_per_launch")


def layer_config(lib, wl, max_tokens, bidirectional=False):
    return lib.make_config(wl.d_model, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.d_ff, wl.max_pos,
                           max_tokens, wl.dtype, wl.rms_eps, wl.rope_base, bidirectional=bidirectional)


GATE_UP_STEP = 5  # the library's step index of the gate/up projection


def ramp_clocks(call, seconds=0.3):
    """Untimed calls for a fixed wall time before the warmup steps: the GPU
    takes tens of milliseconds of sustained load to reach its working clocks,
    more than a handful of warmup steps provide."""
    import torch
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(4):
            call()
        torch.cuda.synchronize()


def per_step_breakdown(lib, layer, call, n):
    """Per-step times from a separate, untimed pass with events around every
    step (they add a few µs per step, so the timed steps do not use them)."""
    import torch
    lib.llama_layer_profile(layer.handle, True)
    for _ in range(n):
        call()
    torch.cuda.synchronize()
    step_ms, calls = lib.llama_layer_profile_read(layer.handle)
    lib.llama_layer_profile(layer.handle, False)
    return {k: v / calls for k, v in step_ms.items()}


def bench_prefill(lib, synth, steps, warmup):
    import torch
    wl = synth.WORKLOADS["llama7b_prefill"]
    B, T = wl.batch, wl.seq
    w = synth.make_weights(wl, "cuda")
    x = synth.make_x(wl, (B, T), device="cuda")
    pos = synth.prefill_positions(B, T, device="cuda")
    kc, vc = synth.make_cache(wl, "cuda")
    y = torch.empty_like(x)
    layer = lib.LlamaLayer(layer_config(lib, wl, B * T), w)
    ramp_clocks(lambda: layer.prefill(x, pos, kc, vc, y=y))
    for _ in range(warmup):
        layer.prefill(x, pos, kc, vc, y=y)
    torch.cuda.synchronize()
    # timed steps: HIP events bracket the gate/up kernel only (two per step),
    # so the rest of the layer runs as it does without measurement
    lib.llama_layer_profile(layer.handle, True, step=GATE_UP_STEP)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer.prefill(x, pos, kc, vc, y=y)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms, calls = lib.llama_layer_profile_read(layer.handle)
    assert calls == steps, (calls, steps)
    gu_ms = step_ms["gate_up_swiglu"] / calls
    avg = per_step_breakdown(lib, layer, lambda: layer.prefill(x, pos, kc, vc, y=y), max(5, steps // 2))
    host = {"w": w, "x": x, "pos": pos, "kc": kc, "vc": vc}
    layer.close()
    return wl, (t1 - t0), gu_ms, avg, host


def bench_prefill_int8(lib, synth, steps, warmup):
    """The headline prefill (a 2048-token prompt into an empty cache) over the
    int8 KV cache: wall time of back-to-back calls, like the headline."""
    import torch
    wl = synth.WORKLOADS["llama7b_prefill"]
    B, T = wl.batch, wl.seq
    w = synth.make_weights(wl, "cuda")
    x = synth.make_x(wl, (B, T), device="cuda")
    pos = synth.prefill_positions(B, T, device="cuda")
    shape = (B, wl.n_kv_heads, wl.max_pos, wl.head_dim)
    kq = torch.zeros(shape, dtype=torch.int8, device="cuda")
    vq = torch.zeros_like(kq)
    ks = torch.zeros(shape[:3], dtype=torch.float32, device="cuda")
    vs = torch.zeros_like(ks)
    y = torch.empty_like(x)
    layer = lib.LlamaLayer(layer_config(lib, wl, B * T), w)

    def call():
        layer.prefill_int8(x, pos, kq, vq, ks, vs, y=y)
    ramp_clocks(call)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    breakdown = per_step_breakdown(lib, layer, call, max(5, steps // 2))
    layer.close()
    flops = prefill_flops(wl, T, B)
    return {"workload": "llama7b_prefill, int8 KV cache (codes + one fp32 scale per row)", "batch": B,
            "seq_len": T, "ms_per_step": ms, "tokens_per_s": B * T / ms * 1e3,
            "tflops": flops / (ms * 1e-3) / 1e12, "mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "step_ms_by_kernel": breakdown}


def bench_decode(lib, synth, steps, warmup):
    import torch
    wl = synth.WORKLOADS["llama7b_decode"]
    B, p = wl.batch, wl.prior
    w = synth.make_weights(wl, "cuda")
    x = synth.make_x(wl, (B,), device="cuda")
    pos = torch.full((B,), p, dtype=torch.int32, device="cuda")
    kc, vc = synth.make_cache(wl, "cuda")
    y = torch.empty_like(x)
    layer = lib.LlamaLayer(layer_config(lib, wl, B), w)
    # evicts L2 and the Infinity Cache between steps by READING 512 MB: the
    # caches then hold clean lines, as after the other layers of a real decode
    # step (a write-based flush would leave dirty lines whose write-back the
    # next step's reads would pay for)
    flush = torch.ones(128 << 20, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    ramp_clocks(lambda: layer.decode(x, pos, kc, vc, y=y))
    for _ in range(warmup):
        layer.decode(x, pos, kc, vc, y=y)
    times = []
    for _ in range(steps):
        flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        layer.decode(x, pos, kc, vc, y=y)  # a repeated decode at one position is idempotent
        e1.record(stream)
        times.append((e0, e1))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in times)
    med = ms[len(ms) // 2]
    nbytes = decode_bytes(wl, B, p)

    def step():
        flush.sum()
        layer.decode(x, pos, kc, vc, y=y)
    breakdown = per_step_breakdown(lib, layer, step, max(5, steps // 2))
    layer.close()
    return {"workload": "llama7b_decode", "batch": B, "position": p, "ms_per_step_median": med,
            "bytes_per_step": nbytes, "GBps": nbytes / med / 1e6,
            "hbm_frac": nbytes / med / 1e6 / PEAK_HBM_GBPS, "tokens_per_s": B / med * 1e3,
            "cache_flush_between_steps": "512 MB read",
            "step_ms_by_kernel": breakdown,
            "step_ms_by_kernel_note": "separate untimed pass with HIP events around every step",
            "step_roofline": step_rooflines(wl, B, 1, breakdown, pos=p)}


def bench_decode_paged(lib, synth, steps, warmup, page=64, int8=False):
    """The 7B decode workload over a paged cache: the same K/V scattered into
    pages of `page` slots in shuffled order (a block table per sequence),
    timed like the contiguous decode (median of event-timed steps, caches
    evicted by a 512 MB read before each).  int8: the cache converted by
    llama_layer_kv_quantize first, then its codes and scales paged alike."""
    import torch
    wl = synth.WORKLOADS["llama7b_decode"]
    B, p, Hkv = wl.batch, wl.prior, wl.n_kv_heads
    w = synth.make_weights(wl, "cuda")
    x = synth.make_x(wl, (B,), device="cuda")
    pos = torch.full((B,), p, dtype=torch.int32, device="cuda")
    kc, vc = synth.make_cache(wl, "cuda")
    layer = lib.LlamaLayer(layer_config(lib, wl, B), w)
    if int8:
        kq = torch.empty(kc.shape, dtype=torch.int8, device="cuda")
        vq = torch.empty_like(kq)
        ks = torch.empty(kc.shape[:3], dtype=torch.float32, device="cuda")
        vs = torch.empty_like(ks)
        layer.kv_quantize(kc, vc, wl.max_pos, kq, vq, ks, vs)
        caches = [kq, vq, ks.unsqueeze(-1), vs.unsqueeze(-1)]  # scales page like rows of one element
    else:
        caches = [kc, vc]
    del kc, vc
    nb = wl.max_pos // page
    perm = torch.randperm(B * nb, generator=torch.Generator().manual_seed(11))
    bt = perm.view(B, nb).to(torch.int32).cuda()
    idx = bt.view(-1).long()
    pools = []
    for c in caches:
        e = c.shape[-1]
        pool = torch.empty(B * nb, Hkv, page, e, dtype=c.dtype, device="cuda")
        pool[idx] = c.reshape(B, Hkv, nb, page, e).transpose(1, 2).reshape(B * nb, Hkv, page, e)
        pools.append(pool if e > 1 else pool.squeeze(-1).contiguous())
    del caches
    torch.cuda.synchronize()
    y = torch.empty_like(x)
    if int8:
        def call():
            layer.decode_paged_int8(x, pos, *pools, bt, y=y)
    else:
        def call():
            layer.decode_paged(x, pos, *pools, bt, y=y)
    flush = torch.ones(128 << 20, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    ramp_clocks(call)
    for _ in range(warmup):
        call()
    times = []
    for _ in range(steps):
        flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()  # a repeated decode at one position is idempotent
        e1.record(stream)
        times.append((e0, e1))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in times)
    med = ms[len(ms) // 2]
    nbytes = decode_int8_bytes(wl, B, p) if int8 else decode_bytes(wl, B, p)
    layer.close()
    return {"workload": "llama7b_decode, paged " + ("int8 KV cache" if int8 else "KV cache"), "page_slots": page,
            "pages": B * nb, "batch": B, "position": p, "ms_per_step_median": med, "bytes_per_step": nbytes,
            "GBps": nbytes / med / 1e6, "hbm_frac": nbytes / med / 1e6 / PEAK_HBM_GBPS,
            "tokens_per_s": B / med * 1e3}


def decode_int8_bytes(wl, B, pos):
    """As decode_bytes with the int8 cache: the prior K/V as int8 codes plus
    a 4-byte scale per row, the appended rows likewise."""
    d, H, Hkv, dh, f = wl.d_model, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.d_ff
    es = 2
    p_lin = d * (H + 2 * Hkv) * dh + H * dh * d + 3 * d * f
    rows = B * 2 * Hkv * (pos + 1)
    return es * (p_lin + 2 * d) + rows * (dh + 4) + 2 * es * B * d


def bench_decode_int8(lib, synth, steps, warmup):
    """The 7B decode workload over the int8 cache: the same random bf16 cache
    converted by llama_layer_kv_quantize, then the step timed like the
    contiguous decode (median of event-timed steps, caches evicted by a
    512 MB read before each)."""
    import torch
    wl = synth.WORKLOADS["llama7b_decode"]
    B, p = wl.batch, wl.prior
    w = synth.make_weights(wl, "cuda")
    x = synth.make_x(wl, (B,), device="cuda")
    pos = torch.full((B,), p, dtype=torch.int32, device="cuda")
    kc, vc = synth.make_cache(wl, "cuda")
    kq = torch.empty(kc.shape, dtype=torch.int8, device="cuda")
    vq = torch.empty_like(kq)
    ks = torch.empty(kc.shape[:3], dtype=torch.float32, device="cuda")
    vs = torch.empty_like(ks)
    y = torch.empty_like(x)
    layer = lib.LlamaLayer(layer_config(lib, wl, B), w)
    layer.kv_quantize(kc, vc, wl.max_pos, kq, vq, ks, vs)
    del kc, vc
    flush = torch.ones(128 << 20, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    ramp_clocks(lambda: layer.decode_int8(x, pos, kq, vq, ks, vs, y=y))
    for _ in range(warmup):
        layer.decode_int8(x, pos, kq, vq, ks, vs, y=y)
    times = []
    for _ in range(steps):
        flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        layer.decode_int8(x, pos, kq, vq, ks, vs, y=y)  # a repeated decode at one position is idempotent
        e1.record(stream)
        times.append((e0, e1))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in times)
    med = ms[len(ms) // 2]
    nbytes = decode_int8_bytes(wl, B, p)

    def step():
        flush.sum()
        layer.decode_int8(x, pos, kq, vq, ks, vs, y=y)
    breakdown = per_step_breakdown(lib, layer, step, max(5, steps // 2))
    layer.close()
    return {"workload": "llama7b_decode, int8 KV cache (codes + one fp32 scale per row)", "batch": B,
            "position": p, "ms_per_step_median": med, "bytes_per_step": nbytes, "GBps": nbytes / med / 1e6,
            "hbm_frac": nbytes / med / 1e6 / PEAK_HBM_GBPS, "tokens_per_s": B / med * 1e3,
            "step_ms_by_kernel": breakdown}


def measure_ceilings(lib, runs=5):
    """What this GPU sustains, measured by the library's ceiling kernels: a
    register-only MFMA loop (dense bf16) and a one-pass 2 GiB streaming read,
    each the median of `runs` event-timed launches after a warm-up."""
    import torch
    stream = torch.cuda.current_stream()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    def timed(launch):
        launch()
        torch.cuda.synchronize()
        ms = []
        for _ in range(runs):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            out = launch()
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return sorted(ms)[len(ms) // 2], out

    mfma_ms, flops = timed(lambda: lib.llama_layer_ceiling_mfma(40000, sink))
    buf = torch.arange(1 << 28, dtype=torch.int64, device="cuda")  # 2 GiB of distinct values
    read_ms, _ = timed(lambda: lib.llama_layer_ceiling_read(buf, sink))
    nbytes = buf.numel() * buf.element_size()
    del buf
    return {"mfma_loop_tflops": flops / (mfma_ms * 1e-3) / 1e12, "mfma_loop_ms": mfma_ms,
            "stream_read_GBps": nbytes / (read_ms * 1e-3) / 1e9, "stream_read_bytes": nbytes,
            "stream_read_ms": read_ms}


def bench_other_configs(lib, synth, steps, warmup):
    """The other layer shapes, timed the same way (not the headline): the 7B
    shape with bidirectional attention (the encoder-style variant), 13B-shape
    prefill (2 x 4096 tokens), 70B-shape GQA prefill (4096 tokens) and the 64
    single-token decode steps that follow it (positions 4096..4159; caches
    evicted by a 512 MB read before each step, as for the 7B decode), and the
    same two at one GPU's share of the 70B layer under 8-way tensor
    parallelism (the all-reduces after o_proj and down are not part of it)."""
    import torch
    res = {}
    flush = torch.ones(128 << 20, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    keys = {"llama70b_gqa": ("llama70b_gqa_prefill", "llama70b_gqa_decode"),
            "llama70b_tp8_shard": ("llama70b_tp8_shard_prefill", "llama70b_tp8_shard_decode")}
    for name in ("llama7b_prefill_bidirectional", "llama13b_prefill", "llama70b_gqa", "llama70b_tp8_shard"):
        bidir = name.endswith("_bidirectional")
        wl = synth.WORKLOADS[name.replace("_bidirectional", "")]
        B, T = wl.batch, wl.seq
        w = synth.make_weights(wl, "cuda")
        x = synth.make_x(wl, (B, T), device="cuda")
        pos = synth.prefill_positions(B, T, device="cuda")
        kc, vc = synth.make_cache(wl, "cuda")
        y = torch.empty_like(x)
        layer = lib.LlamaLayer(layer_config(lib, wl, B * T, bidirectional=bidir), w)
        for _ in range(warmup):
            layer.prefill(x, pos, kc, vc, y=y)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            layer.prefill(x, pos, kc, vc, y=y)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / steps * 1e3
        tfl = prefill_flops(wl, T, B, bidir) / (ms * 1e-3) / 1e12
        res[keys.get(name, (name,))[0]] = {
            "batch": B, "seq_len": T, "ms_per_step": ms, "tokens_per_s": B * T / ms * 1e3,
            "tflops": tfl, "mfma_frac": tfl / PEAK_BF16_TFLOPS,
            "step_ms_by_kernel": per_step_breakdown(lib, layer, lambda: layer.prefill(x, pos, kc, vc, y=y), 3)}
        log(f"{name}: prefill {ms:.3f} ms/step")
        layer.close()
        if wl.decode_steps:
            # the decode steps continue the cache the prefill just wrote
            layer = lib.LlamaLayer(layer_config(lib, wl, B), w)
            xs = [synth.make_x(wl, (B,), tensor_id=100 + s, device="cuda") for s in range(wl.decode_steps)]
            yd = torch.empty_like(xs[0])
            times, nbytes = [], 0
            for s, xd in enumerate(xs):
                p = T + s
                pd = torch.full((B,), p, dtype=torch.int32, device="cuda")
                flush.sum()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                layer.decode(xd, pd, kc, vc, y=yd)
                e1.record(stream)
                times.append((e0, e1))
                nbytes += decode_bytes(wl, B, p)
            torch.cuda.synchronize()
            ms_all = [a.elapsed_time(b) for a, b in times]
            tot = sum(ms_all)
            med = sorted(ms_all)[len(ms_all) // 2]
            res[keys[name][1]] = {
                "batch": B, "positions": [T, T + wl.decode_steps - 1], "steps": wl.decode_steps,
                "ms_per_step_median": med, "GBps": nbytes / tot / 1e6,
                "hbm_frac": nbytes / tot / 1e6 / PEAK_HBM_GBPS}
            log(f"{name}: decode median {med:.3f} ms/step")
            layer.close()
    return res


def bench_prefill_chunks(lib, synth, steps, warmup, sizes=(128, 512)):
    """The 7B-shape layer over short chunks of tokens (one sequence at
    positions 0..T-1), where the tiled GEMMs have fewer tiles than CUs and
    split K: wall time of back-to-back calls."""
    import dataclasses
    import torch
    res = {}
    for T in sizes:
        wl = dataclasses.replace(synth.WORKLOADS["llama7b_prefill"], seq=T)
        w = synth.make_weights(wl, "cuda")
        x = synth.make_x(wl, (1, T), device="cuda")
        pos = synth.prefill_positions(1, T, device="cuda")
        kc, vc = synth.make_cache(wl, "cuda")
        y = torch.empty_like(x)
        layer = lib.LlamaLayer(layer_config(lib, wl, T), w)
        for _ in range(warmup):
            layer.prefill(x, pos, kc, vc, y=y)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            layer.prefill(x, pos, kc, vc, y=y)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / steps * 1e3
        tfl = prefill_flops(wl, T, 1) / (ms * 1e-3) / 1e12
        res[f"llama7b_prefill_{T}"] = {"batch": 1, "seq_len": T, "ms_per_step": ms, "tokens_per_s": T / ms * 1e3,
                                       "tflops": tfl, "mfma_frac": tfl / PEAK_BF16_TFLOPS}
        layer.close()
    return res


def bench_generate(lib, synth, n_layers=32, vocab=32000, B=32, T=128, max_new=64):
    """Greedy generation with a 7B-shape stack (32 layers, LLaMA's 32000-token
    vocabulary, random weights): B prompts of T tokens, then max_new tokens
    each through the library's native loop (sampling, EOS bookkeeping and a
    host sync per step included).  Decode rate = tokens generated / (loop
    time - prefill time); bytes per decode step = every layer's weights and
    gains + the LM head + the K/V read at the mean position."""
    import dataclasses

    import numpy as np
    import torch
    wl = dataclasses.replace(synth.WORKLOADS["llama7b_prefill"], batch=B, seq=T, decode_steps=max_new)
    mw = synth.make_model_weights(wl, n_layers, vocab, "cuda")
    cfg = layer_config(lib, wl, B * T)
    model = lib.LlamaModel(cfg, n_layers, vocab, mw["embed"], mw["final_norm"], mw["lm_head"], mw["layers"])
    del mw
    kc = [torch.zeros(B, wl.n_kv_heads, wl.max_pos, wl.head_dim, dtype=torch.bfloat16, device="cuda")
          for _ in range(n_layers)]
    vc = [torch.zeros_like(k) for k in kc]
    rng = np.random.default_rng(5)
    prompt = rng.integers(0, vocab, size=(B, T)).astype(np.int32)
    ids = torch.tensor(prompt, device="cuda")
    sp = lib.make_sampling()
    model.generate(prompt, 4, sp, kc, vc)  # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(3):
        model.prefill(ids, kc, vc)
    torch.cuda.synchronize()
    pre_ms = (time.perf_counter() - t0) / 3 * 1e3
    t0 = time.perf_counter()
    out = model.generate(prompt, max_new, sp, kc, vc)
    gen_ms = (time.perf_counter() - t0) * 1e3
    n_tok = sum(len(o) for o in out)
    step_ms = (gen_ms - pre_ms) / max_new
    d = wl.d_model
    p_layer = d * (wl.n_heads + 2 * wl.n_kv_heads) * wl.head_dim + wl.n_heads * wl.head_dim * d + 3 * d * wl.d_ff
    kv = 2 * 2 * B * wl.n_kv_heads * wl.head_dim * (T + max_new / 2) * n_layers
    step_bytes = 2 * (n_layers * (p_layer + 2 * d) + vocab * d + d) + kv
    model.close()
    log(f"generate: prefill {pre_ms:.2f} ms, {max_new} steps {gen_ms - pre_ms:.1f} ms")
    return {"layers": n_layers, "vocab": vocab, "batch": B, "prompt": T, "new_tokens": max_new,
            "sampling": "greedy", "prefill_ms": pre_ms, "decode_step_ms": step_ms,
            "decode_tokens_per_s": n_tok / ((gen_ms - pre_ms) * 1e-3),
            "decode_GBps": step_bytes / (step_ms * 1e-3) / 1e9,
            "decode_hbm_frac": step_bytes / (step_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS}


def cpu_baseline(wl, host, budget_s):
    """The oracle as it stands (plain fp64 numpy) on a prefix of the same layer
    call: tokens 0..T'-1 of the sequence, T' doubled from 64 until one run takes
    a third of the budget (causal, so these are exactly the first T' outputs)."""
    import numpy as np
    from oracle import llama_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        cores = os.cpu_count()
    f64 = lambda t: t.detach().cpu().double().numpy()  # noqa: E731
    w64 = {k: f64(v) for k, v in host["w"].items()}
    x, pos, kc, vc = f64(host["x"]), f64(host["pos"]).astype(np.int64), host["kc"], host["vc"]
    kc0 = np.zeros(tuple(kc.shape))
    tp, last = 64, None
    while True:
        t0 = time.perf_counter()
        O.decoder_layer(x[:, :tp], pos[:, :tp], w64, kc0, kc0, n_heads=wl.n_heads,
                        n_kv_heads=wl.n_kv_heads, eps=wl.rms_eps, rope_base=wl.rope_base)
        dt = time.perf_counter() - t0
        last = (tp, dt)
        log(f"cpu oracle: {tp} tokens in {dt:.2f} s")
        if dt >= budget_s / 3 or tp >= wl.seq:
            break
        tp = min(wl.seq, tp * 2)
    tp, dt = last
    # the same oracle limited to one thread, on a prefix sized the same way
    one = None
    try:
        from threadpoolctl import threadpool_limits
        t1 = 64
        with threadpool_limits(limits=1):
            while True:
                t0 = time.perf_counter()
                O.decoder_layer(x[:, :t1], pos[:, :t1], w64, kc0, kc0, n_heads=wl.n_heads,
                                n_kv_heads=wl.n_kv_heads, eps=wl.rms_eps, rope_base=wl.rope_base)
                d1 = time.perf_counter() - t0
                log(f"cpu oracle, 1 thread: {t1} tokens in {d1:.2f} s")
                if d1 >= budget_s / 6 or t1 >= tp:
                    break
                t1 = min(tp, t1 * 2)
        one = {"value": wl.batch * t1 / d1, "unit": "tokens/s", "cores": 1,
               "sample": f"first {t1} tokens, {d1:.2f} s"}
    except ImportError:
        pass
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": wl.batch * tp / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {tp} of the {wl.seq} tokens of the llama7b_prefill layer call, plain "
                      f"fp64 numpy oracle, {dt:.2f} s",
            "host_cpu": cpu, "host_logical_cpus": os.cpu_count(), "one_thread": one}


def cpu_baseline_decode(budget_s):
    """The oracle as it stands on a bounded sample of the 7B decode workload:
    the first k of its 32 sequences (k doubled from 1 until one run takes a
    third of the budget), each at position 4095 over its 4095 prior slots.
    Reported as effective GB/s over the algorithmic bytes of that sample
    (weights and gains once, the k sequences' prior K/V, appended K/V, x and y)."""
    import numpy as np
    import torch
    import synth
    from oracle import llama_oracle as O
    wl = synth.WORKLOADS["llama7b_decode"]
    p = wl.prior
    w = synth.make_weights(wl, "cuda")
    w64 = {k: v.detach().cpu().double().numpy() for k, v in w.items()}
    del w
    x = synth.make_x(wl, (wl.batch,), device="cuda").cpu().double().numpy()
    kc, vc = synth.make_cache(wl, "cuda")
    k, last = 1, None
    while True:
        k64 = kc[:k].cpu().double().numpy()
        v64 = vc[:k].cpu().double().numpy()
        t0 = time.perf_counter()
        O.decoder_layer_decode(x[:k], np.full(k, p), w64, k64, v64, n_heads=wl.n_heads, n_kv_heads=wl.n_kv_heads)
        dt = time.perf_counter() - t0
        last = (k, dt)
        log(f"cpu oracle decode: {k} sequences in {dt:.2f} s")
        if dt >= budget_s / 3 or k >= wl.batch:
            break
        k = min(wl.batch, 2 * k)
    k, dt = last
    nbytes = decode_bytes(wl, k, p)
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"first {k} of the 32 sequences of the llama7b_decode step (position 4095), plain fp64 "
                      f"numpy oracle, {dt:.2f} s; bytes = weights + those sequences' K/V + x, y"}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max((i.get("num_threads", 1) for i in threadpool_info()), default=1))
    except Exception:
        return os.cpu_count()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=30.0)
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the other configs (13B prefill, 70B GQA prefill + 64 decode steps, the "
                         "bidirectional variant, the generation stack, the paged and int8 decode)")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="keep the paged and int8 decode, skip the other configs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}): this library "
              "is a single-GPU decoder layer and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": 1 << 30, "launches": 3}))
        return

    import llama_decoder_block_amd as lib
    import synth

    wl, elapsed, gu_ms, step_avg, host = bench_prefill(lib, synth, args.steps, args.warmup)
    B, T = wl.batch, wl.seq
    ms_per_step = elapsed / args.steps * 1e3
    tokens_per_s = B * T * args.steps / elapsed
    flops = prefill_flops(wl, T, B)
    gu_flops = 2 * B * T * (2 * wl.d_ff) * wl.d_model
    gu_tflops = gu_flops / (gu_ms * 1e-3) / 1e12
    kernel_src = os.path.join(ROOT, "llama_decoder_block_amd", "csrc", "gemm.hip")
    out = {
        "metric": "decoder-layer tokens/s (7B-shape prefill) + decode GB/s; % MFMA/HBM roofline",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights)",
        "config": {"workload": "llama7b_prefill", "global_batch": B, "seq_len": T,
                   "d_model": wl.d_model, "n_heads": wl.n_heads, "n_kv_heads": wl.n_kv_heads,
                   "head_dim": wl.head_dim, "d_ff": wl.d_ff, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "gate_up_swiglu (gemm_kernel<128, 512, EPI_SWIGLU>)",
                     "achieved": gu_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": gu_tflops / PEAK_BF16_TFLOPS,
                     "traffic": traffic_from_profile(kernel_src),
                     "flops_per_launch": gu_flops, "avg_launch_ms": gu_ms,
                     "layer_mfma_frac": flops / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                     "note": "achieved/frac: the dominant kernel (gate/up + SwiGLU, 43% of the layer's flops); "
                             "layer_mfma_frac: the whole layer call's algorithmic flops / its wall time"},
        "layer": {"flops_per_step": flops, "tflops": flops / (ms_per_step * 1e-3) / 1e12,
                  "mfma_frac": flops / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                  "step_ms_by_kernel": step_avg,
                  "step_ms_by_kernel_note": "separate untimed pass with HIP events around every step",
                  "step_roofline": step_rooflines(wl, B, T, step_avg)},
    }
    if not args.headline_only:
        out["prefill_int8"] = bench_prefill_int8(lib, synth, args.steps, args.warmup)
    if not args.no_decode:
        out["decode"] = bench_decode(lib, synth, args.decode_steps, 3)
        if not args.headline_only:
            out["decode_paged"] = bench_decode_paged(lib, synth, args.decode_steps, 3)
            out["decode_int8"] = bench_decode_int8(lib, synth, args.decode_steps, 3)
            out["decode_paged_int8"] = bench_decode_paged(lib, synth, args.decode_steps, 3, int8=True)
    # fractions of what this GPU sustains (the roofline above uses the published peaks)
    ceil = measure_ceilings(lib)
    ceil["prefill_layer_frac_of_mfma_loop"] = out["layer"]["tflops"] / ceil["mfma_loop_tflops"]
    ceil["gate_up_frac_of_mfma_loop"] = gu_tflops / ceil["mfma_loop_tflops"]
    if "decode" in out:
        ceil["decode_frac_of_stream_read"] = out["decode"]["GBps"] / ceil["stream_read_GBps"]
    out["ceilings"] = ceil
    if not args.headline_only and not args.no_other_configs:
        out["other_configs"] = bench_other_configs(lib, synth, max(3, args.steps // 4), 2)
        out["other_configs"].update(bench_prefill_chunks(lib, synth, 20, 5))
        out["other_configs"]["llama7b_generate"] = bench_generate(lib, synth)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, host, args.cpu_budget_s)
        if "decode" in out:
            out["decode"]["cpu_baseline"] = cpu_baseline_decode(args.cpu_budget_s / 2)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
