#!/usr/bin/env python3
"""Benchmark: one Wan-style video DiT denoise step on one MI355X.

Workload (default): the Wan2.1-1.3B-shaped text-to-video step at 480p x 81 frames --
latent [16, 21, 60, 104] -> 32760 tokens, dim 1536, 12 heads x 128, FFN 8960, 512 text
tokens, 32 blocks (the layer count the "图解 Wan2.1 I2V" page gives for 1.3B, §8).
A step = patchify -> patch embedding -> timestep embedding -> 32 blocks -> head ->
unpatchify -> flow-matching Euler update, all through libwan.so; inputs and weights
are resident in HBM before timing starts (context embedding and cross-attention K/V
are computed once per generation, outside the timed region).

Prints one JSON line with ms per step, the self-attention kernel's TFLOP/s against the
bf16 dense MFMA peak (timed with HIP events around that kernel inside the timed
region), a per-kernel breakdown (one extra untimed step) and the CPU oracle's time on
a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA (int8: 5.0 POP/s)
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
METRIC = "ms per DiT denoise step + attention TFLOP/s (% MFMA peak) at 32760 tokens"
BLOCK_COUNTERS_FILE = os.path.join(ROOT, "profiles", "block_kernels_counters.json")
CSRC = os.path.join(ROOT, "video_diffusion_transformer_step_amd", "csrc")
# which source file holds each block launch's kernel (its counters are stale once that file changes)
KERNEL_SOURCE = {"ln1": "norm.hip", "ln2": "norm.hip", "ln3": "norm.hip", "qk_rms": "norm.hip",
                 "attn_prologue": "layout.hip", "mod_combine": "layout.hip", "self_attn": "attention.hip",
                 "cross_attn": "attention.hip", "qkv_gemm": "gemm.hip", "o_gemm": "gemm.hip",
                 "cross_q_gemm": "gemm.hip", "cross_o_gemm": "gemm.hip", "ffn1_gemm": "gemm.hip",
                 "ffn2_gemm": "gemm.hip"}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def block_flops(c):
    """Algorithmic FLOPs of one block (2MNK per GEMM; 4 B S^2 dim for self-attention, the forward
    constant of the cost model on the "Wan 技术深度解析" page, §5.1)."""
    S, d, f, B = c.S, c.dim, c.ffn_dim, c.B
    gemm = 2 * B * S * d * (3 * d) + 2 * B * S * d * d * 3 + 2 * 2 * B * S * d * f
    attn = 4 * B * S * S * d
    cross = 4 * B * S * (c.text_len + c.img_len) * d
    return gemm + attn + cross, attn


def step_flops(c, layers):
    blk, attn = block_flops(c)
    S, d = c.S, c.dim
    extra = 2 * c.B * S * 4 * c.in_channels * d + 2 * c.B * S * d * 4 * c.out_channels
    return layers * blk + extra, attn


def device_block_tensors(c, gen, device="cuda"):
    """Random-init weights of one block, drawn on the device from a seeded generator:
    matrices and biases N(0, 0.02), norm gains 1 + N(0, 0.02)."""
    import torch
    bf = torch.bfloat16 if c.dtype == "bf16" else torch.float32
    d, f = c.dim, c.ffn_dim

    def n(*shape, dtype=torch.float32, mean=0.0):
        return (torch.randn(*shape, generator=gen, device=device) * 0.02 + mean).to(dtype).contiguous()

    g = {"wqkv": n(3 * d, d, dtype=bf), "bqkv": n(3 * d), "wo": n(d, d, dtype=bf), "wcq": n(d, d, dtype=bf),
         "wco": n(d, d, dtype=bf), "w1": n(f, d, dtype=bf), "w2": n(d, f, dtype=bf), "mod_bias": n(6, d),
         "gq": n(d, mean=1.0), "gk": n(d, mean=1.0), "bo": n(d), "ln3_w": n(d, mean=1.0), "ln3_b": n(d),
         "bcq": n(d), "bco": n(d), "b1": n(f), "b2": n(d), "wkv_txt": n(2 * d, d, dtype=bf),
         "bkv_txt": n(2 * d)}
    if c.img_len:
        g["wkv_img"] = n(2 * d, d, dtype=bf)
        g["bkv_img"] = n(2 * d)
    return g


def counters_traffic():
    """HBM bytes per launch of the self-attention kernel (copy-calibrated FETCH_SIZE + WRITE_SIZE) from
    the committed rocprofv3 reduction, only while the kernel source is the one the counters were taken
    on."""
    e = block_counters().get("self_attn")
    return None if e is None or "hbm_bytes" not in e else float(e["hbm_bytes"])


def block_counters():
    """Per-launch counter figures of the block's kernels from the committed rocprofv3 reduction
    (profiles/block_kernels_counters.json, written by video_diffusion_transformer_step_amd.counters), each
    kept only while its kernel's source file is the one the counters were taken on."""
    try:
        with open(BLOCK_COUNTERS_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return {}
    taken = rec.get("meta", {}).get("source_sha256", {})
    out = {}
    for label, e in rec.get("kernels", {}).items():
        src = KERNEL_SOURCE.get(label)
        if src is None or taken.get(src) is None:
            continue
        if hashlib.sha256(open(os.path.join(CSRC, src), "rb").read()).hexdigest() != taken[src]:
            continue
        out[label] = e
    return out


def measure_device():
    """Device ceilings measured beside the nominal ones: compute units and peak engine clock as the
    runtime reports them, the matrix-core rate of a kernel issuing only MFMAs on register operands
    (bf16 and E4M3 on constant operands, bf16 on hashed operands that toggle like real data), and the
    rate of a plain 1 GiB device-to-device copy."""
    import torch

    from video_diffusion_transformer_step_amd import _lib as L
    cus, khz = L.device_info()
    blocks = cus * 8
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    res = {"compute_units": cus, "clock_mhz": round(khz / 1e3, 1),
           "nominal_bf16_tflops": round(cus * khz * 1e3 * 4096 / 1e12, 1)}
    one = {0: 0x3F803F80, 1: 0x38383838}  # bf16 1.0 in both halves; E4M3 1.0 in every byte
    for kind, key, iters in ((0, "bf16", 4000), (1, "fp8_e4m3", 2000)):
        L.mfma_peak_probe(kind, one[kind], one[kind], blocks, 16, out)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        ev0.record()
        for _ in range(reps):
            flop = L.mfma_peak_probe(kind, one[kind], one[kind], blocks, iters, out)
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / reps
        expect = 64.0 * L.MFMA_PROBE_K[kind] * iters
        assert bool((out == expect).all()), f"MFMA probe ({key}) returned wrong sums"
        res[f"measured_{key}_tflops"] = round(flop / (ms * 1e-3) / 1e12, 1)
    # the same bf16 loop on operands that differ per lane and instruction (real data toggles operand
    # bits, which costs matrix-core power; constant operands toggle none)
    L.mfma_peak_probe(2, 0x9E3779B9, 0x7F4A7C15, blocks, 16, out)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(10):
        flop = L.mfma_peak_probe(2, 0x9E3779B9, 0x7F4A7C15, blocks, 4000, out)
    ev1.record()
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), "MFMA probe (bf16, hashed operands) returned non-finite sums"
    res["measured_bf16_random_operands_tflops"] = round(flop / (ev0.elapsed_time(ev1) / 10 * 1e-3) / 1e12, 1)
    res["sustained_mfma_clock_mhz"] = round(res["measured_bf16_tflops"] * 1e12 / (cus * 4096) / 1e6, 1)
    del out
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(5):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    res["copy_gbs"] = round(2 * 4 * n / (ev0.elapsed_time(ev1) / 5 * 1e-3) / 1e9, 1)
    del src, dst
    return res


def measure_sharded(c, ulysses=4, ring=8, reps=10):
    """One GPU's share of the sequence-parallel self-attention on this workload, timed with events:
    Ulysses over `ulysses` GPUs (every token, heads / ulysses heads: the unchanged kernel on a head
    shard), one ring step over `ring` GPUs (an S / ring query shard against one S / ring key/value
    shard, with its log-sum-exp, via wan_attention_partial_fwd, which also transposes the chunk's V),
    and the exact merge of `ring` such partial results (wan_attention_lse_merge)."""
    import torch

    from video_diffusion_transformer_step_amd import _lib as L
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    bf, hd, S = torch.bfloat16, c.head_dim, c.S

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(reps):
            fn()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / reps

    out = {}
    hs = c.heads // ulysses
    q, k, v = (torch.randn(c.B, S, hs, hd, generator=gen, device="cuda").to(bf) for _ in range(3))
    o = torch.empty_like(q)
    ws = torch.empty(L.attention_partial_ws_bytes(L.WAN_BF16, c.B, S, S, hs, hd), dtype=torch.uint8, device="cuda")
    ms = timed(lambda: L.attention_partial_fwd(q, k, v, o, None, ws))
    fl = 4 * c.B * S * S * hs * hd
    out["ulysses_shard"] = {"gpus": ulysses, "heads": hs, "tokens": S, "ms": round(ms, 4),
                            "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                            "frac_of_bf16_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del q, k, v, o, ws
    Sr = (S + ring - 1) // ring
    q, k, v = (torch.randn(c.B, Sr, c.heads, hd, generator=gen, device="cuda").to(bf) for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty(c.B, c.heads, Sr, dtype=torch.float32, device="cuda")
    ws = torch.empty(L.attention_partial_ws_bytes(L.WAN_BF16, c.B, Sr, Sr, c.heads, hd), dtype=torch.uint8,
                     device="cuda")
    ms = timed(lambda: L.attention_partial_fwd(q, k, v, o, lse, ws))
    fl = 4 * c.B * Sr * Sr * c.heads * hd
    out["ring_step"] = {"gpus": ring, "q_tokens": Sr, "kv_tokens": Sr, "heads": c.heads, "ms": round(ms, 4),
                        "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                        "frac_of_bf16_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                        "ring_ms_per_block": round(ms * ring, 3)}
    o_parts = [torch.randn(c.B, Sr, c.heads, hd, generator=gen, device="cuda").to(bf) for _ in range(ring)]
    l_parts = [torch.randn(c.B, c.heads, Sr, generator=gen, device="cuda") for _ in range(ring)]
    ms = timed(lambda: L.attention_lse_merge(o_parts, l_parts, o, lse))
    nbytes = (ring + 1) * c.B * Sr * c.heads * (hd * 2 + 4)
    out["lse_merge"] = {"parts": ring, "tokens": Sr, "ms": round(ms, 4),
                        "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                        "frac_of_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)}
    out["note"] = ("the shard kernels on one GPU at the shapes each GPU would run; no collective is timed "
                   "(ring_ms_per_block = ring steps x one step, without the merge or the K/V exchange)")
    return out


def measure_attention_720p(reps=3):
    """The 720p self-attention stress workload: latent [16, 21, 90, 160] -> 21 x 45 x 80 = 75600 tokens,
    40 heads x 128, q, k, v ~N(0,1) bf16, 3D RoPE on q and k.  One wan_attention_fwd call (RoPE on q and k,
    V transposed into the workspace, the attention kernel) timed with events on the stream it runs on;
    FLOPs 4 S^2 dim."""
    import torch

    import wan_inputs as wi
    from video_diffusion_transformer_step_amd import _lib as L
    c = wi.get_config("attn-720p")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(720)
    q, k, v = (torch.randn(1, c.S, c.heads, c.head_dim, generator=gen, device="cuda").to(torch.bfloat16)
               for _ in range(3))
    o = torch.empty_like(q)
    ws = torch.empty(L.attention_ws_bytes(L.WAN_BF16, c.grid, 1, c.heads, c.head_dim), dtype=torch.uint8,
                     device="cuda")
    L.attention_fwd(q, k, v, c.grid, o, ws)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        L.attention_fwd(q, k, v, c.grid, o, ws)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / reps
    assert bool(torch.isfinite(o).all()), "non-finite 720p attention output"
    fl = 4 * c.S * c.S * c.heads * c.head_dim
    tf = fl / (ms * 1e-3) / 1e12
    del q, k, v, o, ws
    torch.cuda.empty_cache()
    return {"workload": f"{c.name}: [1, {c.S}, {c.heads}, {c.head_dim}] bf16, 3D RoPE on grid {c.grid}",
            "ms": round(ms, 3), "tflops": round(tf, 1), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "flops": fl, "bound_ms_at_half_peak": round(fl / (0.5 * PEAK_BF16_TFLOPS * 1e12) * 1e3, 1),
            "note": "whole wan_attention_fwd call (RoPE pass on q and k, V transpose, attention) per launch"}


def measure_other_step(name, steps, warmup, seed=5):
    """A whole denoise-step workload other than the headline one, on device-drawn random weights:
    i2v-14b = the 14B-shaped image-to-video step (40 blocks, dim 5120, CFG batch 2, text + image
    cross-attention), ti2v-5b = the TI2V-5B-shaped sampling run (30 blocks, dim 3072, CFG batch 2,
    100-channel input, 4 Euler steps from t = 1, timed as one whole run)."""
    import numpy as np
    import torch

    import wan_inputs as wi
    from video_diffusion_transformer_step_amd import _lib as L
    from video_diffusion_transformer_step_amd import runtime as R
    c = wi.get_config(name)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    model = R.DeviceModel(wi.make_model_weights(c, seed=seed), c.dtype)
    blocks = [R.DeviceBlock(None, c.dtype, tensors=device_block_tensors(c, gen)) for _ in range(c.layers)]
    x_t, z = wi.make_latents(c, seed=seed)
    txt, img = wi.make_contexts(c, seed=seed)
    t_emb, i_emb = R.embed_contexts(c, model, txt, img, c.B)
    caches = R.cross_kv_all(c, blocks, t_emb, i_emb, c.B)
    buf = R.alloc_step(c, c.B)
    xg = torch.from_numpy(x_t).cuda()
    zg = torch.from_numpy(z).cuda() if z is not None else None
    nsteps = c.steps if name == "ti2v-5b" else steps
    dt = -1.0 / nsteps
    for k in range(warmup):
        R.denoise_step(c, model, blocks, caches, xg, zg, 1.0 + k * dt, dt, c.guidance, buf, c.B)
    torch.cuda.synchronize()
    xg.copy_(torch.from_numpy(x_t))
    timer = L.KernelTimer(capacity=nsteps * c.layers, kernels=("self_attn",))
    t0 = time.perf_counter()
    with timer:
        for k in range(nsteps):
            R.denoise_step(c, model, blocks, caches, xg, zg, 1.0 + k * dt, dt, c.guidance, buf, c.B)
    torch.cuda.synchronize()
    total_ms = (time.perf_counter() - t0) * 1e3
    assert np.isfinite(xg.float().cpu().numpy()).all(), f"non-finite latent after the {name} steps"
    fl_step, attn_fl = step_flops(c, c.layers)
    ms = total_ms / nsteps
    a = float(np.mean(timer.times_ms().get("self_attn", [float("nan")])))
    out = {"workload": (f"{c.name}: latent [{c.latent_channels},{c.T},{c.H},{c.W}] -> {c.S} tokens, "
                        f"{c.layers} blocks, dim {c.dim}, {c.heads}x{c.head_dim}, FFN {c.ffn_dim}, B {c.B}"
                        + (f", image {c.img_len} keys" if c.img_len else "")),
           "ms_per_step": round(ms, 2), "ms_per_block": round(ms / c.layers, 3),
           "step_tflops": round(fl_step / (ms * 1e-3) / 1e12, 1),
           "step_frac_of_bf16_peak": round(fl_step / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "attention_ms": round(a, 3),
           "attention_frac_of_bf16_peak": round(attn_fl / (a * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    if name == "ti2v-5b":
        out["sampling_run_ms"] = round(total_ms, 1)
        out["steps"] = nsteps
    del blocks, caches, buf, model, xg, zg
    torch.cuda.empty_cache()
    return out


def cpu_tiny_full():
    """The oracle in full on the tiny image-to-video config: build the 36-channel input, one DiT
    evaluation (patchify, patch embedding, time embedding, one block, head, unpatchify) and the Euler
    step, timed end to end on the host (float64 NumPy; best of 3)."""
    import threadpoolctl

    import oracle
    import wan_inputs as wi
    c = wi.get_config("tiny")
    mw = wi.make_model_weights(c, seed=0)
    bw = [wi.make_block_weights(c, 0, seed=0)]
    x_t, z = wi.make_latents(c, seed=0)
    txt, img = wi.make_contexts(c, seed=0)
    cores = len(os.sched_getaffinity(0))
    best = float("inf")
    with threadpoolctl.threadpool_limits(cores):
        for _ in range(3):
            t = time.perf_counter()
            v = oracle.dit_fwd(oracle.build_i2v_input(x_t, z), c.t, mw, bw, txt, img, c.heads, freq_dim=c.freq_dim,
                               out_channels=c.out_channels)
            oracle.euler_step(x_t, v, c.dt)
            best = min(best, time.perf_counter() - t)
    return {"ms_per_step": round(best * 1e3, 2), "cores": cores,
            "sample": (f"{c.name}: the whole step (I2V input, patchify, embeddings, 1 block of dim {c.dim}, head, "
                       f"unpatchify, Euler) on {c.S} tokens, in full, best of 3")}


def cpu_baseline(c, layers, seed=0):
    """The CPU oracle on a bounded sample: one block in sampled-row mode (K/V for all tokens,
    then R1 and R2 query rows), extrapolated to all S rows and `layers` blocks."""
    import numpy as np
    import threadpoolctl

    import oracle
    import wan_inputs as wi
    cores = len(os.sched_getaffinity(0))
    with threadpoolctl.threadpool_limits(cores):
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
        mw = wi.make_model_weights(c, seed=seed)
        bw = wi.make_block_weights(c, 0, seed=seed)
        x = wi.normal(seed, c, "x_block", (1, c.S, c.dim), quantize=False)
        _, e0 = oracle.time_embed(c.t, mw, c.freq_dim)
        txt, _ = wi.make_contexts(c, seed=seed)
        temb = oracle.context_embed(txt[0], mw["wtx1"], mw["btx1"], mw["wtx2"], mw["btx2"])
        kv = [oracle.cross_kv(temb, bw["wck"], bw["bck"], bw["wcv"], bw["bcv"]) + (None, None)]
        # R2 - R1 rows must cost well above the run-to-run noise of the fixed part (~0.1 s)
        R1, R2 = 256, 2048
        rows = wi.sample_rows(c, R2, seed=seed)[:R2]
        oracle.block_fwd(x, e0[None], bw, kv, c.grid, c.heads, rows=rows[:8])  # untimed: threads, page-in
        t = time.perf_counter()
        oracle.block_fwd(x, e0[None], bw, kv, c.grid, c.heads, rows=rows[:R1])
        t1 = time.perf_counter() - t
        t = time.perf_counter()
        oracle.block_fwd(x, e0[None], bw, kv, c.grid, c.heads, rows=rows)
        t2 = time.perf_counter() - t
        blas = [i for i in info if i.get("user_api") == "blas"]
        blas = (f"{blas[0].get('internal_api')} {blas[0].get('version')} ({blas[0].get('architecture')}, "
                f"{blas[0].get('threading_layer')} threads)") if blas else "none found"
    with threadpoolctl.threadpool_limits(1):
        t = time.perf_counter()
        oracle.block_fwd(x, e0[None], bw, kv, c.grid, c.heads, rows=rows[:R1])
        t1_one = time.perf_counter() - t
    per_row = max(t2 - t1, 0.0) / (R2 - R1)
    fixed = max(t1 - R1 * per_row, 0.0)
    block_s = fixed + c.S * per_row
    return {
        "value": round(layers * block_s * 1e3, 1), "unit": "ms/step", "cores": int(threads), "kind": "oracle",
        "sample": (f"one {c.S}-token block in sampled-row mode (LN/K/V for all tokens; after an untimed 8-row "
                   f"call, {R1} and {R2} query rows: {t1:.2f} s and {t2:.2f} s), extrapolated as (fixed "
                   f"{fixed:.2f} s + {c.S} rows x "
                   f"{per_row * 1e3:.1f} ms) x {layers} blocks; float64 NumPy, {threads} BLAS threads "
                   f"of {cores} cores"),
        "blas": blas,
        "one_thread": {"seconds": round(t1_one, 2), "vs_all_threads": round(t1_one / t1, 2),
                       "value_est": round(layers * block_s * 1e3 * t1_one / t1, 1),
                       "sample": (f"the {R1}-row call above on one BLAS thread; value_est scales the step "
                                  f"figure by the two calls' time ratio (an estimate)")},
    }


def measure_two_expert(c, model, blocks, caches, layers, x_t, zg, txt, img, steps, warmup):
    """Wan2.2's two-expert sampling on this workload: a second, independently drawn DiT of the same
    shape is made resident beside the first, and sampling switches from the first (high-noise) to the
    second (low-noise) at t_moe = 1/2.  Times whole sampling runs of 2 * steps Euler steps from t = 1,
    half on each expert."""
    import torch

    from video_diffusion_transformer_step_amd import runtime as R
    import wan_inputs as wi

    gen = torch.Generator(device="cuda")
    gen.manual_seed(4321)
    model2 = R.DeviceModel(wi.make_model_weights(c, seed=1), c.dtype)
    blocks2 = [R.DeviceBlock(None, c.dtype, tensors=device_block_tensors(c, gen)) for _ in range(layers)]
    t_emb, i_emb = R.embed_contexts(c, model2, txt, img, c.B)
    caches2 = R.cross_kv_all(c, blocks2, t_emb, i_emb, c.B)
    experts = [(model, blocks, caches), (model2, blocks2, caches2)]
    buf = R.alloc_step(c, c.B)
    n = 2 * steps
    x = torch.from_numpy(x_t).cuda()
    for _ in range(max(warmup, 1)):
        R.sample_two_expert(c, experts, x, zg, 2, c.guidance, buf, c.B, 0.5)
    torch.cuda.synchronize()
    x = torch.from_numpy(x_t).cuda()
    t0 = time.perf_counter()
    used = R.sample_two_expert(c, experts, x, zg, n, c.guidance, buf, c.B, 0.5)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / n
    gb = sum(p.numel() * p.element_size() for bl in (blocks, blocks2) for b in bl for p in b._keep.t.values()
             if p is not None) / 1e9
    del experts, blocks2, caches2, model2, buf, x
    torch.cuda.empty_cache()
    return {"t_moe": 0.5, "steps": n, "experts_used": used, "ms_per_step": round(ms, 3),
            "block_weights_resident_gb": round(gb, 2),
            "note": ("two independently drawn DiTs of the workload's shape, both resident in HBM; the switch "
                     "at t_moe changes which weights the next step reads (no reload)")}


# Diffusion-cache schedule used for the reported average (a reading: the pages name the two caches and
# their combined gain but give no schedule).  50 Euler steps with CFG; the self-attention output is
# reused on every other step from step 10 to 39, and the unconditional velocity from step 35 on.
CACHE_STEPS = 50
CACHE_ATTN_REUSE = [10 <= k < 40 and k % 2 == 1 for k in range(CACHE_STEPS)]
CACHE_CFG_REUSE = [k >= 35 for k in range(CACHE_STEPS)]


def measure_diffusion_cache(c, model, blocks, layers, x_t, zg, img, steps, warmup):
    """ms per step of the bf16 step in each diffusion-cache mode on this workload's latent: one row
    storing / reusing the attention cache, and the two-row CFG step (conditional + unconditional text),
    storing / reusing; then the average over CACHE_* against the plain two-row CFG step."""
    import numpy as np
    import torch

    from video_diffusion_transformer_step_amd import _lib as L
    from video_diffusion_transformer_step_amd import runtime as R

    import wan_inputs as wi

    c2 = c.replace(B=2)
    txt2, _ = wi.make_contexts(c2, seed=0)  # conditional + unconditional text rows
    t_emb, i_emb = R.embed_contexts(c2, model, txt2, img, 2)
    kv2 = R.cross_kv_all(c2, blocks, t_emb, i_emb, 2)
    buf2 = R.alloc_step(c2, 2)
    ac = R.AttnCache(c2, layers, 2)
    x = torch.from_numpy(x_t).cuda()
    dt = -1.0 / CACHE_STEPS

    def timed(B, mode):
        def one(k):
            R.denoise_step(c2, model, blocks, kv2, x, zg, 1.0 + k * dt, dt, c.guidance, buf2, B,
                           attn_cache=ac.rows(B), attn_mode=mode)
        for k in range(warmup):
            one(k)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            one(warmup + k)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    ms = {}
    ms["cfg_plain"] = timed(2, L.WAN_ATTN_CACHE_OFF)
    ms["cfg_store"] = timed(2, L.WAN_ATTN_CACHE_STORE)
    ms["cfg_reuse"] = timed(2, L.WAN_ATTN_CACHE_REUSE)
    ms["one_row_store"] = timed(1, L.WAN_ATTN_CACHE_STORE)
    ms["one_row_reuse"] = timed(1, L.WAN_ATTN_CACHE_REUSE)
    assert np.isfinite(x.float().cpu().numpy()).all(), "non-finite latent after the cache steps"
    total = 0.0
    for a, g in zip(CACHE_ATTN_REUSE, CACHE_CFG_REUSE):
        total += ms[("one_row_" if g else "cfg_") + ("reuse" if a else "store")]
    avg = total / CACHE_STEPS
    del buf2, ac, kv2, x
    torch.cuda.empty_cache()
    out = {k: round(v, 3) for k, v in ms.items()}
    out.update({
        "schedule": (f"{CACHE_STEPS} CFG Euler steps; attention output reused on {sum(CACHE_ATTN_REUSE)} "
                     f"(odd steps 11..39), unconditional velocity reused on {sum(CACHE_CFG_REUSE)} (steps 35..49)"),
        "avg_ms_per_step": round(avg, 3),
        "speedup_vs_plain_cfg": round(ms["cfg_plain"] / avg, 3),
        "note": ("bf16 step, both CFG rows on the 32760-token latent; cfg_* = two rows, one_row_* = "
                 "conditional row only (CFG reuse); *_store computes self-attention and records its "
                 "layer output, *_reuse skips it"),
    })
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="t2v-1.3b", help="workload preset (t2v-1.3b = 1.3B-shaped 32760-token step)")
    ap.add_argument("--layers", type=int, default=None, help="blocks per step (default: the preset's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the second measurement with the quantised (INT8 Q.K / FP8 P.V) self-attention")
    ap.add_argument("--no-cache", action="store_true",
                    help="skip the diffusion-cache measurement (attention-output and CFG reuse)")
    ap.add_argument("--no-two-expert", action="store_true",
                    help="skip the two-expert (high-noise / low-noise DiT) sampling measurement")
    ap.add_argument("--graph", action="store_true",
                    help="capture each timed step as a HIP graph beforehand and replay it (launch-bound small shapes)")
    ap.add_argument("--no-sharded", action="store_true",
                    help="skip the one-GPU shares of sequence-parallel attention (Ulysses head shard, ring step, merge)")
    ap.add_argument("--no-720p", action="store_true",
                    help="skip the 75600-token self-attention stress measurement")
    ap.add_argument("--no-other-steps", action="store_true",
                    help="skip the 14B-shaped I2V step and the TI2V-5B-shaped sampling run")
    ap.add_argument("--no-device-probe", action="store_true",
                    help="skip the device ceilings (register-only MFMA rate, plain copy rate)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after the timed region, run one plain device copy of this many bytes (a known-size "
                         "reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import wan_inputs as wi
    from video_diffusion_transformer_step_amd import _lib as L
    from video_diffusion_transformer_step_amd import runtime as R

    if not os.path.exists(L.LIB_PATH):
        from video_diffusion_transformer_step_amd.build import build
        build()
    L.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    c = wi.get_config(args.config)
    layers = args.layers or c.layers
    seed = 0
    log(f"workload {c.name}: latent [{c.in_channels},{c.T},{c.H},{c.W}] -> S={c.S}, dim={c.dim}, "
        f"{c.heads}x{c.head_dim}, ffn={c.ffn_dim}, {layers} blocks, B={c.B}")

    # ---- resident inputs and weights
    t = time.perf_counter()
    mw = wi.make_model_weights(c, seed=seed)
    model = R.DeviceModel(mw, c.dtype)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    blocks = [R.DeviceBlock(None, c.dtype, tensors=device_block_tensors(c, gen)) for _ in range(layers)]
    x_t, z = wi.make_latents(c, seed=seed)
    txt, img = wi.make_contexts(c, seed=seed)
    t_emb, i_emb = R.embed_contexts(c, model, txt, img, c.B)
    caches = R.cross_kv_all(c, blocks, t_emb, i_emb, c.B)
    buf = R.alloc_step(c, c.B)
    xg = torch.from_numpy(x_t).cuda()
    zg = torch.from_numpy(z).cuda() if z is not None else None
    torch.cuda.synchronize()
    log(f"setup {time.perf_counter() - t:.1f} s; weights {sum(p.numel() * p.element_size() for b in blocks for p in b._keep.t.values() if p is not None) / 1e9:.2f} GB")

    total = args.warmup + args.steps
    dt = -1.0 / max(total, 1)

    def step(k):
        R.denoise_step(c, model, blocks, caches, xg, zg, 1.0 + k * dt, dt, c.guidance, buf, c.B)

    for k in range(args.warmup):
        step(k)
        torch.cuda.synchronize()
        log(f"warmup step {k} done")

    graphs = None
    if args.graph:  # one captured step per timed step (t differs per step); capturing runs nothing
        graphs = [R.StepGraph(c, model, blocks, caches, xg, zg, 1.0 + (args.warmup + k) * dt, dt, c.guidance, buf,
                              c.B) for k in range(args.steps)]
        log(f"captured {len(graphs)} step graphs")

    # ---- timed region: K steps; self-attention launches bracketed by HIP events on their stream
    # (kernel events are recorded only for eager launches; a replayed graph is timed as a whole)
    timer = L.KernelTimer(capacity=args.steps * layers, kernels=("self_attn",))
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    with timer:
        for k in range(args.steps):
            if graphs is not None:
                graphs[k].replay()
            else:
                step(args.warmup + k)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    gpu_ms_per_step = ev0.elapsed_time(ev1) / args.steps
    attn_ms = timer.times_ms().get("self_attn", [])
    if not attn_ms:  # graph replays record no kernel events: time the launches in one extra eager step
        t_one = L.KernelTimer(capacity=layers, kernels=("self_attn",))
        with t_one:
            step(args.warmup + args.steps)
        attn_ms = t_one.times_ms().get("self_attn", [])
    attn_avg = float(np.mean(attn_ms)) if attn_ms else float("nan")
    log(f"timed {args.steps} steps: {ms_per_step:.2f} ms/step (events {gpu_ms_per_step:.2f}); "
        f"self-attention {attn_avg:.3f} ms/launch over {len(attn_ms)} launches")
    assert np.isfinite(xg.float().cpu().numpy()).all(), "non-finite latent after the timed steps"

    flops_step, attn_flops = step_flops(c, layers)
    attn_tflops = attn_flops / (attn_avg * 1e-3) / 1e12
    step_tflops = flops_step / (ms_per_step * 1e-3) / 1e12

    # ---- per-kernel breakdown (one extra, untimed step with every block kernel bracketed)
    breakdown = None
    if not args.no_breakdown:
        bt = L.KernelTimer(capacity=2 * layers * len(L.KERNEL_IDS), kernels=tuple(L.KERNEL_IDS))
        with bt:
            step(total)
        bd = bt.times_ms()
        blk_flops, _ = block_flops(c)
        S, d, f = c.S, c.dim, c.ffn_dim
        fl = {"qkv_gemm": 2 * S * d * 3 * d, "self_attn": 4 * S * S * d, "o_gemm": 2 * S * d * d,
              "cross_q_gemm": 2 * S * d * d, "cross_attn": 4 * S * (c.text_len + c.img_len) * d,
              "cross_o_gemm": 2 * S * d * d, "ffn1_gemm": 2 * S * d * f, "ffn2_gemm": 2 * S * f * d}
        # algorithmic bytes of the bandwidth-bound kernels: LN reads fp32 x and writes the bf16 operand;
        # the Q/K RMS pass reads the epilogue's sums of squares (2 d / 32 floats per token), reads and
        # writes bf16 k and writes one float r_q per token
        hbm_bytes = {"ln1": 6 * S * d, "ln2": 6 * S * d, "ln3": 6 * S * d, "qk_rms": 4 * S * d + S * d // 4 + 4 * S}
        # algorithmic bytes of every launch (each operand read once, each result written once; the
        # residual products read and write the fp32 x), per batch row except the weights
        L_ctx = c.text_len + c.img_len
        alg_bytes = dict(hbm_bytes)
        alg_bytes.update({
            "qkv_gemm": 2 * S * d + 2 * S * 3 * d + S * d // 4, "o_gemm": 2 * S * d + 8 * S * d,
            "cross_q_gemm": 4 * S * d, "cross_o_gemm": 2 * S * d + 8 * S * d, "ffn1_gemm": 2 * S * d + 2 * S * f,
            "ffn2_gemm": 2 * S * f + 8 * S * d, "self_attn": 8 * S * d, "cross_attn": 4 * S * d + 4 * L_ctx * d})
        w_bytes = {"qkv_gemm": 6 * d * d, "o_gemm": 2 * d * d, "cross_q_gemm": 2 * d * d, "cross_o_gemm": 2 * d * d,
                   "ffn1_gemm": 2 * f * d, "ffn2_gemm": 2 * f * d}
        # counter-backed figures (only for the workload the counters were taken on)
        cnt = block_counters() if args.config == "t2v-1.3b" else {}
        breakdown = {}
        for k_, v in bd.items():
            ms = float(np.sum(v)) / layers  # per block (the I2V cross-attention is two launches)
            e = {"ms": round(ms, 4)}
            if k_ in fl:
                e["tflops"] = round(fl[k_] * c.B / (ms * 1e-3) / 1e12, 1)
                e["frac_of_bf16_peak"] = round(e["tflops"] / PEAK_BF16_TFLOPS, 4)
            if k_ in alg_bytes:
                e["alg_bytes"] = alg_bytes[k_] * c.B + w_bytes.get(k_, 0)
            if k_ in hbm_bytes:
                e["gbs"] = round(hbm_bytes[k_] * c.B / (ms * 1e-3) / 1e9, 1)
                e["frac_of_hbm"] = round(e["gbs"] / PEAK_HBM_GBS, 3)
            ce = cnt.get(k_)
            if ce is not None:
                # L2-miss bytes (FETCH_SIZE + WRITE_SIZE, copy-calibrated; MALL hits included) per launch,
                # and the MFMA busy fraction relative to the register-only probe, from the counter runs
                if "hbm_bytes" in ce:
                    e["counter_bytes"] = round(ce["hbm_bytes"])
                    e["counter_gbs"] = round(ce["hbm_bytes"] / (ms * 1e-3) / 1e9, 1)
                    if k_ in hbm_bytes:
                        e["counter_frac_of_hbm"] = round(e["counter_gbs"] / PEAK_HBM_GBS, 3)
                if ce.get("mfma_busy_vs_probe"):
                    e["counter_mfma_busy_vs_probe"] = round(ce["mfma_busy_vs_probe"], 3)
            breakdown[k_] = e
        breakdown["block_sum_ms"] = round(sum(e["ms"] for e in breakdown.values()), 3)
        log(f"breakdown: {json.dumps(breakdown)}")

    if args.copy_bytes > 0:
        n = args.copy_bytes // 4
        src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {n * 4} bytes (counter calibration)")
        del src, dst

    device = None
    if not args.no_device_probe:
        device = measure_device()
        log(f"device: {json.dumps(device)}")

    sharded = None
    if not args.no_sharded and c.dtype == "bf16" and c.heads % 4 == 0:
        sharded = measure_sharded(c)
        log(f"sharded attention: {json.dumps(sharded)}")

    # ---- the same step on the FP8 paths (reported beside the bf16 headline): the quantised
    # self-attention alone, then with the E4M3 Q/K/V, O, FFN1, FFN2 products as well
    fp8 = {}
    if not args.no_fp8 and c.dtype == "bf16" and c.head_dim == 128 and c.dim % 256 == 0 and c.ffn_dim % 256 == 0:
        for b in blocks:
            b.enable_e4m3()
        for key, gemm8, note in (
                ("fp8_attention_step", False,
                 "self-attention in INT8 (Q.K) / FP8 E4M3 (P.V); every other kernel as in the bf16 step"),
                ("fp8_step", True,
                 "self-attention as above; Q/K/V, O, FFN1, FFN2 products in E4M3 (per-token activation, per-tensor "
                 "weight scales); the rest (norms, cross-attention, head) as in the bf16 step")):
            buf8 = R.alloc_step(c, c.B, fp8_attn=True, fp8_gemm=gemm8)
            x8 = torch.from_numpy(x_t).cuda()

            def step8(k):
                R.denoise_step(c, model, blocks, caches, x8, zg, 1.0 + k * dt, dt, c.guidance, buf8, c.B,
                               fp8_attn=True, fp8_gemm=gemm8)

            for k in range(args.warmup):
                step8(k)
            torch.cuda.synchronize()
            t8 = L.KernelTimer(capacity=args.steps * layers * 8, kernels=("self_attn", "quant"))
            t0 = time.perf_counter()
            with t8:
                for k in range(args.steps):
                    step8(args.warmup + k)
            torch.cuda.synchronize()
            ms8 = (time.perf_counter() - t0) * 1e3 / args.steps
            tm = t8.times_ms()
            a8 = float(np.mean(tm.get("self_attn", [float("nan")])))
            q8 = float(np.sum(tm.get("quant", [0.0]))) / (args.steps * layers)
            tf8 = attn_flops / (a8 * 1e-3) / 1e12
            assert np.isfinite(x8.float().cpu().numpy()).all(), "non-finite latent after the FP8 steps"
            fp8[key] = {"ms_per_step": round(ms8, 3), "ms_per_block": round(ms8 / layers, 3),
                        "attention_ms": round(a8, 4), "attention_tflops": round(tf8, 1),
                        "attention_frac_of_fp8_peak": round(tf8 / PEAK_FP8_TFLOPS, 4),
                        "attention_frac_of_bf16_peak": round(tf8 / PEAK_BF16_TFLOPS, 4),
                        "attention_frac_of_measured_fp8_peak": (round(tf8 / device["measured_fp8_e4m3_tflops"], 4)
                                                                if device else None),
                        "quantise_ms_per_block": round(q8, 4),
                        "step_speedup_vs_bf16": round(ms_per_step / ms8, 3), "note": note}
            log(f"{key}: {ms8:.2f} ms/step, attention {a8:.3f} ms ({tf8:.0f} TFLOP/s), quantisers {q8:.3f} ms/block")
            del buf8, x8

    cache = None
    if not args.no_cache and c.B == 1:
        cache = measure_diffusion_cache(c, model, blocks, layers, x_t, zg, img, args.steps, args.warmup)
        log(f"diffusion cache: {json.dumps(cache)}")

    two_expert = None
    if not args.no_two_expert:
        two_expert = measure_two_expert(c, model, blocks, caches, layers, x_t, zg, txt, img, args.steps,
                                        args.warmup)
        two_expert["ms_per_step_vs_one_expert"] = round(two_expert["ms_per_step"] / ms_per_step, 3)
        log(f"two experts: {json.dumps(two_expert)}")

    attn720 = None
    if not args.no_720p:
        attn720 = measure_attention_720p()
        log(f"720p attention: {json.dumps(attn720)}")

    other = None
    if not args.no_other_steps and args.config == "t2v-1.3b":
        other = {}
        for name in ("i2v-14b", "ti2v-5b"):
            other[name] = measure_other_step(name, steps=2, warmup=1)
            log(f"{name}: {json.dumps(other[name])}")

    cpu = None
    if not args.no_cpu_baseline:
        t = time.perf_counter()
        cpu = cpu_baseline(c, layers, seed=seed)
        cpu["tiny_full"] = cpu_tiny_full()
        log(f"cpu baseline {time.perf_counter() - t:.1f} s: {cpu['value']} ms/step; tiny in full "
            f"{cpu['tiny_full']['ms_per_step']} ms")

    traffic = counters_traffic() if args.config == "t2v-1.3b" else None  # counters are of that workload
    out = {
        "metric": METRIC,
        "value": round(ms_per_step, 3),
        "unit": "ms/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c.dtype,
        "data": "synthetic (seeded N(0,1) latent and text context; random-init N(0,0.02) weights)",
        "config": {"workload": (f"{c.name}: Wan2.1-1.3B-shaped text-to-video denoise step, latent "
                                f"[{c.latent_channels},{c.T},{c.H},{c.W}] -> {c.S} tokens, {layers} blocks"),
                   "global_batch": c.B, "seq_len": c.S, "layers": layers, "dim": c.dim, "heads": c.heads,
                   "head_dim": c.head_dim, "ffn_dim": c.ffn_dim, "text_len": c.text_len,
                   "parallelism": "single GPU", "launch": "hip graph per step" if args.graph else "eager"},
        "ms_per_block": round(ms_per_step / layers, 3),
        "step_tflops": round(step_tflops, 1),
        "step_frac_of_bf16_peak": round(step_tflops / PEAK_BF16_TFLOPS, 4),
        "step_frac_of_measured_bf16_peak": (round(step_tflops / device["measured_bf16_tflops"], 4)
                                            if device else None),
        "attention_tflops": round(attn_tflops, 1),
        "attention_frac_of_bf16_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": {"kernel": "self-attention (flash, bf16 MFMA)", "bound": "mfma",
                     "achieved": round(attn_tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "launch_ms": round(attn_avg, 4), "flops_per_launch": attn_flops,
                     "peak_measured": device["measured_bf16_tflops"] if device else None,
                     "frac_of_measured_peak": (round(attn_tflops / device["measured_bf16_tflops"], 4)
                                               if device else None),
                     "peak_measured_random_operands": (device["measured_bf16_random_operands_tflops"]
                                                       if device else None),
                     "frac_of_measured_random_operand_peak": (
                         round(attn_tflops / device["measured_bf16_random_operands_tflops"], 4) if device else None)},
        "device": device,
        "breakdown_ms_per_block": breakdown,
        "fp8_attention_step": fp8.get("fp8_attention_step"),
        "fp8_step": fp8.get("fp8_step"),
        "sharded_attention": sharded,
        "attention_720p": attn720,
        "other_workloads": other,
        "diffusion_cache": cache,
        "two_expert": two_expert,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
