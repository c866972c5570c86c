"""Device-resident weights and the denoise-step call sequence over the C ABI.

Uploads weights once (packing W_q/W_k/W_v and the cross-attention W_k/W_v into
the fused layouts include/wan.h documents), keeps the ctypes structs that point
at them, and calls the library's entry points in the order of one DiT
evaluation ("图解 Wan2.1 I2V" §7): [I2V input] -> patchify -> patch embedding ->
timestep embedding -> blocks -> head -> unpatchify -> CFG + Euler.  No
arithmetic happens here.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np
import torch

from . import _lib as L


def _dt(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_dev(a, dtype=torch.float32, device="cuda"):
    """Upload a host array (values already representable in `dtype`)."""
    t = torch.from_numpy(np.array(a, dtype=np.float32, copy=True))
    return t.to(device=device).to(dtype).contiguous()


class _Keep:
    """Holds device tensors referenced by a ctypes struct."""

    def __init__(self):
        self.t = {}

    def put(self, name, tensor):
        self.t[name] = tensor
        return None if tensor is None else tensor.data_ptr()


def cfg_of(c, dtype=None, fp8_attn=False, fp8_gemm=False):
    """BlockCfg from a workload description (attributes dim, heads, head_dim, ffn_dim,
    text_len, img_len, dtype, ln_eps, rms_eps, rope_theta); fp8_attn selects the quantised
    self-attention (WAN_FLAG_FP8_ATTN), fp8_gemm the E4M3 products (WAN_FLAG_FP8_GEMM; the blocks
    need DeviceBlock.enable_e4m3())."""
    d = dtype if dtype is not None else c.dtype
    flags = (L.WAN_FLAG_FP8_ATTN if fp8_attn else 0) | (L.WAN_FLAG_FP8_GEMM if fp8_gemm else 0)
    return L.block_cfg(c.dim, c.heads, c.head_dim, c.ffn_dim, max(c.text_len, 1), c.img_len,
                       L.WAN_BF16 if d == "bf16" else L.WAN_F32, c.ln_eps, c.rms_eps, c.rope_theta, flags)


# The block matrices the products read in K panels (wan_pack_weight), packed once at set-up.
PANEL_MATRICES = ("wqkv", "wo", "wcq", "wco", "w1", "w2")


class DeviceBlock:
    """One block's weights on the device + its BlockWeights / CrossKVWeights structs.  The six product
    matrices are held in K panels only (the row-major tensors passed in are not kept)."""

    def __init__(self, w: dict, dtype: str, device="cuda", tensors=None):
        wd = _dt(dtype)
        k = _Keep()
        if tensors is not None:  # already-on-device tensors (benchmark path)
            g = tensors
        else:
            g = {}
            g["wqkv"] = to_dev(np.concatenate([w["wq"], w["wk"], w["wv"]]), wd, device)
            g["bqkv"] = to_dev(np.concatenate([w["bq"], w["bk"], w["bv"]]), torch.float32, device)
            for n in ("wo", "wcq", "wco", "w1", "w2"):
                g[n] = to_dev(w[n], wd, device)
            for n in ("mod_bias", "gq", "gk", "bo", "ln3_w", "ln3_b", "bcq", "bco", "b1", "b2"):
                g[n] = to_dev(w[n], torch.float32, device)
            g["wkv_txt"] = to_dev(np.concatenate([w["wck"], w["wcv"]]), wd, device)
            g["bkv_txt"] = to_dev(np.concatenate([w["bck"], w["bcv"]]), torch.float32, device)
            if "wki" in w:
                g["wkv_img"] = to_dev(np.concatenate([w["wki"], w["wvi"]]), wd, device)
                g["bkv_img"] = to_dev(np.concatenate([w["bki"], w["bvi"]]), torch.float32, device)
        g = dict(g)
        for n in PANEL_MATRICES:
            g[n] = L.pack_weight(g[n].contiguous())
        self.bw = L.BlockWeights(*[k.put(n, g[n]) for n in (
            "mod_bias", "wqkv", "bqkv", "gq", "gk", "wo", "bo", "ln3_w", "ln3_b", "wcq", "bcq", "wco", "bco",
            "w1", "b1", "w2", "b2")])
        self.kvw = L.CrossKVWeights(k.put("wkv_txt", g["wkv_txt"]), k.put("bkv_txt", g["bkv_txt"]),
                                    k.put("wkv_img", g.get("wkv_img")), k.put("bkv_img", g.get("bkv_img")))
        self._keep = k

    def enable_e4m3(self):
        """E4M3 codes of wqkv, wo, w1, w2 with one scale each (wan_quantize_tensor_e4m3 of the packed
        matrices: per-element codes of packed values are the packed codes), linked into bw for
        WAN_FLAG_FP8_GEMM.  bf16 blocks only."""
        k = self._keep
        ws = torch.empty(256, dtype=torch.uint8, device=k.t["wqkv"].device)
        ptrs, scales = [], []
        for n in ("wqkv", "wo", "w1", "w2"):
            src = k.t[n]
            codes = torch.empty(src.shape, dtype=torch.uint8, device=src.device)
            scale = torch.empty(1, dtype=torch.float32, device=src.device)
            L.quantize_tensor_e4m3(src, codes, scale, ws)
            ptrs.append(k.put(n + "_e4m3", codes))
            scales.append(k.put(n + "_scale", scale))
        self._e4m3 = L.BlockWeightsE4M3(*ptrs, *scales)
        self.bw.e4m3 = ctypes.pointer(self._e4m3)
        return self


class CrossKVCache:
    """Per-block cross-attention K / V^T buffers (computed once per generation)."""

    def __init__(self, cfg: L.BlockCfg, B: int, device="cuda"):
        self.bufs = [torch.empty(max(L.cross_kv_buffer_bytes(cfg, B, i), 16), dtype=torch.uint8, device=device)
                     if (i < 2 or cfg.img_len > 0) else None for i in range(4)]
        self.kv = L.CrossKV(*[None if b is None else b.data_ptr() for b in self.bufs])


class DeviceModel:
    """Model-level weights: patch embedding, timestep MLP, context MLPs, head."""

    def __init__(self, w: dict, dtype: str, device="cuda"):
        wd = _dt(dtype)
        k = _Keep()
        f = lambda n: to_dev(w[n], torch.float32, device)
        m = lambda n: to_dev(w[n], wd, device)
        self.w_pe, self.b_pe = m("w_pe"), f("b_pe")
        self.tw = L.TimeWeights(k.put("wt1", m("wt1")), k.put("bt1", f("bt1")), k.put("wt2", m("wt2")),
                                k.put("bt2", f("bt2")), k.put("wtp", m("wtp")), k.put("btp", f("btp")))
        self.hw = L.HeadWeights(k.put("head_mod", f("head_mod")), k.put("wh", m("wh")), k.put("bh", f("bh")))
        self.txt = (m("wtx1"), f("btx1"), m("wtx2"), f("btx2"))
        self.img = (m("wim1"), f("bim1"), m("wim2"), f("bim2")) if "wim1" in w else None
        self._keep = k


@dataclass
class StepBuffers:
    x_in: torch.Tensor
    p: torch.Tensor
    x: torch.Tensor
    e: torch.Tensor
    e0: torch.Tensor
    head_out: torch.Tensor
    v: torch.Tensor
    ws: torch.Tensor


def embed_contexts(c, model: DeviceModel, ctx_txt, ctx_img, B, device="cuda"):
    """Context MLPs, once per generation.  ctx_txt [B, L, text_dim] host; ctx_img [Li, img_dim] host
    (shared by all rows).  Returns (txt_emb [B, L, dim], img_emb [B, Li, dim] or None) device tensors."""
    cfg = cfg_of(c)
    wd = _dt(c.dtype)
    txt = to_dev(ctx_txt, wd, device)
    out_t = torch.empty((B, c.text_len, c.dim), dtype=wd, device=device)
    rows = B * max(c.text_len, c.img_len)
    ws = torch.empty(max(L.context_embed_ws_bytes(cfg, rows), 16), dtype=torch.uint8, device=device)
    L.context_embed(cfg, txt, *model.txt, out_t, ws)
    out_i = None
    if c.img_len > 0:
        img = to_dev(np.broadcast_to(ctx_img[None], (B,) + ctx_img.shape), wd, device)
        out_i = torch.empty((B, c.img_len, c.dim), dtype=wd, device=device)
        L.context_embed(cfg, img, *model.img, out_i, ws)
    return out_t, out_i


def cross_kv_all(c, blocks, txt_emb, img_emb, B, device="cuda"):
    cfg = cfg_of(c)
    ws = torch.empty(max(L.cross_kv_ws_bytes(cfg, B), 16), dtype=torch.uint8, device=device)
    caches = []
    for blk in blocks:
        kc = CrossKVCache(cfg, B, device)
        L.cross_kv_fwd(cfg, blk.kvw, txt_emb, img_emb, B, kc.kv, ws)
        caches.append(kc)
    return caches


def alloc_step(c, B, device="cuda", fp8_attn=False, fp8_gemm=False) -> StepBuffers:
    cfg = cfg_of(c, fp8_attn=fp8_attn, fp8_gemm=fp8_gemm)
    S = c.S
    ws_bytes = max(L.block_ws_bytes(cfg, c.grid, B), L.patch_embed_ws_bytes(cfg, B * S, c.in_channels),
                   L.head_ws_bytes(cfg, B * S), 16)
    f32 = torch.float32
    return StepBuffers(
        x_in=torch.empty((B, c.in_channels, c.T, c.H, c.W), dtype=f32, device=device),
        p=torch.empty((B, S, 4 * c.in_channels), dtype=f32, device=device),
        x=torch.empty((B, S, c.dim), dtype=f32, device=device),
        e=torch.empty((B, c.dim), dtype=f32, device=device),
        e0=torch.empty((B, 6, c.dim), dtype=f32, device=device),
        head_out=torch.empty((B, S, 4 * c.out_channels), dtype=f32, device=device),
        v=torch.empty((B, c.out_channels, c.T, c.H, c.W), dtype=f32, device=device),
        ws=torch.empty(ws_bytes, dtype=torch.uint8, device=device),
    )


def dit_forward(c, model: DeviceModel, blocks, caches, x_latent, z_img, t, buf: StepBuffers, B,
                known_pixel_frames=None, fp8_attn=False, fp8_gemm=False, attn_cache=None,
                attn_mode=0, tap=None):
    """One DiT evaluation over B rows sharing the latent x_latent [1, C, T, H, W] (CFG rows see the same
    x_in).  Result in buf.v [B, C_out, T, H, W].  fp8_attn / fp8_gemm: quantised self-attention / E4M3
    products in every block (buf from alloc_step with the same flags).  attn_cache / attn_mode: the
    attention cache of every block (AttnCache, its rows 0 .. B-1) and WAN_ATTN_CACHE_STORE / _REUSE.
    tap: None, or {block index: list}; for each listed block a dict of device copies of its input x,
    its e0 and its output x is appended (for checking one block inside a running chain)."""
    cfg = cfg_of(c, fp8_attn=fp8_attn, fp8_gemm=fp8_gemm)
    one = x_latent.shape[0]
    for b in range(B):
        src = x_latent[b % one:b % one + 1]
        if c.i2v:
            L.build_i2v_input(src, z_img[b % one:b % one + 1], buf.x_in[b:b + 1], known_pixel_frames)
            L.patchify(buf.x_in[b:b + 1], buf.p[b:b + 1])
        else:
            L.patchify(src, buf.p[b:b + 1])
    L.patch_embed(cfg, buf.p[:B], c.in_channels, model.w_pe, model.b_pe, buf.x, buf.ws)
    L.time_embed(cfg, c.freq_dim, model.tw, [t] * B, buf.e, buf.e0)
    for i, (blk, kc) in enumerate(zip(blocks, caches)):
        if tap is not None and i in tap:
            tap[i].append({"x_in": buf.x[:B].clone(), "e0": buf.e0[:B].clone()})
        if attn_cache is None or attn_mode == L.WAN_ATTN_CACHE_OFF:
            L.dit_block_fwd(cfg, blk.bw, c.grid, B, buf.x, buf.e0, kc.kv, buf.ws)
        else:
            L.dit_block_fwd(cfg, blk.bw, c.grid, B, buf.x, buf.e0, kc.kv, buf.ws, attn_y=attn_cache.t[i],
                            attn_mode=attn_mode)
        if tap is not None and i in tap:
            tap[i][-1]["x_out"] = buf.x[:B].clone()
    L.head_fwd(cfg, model.hw, c.out_channels, B, c.S, buf.x, buf.e, buf.head_out, buf.ws)
    L.unpatchify(buf.head_out, buf.v)
    return buf.v


def denoise_step(c, model, blocks, caches, x_latent, z_img, t, dt, guidance, buf: StepBuffers, B,
                 known_pixel_frames=None, fp8_attn=False, fp8_gemm=False, attn_cache=None, attn_mode=0, tap=None):
    """x_latent <- x_latent + dt * v, v = CFG(v_cond, v_uncond) when B == 2 (row 0 conditional)."""
    v = dit_forward(c, model, blocks, caches, x_latent, z_img, t, buf, B, known_pixel_frames, fp8_attn, fp8_gemm,
                    attn_cache, attn_mode, tap)
    L.fm_euler_step(x_latent, v[0:1], v[1:2] if B > 1 else None, guidance, dt)
    return x_latent


class StepGraph:
    """One denoise_step captured as a HIP graph (torch.cuda.CUDAGraph) and replayed with one call.

    The library enqueues kernels only (no allocation, memset or synchronisation) and this module adds
    no device work of its own, so the graph holds exactly the eager step's launches.  The captured
    step is fixed to its buffers, its t and dt (the time embedding takes t as a host value, baked into
    the launch), and its guidance: a sampling schedule captures one graph per step.  Capturing
    records the launches without running them."""

    def __init__(self, c, model, blocks, caches, x_latent, z_img, t, dt, guidance, buf: StepBuffers, B, **kw):
        self.graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(self.graph):
            denoise_step(c, model, blocks, caches, x_latent, z_img, t, dt, guidance, buf, B, **kw)

    def replay(self):
        self.graph.replay()


class AttnCache:
    """The attention cache of every block: y [B, S, dim] float32 per block (the self-attention layer
    output before its gate, as wan_dit_block_fwd_cached keeps it)."""

    def __init__(self, c, nblocks, B, device="cuda"):
        self.t = [torch.zeros((B, c.S, c.dim), dtype=torch.float32, device=device) for _ in range(nblocks)]

    def rows(self, B):
        """A view on the first B batch rows (same storage)."""
        v = AttnCache.__new__(AttnCache)
        v.t = [t[:B] for t in self.t]
        return v


def sample_cached(c, model, blocks, caches, x_latent, z_img, steps, guidance, buf: StepBuffers, B, attn_reuse,
                  cfg_reuse, attn_cache: AttnCache, t0=1.0, known_pixel_frames=None, fp8_attn=False, fp8_gemm=False):
    """Euler sampling with the diffusion cache: on steps with attn_reuse[k] every block reuses its cached
    self-attention output; on steps with cfg_reuse[k] only the conditional row runs and the unconditional
    velocity of the last full step is reused.  Both lists start with False.  Returns the latent (in place)."""
    assert not attn_reuse[0] and not cfg_reuse[0]
    dt = -t0 / steps
    v_u = torch.empty_like(buf.v[0:1]) if B > 1 else None
    for k in range(steps):
        t = t0 + k * dt
        Bk = 1 if (cfg_reuse[k] and B > 1) else B
        mode = L.WAN_ATTN_CACHE_REUSE if attn_reuse[k] else L.WAN_ATTN_CACHE_STORE
        v = dit_forward(c, model, blocks, caches, x_latent, z_img, t, buf, Bk, known_pixel_frames, fp8_attn,
                        fp8_gemm, attn_cache.rows(Bk), mode)
        if B > 1 and Bk > 1:
            v_u.copy_(v[1:2])
        L.fm_euler_step(x_latent, v[0:1], v_u, guidance, dt)
    return x_latent


def expert_for_step(t, t_moe):
    """Wan2.2's timestep-level expert choice ("Wan 技术深度解析" §7.2): 0 = the high-noise expert while
    t > t_moe, 1 = the low-noise expert from t <= t_moe on."""
    return 0 if t > t_moe else 1


def sample_two_expert(c, experts, x_latent, z_img, steps, guidance, buf: StepBuffers, B, t_moe, t0=1.0,
                      known_pixel_frames=None, fp8_attn=False, fp8_gemm=False):
    """Euler sampling over two whole DiTs that split the schedule at t_moe: experts = ((model, blocks,
    caches) of the high-noise expert, (model, blocks, caches) of the low-noise one), both resident.
    Returns the expert index of each step; the latent is updated in place."""
    dt = -t0 / steps
    used = []
    for k in range(steps):
        t = t0 + k * dt
        e = expert_for_step(t, t_moe)
        model, blocks, caches = experts[e]
        denoise_step(c, model, blocks, caches, x_latent, z_img, t, dt, guidance, buf, B, known_pixel_frames,
                     fp8_attn, fp8_gemm)
        used.append(e)
    return used

