"""Seeded synthetic inputs for the Wan-style video DiT denoise step.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark.  It draws random numbers and rounds them to bf16-representable values;
it holds none of the method's arithmetic (no norm, no projection, no attention).

Every tensor is drawn from its own NumPy PCG64 stream keyed by
``SeedSequence([seed, stream_id, tensor_id, block])`` so any one tensor can be
regenerated on its own.  Distributions follow the workload description:
latents, contexts and self-attention stress inputs ~N(0,1); weight matrices and
biases ~N(0, 0.02); norm gains 1 + N(0, 0.02).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

__all__ = ["WanConfig", "CONFIGS", "get_config", "rng", "bf16_round", "normal",
           "make_block_weights", "make_blocks_weights", "make_model_weights", "make_latents",
           "make_contexts", "make_attention_qkv", "sample_rows", "TENSOR_IDS",
           "BLOCK_MATRICES"]


@dataclass(frozen=True)
class WanConfig:
    """Shapes of one workload.  Latent dims are (C, T, H, W); tokens S = T*(H/2)*(W/2)."""
    name: str
    stream_id: int
    dtype: str            # "f32" or "bf16": the arithmetic type of GEMM / attention operands
    B: int                # batch rows seen by the DiT (2 with classifier-free guidance)
    latent_channels: int  # C of x_t (16 for Wan2.1, 48 for the TI2V-5B-shaped case)
    i2v: bool             # True: input = [x_t, 4-channel mask, image latent]
    T: int
    H: int
    W: int
    dim: int
    heads: int
    head_dim: int
    ffn_dim: int
    text_len: int
    text_dim: int
    img_len: int          # 0 = single-stream (text only) cross-attention
    img_dim: int
    layers: int
    freq_dim: int = 256
    t: float = 0.5
    dt: float = -0.1
    guidance: float = 5.0
    steps: int = 1
    ln_eps: float = 1e-6
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0

    @property
    def in_channels(self) -> int:
        return 2 * self.latent_channels + 4 if self.i2v else self.latent_channels

    @property
    def out_channels(self) -> int:
        return self.latent_channels

    @property
    def grid(self):
        return (self.T, self.H // 2, self.W // 2)

    @property
    def S(self) -> int:
        return self.T * (self.H // 2) * (self.W // 2)

    def replace(self, **kw) -> "WanConfig":
        return dataclasses.replace(self, **kw)


# The five workloads.  The 1.3B layer count (32) comes from the
# "图解 Wan2.1 I2V" page's summary table (§8); the 14B one (40) is there too.
CONFIGS = {
    "tiny": WanConfig("tiny-i2v-block-f32", 0, "f32", 1, 16, True, 2, 8, 8,
                   128, 2, 64, 512, 16, 64, 0, 0, 1, t=0.5, dt=-0.1),
    "t2v-1.3b": WanConfig("wan2.1-1.3b-t2v-block-bf16", 1, "bf16", 1, 16, False, 21, 60, 104,
                   1536, 12, 128, 8960, 512, 4096, 0, 0, 32, t=0.5, dt=-0.1),
    "i2v-14b": WanConfig("wan-14b-i2v-block-bf16", 2, "bf16", 2, 16, True, 21, 60, 104,
                   5120, 40, 128, 13824, 512, 4096, 257, 1280, 40, t=0.5, dt=-0.1),
    "attn-720p": WanConfig("720p-self-attention-bf16", 3, "bf16", 1, 16, False, 21, 90, 160,
                   5120, 40, 128, 0, 0, 0, 0, 0, 0),
    "ti2v-5b": WanConfig("ti2v-5b-sampling-bf16", 4, "bf16", 2, 48, True, 31, 44, 80,
                   3072, 24, 128, 14336, 512, 4096, 0, 0, 30, t=1.0, dt=-0.25,
                    guidance=5.0, steps=4),
}


def get_config(name: str) -> WanConfig:
    return CONFIGS[name]


# Fixed tensor-id list: a tensor's stream depends only on (seed, config, id, block).
TENSOR_IDS = {name: i for i, name in enumerate([
    # per-block
    "mod_bias", "wq", "bq", "wk", "bk", "wv", "bv", "gq", "gk", "wo", "bo",
    "ln3_w", "ln3_b", "wcq", "bcq", "wck", "bck", "wcv", "bcv", "wki", "bki",
    "wvi", "bvi", "wco", "bco", "w1", "b1", "w2", "b2",
    # model-level
    "w_pe", "b_pe", "wt1", "bt1", "wt2", "bt2", "wtp", "btp",
    "wtx1", "btx1", "wtx2", "btx2", "wim1", "bim1", "wim2", "bim2",
    "head_mod", "wh", "bh",
    # activations / inputs
    "x_t", "z_img", "ctx_txt", "ctx_txt_uncond", "ctx_img", "x_block",
    "q", "k", "v", "v_cond", "v_uncond", "x0", "x1", "rows",
    # drawn directly where the producing MLP is not under test (appended: earlier ids are unchanged)
    "e0", "t_emb",
])}

# Which per-block tensors are weight matrices (bf16 operands in bf16 mode).
BLOCK_MATRICES = ("wq", "wk", "wv", "wo", "wcq", "wck", "wcv", "wki", "wvi", "wco", "w1", "w2")
MODEL_MATRICES = ("w_pe", "wt1", "wt2", "wtp", "wtx1", "wtx2", "wim1", "wim2", "wh")


def rng(seed: int, stream_id: int, tensor: str, block: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([seed, stream_id, TENSOR_IDS[tensor], block])
    return np.random.Generator(np.random.PCG64(ss))


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even); result is float32.
    (bits + 0x7FFF + lsb) with the low 16 bits cleared, in wrapping 32-bit arithmetic."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u >> 16) & 1
    r += 0x7FFF
    r += u
    r &= 0xFFFF0000
    return r.view(np.float32)


def normal(seed, cfg: WanConfig, tensor: str, shape, std=1.0, mean=0.0, block=0,
           quantize=None) -> np.ndarray:
    """float32 N(mean, std^2) draw; bf16-representable when the config is bf16 and
    ``quantize`` is not False (``quantize=True`` forces it)."""
    g = rng(seed, cfg.stream_id, tensor, block)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    q = (cfg.dtype == "bf16") if quantize is None else quantize
    return bf16_round(a) if q else a


def make_block_weights(cfg: WanConfig, block: int = 0, seed: int = 0, std: float = 0.02):
    """Weights of one DiT block, W as [out, in].  Matrices are bf16-representable in bf16
    mode; biases, norm gains and the modulation bias stay float32."""
    d, f = cfg.dim, cfg.ffn_dim
    n = lambda name, shape, **kw: normal(seed, cfg, name, shape, std=std, block=block, **kw)
    w = {
        "mod_bias": n("mod_bias", (6, d), quantize=False),
        "wq": n("wq", (d, d)), "bq": n("bq", (d,), quantize=False),
        "wk": n("wk", (d, d)), "bk": n("bk", (d,), quantize=False),
        "wv": n("wv", (d, d)), "bv": n("bv", (d,), quantize=False),
        "gq": normal(seed, cfg, "gq", (d,), std=std, mean=1.0, block=block, quantize=False),
        "gk": normal(seed, cfg, "gk", (d,), std=std, mean=1.0, block=block, quantize=False),
        "wo": n("wo", (d, d)), "bo": n("bo", (d,), quantize=False),
        "ln3_w": normal(seed, cfg, "ln3_w", (d,), std=std, mean=1.0, block=block, quantize=False),
        "ln3_b": n("ln3_b", (d,), quantize=False),
        "wcq": n("wcq", (d, d)), "bcq": n("bcq", (d,), quantize=False),
        "wck": n("wck", (d, d)), "bck": n("bck", (d,), quantize=False),
        "wcv": n("wcv", (d, d)), "bcv": n("bcv", (d,), quantize=False),
        "wco": n("wco", (d, d)), "bco": n("bco", (d,), quantize=False),
        "w1": n("w1", (f, d)), "b1": n("b1", (f,), quantize=False),
        "w2": n("w2", (d, f)), "b2": n("b2", (d,), quantize=False),
    }
    if cfg.img_len > 0:
        w.update({"wki": n("wki", (d, d)), "bki": n("bki", (d,), quantize=False),
                  "wvi": n("wvi", (d, d)), "bvi": n("bvi", (d,), quantize=False)})
    return w


def make_blocks_weights(cfg: WanConfig, nblocks: int, seed: int = 0, std: float = 0.02, workers: int = 16):
    """``make_block_weights`` for blocks 0 .. nblocks-1, drawn on `workers` threads (every tensor has its
    own stream, so the values do not depend on the thread count)."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=max(1, min(workers, nblocks))) as ex:
        return list(ex.map(lambda i: make_block_weights(cfg, i, seed, std), range(nblocks)))


def make_model_weights(cfg: WanConfig, seed: int = 0, std: float = 0.02):
    """Model-level weights: patch embedding, time MLP + projection, context MLPs, head."""
    d = cfg.dim
    n = lambda name, shape, **kw: normal(seed, cfg, name, shape, std=std, **kw)
    w = {
        "w_pe": n("w_pe", (d, 4 * cfg.in_channels)), "b_pe": n("b_pe", (d,), quantize=False),
        "wt1": n("wt1", (d, cfg.freq_dim)), "bt1": n("bt1", (d,), quantize=False),
        "wt2": n("wt2", (d, d)), "bt2": n("bt2", (d,), quantize=False),
        "wtp": n("wtp", (6 * d, d)), "btp": n("btp", (6 * d,), quantize=False),
        "wtx1": n("wtx1", (d, cfg.text_dim)), "btx1": n("btx1", (d,), quantize=False),
        "wtx2": n("wtx2", (d, d)), "btx2": n("btx2", (d,), quantize=False),
        "head_mod": n("head_mod", (2, d), quantize=False),
        "wh": n("wh", (4 * cfg.out_channels, d)), "bh": n("bh", (4 * cfg.out_channels,), quantize=False),
    }
    if cfg.img_len > 0:
        w.update({"wim1": n("wim1", (d, cfg.img_dim)), "bim1": n("bim1", (d,), quantize=False),
                  "wim2": n("wim2", (d, d)), "bim2": n("bim2", (d,), quantize=False)})
    return w


def make_latents(cfg: WanConfig, seed: int = 0):
    """x_t and (for image-to-video) the image latent z_img, both [1, C, T, H, W] ~N(0,1) fp32."""
    shape = (1, cfg.latent_channels, cfg.T, cfg.H, cfg.W)
    x_t = normal(seed, cfg, "x_t", shape, quantize=False)
    z = normal(seed, cfg, "z_img", shape, quantize=False) if cfg.i2v else None
    return x_t, z


def make_contexts(cfg: WanConfig, seed: int = 0):
    """Text context [B, text_len, text_dim] (row 1 is an independent 'unconditional' draw
    when B = 2) and CLIP image tokens [img_len, img_dim] shared by all rows; bf16 values
    in bf16 mode."""
    txt = [normal(seed, cfg, "ctx_txt", (cfg.text_len, cfg.text_dim))]
    if cfg.B > 1:
        txt.append(normal(seed, cfg, "ctx_txt_uncond", (cfg.text_len, cfg.text_dim)))
    txt = np.stack(txt[:cfg.B]) if cfg.B <= 2 else np.stack([txt[i % 2] for i in range(cfg.B)])
    img = normal(seed, cfg, "ctx_img", (cfg.img_len, cfg.img_dim)) if cfg.img_len else None
    return txt, img


def make_attention_qkv(cfg: WanConfig, seed: int = 0):
    """Self-attention stress inputs q, k, v [B, S, heads, head_dim] ~N(0,1)."""
    shape = (cfg.B, cfg.S, cfg.heads, cfg.head_dim)
    return tuple(normal(seed, cfg, name, shape) for name in ("q", "k", "v"))


def sample_rows(cfg: WanConfig, R: int, seed: int = 0) -> np.ndarray:
    """R sorted, distinct query rows: always row 0, row S-1 and the first row of frames
    0..2, plus seeded uniform draws."""
    S = cfg.S
    hw = (cfg.H // 2) * (cfg.W // 2)
    fixed = {0, S - 1} | {f * hw for f in range(min(3, cfg.T))}
    g = rng(seed, cfg.stream_id, "rows")
    rest = g.choice(S, size=min(S, R + len(fixed)), replace=False)
    rows = list(sorted(fixed))
    for r in rest:
        if len(rows) >= R:
            break
        if int(r) not in fixed:
            rows.append(int(r))
    return np.array(sorted(rows[:R]), dtype=np.int64)
