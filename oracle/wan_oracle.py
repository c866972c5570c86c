"""Plain float64 definitions of every step of the Wan-style video DiT denoise step.

TEST INFRASTRUCTURE ONLY (see the package docstring): never called by the product path.

Conventions
-----------
* Latents are [B, C, T, H, W]; tokens are [B, S, dim] with S = T * (H/2) * (W/2).
* Linear layers store W as [out, in]: y = x @ W.T + b.
* Multi-head tensors use channel index h * head_dim + d (heads concatenated).
* All arithmetic is float64; inputs are decoded from whatever the caller gives.

Readings of points the pages leave open are marked "Reading:" in the docstrings.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

__all__ = [
    "i2v_mask", "build_i2v_input", "patchify", "unpatchify", "linear", "patch_embed",
    "conv3d_patch_embed_direct", "sinusoidal_embedding", "silu", "gelu", "time_embed",
    "layer_norm", "modulate", "rms_norm", "rope_segments", "rope_3d", "token_positions",
    "attention", "attention_lse", "lse_merge", "multihead_attention", "context_embed", "cross_kv", "block_fwd",
    "head_fwd", "cfg_combine", "euler_step", "cfg_euler", "dit_fwd", "sample", "sample_cached",
    "self_attention_rope_only", "snr", "t_moe_from_snr", "expert_for_step", "sample_two_expert",
]

f64 = np.float64


def _a(x):
    return np.asarray(x, dtype=f64)


# ---------------------------------------------------------------------------
# a1: image-to-video mask and channel concatenation
# ---------------------------------------------------------------------------
def i2v_mask(T: int, H: int, W: int, known_pixel_frames=None) -> np.ndarray:
    """Four-channel frame mask [4, T, H, W] for image-to-video.

    [I2V-illustrated §4.1, step 3]: a per-pixel-frame mask (1 = known frame,
    first frame only by default) over F = 4(T-1)+1 pixel frames; frame 0's
    entry is repeated 4 times along time and joined with frames 1..F-1, giving
    4T entries, then laid out as [4, T].  Reading: the 4T entries are grouped
    4 per latent frame (latent frame tau covers entries 4*tau .. 4*tau+3) and
    channel c holds entry 4*tau + c -- the layout the Q3 answer in
    [I2V-illustrated §10] describes (each latent frame's 4 channels flag its 4
    pixel frames).  Multi-frame masks follow the Q6 answer there.
    """
    F = 4 * (T - 1) + 1
    if known_pixel_frames is None:
        known = np.zeros(F, dtype=f64)
        known[0] = 1.0
    else:
        known = _a(known_pixel_frames).reshape(-1)
        assert known.shape[0] == F, "known_pixel_frames must have 4(T-1)+1 entries"
        known = (known != 0).astype(f64)
    seq = np.concatenate([np.repeat(known[:1], 4), known[1:]])  # 4T entries
    m = np.empty((4, T), dtype=f64)
    for tau in range(T):
        for c in range(4):
            m[c, tau] = seq[4 * tau + c]
    return np.broadcast_to(m[:, :, None, None], (4, T, H, W)).copy()


def build_i2v_input(x_t, z_img, known_pixel_frames=None) -> np.ndarray:
    """x_in = [x_t, mask, z_img] along channels: 16 + 4 + 16 = 36 channels.

    [I2V-illustrated §4.1 step 4 and §4.2]: y = concat(mask, image latent)
    (4 + 16 = 20 channels), then x = concat(x_t, y).  The order [x_t, mask,
    z_img] is the one these sections give (the TI2V-5B page §4.2 lists another
    order; this build follows the Wan2.1 page).
    """
    x_t, z_img = _a(x_t), _a(z_img)
    B, C, T, H, W = x_t.shape
    m = i2v_mask(T, H, W, known_pixel_frames)
    m = np.broadcast_to(m[None], (B, 4, T, H, W))
    return np.concatenate([x_t, m, z_img], axis=1)


# ---------------------------------------------------------------------------
# a2 / a11: (1,2,2) patchify and its inverse
# ---------------------------------------------------------------------------
def patchify(x) -> np.ndarray:
    """[B, C, T, H, W] -> [B, S, 4C] patch vectors.

    [I2V-illustrated §5.1]: a Conv3d with kernel = stride = (1,2,2) turns each
    1x2x2 block into one token; S = T * (H/2) * (W/2).  Reading: token order
    is (frame, row, column) row-major, and the patch vector is ordered like a
    flattened Conv3d weight (c, kt, kh, kw), i.e. index c*4 + kh*2 + kw.
    """
    x = _a(x)
    B, C, T, H, W = x.shape
    assert H % 2 == 0 and W % 2 == 0
    Hp, Wp = H // 2, W // 2
    S = T * Hp * Wp
    p = np.empty((B, S, 4 * C), dtype=f64)
    for f in range(T):
        for i in range(Hp):
            for j in range(Wp):
                s = (f * Hp + i) * Wp + j
                blk = x[:, :, f, 2 * i:2 * i + 2, 2 * j:2 * j + 2]  # [B, C, 2(kh), 2(kw)]
                p[:, s, :] = blk.reshape(B, 4 * C)
    return p


def unpatchify(p, C: int, T: int, H: int, W: int) -> np.ndarray:
    """Exact inverse of ``patchify``: [B, S, 4C] -> [B, C, T, H, W]  ([I2V-illustrated §5.5]:
    the head 'with unpatchify' maps [B, S, dim] back to [C, T, H, W])."""
    p = _a(p)
    B = p.shape[0]
    Hp, Wp = H // 2, W // 2
    assert p.shape[1] == T * Hp * Wp and p.shape[2] == 4 * C
    x = np.empty((B, C, T, H, W), dtype=f64)
    for f in range(T):
        for i in range(Hp):
            for j in range(Wp):
                s = (f * Hp + i) * Wp + j
                x[:, :, f, 2 * i:2 * i + 2, 2 * j:2 * j + 2] = p[:, s, :].reshape(B, C, 2, 2)
    return x


# ---------------------------------------------------------------------------
# linear algebra helpers and a3 patch embedding
# ---------------------------------------------------------------------------
def linear(x, w, b=None) -> np.ndarray:
    y = _a(x) @ _a(w).T
    if b is not None:
        y = y + _a(b)
    return y


def patch_embed(p, w_pe, b_pe) -> np.ndarray:
    """z = P @ W_pe.T + b: the Conv3d patch embedding of [I2V-illustrated §5.1] written as
    a matrix product over patch vectors (W_pe is the Conv3d weight [dim, C, 1, 2, 2]
    flattened to [dim, 4C])."""
    return linear(p, w_pe, b_pe)


def conv3d_patch_embed_direct(x, w_pe, b_pe) -> np.ndarray:
    """Direct Conv3d (kernel = stride = (1,2,2)) by explicit loops, tokens in (f, i, j)
    order.  Used only to pin ``patchify`` + ``patch_embed`` on tiny inputs."""
    x, w, b = _a(x), _a(w_pe), _a(b_pe)
    B, C, T, H, W = x.shape
    dim = w.shape[0]
    wk = w.reshape(dim, C, 1, 2, 2)
    Hp, Wp = H // 2, W // 2
    out = np.zeros((B, T * Hp * Wp, dim), dtype=f64)
    for bb in range(B):
        for f in range(T):
            for i in range(Hp):
                for j in range(Wp):
                    s = (f * Hp + i) * Wp + j
                    for o in range(dim):
                        acc = b[o]
                        for c in range(C):
                            for kh in range(2):
                                for kw in range(2):
                                    acc += wk[o, c, 0, kh, kw] * x[bb, c, f, 2 * i + kh, 2 * j + kw]
                        out[bb, s, o] = acc
    return out


# ---------------------------------------------------------------------------
# a4: timestep embedding and shared modulation MLP
# ---------------------------------------------------------------------------
def sinusoidal_embedding(t: float, freq_dim: int = 256, t_scale: float = 1000.0,
                         base: float = 10000.0) -> np.ndarray:
    """Scalar t -> freq_dim-vector [cos(tau * f_i) | sin(tau * f_i)], f_i = base^(-i/half).

    [I2V-illustrated §5.2]: 'sinusoidal_embedding_1d(256, t)'.  Reading (parity
    unpinned beyond its special cases): tau = 1000 t (t in [0, 1] mapped onto a
    1000-step scale), base 10000, cosines first.
    """
    half = freq_dim // 2
    tau = t_scale * float(t)
    freqs = np.array([base ** (-i / half) for i in range(half)], dtype=f64)
    return np.concatenate([np.cos(tau * freqs), np.sin(tau * freqs)])


def silu(x):
    x = _a(x)
    return x / (1.0 + np.exp(-x))


def gelu(x):
    """Exact GELU x * Phi(x).  Reading: the pages say 'GELU' without a variant."""
    x = _a(x)
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


def time_embed(t: float, w: dict, freq_dim: int = 256):
    """(e [dim], e0 [6, dim]) from a scalar t.

    [I2V-illustrated §5.2]: e = time_embedding(sinusoid(t)) (an MLP to dim),
    e0 = time_projection(e) reshaped to [6, dim].  [Wan-deep-dive §2.5]: one
    MLP shared by all blocks predicts the 6 modulation vectors.  Reading: both
    MLPs use SiLU (Linear -> SiLU -> Linear; SiLU -> Linear).
    """
    emb = sinusoidal_embedding(t, freq_dim)
    h = silu(linear(emb, w["wt1"], w["bt1"]))
    e = linear(h, w["wt2"], w["bt2"])
    e0 = linear(silu(e), w["wtp"], w["btp"])
    return e, e0.reshape(6, -1)


# ---------------------------------------------------------------------------
# norms
# ---------------------------------------------------------------------------
def layer_norm(x, eps: float = 1e-6, weight=None, bias=None):
    """LayerNorm over the last axis: (x - mean) / sqrt(var + eps) [* weight + bias].
    Biased variance (divide by n)."""
    x = _a(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    y = (x - mu) / np.sqrt(var + eps)
    if weight is not None:
        y = y * _a(weight)
    if bias is not None:
        y = y + _a(bias)
    return y


def modulate(xn, shift, scale):
    """adaLN modulation x' = norm(x) * (1 + scale) + shift  ([I2V-illustrated §5.2])."""
    return _a(xn) * (1.0 + _a(scale)) + _a(shift)


def rms_norm(x, g, eps: float = 1e-6):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g.

    [I2V-illustrated §5.3 ①]: q = RMSNorm(Linear_q(x)), k likewise.  Reading:
    the norm spans the full model dim (all heads together) and has a learned
    gain g; eps = 1e-6.
    """
    x = _a(x)
    r = 1.0 / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    return x * r * _a(g)


# ---------------------------------------------------------------------------
# 3D RoPE
# ---------------------------------------------------------------------------
def rope_segments(head_dim: int):
    """Channel split of one head for (time, height, width): [I2V-illustrated §5.3 ②]
    gives d - 4*(d/6), 2*(d/6), 2*(d/6) with d/6 rounded down."""
    q6 = head_dim // 6
    return head_dim - 4 * q6, 2 * q6, 2 * q6


def token_positions(grid):
    """(f, i, j) of every token in (frame, row, column) row-major order -> int [S, 3]."""
    T, Hp, Wp = grid
    f, i, j = np.meshgrid(np.arange(T), np.arange(Hp), np.arange(Wp), indexing="ij")
    return np.stack([f.reshape(-1), i.reshape(-1), j.reshape(-1)], axis=1)


def rope_3d(x, pos, theta: float = 10000.0):
    """Rotate [N, heads, hd] by 3D factorised RoPE at positions pos [N, 3] = (f, i, j).

    [I2V-illustrated §5.3 ②]: each head's channels split into time / height /
    width segments; each segment is rotated by a 1D RoPE (complex rotation) of
    its own axis' index, then the segments are joined back.  Reading (RoFormer,
    which the page cites): a segment of width n rotates channel pairs (2m, 2m+1)
    as a complex number by angle pos * theta^(-2m/n), theta = 10000, i.e.
    (a, b) -> (a cos - b sin, a sin + b cos).
    """
    x = _a(x)
    N, H, hd = x.shape
    pos = np.asarray(pos)
    segs = rope_segments(hd)
    out = x.copy()
    c0 = 0
    for axis, n in enumerate(segs):
        for m in range(n // 2):
            ang = pos[:, axis].astype(f64) * (theta ** (-2.0 * m / n))  # [N]
            c, s = np.cos(ang)[:, None], np.sin(ang)[:, None]
            a = x[:, :, c0 + 2 * m]
            b = x[:, :, c0 + 2 * m + 1]
            out[:, :, c0 + 2 * m] = a * c - b * s
            out[:, :, c0 + 2 * m + 1] = a * s + b * c
        c0 += n
    return out


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def attention(q, k, v):
    """softmax(q k^T / sqrt(d)) v for one head: q [Nq, d], k [Nk, d], v [Nk, dv].

    Full, non-causal, unmasked ([I2V-illustrated §5.3]: every video token sees
    every other; [Wan-deep-dive §2.5]: global, non-causal attention).  The
    softmax subtracts the row maximum before exponentiating.
    """
    q, k, v = _a(q), _a(k), _a(v)
    s = (q @ k.T) / math.sqrt(q.shape[-1])
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return p @ v


def attention_lse(q, k, v):
    """(o, lse) for one head: o = attention(q, k, v) and lse [Nq] the natural
    log of the softmax normaliser, lse_i = log sum_j exp(<q_i, k_j> / sqrt(d)).

    [Wan-deep-dive §5.2] shards the sequence across GPUs with RingAttention (the
    outer level of 2D context parallelism): each GPU attends its queries to one
    key/value shard at a time.  Reading: the page does not spell out how the
    per-shard results combine; the normaliser of each shard travels with its
    output as this log-sum-exp, and ``lse_merge`` combines them exactly.
    """
    q, k, v = _a(q), _a(k), _a(v)
    s = (q @ k.T) / math.sqrt(q.shape[-1])
    m = s.max(axis=-1, keepdims=True)
    p = np.exp(s - m)
    z = p.sum(axis=-1, keepdims=True)
    return (p / z) @ v, (m + np.log(z))[:, 0]


def lse_merge(outs, lses):
    """Combine attention results over disjoint key chunks of the same queries.

    outs[n] [Nq, dv] and lses[n] [Nq] from ``attention_lse`` on chunk n.  The
    softmax over the union of the chunks weighs chunk n's normalised output by
    its share of the total normaliser: with lse = log sum_n exp(lses[n]),
    o = sum_n exp(lses[n] - lse) * outs[n].  Returns (o, lse).
    """
    L = np.stack([_a(x) for x in lses])          # [N, Nq]
    m = L.max(axis=0)
    lse = m + np.log(np.exp(L - m).sum(axis=0))
    o = sum(np.exp(L[n] - lse)[:, None] * _a(outs[n]) for n in range(len(outs)))
    return o, lse


def multihead_attention(q, k, v, heads: int):
    """q [Nq, heads*hd], k/v [Nk, heads*hd] -> o [Nq, heads*hd], head by head."""
    q, k, v = _a(q), _a(k), _a(v)
    hd = q.shape[-1] // heads
    o = np.empty_like(q)
    for h in range(heads):
        sl = slice(h * hd, (h + 1) * hd)
        o[:, sl] = attention(q[:, sl], k[:, sl], v[:, sl])
    return o


def self_attention_rope_only(q, k, v, grid, rows=None, theta: float = 10000.0):
    """Self-attention core with 3D RoPE on q and k (no projections, no norms):
    q, k, v [S, heads, hd] -> o [R, heads, hd] for the query rows ``rows``."""
    q, k, v = _a(q), _a(k), _a(v)
    S, H, hd = q.shape
    pos = token_positions(grid)
    rows = np.arange(S) if rows is None else np.asarray(rows)
    qr = rope_3d(q[rows], pos[rows], theta)
    kr = rope_3d(k, pos, theta)
    o = np.empty((len(rows), H, hd), dtype=f64)
    for h in range(H):
        o[:, h, :] = attention(qr[:, h, :], kr[:, h, :], v[:, h, :])
    return o


# ---------------------------------------------------------------------------
# context embedding and cross-attention K/V
# ---------------------------------------------------------------------------
def context_embed(ctx, w1, b1, w2, b2):
    """Two-layer GELU MLP to the model dim.  [I2V-illustrated §7 steps 1-2]: umT5 output
    [512, 4096] -> MLP -> [512, dim]; CLIP tokens [257, 1280] -> MLPProj -> [257, dim].
    Reading: Linear -> GELU -> Linear for both (the implementation is pinned against PyTorch
    modules; the MLP shape is not on the pages)."""
    return linear(gelu(linear(ctx, w1, b1)), w2, b2)


def cross_kv(ctx_emb, wk, bk, wv, bv):
    """K, V of one cross-attention stream from embedded context [L, dim]
    ([I2V-illustrated §5.4]: k = Linear_k(context), v = Linear_v(context))."""
    return linear(ctx_emb, wk, bk), linear(ctx_emb, wv, bv)


# ---------------------------------------------------------------------------
# a5..a10: one DiT block
# ---------------------------------------------------------------------------
def block_fwd(x, e0, w: dict, kv, grid, heads: int, rows=None,
              ln_eps: float = 1e-6, rms_eps: float = 1e-6, theta: float = 10000.0, attn_cache=None):
    """One DiT block on [B, S, dim] tokens.

    Follows [I2V-illustrated §5.2-§5.5] in the order self-attention ->
    cross-attention -> FFN:
      mod = e0[b] + b_i -> (shift1, scale1, gate1, shift2, scale2, gate2)
        ([I2V-illustrated §5.2]; per-block bias [Wan-deep-dive §2.5]);
      u  = LN(x) (1 + scale1) + shift1;
      q  = RoPE(RMSNorm(u Wq^T + bq)), k = RoPE(RMSNorm(u Wk^T + bk)), v = u Wv^T + bv;
      x += gate1 * (Attn(q, k, v) Wo^T + bo)            (full non-causal, §5.3);
      c  = LN(x) * ln3_w + ln3_b                         (no adaLN on cross-attention, §5.2);
      qc = c Wcq^T + bcq;  o = Attn(qc, K_txt, V_txt) [+ Attn(qc, K_img, V_img)]  (§5.4);
      x += o Wco^T + bco;
      u2 = LN(x) (1 + scale2) + shift2;
      x += gate2 * (GELU(u2 W1^T + b1) W2^T + b2)         (§5.5).
    Readings: LayerNorms have eps 1e-6 and no affine except the cross-attention
    pre-norm, which is affine; cross-attention has no RoPE and no q/k norm;
    attention scale 1/sqrt(head_dim).

    ``kv[b]`` = (K_txt, V_txt, K_img, V_img) with the image pair None for
    single-stream cross-attention.  With ``rows`` given, K/V of self-attention
    are computed for all S tokens and everything else only for those query
    rows; the result is then [B, len(rows), dim] and equals those rows of the
    full output exactly (every step but self-attention is token-local).

    attn_cache (the attention cache of [Wan-deep-dive §5.3], which reuses attention outputs across
    sampling steps): None, or {"mode": "store" | "reuse", "y": array [B, len(rows), dim]}.  Reading:
    the cached quantity is the self-attention layer's output y = o W_o^T + b_o before the gate; "store"
    computes and records it, "reuse" skips the self-attention layer and uses the recorded y, with
    the current step's gate1.
    """
    x, e0 = _a(x), _a(e0)
    B, S, dim = x.shape
    pos = token_positions(grid)
    assert pos.shape[0] == S
    rows = np.arange(S) if rows is None else np.asarray(rows)
    hd = dim // heads
    out = np.empty((B, len(rows), dim), dtype=f64)
    for b in range(B):
        mod = e0[b] + _a(w["mod_bias"])
        shift1, scale1, gate1, shift2, scale2, gate2 = mod
        # self-attention
        if attn_cache is not None and attn_cache["mode"] == "reuse":
            ya = _a(attn_cache["y"][b])
        else:
            u = modulate(layer_norm(x[b], ln_eps), shift1, scale1)
            k = rms_norm(linear(u, w["wk"], w["bk"]), w["gk"], rms_eps)
            v = linear(u, w["wv"], w["bv"])
            q = rms_norm(linear(u[rows], w["wq"], w["bq"]), w["gq"], rms_eps)
            q = rope_3d(q.reshape(len(rows), heads, hd), pos[rows], theta).reshape(len(rows), dim)
            k = rope_3d(k.reshape(S, heads, hd), pos, theta).reshape(S, dim)
            o = multihead_attention(q, k, v, heads)
            ya = linear(o, w["wo"], w["bo"])
            if attn_cache is not None:
                attn_cache["y"][b] = ya
        xr = x[b, rows] + gate1 * ya
        # cross-attention
        c = layer_norm(xr, ln_eps, w["ln3_w"], w["ln3_b"])
        qc = linear(c, w["wcq"], w["bcq"])
        k_txt, v_txt, k_img, v_img = kv[b]
        oc = multihead_attention(qc, k_txt, v_txt, heads)
        if k_img is not None:
            oc = oc + multihead_attention(qc, k_img, v_img, heads)
        xr = xr + linear(oc, w["wco"], w["bco"])
        # FFN
        u2 = modulate(layer_norm(xr, ln_eps), shift2, scale2)
        y = linear(gelu(linear(u2, w["w1"], w["b1"])), w["w2"], w["b2"])
        out[b] = xr + gate2 * y
    return out


# ---------------------------------------------------------------------------
# a11: head
# ---------------------------------------------------------------------------
def head_fwd(x, e, w: dict, ln_eps: float = 1e-6):
    """Head: (shift, scale) = head_mod + e; out = (LN(x)(1 + scale) + shift) Wh^T + bh.

    [I2V-illustrated §5.5]: a head 'also with AdaLN and unpatchify' maps
    [B, S, dim] back to the latent.  Reading (not on the pages; the implementation is pinned
    against PyTorch's layer_norm + linear): two modulation vectors (shift first) from a learned
    [2, dim] bias plus e.
    x [B, S, dim], e [B, dim] -> [B, S, 4*C_out].
    """
    x, e = _a(x), _a(e)
    out = []
    for b in range(x.shape[0]):
        mod = _a(w["head_mod"]) + e[b][None, :]
        u = modulate(layer_norm(x[b], ln_eps), mod[0], mod[1])
        out.append(linear(u, w["wh"], w["bh"]))
    return np.stack(out)


# ---------------------------------------------------------------------------
# a12: classifier-free guidance and the flow-matching Euler step
# ---------------------------------------------------------------------------
def cfg_combine(v_cond, v_uncond, s: float):
    """v = v_u + s (v_c - v_u)  ([I2V-illustrated §7], CFG note)."""
    v_cond, v_uncond = _a(v_cond), _a(v_uncond)
    return v_uncond + s * (v_cond - v_uncond)


def euler_step(x, v, dt: float):
    """x <- x + dt * v with a signed dt.  [I2V-illustrated §7]: x_{t-Δt} = x_t - v Δt
    with t going 1 -> 0 (dt = -Δt); [Wan-deep-dive §2.7]: Euler integration of the
    flow-matching ODE."""
    return _a(x) + dt * _a(v)


def cfg_euler(x, v_cond, v_uncond, s: float, dt: float):
    v = _a(v_cond) if v_uncond is None else cfg_combine(v_cond, v_uncond, s)
    return euler_step(x, v, dt)


# ---------------------------------------------------------------------------
# a13: one DiT evaluation and the sampling loop
# ---------------------------------------------------------------------------
def dit_fwd(x_in, t, model_w: dict, blocks_w, ctx_txt, ctx_img, heads: int,
            ln_eps: float = 1e-6, rms_eps: float = 1e-6, theta: float = 10000.0,
            freq_dim: int = 256, out_channels: int = 16, attn_caches=None):
    """One DiT call v = DiT(x_in, t, context) ([I2V-illustrated §7], sampling loop).

    x_in [B, C_in, T, H, W]; t scalar or [B]; ctx_txt [B, L, text_dim];
    ctx_img [L_img, img_dim] or None (shared by every row).  ``blocks_w`` is a
    sequence of per-block weight dicts (or a callable i -> dict).
    """
    x_in = _a(x_in)
    B, C_in, T, H, W = x_in.shape
    grid = (T, H // 2, W // 2)
    tt = np.broadcast_to(_a(t), (B,))
    x = patch_embed(patchify(x_in), model_w["w_pe"], model_w["b_pe"])
    es, e0s = zip(*[time_embed(tt[b], model_w, freq_dim) for b in range(B)])
    e, e0 = np.stack(es), np.stack(e0s)
    txt = np.stack([context_embed(ctx_txt[b], model_w["wtx1"], model_w["btx1"],
                                  model_w["wtx2"], model_w["btx2"]) for b in range(B)])
    img = None
    if ctx_img is not None:
        img = context_embed(ctx_img, model_w["wim1"], model_w["bim1"],
                            model_w["wim2"], model_w["bim2"])
    nblocks = len(blocks_w) if not callable(blocks_w) else None
    i = 0
    while True:
        if nblocks is not None and i >= nblocks:
            break
        w = blocks_w[i] if nblocks is not None else blocks_w(i)
        if w is None:
            break
        kv = []
        for b in range(B):
            kt, vt = cross_kv(txt[b], w["wck"], w["bck"], w["wcv"], w["bcv"])
            ki = vi = None
            if img is not None:
                ki, vi = cross_kv(img, w["wki"], w["bki"], w["wvi"], w["bvi"])
            kv.append((kt, vt, ki, vi))
        x = block_fwd(x, e0, w, kv, grid, heads, ln_eps=ln_eps, rms_eps=rms_eps, theta=theta,
                      attn_cache=None if attn_caches is None else attn_caches[i])
        i += 1
    out = head_fwd(x, e, model_w, ln_eps)
    return unpatchify(out, out_channels, T, H, W)


def sample(x_T, z_img, steps: int, guidance: float, model_w, blocks_w, ctx_txt, ctx_img,
           heads: int, t0: float = 1.0, known_pixel_frames=None, **kw):
    """Flow-matching Euler sampling with optional CFG ([I2V-illustrated §7]).

    Schedule t_k = t0 - k*t0/steps, dt = -t0/steps.  x_T [1, C, T, H, W].  With
    ctx_txt holding two rows (conditional, unconditional) both DiT rows see the
    same x_in and v = v_u + s (v_c - v_u); with one row v = v_c.  z_img None means
    text-to-video (x_in = x_t).  Returns the final latent and the per-step list.
    """
    x = _a(x_T)
    B = _a(ctx_txt).shape[0]
    dt = -t0 / steps
    traj = []
    for k in range(steps):
        t = t0 + k * dt
        x_in = x if z_img is None else build_i2v_input(x, z_img, known_pixel_frames)
        x_in = np.repeat(x_in, B, axis=0)
        v = dit_fwd(x_in, t, model_w, blocks_w, ctx_txt, ctx_img, heads, **kw)
        x = cfg_euler(x, v[0:1], v[1:2] if B > 1 else None, guidance, dt)
        traj.append(x.copy())
    return x, traj


def sample_cached(x_T, z_img, steps: int, guidance: float, model_w, blocks_w, ctx_txt, ctx_img,
                  heads: int, attn_reuse, cfg_reuse, t0: float = 1.0, known_pixel_frames=None, **kw):
    """``sample`` with the diffusion cache of [Wan-deep-dive §5.3] (attention cache + CFG cache).

    Reading (the page gives neither the cached quantities nor the schedule):
    * attention cache: on a step with attn_reuse[k], every block reuses the self-attention layer
      output y = o W_o^T + b_o it recorded at the last step that computed it (per CFG row), with the
      current gate (see ``block_fwd``); other steps compute and record it.  attn_reuse[0] must be
      False.
    * CFG cache: on a step with cfg_reuse[k], the unconditional row is not evaluated and v_u is the
      one of the last step that evaluated it; cfg_reuse[0] must be False.  Only the conditional row
      then runs (its attention cache is updated as usual; the unconditional row's is left as is).
    With both lists all False this is exactly ``sample``.
    """
    x = _a(x_T)
    Bfull = _a(ctx_txt).shape[0]
    assert not attn_reuse[0] and not cfg_reuse[0]
    dt = -t0 / steps
    nblocks = len(blocks_w)
    S = x.shape[2] * (x.shape[3] // 2) * (x.shape[4] // 2)
    dim = _a(model_w["b_pe"]).shape[0]
    ycache = [np.zeros((Bfull, S, dim)) for _ in range(nblocks)]
    v_u = None
    traj = []
    for k in range(steps):
        t = t0 + k * dt
        B = 1 if (cfg_reuse[k] and Bfull > 1) else Bfull
        x_in = x if z_img is None else build_i2v_input(x, z_img, known_pixel_frames)
        x_in = np.repeat(x_in, B, axis=0)
        mode = "reuse" if attn_reuse[k] else "store"
        caches = [{"mode": mode, "y": ycache[i][:B]} for i in range(nblocks)]
        v = dit_fwd(x_in, t, model_w, blocks_w, _a(ctx_txt)[:B], ctx_img, heads, attn_caches=caches, **kw)
        if Bfull > 1 and B > 1:
            v_u = v[1:2].copy()
        x = cfg_euler(x, v[0:1], v_u if Bfull > 1 else None, guidance, dt)
        traj.append(x.copy())
    return x, traj


# ---------------------------------------------------------------------------
# next row: the Wan2.2 timestep-level two-expert switch
# ---------------------------------------------------------------------------
def snr(t):
    """Signal-to-noise ratio of the straight path x_t = (1 - t) x0 + t eps ([I2V-illustrated §7]):
    the signal weight squared over the noise weight squared, ((1 - t) / t)^2; infinite at t = 0."""
    t = _a(t)
    with np.errstate(divide="ignore"):
        return ((1.0 - t) / t) ** 2


def t_moe_from_snr(snr_min: float) -> float:
    """The switch time of [Wan-deep-dive §7.2]: the t at which the SNR is half of snr_min.

    On the straight path SNR falls monotonically from infinity (t = 0) to 0 (t = 1), so the
    solution is unique: (1 - t) / t = sqrt(snr_min / 2).  With snr_min = 0 (a schedule that starts at
    pure noise, t = 1) it is t = 1 and the high-noise expert never runs.
    """
    return 1.0 / (1.0 + math.sqrt(snr_min / 2.0))


def expert_for_step(t: float, t_moe: float) -> int:
    """0 = the high-noise expert (t > t_moe), 1 = the low-noise expert (t <= t_moe)
    ([Wan-deep-dive §7.2], its phase table)."""
    return 0 if t > t_moe else 1


def sample_two_expert(x_T, z_img, steps: int, guidance: float, experts, t_moe: float, ctx_txt, ctx_img,
                      heads: int, t0: float = 1.0, known_pixel_frames=None, **kw):
    """``sample`` with the timestep-level two-expert switch of [Wan-deep-dive §7.2]: experts =
    ((model_w, blocks_w) of the high-noise expert, (model_w, blocks_w) of the low-noise one), each a
    whole DiT; step k evaluates the expert ``expert_for_step(t_k, t_moe)`` selects.  Schedule, CFG and
    the Euler update as in ``sample``.  Returns the final latent, the per-step list and the expert
    index of each step."""
    x = _a(x_T)
    B = _a(ctx_txt).shape[0]
    dt = -t0 / steps
    traj, used = [], []
    for k in range(steps):
        t = t0 + k * dt
        e = expert_for_step(t, t_moe)
        model_w, blocks_w = experts[e]
        x_in = x if z_img is None else build_i2v_input(x, z_img, known_pixel_frames)
        x_in = np.repeat(x_in, B, axis=0)
        v = dit_fwd(x_in, t, model_w, blocks_w, ctx_txt, ctx_img, heads, **kw)
        x = cfg_euler(x, v[0:1], v[1:2] if B > 1 else None, guidance, dt)
        traj.append(x.copy())
        used.append(e)
    return x, traj, used

# Parity status of each function, as checked by the CPU tests.
PARITY = {
    "i2v_mask": "pinned: hand-worked fixtures (first frame; first+last frame); 4+16=20 channels",
    "build_i2v_input": "pinned: 16+20=36 channels; channel blocks equal x_t / mask / z_img",
    "patchify": "pinned: hand-worked fixture; S = T*(H/2)*(W/2); round trip; direct Conv3d loop",
    "unpatchify": "pinned: exact inverse of patchify (round trip), hand-worked fixture",
    "patch_embed": "pinned: equals a direct Conv3d (kernel = stride = (1,2,2)) loop",
    "sinusoidal_embedding": "pinned: t = 0 gives [1..1 | 0..0]; unit-modulus (cos,sin) pairs",
    "time_embed": "parity unpinned (the pages name the MLP and its [6, dim] output, not its layers): "
                  "the reading's implementation is checked against PyTorch float64 Linear/SiLU modules "
                  "with the same weights and an identity-weight special case",
    "layer_norm": "pinned: zero mean / unit variance; constant row -> bias; numpy.var cross-check",
    "rms_norm": "pinned: constant row c -> g c / sqrt(c^2 + eps); unit RMS for g = 1",
    "rope_3d": "pinned: segment sizes 44/42/42 and 24/20/20; identity at (0,0,0); norm "
               "preserved; relative-position property per axis; per-axis segment isolation; "
               "1D complex-exponential RoPE special case",
    "attention": "pinned: brute-force pure-Python softmax; K = 0 -> mean of V; single key; "
                 "joint permutation of keys; key-chunked log-sum-exp merge",
    "attention_lse": "pinned: K = 0 -> lse = log Nk; single key -> lse = its scaled score; "
                     "brute-force pure-Python log of the normaliser",
    "lse_merge": "pinned: merging key chunks reproduces attention() and attention_lse() over "
                 "all keys (for several chunkings, one-key chunks included); one part -> itself",
    "block_fwd": "pinned: adaLN-Zero identity; closed forms of each branch with the others switched "
                 "off (scale1 = -1 and scale2 = -1 make the branch input equal its shift; uniform "
                 "attention with identity value/output projections; a constant cross-attention input "
                 "from ln3_w = 0 with two text keys and one image key; the sign of a two-token RoPE "
                 "score from the q and k gains); self-attention before cross-attention; sampled-row "
                 "mode; non-causality",
    "head_fwd": "parity unpinned (the pages say only that the head has adaLN and unpatchify): the "
                "reading's implementation equals PyTorch layer_norm with weight 1 + scale and bias "
                "shift, then linear",
    "context_embed": "parity unpinned (the pages name an MLP, not its layers): the reading's "
                     "implementation equals PyTorch Linear -> exact GELU -> Linear with the same weights",
    "cfg_combine": "pinned: s = 1 -> v_c, s = 0 -> v_u",
    "euler_step": "pinned: straight-line path lands exactly on the endpoint",
    "sample": "pinned through cfg_combine / euler_step; DiT part as block_fwd",
    "snr": "pinned: t = 1 -> 0, t = 1/2 -> 1, t -> 0 -> infinity; equals the squared ratio of the "
           "coefficients of x0 and eps in the straight path at hand-picked t",
    "t_moe_from_snr": "pinned: snr_min = 2 -> 1/2; snr_min = 0 -> 1; snr(t_moe) = snr_min / 2 by "
                      "bisection on the monotone snr",
    "expert_for_step": "pinned: the boundary t = t_moe goes to the low-noise expert; hand-worked "
                       "sequence for 4 steps from t = 1 at t_moe = 1/2",
    "sample_two_expert": "pinned: the same expert twice -> sample; t_moe >= t0 -> sample with the "
                         "low-noise expert; a mixed run equals the high expert's first k steps of "
                         "sample followed by sample with the low expert from t_k",
    "sample_cached": "pinned: no reuse -> sample; attention reuse with gate1 = 0 -> sample; CFG reuse "
                     "with guidance 1 -> sample; storing changes nothing; reuse of a zero cache -> "
                     "the block without its self-attention branch",
}
