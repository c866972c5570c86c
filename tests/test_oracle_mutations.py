"""Planted mistakes in the CPU oracle must be caught by its pins (no GPU).

Each case swaps one oracle function for a plausible wrong version (a dropped
term, a wrong sign, index or layout) inside the oracle module and requires that
at least one pin in ``oracle_pins`` fails.  The mistakes are planted in the
oracle, on the CPU, never in the HIP path.
"""
import math

import numpy as np
import pytest

from oracle import wan_oracle as wo
from tests import oracle_pins as pins


def _mask_raw_reshape(T, H, W, known_pixel_frames=None):
    F = 4 * (T - 1) + 1
    known = np.zeros(F) if known_pixel_frames is None else np.asarray(known_pixel_frames, float)
    if known_pixel_frames is None:
        known[0] = 1
    seq = np.concatenate([np.repeat(known[:1], 4), known[1:]])
    m = seq.reshape(4, T)  # raw reshape instead of grouping 4 entries per latent frame
    return np.broadcast_to(m[:, :, None, None], (4, T, H, W)).copy()


def _patchify_kw_kh(x):
    x = np.asarray(x, float)
    B, C, T, H, W = x.shape
    p = wo.__dict__["_orig_patchify"](x)
    return p.reshape(B, -1, C, 2, 2).transpose(0, 1, 2, 4, 3).reshape(B, -1, 4 * C)


def _rope_variant(kind):
    def rope(x, pos, theta=10000.0):
        x = np.asarray(x, float)
        N, H, hd = x.shape
        segs = list(wo.rope_segments(hd))
        if kind == "segments_swapped":
            segs = [segs[1], segs[0], segs[2]]
        out = x.copy()
        c0 = 0
        for axis, n in enumerate(segs):
            for m in range(n // 2):
                width = hd if kind == "freq_over_head_dim" else n
                ang = pos[:, axis] * theta ** (-2.0 * m / width)
                c, s = np.cos(ang)[:, None], np.sin(ang)[:, None]
                if kind == "rotate_half":
                    i0, i1 = c0 + m, c0 + m + n // 2
                else:
                    i0, i1 = c0 + 2 * m, c0 + 2 * m + 1
                a, b = x[:, :, i0], x[:, :, i1]
                if kind == "sign":
                    out[:, :, i0], out[:, :, i1] = a * c + b * s, -a * s + b * c
                else:
                    out[:, :, i0], out[:, :, i1] = a * c - b * s, a * s + b * c
            c0 += n
        return out
    return rope


def _attention_variant(kind):
    def attn(q, k, v):
        q, k, v = (np.asarray(a, float) for a in (q, k, v))
        scale = 1.0 / q.shape[-1] if kind == "scale_1_over_d" else 1.0 / math.sqrt(q.shape[-1])
        s = q @ k.T * scale
        axis = 0 if kind == "softmax_over_queries" else -1
        p = np.exp(s - s.max(axis=axis, keepdims=True))
        p = p / p.sum(axis=axis, keepdims=True)
        return p @ v
    return attn


def _lse_variant(kind):
    def attention_lse(q, k, v):
        q, k, v = (np.asarray(a, float) for a in (q, k, v))
        s = q @ k.T / math.sqrt(q.shape[-1])
        m = s.max(-1, keepdims=True)
        p = np.exp(s - m)
        z = p.sum(-1, keepdims=True)
        if kind == "log2":
            lse = (m + np.log2(z))[:, 0]
        elif kind == "no_scale":
            lse = np.log(np.exp(q @ k.T).sum(-1))
        else:  # max dropped
            lse = np.log(z)[:, 0]
        return (p / z) @ v, lse
    return attention_lse


def _lse_merge_max_weights(outs, lses):
    # weights relative to the largest chunk normaliser instead of the total one
    L = np.stack([np.asarray(x, float) for x in lses])
    m = L.max(0)
    o = sum(np.exp(L[n] - m)[:, None] * np.asarray(outs[n], float) for n in range(len(outs)))
    return o, m + np.log(np.exp(L - m).sum(0))


def _ln_unbiased(x, eps=1e-6, weight=None, bias=None):
    x = np.asarray(x, float)
    mu = x.mean(-1, keepdims=True)
    y = (x - mu) / np.sqrt(x.var(-1, ddof=1, keepdims=True) + eps)
    if weight is not None:
        y = y * weight
    if bias is not None:
        y = y + bias
    return y


def _rms_sum(x, g, eps=1e-6):
    x = np.asarray(x, float)
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + eps) * g


def _modulate_no_one(xn, shift, scale):
    return np.asarray(xn) * np.asarray(scale) + np.asarray(shift)


def _euler_wrong_sign(x, v, dt):
    return np.asarray(x) - dt * np.asarray(v)


def _cfg_swapped(v_cond, v_uncond, s):
    return np.asarray(v_cond) + s * (np.asarray(v_uncond) - np.asarray(v_cond))


def _sinusoid_sin_first(t, freq_dim=256, t_scale=1000.0, base=10000.0):
    e = wo.__dict__["_orig_sinusoidal_embedding"](t, freq_dim, t_scale, base)
    h = freq_dim // 2
    return np.concatenate([e[h:], e[:h]])


def _time_embed_no_silu(t, w, freq_dim=256):
    emb = wo.sinusoidal_embedding(t, freq_dim)
    e = wo.linear(wo.silu(wo.linear(emb, w["wt1"], w["bt1"])), w["wt2"], w["bt2"])
    return e, wo.linear(e, w["wtp"], w["btp"]).reshape(6, -1)


def _mha_joint_softmax_factory():
    orig_block = wo.block_fwd

    def block(x, e0, w, kv, grid, heads, rows=None, **kw):
        # one softmax over the concatenated image + text keys instead of two
        kv2 = []
        for kt, vt, ki, vi in kv:
            if ki is None:
                kv2.append((kt, vt, None, None))
            else:
                kv2.append((np.concatenate([ki, kt]), np.concatenate([vi, vt]), None, None))
        return orig_block(x, e0, w, kv2, grid, heads, rows=rows, **kw)
    return block


def _block_ungated_factory():
    orig_block = wo.block_fwd

    def block(x, e0, w, kv, grid, heads, rows=None, **kw):
        # gate1 dropped: the self-attention branch is added with weight 1
        w2 = dict(w)
        mb = np.array(w["mod_bias"], float).copy()
        e0 = np.array(e0, float).copy()
        e0[:, 2, :] = 1.0
        mb[2] = 0.0
        w2["mod_bias"] = mb
        return orig_block(x, e0, w2, kv, grid, heads, rows=rows, **kw)
    return block


def _expert_boundary_high(t, t_moe):
    return 0 if t >= t_moe else 1  # the boundary step given to the high-noise expert


def _expert_swapped(t, t_moe):
    return 1 if t > t_moe else 0


def _t_moe_full_snr(snr_min):
    return 1.0 / (1.0 + math.sqrt(snr_min))  # SNR(t) = snr_min instead of snr_min / 2


def _snr_not_squared(t):
    t = np.asarray(t, float)
    with np.errstate(divide="ignore"):
        return (1.0 - t) / t


def _head_scale_without_one(x, e, w, ln_eps=1e-6):
    x, e = np.asarray(x, float), np.asarray(e, float)
    out = []
    for b in range(x.shape[0]):
        mod = np.asarray(w["head_mod"], float) + e[b][None, :]
        u = wo.layer_norm(x[b], ln_eps) * mod[1] + mod[0]  # scale used without the 1 +
        out.append(wo.linear(u, w["wh"], w["bh"]))
    return np.stack(out)


def _head_shift_scale_swapped(x, e, w, ln_eps=1e-6):
    x, e = np.asarray(x, float), np.asarray(e, float)
    out = []
    for b in range(x.shape[0]):
        mod = np.asarray(w["head_mod"], float) + e[b][None, :]
        u = wo.modulate(wo.layer_norm(x[b], ln_eps), mod[1], mod[0])
        out.append(wo.linear(u, w["wh"], w["bh"]))
    return np.stack(out)


def _context_embed_tanh_gelu(ctx, w1, b1, w2, b2):
    h = wo.linear(ctx, w1, b1)
    g = 0.5 * h * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (h + 0.044715 * h ** 3)))
    return wo.linear(g, w2, b2)


def _time_embed_silu_on_e0(t, w, freq_dim=256):
    emb = wo.sinusoidal_embedding(t, freq_dim)
    h = wo.silu(wo.linear(emb, w["wt1"], w["bt1"]))
    e = wo.linear(h, w["wt2"], w["bt2"])
    e0 = wo.silu(wo.linear(e, w["wtp"], w["btp"]))  # SiLU after the projection instead of before
    return e, e0.reshape(6, -1)


def _block_source_mutant(*edits):
    """block_fwd with text substitutions (old -> new) made in its source, so that one line of the
    composition is planted wrong while the rest stays as written."""
    def factory():
        import inspect
        src = inspect.getsource(wo.__dict__["_orig_block_fwd"])
        for old, new in edits:
            assert old in src, old
            src = src.replace(old, new)
        ns = {}
        exec(compile(src, "<block_fwd mutant>", "exec"), wo.__dict__, ns)
        return ns["block_fwd"]
    return factory


def _block_cross_before_self_factory():
    # cross-attention first, then self-attention, then the FFN (the order of another page's diagram)
    def block(x, e0, w, kv, grid, heads, rows=None, ln_eps=1e-6, rms_eps=1e-6, theta=10000.0, attn_cache=None):
        x, e0 = np.asarray(x, float), np.asarray(e0, float)
        B, S, dim = x.shape
        rows = np.arange(S) if rows is None else np.asarray(rows)
        hd = dim // heads
        pos = wo.token_positions(grid)
        out = np.empty((B, len(rows), dim))
        for b in range(B):
            shift1, scale1, gate1, shift2, scale2, gate2 = e0[b] + np.asarray(w["mod_bias"], float)
            kt, vt, ki, vi = kv[b]
            qc = wo.linear(wo.layer_norm(x[b], ln_eps, w["ln3_w"], w["ln3_b"]), w["wcq"], w["bcq"])
            oc = wo.multihead_attention(qc, kt, vt, heads)
            if ki is not None:
                oc = oc + wo.multihead_attention(qc, ki, vi, heads)
            xc = x[b] + wo.linear(oc, w["wco"], w["bco"])
            u = wo.modulate(wo.layer_norm(xc, ln_eps), shift1, scale1)
            k = wo.rope_3d(wo.rms_norm(wo.linear(u, w["wk"], w["bk"]), w["gk"], rms_eps).reshape(S, heads, hd), pos,
                           theta).reshape(S, dim)
            q = wo.rope_3d(wo.rms_norm(wo.linear(u[rows], w["wq"], w["bq"]), w["gq"], rms_eps)
                           .reshape(len(rows), heads, hd), pos[rows], theta).reshape(len(rows), dim)
            v = wo.linear(u, w["wv"], w["bv"])
            xr = xc[rows] + gate1 * wo.linear(wo.multihead_attention(q, k, v, heads), w["wo"], w["bo"])
            u2 = wo.modulate(wo.layer_norm(xr, ln_eps), shift2, scale2)
            out[b] = xr + gate2 * wo.linear(wo.gelu(wo.linear(u2, w["w1"], w["b1"])), w["w2"], w["b2"])
        return out
    return block


_UNPACK = "shift1, scale1, gate1, shift2, scale2, gate2 = mod"
_LN3 = 'c = layer_norm(xr, ln_eps, w["ln3_w"], w["ln3_b"])'
_CROSS_ADD = 'xr = xr + linear(oc, w["wco"], w["bco"])'
_GQ = 'w["gq"], rms_eps)'
_GK = 'w["gk"], rms_eps)'

MUTANTS = {
    "mask_raw_reshape": ("i2v_mask", lambda: _mask_raw_reshape),
    "patch_vector_kw_kh": ("patchify", lambda: _patchify_kw_kh),
    "rope_rotate_half_pairs": ("rope_3d", lambda: _rope_variant("rotate_half")),
    "rope_freq_over_head_dim": ("rope_3d", lambda: _rope_variant("freq_over_head_dim")),
    "rope_sign": ("rope_3d", lambda: _rope_variant("sign")),
    "rope_segments_swapped": ("rope_3d", lambda: _rope_variant("segments_swapped")),
    "attention_scale_1_over_d": ("attention", lambda: _attention_variant("scale_1_over_d")),
    "attention_softmax_axis": ("attention", lambda: _attention_variant("softmax_over_queries")),
    "lse_log2": ("attention_lse", lambda: _lse_variant("log2")),
    "lse_no_scale": ("attention_lse", lambda: _lse_variant("no_scale")),
    "lse_max_dropped": ("attention_lse", lambda: _lse_variant("max_dropped")),
    "lse_merge_max_weights": ("lse_merge", lambda: _lse_merge_max_weights),
    "layer_norm_unbiased_var": ("layer_norm", lambda: _ln_unbiased),
    "rms_norm_sum_not_mean": ("rms_norm", lambda: _rms_sum),
    "modulate_drops_one": ("modulate", lambda: _modulate_no_one),
    "euler_wrong_sign": ("euler_step", lambda: _euler_wrong_sign),
    "cfg_roles_swapped": ("cfg_combine", lambda: _cfg_swapped),
    "sinusoid_sin_first": ("sinusoidal_embedding", lambda: _sinusoid_sin_first),
    "time_projection_no_silu": ("time_embed", lambda: _time_embed_no_silu),
    "cross_joint_softmax": ("block_fwd", _mha_joint_softmax_factory),
    "self_attention_ungated": ("block_fwd", _block_ungated_factory),
    "expert_boundary_to_high": ("expert_for_step", lambda: _expert_boundary_high),
    "experts_swapped": ("expert_for_step", lambda: _expert_swapped),
    "t_moe_full_snr": ("t_moe_from_snr", lambda: _t_moe_full_snr),
    "snr_not_squared": ("snr", lambda: _snr_not_squared),
    "head_scale_without_one": ("head_fwd", lambda: _head_scale_without_one),
    "head_shift_scale_swapped": ("head_fwd", lambda: _head_shift_scale_swapped),
    "context_embed_tanh_gelu": ("context_embed", lambda: _context_embed_tanh_gelu),
    "time_embed_silu_after_projection": ("time_embed", lambda: _time_embed_silu_on_e0),
    "block_shift_scale_swapped": ("block_fwd", _block_source_mutant(
        (_UNPACK, "scale1, shift1, gate1, scale2, shift2, gate2 = mod"))),
    "block_ffn_shift_scale_swapped": ("block_fwd", _block_source_mutant(
        (_UNPACK, "shift1, scale1, gate1, scale2, shift2, gate2 = mod"))),
    "block_gate_before_scale": ("block_fwd", _block_source_mutant(
        (_UNPACK, "shift1, gate1, scale1, shift2, gate2, scale2 = mod"))),
    "block_chunks_ffn_first": ("block_fwd", _block_source_mutant(
        (_UNPACK, "shift2, scale2, gate2, shift1, scale1, gate1 = mod"))),
    "block_ln3_affine_dropped": ("block_fwd", _block_source_mutant((_LN3, "c = layer_norm(xr, ln_eps)"))),
    "block_ln3_weight_bias_swapped": ("block_fwd", _block_source_mutant(
        (_LN3, 'c = layer_norm(xr, ln_eps, w["ln3_b"], w["ln3_w"])'))),
    "block_cross_input_adaln": ("block_fwd", _block_source_mutant(
        (_LN3, "c = modulate(layer_norm(xr, ln_eps), shift2, scale2)"))),
    "block_cross_gated_by_gate2": ("block_fwd", _block_source_mutant(
        (_CROSS_ADD, 'xr = xr + gate2 * linear(oc, w["wco"], w["bco"])'))),
    "block_cross_gated_by_gate1": ("block_fwd", _block_source_mutant(
        (_CROSS_ADD, 'xr = xr + gate1 * linear(oc, w["wco"], w["bco"])'))),
    "block_ffn_gated_by_gate1": ("block_fwd", _block_source_mutant(("out[b] = xr + gate2 * y", "out[b] = xr + gate1 * y"))),
    "block_qk_gains_swapped": ("block_fwd", _block_source_mutant((_GQ, "@@GK@@"), (_GK, _GQ), ("@@GK@@", _GK))),
    "block_image_stream_dropped": ("block_fwd", _block_source_mutant(
        ("oc = oc + multihead_attention(qc, k_img, v_img, heads)", "oc = oc"))),
    "block_rope_before_rmsnorm": ("block_fwd", _block_source_mutant(
        ('q = rms_norm(linear(u[rows], w["wq"], w["bq"]), w["gq"], rms_eps)', 'q = linear(u[rows], w["wq"], w["bq"])'),
        ('q = rope_3d(q.reshape(len(rows), heads, hd), pos[rows], theta).reshape(len(rows), dim)',
         'q = rms_norm(rope_3d(q.reshape(len(rows), heads, hd), pos[rows], theta).reshape(len(rows), dim), '
         'w["gq"], rms_eps)'))),
    "block_values_from_unmodulated_norm": ("block_fwd", _block_source_mutant(
        ('v = linear(u, w["wv"], w["bv"])', 'v = linear(layer_norm(x[b], ln_eps), w["wv"], w["bv"])'))),
    "block_cross_before_self": ("block_fwd", _block_cross_before_self_factory),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    target, factory = MUTANTS[name]
    monkeypatch.setitem(wo.__dict__, "_orig_patchify", wo.patchify)
    monkeypatch.setitem(wo.__dict__, "_orig_sinusoidal_embedding", wo.sinusoidal_embedding)
    monkeypatch.setitem(wo.__dict__, "_orig_block_fwd", wo.block_fwd)
    mutant = factory()
    monkeypatch.setattr(wo, target, mutant)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(wo)
        except AssertionError:
            caught.append(pin.__name__)
        except Exception as exc:  # a crash on a planted mistake also counts as caught
            caught.append(f"{pin.__name__}({type(exc).__name__})")
    assert caught, f"no pin caught the planted mistake {name}"
