"""Checks that pin the CPU oracle to facts other than itself.

Each ``pin_*`` function takes the oracle module (or an object with the same
functions) and raises AssertionError when the oracle disagrees with a fixed
fact: a hand-worked fixture, a closed form, an invariant, a textbook special
case or brute force.  ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutations.py`` runs them on deliberately broken copies of oracle
functions and requires that some pin fails, so the pins are shown to bite.
"""
from __future__ import annotations

import cmath
import itertools
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------- layout
def pin_mask_golden(o):
    """Hand-worked masks ("图解 Wan2.1 I2V" §4.1 step 3, §10 Q3/Q6)."""
    for case in _golden("i2v_mask.json")["cases"]:
        T = case["T"]
        m = o.i2v_mask(T, 2, 4, case["known_pixel_frames"])
        exp = np.array(case["mask_c_by_tau"], dtype=np.float64)
        assert m.shape == (4, T, 2, 4)
        for hh in range(2):
            for ww in range(4):
                assert np.array_equal(m[:, :, hh, ww], exp), (case, m[:, :, 0, 0])
    # default = first pixel frame only
    m = o.i2v_mask(4, 2, 2)
    assert m[:, 0].min() == 1.0 and m[:, 1:].max() == 0.0


def pin_i2v_input(o):
    """4 + 16 = 20-channel y and a 16 + 20 = 36-channel input ("图解 Wan2.1 I2V" §4.1, §4.2, §8)."""
    rng = np.random.default_rng(1)
    x_t = rng.standard_normal((2, 16, 3, 4, 6))
    z = rng.standard_normal((2, 16, 3, 4, 6))
    x_in = o.build_i2v_input(x_t, z)
    assert x_in.shape == (2, 36, 3, 4, 6)
    assert np.array_equal(x_in[:, :16], x_t)
    assert np.array_equal(x_in[:, 20:], z)
    y = x_in[:, 16:]
    assert y.shape[1] == 20
    assert np.array_equal(x_in[:, 16:20], np.broadcast_to(o.i2v_mask(3, 4, 6), (2, 4, 3, 4, 6)))
    # 48-channel latent (TI2V-5B-shaped): 48 + 4 + 48 = 100
    assert o.build_i2v_input(np.zeros((1, 48, 2, 2, 2)), np.zeros((1, 48, 2, 2, 2))).shape[1] == 100


def pin_patchify_golden(o):
    g = _golden("patchify.json")
    B, C, T, H, W = g["shape"]
    x = np.zeros(g["shape"])
    for c, f, r, col in itertools.product(range(C), range(T), range(H), range(W)):
        x[0, c, f, r, col] = 1000 * c + 100 * f + 4 * r + col
    p = o.patchify(x)
    assert np.array_equal(p[0], np.array(g["tokens"], dtype=np.float64)), p[0]
    assert np.array_equal(o.unpatchify(p, C, T, H, W), x)


def pin_token_counts(o):
    for case in _golden("token_counts.json")["cases"]:
        C, T, H, W = case["latent"]
        p = o.patchify(np.zeros((1, 1, T, H, W)))
        assert p.shape[1] == case["S"], (case, p.shape)


def pin_patch_round_trip(o):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 3, 3, 4, 6))
    p = o.patchify(x)
    assert p.shape == (2, 3 * 2 * 3, 12)
    assert np.array_equal(o.unpatchify(p, 3, 3, 4, 6), x)


def pin_patch_embed_conv(o):
    """patchify + matrix product equals a direct Conv3d with kernel = stride = (1,2,2)."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 3, 2, 4, 6))
    w = rng.standard_normal((5, 12))
    b = rng.standard_normal(5)
    direct = o.conv3d_patch_embed_direct(x, w, b)
    via = o.patch_embed(o.patchify(x), w, b)
    assert np.allclose(direct, via, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ embedding
def pin_sinusoid(o):
    e = o.sinusoidal_embedding(0.0, 256)
    assert e.shape == (256,)
    assert np.array_equal(e, np.concatenate([np.ones(128), np.zeros(128)]))
    e = o.sinusoidal_embedding(0.37, 256)
    assert np.allclose(e[:128] ** 2 + e[128:] ** 2, 1.0, atol=1e-14)
    # frequency 0 (i = 0) is 1: the first pair is (cos 370, sin 370)
    assert abs(e[0] - math.cos(370.0)) < 1e-12 and abs(e[128] - math.sin(370.0)) < 1e-12


def pin_time_embed_identity(o):
    """With identity weights and zero biases: e = SiLU(emb), e0[j] = SiLU(SiLU(emb))."""
    d = 256
    eye = np.eye(d)
    w = {"wt1": eye, "bt1": np.zeros(d), "wt2": eye, "bt2": np.zeros(d),
         "wtp": np.concatenate([eye] * 6), "btp": np.zeros(6 * d)}
    e, e0 = o.time_embed(0.0, w, 256)
    silu1 = np.array([1.0 / (1.0 + math.exp(-1.0))] * 128 + [0.0] * 128)
    assert np.allclose(e, silu1, atol=1e-15)
    s2 = np.array([v / (1.0 + math.exp(-v)) for v in silu1])
    assert e0.shape == (6, d) and np.allclose(e0, s2[None, :], atol=1e-15)


def _torch64():
    import torch
    return torch


def pin_gelu_library(o):
    """GELU is the exact x * Phi(x): PyTorch's erf-based GELU (approximate='none'), float64."""
    torch = _torch64()
    x = np.linspace(-8.0, 8.0, 2001)
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="none").numpy()
    assert np.allclose(o.gelu(x), ref, rtol=0, atol=1e-14)


def pin_time_embed_library(o):
    """e = Linear(SiLU(Linear(sinusoid))), e0 = Linear(SiLU(e)) reshaped [6, dim], against the same
    composition of PyTorch float64 modules holding the same random weights (sinusoid pinned above)."""
    torch = _torch64()
    rng = np.random.default_rng(41)
    fd, dim = 64, 24
    w = {"wt1": rng.standard_normal((dim, fd)), "bt1": rng.standard_normal(dim),
         "wt2": rng.standard_normal((dim, dim)), "bt2": rng.standard_normal(dim),
         "wtp": rng.standard_normal((6 * dim, dim)), "btp": rng.standard_normal(6 * dim)}

    def lin(a, b):
        m = torch.nn.Linear(a.shape[1], a.shape[0], dtype=torch.float64)
        with torch.no_grad():
            m.weight.copy_(torch.from_numpy(a))
            m.bias.copy_(torch.from_numpy(b))
        return m
    mlp = torch.nn.Sequential(lin(w["wt1"], w["bt1"]), torch.nn.SiLU(), lin(w["wt2"], w["bt2"]))
    proj = torch.nn.Sequential(torch.nn.SiLU(), lin(w["wtp"], w["btp"]))
    for t in (0.0, 0.37, 1.0):
        emb = torch.from_numpy(o.sinusoidal_embedding(t, fd))
        with torch.no_grad():
            e_ref = mlp(emb)
            e0_ref = proj(e_ref).reshape(6, dim)
        e, e0 = o.time_embed(t, w, fd)
        assert np.allclose(e, e_ref.numpy(), rtol=1e-12, atol=1e-12)
        assert np.allclose(e0, e0_ref.numpy(), rtol=1e-12, atol=1e-12)


def pin_context_embed_library(o):
    """Linear -> exact GELU -> Linear against PyTorch float64 modules with the same weights."""
    torch = _torch64()
    rng = np.random.default_rng(43)
    n, din, dim = 7, 20, 12
    ctx = rng.standard_normal((n, din))
    w1, b1 = rng.standard_normal((dim, din)), rng.standard_normal(dim)
    w2, b2 = rng.standard_normal((dim, dim)), rng.standard_normal(dim)
    l1 = torch.nn.Linear(din, dim, dtype=torch.float64)
    l2 = torch.nn.Linear(dim, dim, dtype=torch.float64)
    with torch.no_grad():
        l1.weight.copy_(torch.from_numpy(w1)); l1.bias.copy_(torch.from_numpy(b1))
        l2.weight.copy_(torch.from_numpy(w2)); l2.bias.copy_(torch.from_numpy(b2))
        ref = l2(torch.nn.functional.gelu(l1(torch.from_numpy(ctx)), approximate="none")).numpy()
    assert np.allclose(o.context_embed(ctx, w1, b1, w2, b2), ref, rtol=1e-12, atol=1e-12)


def pin_head_library(o):
    """The head's adaLN is a LayerNorm whose affine weight is 1 + scale and bias is shift: PyTorch's
    layer_norm with that weight and bias, then its linear, per batch row (scale and shift from
    head_mod + e, shift first)."""
    torch = _torch64()
    rng = np.random.default_rng(47)
    B, S, dim, cout = 2, 5, 16, 8
    x = rng.standard_normal((B, S, dim))
    e = rng.standard_normal((B, dim))
    w = {"head_mod": rng.standard_normal((2, dim)), "wh": rng.standard_normal((cout, dim)),
         "bh": rng.standard_normal(cout)}
    got = o.head_fwd(x, e, w, 1e-6)
    for b in range(B):
        shift = torch.from_numpy(w["head_mod"][0] + e[b])
        scale = torch.from_numpy(w["head_mod"][1] + e[b])
        u = torch.nn.functional.layer_norm(torch.from_numpy(x[b]), (dim,), weight=1.0 + scale, bias=shift, eps=1e-6)
        ref = torch.nn.functional.linear(u, torch.from_numpy(w["wh"]), torch.from_numpy(w["bh"])).numpy()
        assert np.allclose(got[b], ref, rtol=1e-12, atol=1e-12)

# ---------------------------------------------------------------------- norms
def pin_layer_norm(o):
    rng = np.random.default_rng(4)
    x = 3.0 + 2.5 * rng.standard_normal((7, 64))
    y = o.layer_norm(x, eps=0.0)
    assert np.allclose(y.mean(-1), 0.0, atol=1e-12)
    assert np.allclose(y.var(-1), 1.0, atol=1e-12)
    # eps enters under the square root with the biased variance
    y = o.layer_norm(x, eps=0.5)
    ref = (x - x.mean(-1, keepdims=True)) / np.sqrt(np.var(x, -1, keepdims=True) + 0.5)
    assert np.allclose(y, ref, atol=1e-12)
    # a constant row normalises to 0, so modulation returns the shift exactly
    c = np.full((1, 16), 4.0)
    shift, scale = rng.standard_normal(16), rng.standard_normal(16)
    assert np.array_equal(o.modulate(o.layer_norm(c), shift, scale), shift[None])
    # scale = shift = 0 keeps the normalised row
    z = np.zeros(64)
    assert np.array_equal(o.modulate(o.layer_norm(x), z, z), o.layer_norm(x))
    # affine form
    wgt, bias = rng.standard_normal(64), rng.standard_normal(64)
    assert np.allclose(o.layer_norm(x, 1e-6, wgt, bias), o.layer_norm(x, 1e-6) * wgt + bias, atol=1e-12)


def pin_rms_norm(o):
    g = np.linspace(0.5, 1.5, 32)
    for c in (0.0, 1e-4, 0.3, -2.0, 7.0):
        y = o.rms_norm(np.full((1, 32), c), g, eps=1e-6)
        assert np.allclose(y[0], g * c / math.sqrt(c * c + 1e-6), rtol=1e-13, atol=0)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((5, 48)) * 3
    y = o.rms_norm(x, np.ones(48), eps=0.0)
    assert np.allclose(np.sqrt((y * y).mean(-1)), 1.0, atol=1e-13)
    # per-token scalar: rows scale independently
    assert np.allclose(o.rms_norm(x * 4.0, np.ones(48), 0.0), y, atol=1e-13)


# ----------------------------------------------------------------------- RoPE
def _textbook_rope_1d(z_pairs, pos, width, base=10000.0):
    """RoFormer's 1D rotary embedding in complex form: pair m of a width-`width`
    vector is multiplied by exp(i * pos * base^(-2m/width))."""
    out = []
    for m, (a, b) in enumerate(z_pairs):
        z = complex(a, b) * cmath.exp(1j * pos * base ** (-2.0 * m / width))
        out.append((z.real, z.imag))
    return out


def pin_rope_segments(o):
    assert tuple(o.rope_segments(128)) == (44, 42, 42)
    assert tuple(o.rope_segments(64)) == (24, 20, 20)


def pin_rope_identity_and_norm(o):
    rng = np.random.default_rng(6)
    for hd in (64, 128):
        x = rng.standard_normal((5, 3, hd))
        assert np.array_equal(o.rope_3d(x, np.zeros((5, 3), dtype=int)), x)
        pos = rng.integers(0, 60, size=(5, 3))
        y = o.rope_3d(x, pos)
        # every adjacent channel pair keeps its norm
        assert np.allclose(y[..., 0::2] ** 2 + y[..., 1::2] ** 2,
                           x[..., 0::2] ** 2 + x[..., 1::2] ** 2, atol=1e-12)


def pin_rope_relative(o):
    """<R(p) q, R(p') k> depends on p - p' only (per axis)."""
    rng = np.random.default_rng(7)
    for hd in (64, 128):
        q = rng.standard_normal((1, 1, hd))
        k = rng.standard_normal((1, 1, hd))
        p1, p2 = np.array([[3, 5, 7]]), np.array([[1, 9, 2]])
        d = p1 - p2
        base = (o.rope_3d(q, p1) * o.rope_3d(k, p2)).sum()
        for shift in ([4, 0, 0], [0, 11, 0], [0, 0, 6], [2, 3, 13]):
            s = np.array([shift])
            val = (o.rope_3d(q, p1 + s) * o.rope_3d(k, p2 + s)).sum()
            assert abs(val - base) < 1e-10, (hd, shift)
        # and changes when the offset changes
        val = (o.rope_3d(q, p1 + np.array([[1, 0, 0]])) * o.rope_3d(k, p2)).sum()
        assert abs(val - base) > 1e-6
        del d


def pin_rope_axes_textbook(o):
    """Moving along one axis rotates only that axis' channel segment, exactly as the
    textbook 1D RoPE of the segment's width; the other segments are untouched."""
    rng = np.random.default_rng(8)
    for hd in (64, 128):
        segs = o.rope_segments(hd)
        starts = [0, segs[0], segs[0] + segs[1]]
        x = rng.standard_normal((1, 2, hd))
        for axis in range(3):
            for p in (1, 5, 37):
                pos = np.zeros((1, 3), dtype=int)
                pos[0, axis] = p
                y = o.rope_3d(x, pos)
                for h in range(2):
                    for a2 in range(3):
                        sl = slice(starts[a2], starts[a2] + segs[a2])
                        if a2 != axis:
                            assert np.array_equal(y[0, h, sl], x[0, h, sl])
                        else:
                            pairs = list(zip(x[0, h, sl][0::2], x[0, h, sl][1::2]))
                            ref = _textbook_rope_1d(pairs, p, segs[a2])
                            got = list(zip(y[0, h, sl][0::2], y[0, h, sl][1::2]))
                            assert np.allclose(np.array(got), np.array(ref), atol=1e-12), (hd, axis, p)


# ------------------------------------------------------------------ attention
def _brute_attention(q, k, v):
    """Softmax attention with pure-Python loops: out_i = sum_j w_ij v_j,
    w_ij = exp(s_ij) / sum_l exp(s_il), s_ij = <q_i, k_j> / sqrt(d)."""
    nq, d = len(q), len(q[0])
    out = []
    for i in range(nq):
        s = [sum(q[i][c] * k[j][c] for c in range(d)) / math.sqrt(d) for j in range(len(k))]
        ex = [math.exp(val) for val in s]
        z = sum(ex)
        out.append([sum(ex[j] / z * v[j][c] for j in range(len(k))) for c in range(len(v[0]))])
    return np.array(out)


def pin_attention_bruteforce(o):
    rng = np.random.default_rng(9)
    for nq, nk, d in ((3, 5, 4), (4, 7, 8), (1, 1, 2)):
        q, k, v = (rng.standard_normal((n, d)) for n in (nq, nk, nk))
        assert np.allclose(o.attention(q, k, v), _brute_attention(q.tolist(), k.tolist(), v.tolist()),
                           atol=1e-12)


def pin_attention_special(o):
    rng = np.random.default_rng(10)
    q = rng.standard_normal((6, 16)) * 3
    v = rng.standard_normal((9, 16))
    # K = 0: uniform weights -> mean of V's rows
    assert np.allclose(o.attention(q, np.zeros((9, 16)), v), v.mean(0)[None], atol=1e-12)
    # one key: output is that value row
    k1, v1 = rng.standard_normal((1, 16)), rng.standard_normal((1, 16))
    assert np.allclose(o.attention(q, k1, v1), np.repeat(v1, 6, 0), atol=1e-12)
    # joint permutation of (K, V) rows leaves the output unchanged: no mask, no causality
    k = rng.standard_normal((9, 16))
    perm = rng.permutation(9)
    assert np.allclose(o.attention(q, k, v), o.attention(q, k[perm], v[perm]), atol=1e-12)


def pin_attention_lse_special(o):
    """Closed forms of the log-sum-exp: all-zero keys give log(Nk) (every score is 0); a single
    key gives its own scaled score; small cases match a pure-Python sum of exponentials."""
    rng = np.random.default_rng(11)
    q = rng.standard_normal((6, 16)) * 3
    v = rng.standard_normal((9, 16))
    _, lse = o.attention_lse(q, np.zeros((9, 16)), v)
    assert np.allclose(lse, math.log(9.0), atol=1e-12)
    k1 = rng.standard_normal((1, 16))
    _, lse1 = o.attention_lse(q, k1, v[:1])
    assert np.allclose(lse1, (q @ k1[0]) / 4.0, atol=1e-12)
    for nq, nk, d in ((3, 5, 4), (2, 7, 8)):
        qq, kk, vv = (rng.standard_normal((n, d)) for n in (nq, nk, nk))
        out, lse = o.attention_lse(qq, kk, vv)
        ref = [math.log(sum(math.exp(sum(qq[i][c] * kk[j][c] for c in range(d)) / math.sqrt(d))
                            for j in range(nk))) for i in range(nq)]
        assert np.allclose(lse, ref, atol=1e-12)
        assert np.allclose(out, _brute_attention(qq.tolist(), kk.tolist(), vv.tolist()), atol=1e-12)


def pin_attention_lse_merge(o):
    """Attention over disjoint key chunks, merged through their log-sum-exp, equals attention
    over all keys -- the identity that tile-by-tile and sequence-sharded (ring) attention rely
    on.  Several chunkings, one-key chunks included; a single part merges to itself."""
    rng = np.random.default_rng(12)
    q, k, v = rng.standard_normal((5, 8)) * 2, rng.standard_normal((23, 8)), rng.standard_normal((23, 8))
    full, full_lse = o.attention_lse(q, k, v)
    assert np.allclose(full, o.attention(q, k, v), atol=1e-12)
    for cuts in ((0, 7, 14, 21, 23), (0, 1, 23), (0, 11, 12, 23), (0, 23)):
        outs, lses = [], []
        for lo, hi in zip(cuts[:-1], cuts[1:]):
            oo, ll = o.attention_lse(q, k[lo:hi], v[lo:hi])
            outs.append(oo)
            lses.append(ll)
        merged, mlse = o.lse_merge(outs, lses)
        assert np.allclose(merged, full, atol=1e-12), cuts
        assert np.allclose(mlse, full_lse, atol=1e-12), cuts


# ----------------------------------------------------------------- block / FM
def _tiny_block_inputs(seed=12, S_grid=(2, 2, 3), dim=24, heads=2, ffn=40, L=5, Li=3):
    rng = np.random.default_rng(seed)
    n = lambda *s: 0.2 * rng.standard_normal(s)
    w = {"mod_bias": n(6, dim), "wq": n(dim, dim), "bq": n(dim), "wk": n(dim, dim), "bk": n(dim),
         "wv": n(dim, dim), "bv": n(dim), "gq": 1 + n(dim), "gk": 1 + n(dim), "wo": n(dim, dim),
         "bo": n(dim), "ln3_w": 1 + n(dim), "ln3_b": n(dim), "wcq": n(dim, dim), "bcq": n(dim),
         "wco": n(dim, dim), "bco": n(dim), "w1": n(ffn, dim), "b1": n(ffn), "w2": n(dim, ffn),
         "b2": n(dim)}
    S = S_grid[0] * S_grid[1] * S_grid[2]
    x = rng.standard_normal((2, S, dim))
    e0 = n(2, 6, dim)
    kv = [(n(L, dim), n(L, dim), n(Li, dim), n(Li, dim)) for _ in range(2)]
    return x, e0, w, kv, S_grid, heads


def pin_block_adaln_zero(o):
    """gate1 = gate2 = 0 and a zero cross-attention output projection make the block the
    identity, bit for bit ("图解 Wan2.1 I2V" §5.2: gates start at zero so each block starts
    as the identity)."""
    x, e0, w, kv, grid, heads = _tiny_block_inputs()
    w = dict(w)
    mb = w["mod_bias"].copy()
    e0 = e0.copy()
    e0[:, 2, :] = 0.0
    e0[:, 5, :] = 0.0
    mb[2] = 0.0
    mb[5] = 0.0
    w["mod_bias"] = mb
    w["wco"] = np.zeros_like(w["wco"])
    w["bco"] = np.zeros_like(w["bco"])
    y = o.block_fwd(x, e0, w, kv, grid, heads)
    assert np.array_equal(y, x)
    # with only the FFN gate open, the block changes x
    e0[:, 5, :] = 0.3
    assert not np.allclose(o.block_fwd(x, e0, w, kv, grid, heads), x)


def pin_block_dual_stream_reduces(o):
    """With a zero image value projection the dual-stream (image + text) cross-attention
    equals the text-only one ("图解 Wan2.1 I2V" §5.4: the two streams are added)."""
    x, e0, w, kv, grid, heads = _tiny_block_inputs()
    kv0 = [(kt, vt, ki, np.zeros_like(vi)) for kt, vt, ki, vi in kv]
    kv1 = [(kt, vt, None, None) for kt, vt, _, _ in kv]
    assert np.array_equal(o.block_fwd(x, e0, w, kv0, grid, heads),
                          o.block_fwd(x, e0, w, kv1, grid, heads))


def pin_block_rows_mode(o):
    """Sampled-row mode returns exactly those rows of the full block output."""
    x, e0, w, kv, grid, heads = _tiny_block_inputs()
    full = o.block_fwd(x, e0, w, kv, grid, heads)
    rows = np.array([0, 3, 11])
    assert np.allclose(o.block_fwd(x, e0, w, kv, grid, heads, rows=rows), full[:, rows], atol=1e-13)


def pin_block_non_causal(o):
    """Full, non-causal self-attention: perturbing only the last token changes the first
    token's block output ("图解 Wan2.1 I2V" §5.3; "Wan 技术深度解析" §2.5)."""
    x, e0, w, kv, grid, heads = _tiny_block_inputs()
    y = o.block_fwd(x, e0, w, kv, grid, heads)
    x2 = x.copy()
    x2[:, -1] += np.linspace(-1.0, 2.0, x.shape[-1])  # perturb the last token only (not by a
    # constant: LayerNorm would cancel it)
    y2 = o.block_fwd(x2, e0, w, kv, grid, heads)
    assert np.all(np.abs(y2[:, 0] - y[:, 0]).max(-1) > 1e-6), "first token must see the last one"
    # and the perturbation reaches the first token only through self-attention
    w0 = dict(w)
    e0z = e0.copy()
    e0z[:, 2, :] = 0.0
    w0["mod_bias"] = np.array(w["mod_bias"]).copy()
    w0["mod_bias"][2] = 0.0
    assert np.array_equal(o.block_fwd(x2, e0z, w0, kv, grid, heads)[:, 0],
                          o.block_fwd(x, e0z, w0, kv, grid, heads)[:, 0])


# ------------------------------------------------------ block composition
# Closed forms of the whole block, each with all but one branch switched off by the pages' own
# switches (a zero gate, a zero output projection), so that the remaining branch's output is known
# without running the block's arithmetic: "图解 Wan2.1 I2V" §5.2 (chunk order shift1, scale1, gate1,
# shift2, scale2, gate2; x' = norm(x)(1 + scale) + shift; x = x + gate * f(x')), §5.3 (q, k through
# RMSNorm with their own gains, then RoPE), §5.4 (cross-attention takes the plain, not the modulated,
# norm and is added without a gate), §5.5 (FFN with gate2).
def _set_mod(e0, w, chunk, value):
    """Make mod chunk `chunk` (= e0[:, chunk] + mod_bias[chunk]) equal `value` for every row."""
    e0 = np.array(e0, float).copy()
    w = dict(w)
    mb = np.array(w["mod_bias"], float).copy()
    mb[chunk] = 0.0
    e0[:, chunk, :] = value
    w["mod_bias"] = mb
    return e0, w


def _mod(e0, w, b, chunk):
    return np.asarray(e0, float)[b, chunk] + np.asarray(w["mod_bias"], float)[chunk]


def _branch_off(e0, w, which):
    """Switch branches off: "self" gate1 = 0; "cross" W_co = b_co = 0; "ffn" gate2 = 0."""
    if "self" in which:
        e0, w = _set_mod(e0, w, 2, 0.0)
    if "ffn" in which:
        e0, w = _set_mod(e0, w, 5, 0.0)
    if "cross" in which:
        w = dict(w)
        w["wco"] = np.zeros_like(w["wco"])
        w["bco"] = np.zeros_like(w["bco"])
    return e0, w


def _zero_mean_unit_rows(rng, n, dim):
    """Rows d with mean 0 and mean(d^2) = 1 exactly (up to rounding)."""
    d = rng.standard_normal((n, dim))
    d -= d.mean(-1, keepdims=True)
    return d / np.sqrt((d * d).mean(-1, keepdims=True))


def pin_block_self_branch_scale_minus_one(o):
    """scale1 = -1 makes u = shift1 for every token whatever x is, so every value row is
    shift1 W_v^T + b_v, attention returns it unchanged (its weights sum to one), and with the cross
    and FFN branches off the block output is x + gate1 * ((shift1 W_v^T + b_v) W_o^T + b_o).  A swap
    of shift1 and scale1, or a scale used without its 1 +, makes u depend on x."""
    x, e0, w, kv, grid, heads = _tiny_block_inputs(seed=31)
    e0, w = _set_mod(e0, w, 1, -1.0)
    e0, w = _branch_off(e0, w, ("cross", "ffn"))
    got = o.block_fwd(x, e0, w, kv, grid, heads)
    for b in range(x.shape[0]):
        v = _mod(e0, w, b, 0) @ np.asarray(w["wv"]).T + w["bv"]
        y = v @ np.asarray(w["wo"]).T + w["bo"]
        assert np.allclose(got[b], x[b] + _mod(e0, w, b, 2) * y[None, :], rtol=0, atol=1e-12)


def pin_block_self_branch_uniform_identity(o):
    """W_q = W_k = 0 (zero biases) makes q = k = 0, so every score is 0 and attention averages the
    values; with W_v = W_o = I (zero biases) the self-attention layer returns mean_s(u_s).  Rows
    x_s = a_s d + c_s with mean(d) = 0 and mean(d^2) = 1 have LN(x_s) = d a_s / sqrt(a_s^2 + eps), so
    with cross and FFN off the block output is x + gate1 * (d mean_s(a_s / sqrt(a_s^2 + eps))
    (1 + scale1) + shift1)."""
    x, e0, w, kv, grid, heads = _tiny_block_inputs(seed=32)
    rng = np.random.default_rng(32)
    B, S, dim = x.shape
    d = _zero_mean_unit_rows(rng, 1, dim)[0]
    a = rng.uniform(0.5, 2.0, size=(B, S))
    x = a[:, :, None] * d[None, None, :] + rng.standard_normal((B, S, 1))
    w = dict(w)
    for k in ("wq", "wk"):
        w[k] = np.zeros((dim, dim))
    for k in ("bq", "bk", "bv", "bo"):
        w[k] = np.zeros(dim)
    w["wv"] = np.eye(dim)
    w["wo"] = np.eye(dim)
    e0, w = _branch_off(e0, w, ("cross", "ffn"))
    got = o.block_fwd(x, e0, w, kv, grid, heads)
    for b in range(B):
        mean_ln = d * np.mean(a[b] / np.sqrt(a[b] ** 2 + 1e-6))
        y = mean_ln * (1.0 + _mod(e0, w, b, 1)) + _mod(e0, w, b, 0)
        assert np.allclose(got[b], x[b] + _mod(e0, w, b, 2) * y[None, :], rtol=0, atol=1e-12)


def pin_block_ffn_branch_scale_minus_one(o):
    """scale2 = -1 makes the FFN input u2 = shift2 for every token; with the self-attention and
    cross branches off the block output is x + gate2 * (GELU(shift2 W_1^T + b_1) W_2^T + b_2).  GELU
    here is PyTorch's exact (erf) GELU in float64."""
    import torch
    x, e0, w, kv, grid, heads = _tiny_block_inputs(seed=33)
    e0, w = _set_mod(e0, w, 4, -1.0)
    e0, w = _branch_off(e0, w, ("self", "cross"))
    got = o.block_fwd(x, e0, w, kv, grid, heads)
    for b in range(x.shape[0]):
        h = _mod(e0, w, b, 3) @ np.asarray(w["w1"]).T + w["b1"]
        h = torch.nn.functional.gelu(torch.from_numpy(h)).numpy()
        y = h @ np.asarray(w["w2"]).T + w["b2"]
        assert np.allclose(got[b], x[b] + _mod(e0, w, b, 5) * y[None, :], rtol=0, atol=1e-12)


def _cross_constant(w, kv_b, heads):
    """Cross branch output when its normalised input is the constant ln3_b (ln3_w = 0): q_c is the
    same for every token; text has two keys per head, so the softmax is the logistic function of
    the score difference; the image stream has one key, so its attention returns its value row."""
    kt, vt, ki, vi = kv_b
    dim = kt.shape[1]
    hd = dim // heads
    q = np.asarray(w["ln3_b"]) @ np.asarray(w["wcq"]).T + w["bcq"]
    o = np.empty(dim)
    for h in range(heads):
        sl = slice(h * hd, (h + 1) * hd)
        z = (q[sl] @ kt[0, sl] - q[sl] @ kt[1, sl]) / math.sqrt(hd)
        p0 = 1.0 / (1.0 + math.exp(-z))
        o[sl] = p0 * vt[0, sl] + (1.0 - p0) * vt[1, sl]
    if ki is not None:
        o = o + vi[0]
    return o @ np.asarray(w["wco"]).T + w["bco"]


def _cross_pin_inputs(seed):
    x, e0, w, kv, grid, heads = _tiny_block_inputs(seed=seed, L=2, Li=1)
    rng = np.random.default_rng(seed)
    kv = [(2.0 * kt, vt, ki, vi) for kt, vt, ki, vi in kv]  # sharper text scores
    w = dict(w)
    w["ln3_w"] = np.zeros(x.shape[-1])
    w["ln3_b"] = rng.standard_normal(x.shape[-1])
    w["wcq"] = 3.0 * np.asarray(w["wcq"])
    return x, e0, w, kv, grid, heads


def pin_block_cross_branch_plain_norm_no_gate(o):
    """The cross branch takes the affine LayerNorm of x (not the adaLN-modulated one) and adds its
    output without a gate.  With ln3_w = 0 its normalised input is ln3_b for every token, so with the
    self-attention branch off (gate1 = 0) and the FFN's weights zero (its output is GELU(0) W_2^T = 0
    while gate2, shift2 and scale2 stay generic) the block output is x + the closed form of
    ``_cross_constant`` for every token (two text keys, one image key)."""
    x, e0, w, kv, grid, heads = _cross_pin_inputs(34)
    e0, w = _branch_off(e0, w, ("self",))
    for k in ("w1", "w2"):
        w[k] = np.zeros_like(w[k])
    for k in ("b1", "b2"):
        w[k] = np.zeros_like(w[k])
    got = o.block_fwd(x, e0, w, kv, grid, heads)
    for b in range(x.shape[0]):
        assert np.allclose(got[b], x[b] + _cross_constant(w, kv[b], heads)[None, :], rtol=0, atol=1e-12)


def pin_block_order_self_then_cross(o):
    """Self-attention runs before cross-attention ("图解 Wan2.1 I2V" §5.3-§5.4): with the self branch
    of ``pin_block_self_branch_uniform_identity`` (output depends on x through LN) and the constant
    cross branch of ``pin_block_cross_branch_plain_norm_no_gate`` both on, the output is
    x + gate1 * y(x) + cross; running cross-attention first would feed x + cross to the self branch."""
    x, e0, w, kv, grid, heads = _cross_pin_inputs(35)
    rng = np.random.default_rng(35)
    B, S, dim = x.shape
    d = _zero_mean_unit_rows(rng, 1, dim)[0]
    a = rng.uniform(0.5, 2.0, size=(B, S))
    x = a[:, :, None] * d[None, None, :] + rng.standard_normal((B, S, 1))
    for k in ("wq", "wk"):
        w[k] = np.zeros((dim, dim))
    for k in ("bq", "bk", "bv", "bo"):
        w[k] = np.zeros(dim)
    w["wv"] = np.eye(dim)
    w["wo"] = np.eye(dim)
    e0, w = _branch_off(e0, w, ("ffn",))
    got = o.block_fwd(x, e0, w, kv, grid, heads)
    for b in range(B):
        mean_ln = d * np.mean(a[b] / np.sqrt(a[b] ** 2 + 1e-6))
        y = mean_ln * (1.0 + _mod(e0, w, b, 1)) + _mod(e0, w, b, 0)
        want = x[b] + _mod(e0, w, b, 2) * y[None, :] + _cross_constant(w, kv[b], heads)[None, :]
        assert np.allclose(got[b], want, rtol=0, atol=1e-12)


def pin_block_qk_gains_own_projection(o):
    """Each of q and k is RMS-normalised with its own gain before RoPE.  Two tokens at frames 0 and 1
    (grid (2, 1, 1)), one head of width 12 (time segment = channels 0-3, first pair rotating by the
    frame index times theta^0 = 1 radian).  W_q = W_k = 0 and b_q = b_k = 1 give q = k = 1 (RMS 1),
    so q^ = R(f) g_q / sqrt(1 + eps) and k^ = R(f) g_k / sqrt(1 + eps).  With g_q = e_0 and
    g_k = gamma e_1 the scores are s_ij = gamma sin(f_i - f_j) / ((1 + eps) sqrt(12)): zero on the
    diagonal, -kappa and +kappa off it.  Rows x_0 = d, x_1 = -d (mean 0, mean square 1), shift1 =
    scale1 = 0 and W_v = W_o = I give u = v = +-d / sqrt(1 + eps), and both outputs equal
    tanh(kappa / 2) d / sqrt(1 + eps).  Swapping the gains flips kappa's sign."""
    rng = np.random.default_rng(36)
    dim, heads, eps, gamma = 12, 1, 1e-6, 6.0
    n = lambda *s: 0.2 * rng.standard_normal(s)
    d = _zero_mean_unit_rows(rng, 1, dim)[0]
    x = np.stack([d, -d])[None]  # [1, 2, dim]
    w = {"mod_bias": n(6, dim), "wq": np.zeros((dim, dim)), "bq": np.ones(dim), "wk": np.zeros((dim, dim)),
         "bk": np.ones(dim), "wv": np.eye(dim), "bv": np.zeros(dim), "gq": np.eye(dim)[0],
         "gk": gamma * np.eye(dim)[1], "wo": np.eye(dim), "bo": np.zeros(dim), "ln3_w": 1 + n(dim),
         "ln3_b": n(dim), "wcq": n(dim, dim), "bcq": n(dim), "wco": n(dim, dim), "bco": n(dim),
         "w1": n(20, dim), "b1": n(20), "w2": n(dim, 20), "b2": n(dim)}
    e0 = n(1, 6, dim)
    kv = [(n(3, dim), n(3, dim), None, None)]
    e0, w = _set_mod(e0, w, 0, 0.0)
    e0, w = _set_mod(e0, w, 1, 0.0)
    e0, w = _branch_off(e0, w, ("cross", "ffn"))
    got = o.block_fwd(x, e0, w, kv, (2, 1, 1), heads)
    kappa = gamma * math.sin(1.0) / ((1.0 + eps) * math.sqrt(dim))
    y = math.tanh(kappa / 2.0) * d / math.sqrt(1.0 + eps)
    want = x[0] + _mod(e0, w, 0, 2)[None, :] * y[None, :]
    assert np.allclose(got[0], want, rtol=0, atol=1e-12)


def pin_fm_straight_line(o):
    """Straight path x_t = (1-t) x0 + t x1 with constant velocity x1 - x0: N exact-velocity
    Euler steps from t = 0 land on x1 ("Wan 技术深度解析" §2.7, §8.3); in the mirrored
    convention x_t = (1-t) x0 + t eps, v = eps - x0, N steps with dt = -1/N from t = 1 land
    on x0 ("图解 Wan2.1 I2V" §6, §7)."""
    rng = np.random.default_rng(13)
    x0, x1 = rng.standard_normal(1000), rng.standard_normal(1000)
    for N in (1, 4, 25, 50):
        x = x0.copy()
        for _ in range(N):
            x = o.euler_step(x, x1 - x0, 1.0 / N)
        assert np.allclose(x, x1, rtol=0, atol=1e-13), N
        eps = x1
        x = eps.copy()
        for _ in range(N):
            x = o.euler_step(x, eps - x0, -1.0 / N)
        assert np.allclose(x, x0, rtol=0, atol=1e-13), N
    # a single step of any size along the line stays on the line
    t, dt = 0.3, 0.45
    xt = (1 - t) * x0 + t * x1
    assert np.allclose(o.euler_step(xt, x1 - x0, dt), (1 - t - dt) * x0 + (t + dt) * x1, atol=1e-13)


def pin_cfg(o):
    """v = v_u + s (v_c - v_u): s = 0 gives v_u, s = 1 gives v_c ("图解 Wan2.1 I2V" §7)."""
    rng = np.random.default_rng(14)
    vc, vu = rng.standard_normal(100), rng.standard_normal(100)
    assert np.array_equal(o.cfg_combine(vc, vu, 0.0), vu)
    assert np.allclose(o.cfg_combine(vc, vu, 1.0), vc, rtol=0, atol=1e-15)
    assert np.allclose(o.cfg_combine(vc, vu, 5.0), vu + 5.0 * (vc - vu), atol=1e-14)
    x = rng.standard_normal(100)
    assert np.array_equal(o.cfg_euler(x, vc, None, 7.0, -0.1), o.euler_step(x, vc, -0.1))


# ------------------------------------------------------------- diffusion cache
def _tiny_sampling(seed=21):
    import wan_inputs as wi
    c = wi.get_config("tiny").replace(B=2, img_len=5, img_dim=32)
    mw = wi.make_model_weights(c, seed=seed)
    bws = [wi.make_block_weights(c, i, seed=seed) for i in range(2)]
    x_t, z = wi.make_latents(c, seed=seed)
    txt, img = wi.make_contexts(c, seed=seed)
    kw = dict(ln_eps=c.ln_eps, rms_eps=c.rms_eps, theta=c.rope_theta, freq_dim=c.freq_dim,
              out_channels=c.out_channels)
    return c, mw, bws, x_t, z, txt, img, kw


def pin_sample_cached_reductions(o):
    """The cached sampler reduces to the plain one: no reuse gives ``sample`` bit for bit; attention
    reuse with gate1 = 0 at every t (time projection rows and block bias of that chunk zeroed)
    gives ``sample`` bit for bit; CFG reuse with guidance 1 gives ``sample`` (v = v_c)."""
    c, mw, bws, x_t, z, txt, img, kw = _tiny_sampling()
    steps = 4
    ref, _ = o.sample(x_t, z, steps, c.guidance, mw, bws, txt, img, c.heads, **kw)
    got, _ = o.sample_cached(x_t, z, steps, c.guidance, mw, bws, txt, img, c.heads, [False] * 4, [False] * 4, **kw)
    assert np.array_equal(got, ref)
    dim = c.dim
    mw0 = dict(mw)
    mw0["wtp"] = np.array(mw["wtp"], float).copy()
    mw0["btp"] = np.array(mw["btp"], float).copy()
    mw0["wtp"][2 * dim:3 * dim] = 0.0
    mw0["btp"][2 * dim:3 * dim] = 0.0
    bws0 = []
    for w in bws:
        w0 = dict(w)
        w0["mod_bias"] = np.array(w["mod_bias"], float).copy()
        w0["mod_bias"][2] = 0.0
        bws0.append(w0)
    ref0, _ = o.sample(x_t, z, steps, c.guidance, mw0, bws0, txt, img, c.heads, **kw)
    got0, _ = o.sample_cached(x_t, z, steps, c.guidance, mw0, bws0, txt, img, c.heads,
                              [False, True, False, True], [False] * 4, **kw)
    assert np.array_equal(got0, ref0)
    ref1, _ = o.sample(x_t, z, steps, 1.0, mw, bws, txt, img, c.heads, **kw)
    got1, _ = o.sample_cached(x_t, z, steps, 1.0, mw, bws, txt, img, c.heads, [False] * 4,
                              [False, False, True, True], **kw)
    assert np.allclose(got1, ref1, rtol=0, atol=1e-12)


def pin_attention_cache_modes(o):
    """Storing the self-attention output changes nothing; reusing a zero cache equals the block with
    its self-attention branch gated off; reusing the stored value at the same inputs reproduces the
    block."""
    x, e0, w, kv, grid, heads = _tiny_block_inputs()
    ref = o.block_fwd(x, e0, w, kv, grid, heads)
    cache = {"mode": "store", "y": np.zeros(x.shape)}
    assert np.array_equal(o.block_fwd(x, e0, w, kv, grid, heads, attn_cache=cache), ref)
    assert np.abs(cache["y"]).max() > 0
    again = o.block_fwd(x, e0, w, kv, grid, heads, attn_cache={"mode": "reuse", "y": cache["y"]})
    assert np.array_equal(again, ref)
    e0z, wz = np.array(e0, float).copy(), dict(w)
    e0z[:, 2] = 0.0
    wz["mod_bias"] = np.array(w["mod_bias"], float).copy()
    wz["mod_bias"][2] = 0.0
    off = o.block_fwd(x, e0z, wz, kv, grid, heads)
    zero = o.block_fwd(x, e0, w, kv, grid, heads, attn_cache={"mode": "reuse", "y": np.zeros(x.shape)})
    assert np.array_equal(zero, off)


def pin_cfg_cache_uses_last_uncond(o):
    """A CFG-reuse step combines the fresh conditional velocity with the unconditional one of the
    previous step, composed here from ``dit_fwd`` and ``cfg_euler`` directly."""
    c, mw, bws, x_t, z, txt, img, kw = _tiny_sampling()
    steps, dt = 3, -1.0 / 3
    got, _ = o.sample_cached(x_t, z, steps, c.guidance, mw, bws, txt, img, c.heads, [False] * 3,
                             [False, False, True], **kw)
    x = np.array(x_t, float)
    for k in range(steps):
        t = 1.0 + k * dt
        x_in = o.build_i2v_input(x, z)
        if k < 2:
            v = o.dit_fwd(np.repeat(x_in, 2, axis=0), t, mw, bws, txt, img, c.heads, **kw)
            v_u = v[1:2]
            x = o.cfg_euler(x, v[0:1], v_u, c.guidance, dt)
        else:
            v_c = o.dit_fwd(x_in, t, mw, bws, np.asarray(txt)[:1], img, c.heads, **kw)
            x = o.cfg_euler(x, v_c, v_u, c.guidance, dt)
    assert np.allclose(got, x, rtol=0, atol=1e-12)


def pin_snr_and_switch_time(o):
    """SNR of the straight path: 0 at pure noise, 1 where signal and noise weigh the same, and the
    empirical power ratio of (1 - t) x0 against t eps on unit-variance draws.  The switch time: the
    hand-worked values snr_min = 2 -> t = 1/2 and snr_min = 0 -> t = 1, and elsewhere the root of
    snr(t) = snr_min / 2 found by bisection."""
    assert o.snr(1.0) == 0.0 and o.snr(0.5) == 1.0 and o.snr(0.2) == 16.0
    assert o.snr(1e-9) > 1e15
    rng = np.random.default_rng(3)
    x0, eps = rng.standard_normal(400000), rng.standard_normal(400000)
    for t in (0.1, 0.3, 0.75, 0.95):
        ratio = np.mean(((1 - t) * x0) ** 2) / np.mean((t * eps) ** 2)
        assert abs(ratio / o.snr(t) - 1) < 0.02, (t, ratio)
    assert o.t_moe_from_snr(2.0) == 0.5 and o.t_moe_from_snr(0.0) == 1.0
    for snr_min in (0.01, 1.0, 7.0, 100.0):
        lo, hi = 1e-12, 1.0  # snr decreases in t: snr(lo) > target > snr(hi) = 0
        for _ in range(200):
            mid = 0.5 * (lo + hi)
            lo, hi = (mid, hi) if o.snr(mid) > snr_min / 2 else (lo, mid)
        assert abs(o.t_moe_from_snr(snr_min) - 0.5 * (lo + hi)) < 1e-12


def pin_expert_switch_sequence(o):
    """The boundary step t = t_moe runs the low-noise expert; 4 steps from t = 1 with t_moe = 1/2 visit
    t = 1, 3/4, 1/2, 1/4 -> high, high, low, low."""
    assert o.expert_for_step(0.5, 0.5) == 1 and o.expert_for_step(0.5 + 1e-9, 0.5) == 0
    assert o.expert_for_step(1.0, 1.0) == 1 and o.expert_for_step(0.0, 0.0) == 1
    c, mw, bws, x_t, z, txt, img, kw = _tiny_sampling()
    _, _, used = o.sample_two_expert(x_t, z, 4, c.guidance, [(mw, bws), (mw, bws)], 0.5, txt, img, c.heads, **kw)
    assert used == [0, 0, 1, 1]


def pin_sample_two_expert_reductions(o):
    """The same expert twice is ``sample``; t_moe >= t0 runs only the low-noise expert; a run that
    switches after k steps equals the high expert's first k steps of ``sample`` followed by ``sample``
    with the low expert from t_k for the remaining steps (same step size)."""
    import wan_inputs as wi
    c, mw, bws, x_t, z, txt, img, kw = _tiny_sampling()
    mw2 = wi.make_model_weights(c, seed=77)
    bws2 = [wi.make_block_weights(c, i, seed=77) for i in range(2)]
    hi, lo = (mw, bws), (mw2, bws2)
    steps = 4
    ref_hi, traj_hi = o.sample(x_t, z, steps, c.guidance, mw, bws, txt, img, c.heads, **kw)
    got, _, _ = o.sample_two_expert(x_t, z, steps, c.guidance, [hi, hi], 0.5, txt, img, c.heads, **kw)
    assert np.array_equal(got, ref_hi)
    ref_lo, _ = o.sample(x_t, z, steps, c.guidance, mw2, bws2, txt, img, c.heads, **kw)
    got, _, used = o.sample_two_expert(x_t, z, steps, c.guidance, [hi, lo], 1.0, txt, img, c.heads, **kw)
    assert used == [1] * steps and np.array_equal(got, ref_lo)
    got, _, used = o.sample_two_expert(x_t, z, steps, c.guidance, [hi, lo], 0.5, txt, img, c.heads, **kw)
    assert used == [0, 0, 1, 1]
    ref, _ = o.sample(traj_hi[1], z, 2, c.guidance, mw2, bws2, txt, img, c.heads, t0=0.5, **kw)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)
    assert not np.allclose(got, ref_hi, rtol=0, atol=1e-3)  # the second expert matters

ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
