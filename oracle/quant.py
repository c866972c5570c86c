"""Plain definitions of the quantised attention path (INT8 / FP8 codes and scales).

TEST INFRASTRUCTURE ONLY: called by tests, never by the product path.

[Wan-deep-dive §5.3] lists an FP8 FlashAttention-3 variant among the inference optimisations:
Q.K inner products in INT8, O = P.V in FP8, accumulation across key blocks in FP32.  The page
names the number formats and nothing else.

Readings (the page gives no granularity, rounding or encoding):
* INT8 codes are symmetric: scale = amax / 127, code = round-half-even(x * (127 / amax)) clamped to
  [-127, 127], both quotients and the product rounded to float32 (so that the codes are a fixed
  function of the float32 inputs).  A group whose amax is 0 gets scale 0 and all-zero codes.
  Q is quantised per (token, head); K per (head, block of 64 consecutive keys).
* FP8 is the OCP 8-bit E4M3 format ("e4m3fn"): sign, 4 exponent bits with bias 7, 3 mantissa bits,
  subnormals, no infinities, S.1111.111 is NaN, largest finite magnitude 448; conversion rounds to
  the nearest representable value, ties to the even code.
  V is quantised per (head, channel) over all tokens: scale = amax / 448,
  code = e4m3(clamp(x * (448 / amax), -448, 448)).
* The attention result is softmax(q k^T / sqrt(d)) v as in ``wan_oracle.attention``; the quantised
  path is compared with that definition within an error bound derived from the code precisions.

[Wan-deep-dive §5.3] also lists FP8 GEMMs: weights quantised per tensor, activations per token.
Reading: both in E4M3 with scale = amax / 448 and code = e4m3(clamp(x * (448 / amax), -448, 448)) (the
same rule as V); the product is y = (sum_k a_code w_code) * (s_row * s_w) + bias.
"""
from __future__ import annotations

import numpy as np

__all__ = ["e4m3_values", "e4m3_encode", "e4m3_decode", "int8_group", "quant_q_int8", "quant_k_int8",
           "quant_v_e4m3", "e4m3_group", "quant_rows_e4m3", "quant_tensor_e4m3", "gemm_e4m3"]

KEY_BLOCK = 64  # keys per K scale group


def e4m3_values() -> np.ndarray:
    """Magnitude of every non-negative E4M3 code 0..127 (code 127 = S.1111.111 is NaN)."""
    vals = np.empty(128, dtype=np.float64)
    for code in range(128):
        e, m = code >> 3, code & 7
        if e == 0:
            vals[code] = m * 2.0 ** -9            # subnormal: 0.m x 2^(1-7)
        else:
            vals[code] = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    vals[127] = np.nan
    return vals


_MAG = e4m3_values()


def e4m3_decode(codes) -> np.ndarray:
    c = np.asarray(codes).astype(np.int64) & 0xFF
    mag = _MAG[c & 0x7F]
    return np.where(c & 0x80, -mag, mag)


def e4m3_encode(x) -> np.ndarray:
    """Round each value to the nearest E4M3 code, ties to the even code.

    Magnitudes that round beyond 448 land on the NaN code (the format has no infinity): the grid is
    extended by 480 = the value S.1111.111 would have, and that code is NaN."""
    x = np.asarray(x, dtype=np.float64)
    grid = _MAG.copy()
    grid[127] = 480.0
    a = np.abs(x)
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, 127)  # first grid value >= a
    lo = np.clip(hi - 1, 0, 127)
    d_lo, d_hi = a - grid[lo], grid[hi] - a
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a > 480.0, 127, pick)
    pick = np.where(np.isnan(a), 127, pick)
    sign = np.signbit(x).astype(np.int64) << 7
    return (pick | sign).astype(np.uint8)


def int8_group(x):
    """Symmetric INT8 codes of one group of float32 values: (codes int8, scale float32)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    if amax == 0:
        return np.zeros(x.shape, np.int8), np.float32(0)
    inv = np.float32(127) / amax
    codes = np.clip(np.rint(x * inv), -127, 127).astype(np.int8)
    return codes, np.float32(amax / np.float32(127))


def quant_q_int8(q):
    """q [B, S, H, d] -> (codes [B, S, H, d] int8, scales [B, H, S] float32): one group per (token, head)."""
    q = np.asarray(q, dtype=np.float32)
    B, S, H, _ = q.shape
    codes = np.empty(q.shape, np.int8)
    scales = np.empty((B, H, S), np.float32)
    for b in range(B):
        for s in range(S):
            for h in range(H):
                codes[b, s, h], scales[b, h, s] = int8_group(q[b, s, h])
    return codes, scales


def quant_k_int8(k):
    """k [B, S, H, d] -> (codes int8 [B, S, H, d], scales [B, H, ceil(S / 64)] float32): one group per
    (head, block of 64 consecutive keys); the last block holds the S mod 64 remaining keys."""
    k = np.asarray(k, dtype=np.float32)
    B, S, H, _ = k.shape
    nb = -(-S // KEY_BLOCK)
    codes = np.empty(k.shape, np.int8)
    scales = np.empty((B, H, nb), np.float32)
    for b in range(B):
        for h in range(H):
            for t in range(nb):
                sl = slice(t * KEY_BLOCK, min(S, (t + 1) * KEY_BLOCK))
                codes[b, sl, h], scales[b, h, t] = int8_group(k[b, sl, h])
    return codes, scales


def quant_v_e4m3(v):
    """v [B, S, H, d] -> (codes uint8 [B, S, H, d] in E4M3, scales [B, H, d] float32): one group per
    (head, channel) over all tokens."""
    v = np.asarray(v, dtype=np.float32)
    B, S, H, d = v.shape
    codes = np.empty(v.shape, np.uint8)
    scales = np.empty((B, H, d), np.float32)
    for b in range(B):
        for h in range(H):
            amax = np.max(np.abs(v[b, :, h, :]), axis=0).astype(np.float32)  # [d]
            safe = np.where(amax > 0, amax, np.float32(1))
            inv = (np.float32(448) / safe).astype(np.float32)
            y = np.clip((v[b, :, h, :] * inv[None, :]).astype(np.float32), -448, 448)
            c = e4m3_encode(y)
            codes[b, :, h, :] = np.where(amax[None, :] > 0, c, 0)
            scales[b, h] = np.where(amax > 0, (amax / np.float32(448)).astype(np.float32), 0)
    return codes, scales


def e4m3_group(x):
    """E4M3 codes of one group of float32 values: (codes uint8, scale float32), scale = amax / 448."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    if amax == 0:
        return np.zeros(x.shape, np.uint8), np.float32(0)
    inv = np.float32(448) / amax
    y = np.clip((x * inv).astype(np.float32), -448, 448)
    return e4m3_encode(y), np.float32(amax / np.float32(448))


def quant_rows_e4m3(x):
    """Per-token activation codes: x [M, K] -> (codes [M, K], scales [M])."""
    x = np.asarray(x, dtype=np.float32)
    codes = np.empty(x.shape, np.uint8)
    scales = np.empty(x.shape[0], np.float32)
    for m in range(x.shape[0]):
        codes[m], scales[m] = e4m3_group(x[m])
    return codes, scales


def quant_tensor_e4m3(w):
    """Per-tensor weight codes: w [N, K] -> (codes [N, K], scale)."""
    return e4m3_group(np.asarray(w, dtype=np.float32))


def gemm_e4m3(a_codes, a_scales, w_codes, w_scale, bias=None):
    """y [M, N] = (decode(a) decode(w)^T) * (a_scale[m] * w_scale) + bias, in float64."""
    a = e4m3_decode(a_codes) * np.asarray(a_scales, np.float64)[:, None]
    w = e4m3_decode(w_codes) * float(w_scale)
    y = a @ w.T
    return y if bias is None else y + np.asarray(bias, np.float64)
