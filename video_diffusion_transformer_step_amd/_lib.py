"""ctypes binding of libwan.so (include/wan.h): argument marshalling only.

Tensors are torch tensors on a ROCm device (PyTorch provides device memory and
streams); every computation runs in the library's HIP kernels.  Loading fails
loudly when the library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libwan.so")

WAN_OK, WAN_EINVAL, WAN_EUNSUPPORTED, WAN_EWORKSPACE, WAN_EHIP = 0, -1, -2, -3, -4
WAN_F32, WAN_BF16 = 0, 1

vp = C.c_void_p
fp = C.c_void_p  # float* passed as an address


class LatentShape(C.Structure):
    _fields_ = [("B", C.c_int32), ("C", C.c_int32), ("T", C.c_int32), ("H", C.c_int32), ("W", C.c_int32)]


class Grid(C.Structure):
    _fields_ = [("T", C.c_int32), ("Hp", C.c_int32), ("Wp", C.c_int32)]


class BlockCfg(C.Structure):
    _fields_ = [("dim", C.c_int32), ("heads", C.c_int32), ("head_dim", C.c_int32), ("ffn_dim", C.c_int32),
                ("text_len", C.c_int32), ("img_len", C.c_int32), ("dtype", C.c_int32), ("flags", C.c_uint32),
                ("ln_eps", C.c_float), ("rms_eps", C.c_float), ("rope_theta", C.c_float)]


class BlockWeightsE4M3(C.Structure):
    _fields_ = [(n, vp) for n in ("wqkv", "wo", "w1", "w2", "s_wqkv", "s_wo", "s_w1", "s_w2")]


class BlockWeights(C.Structure):
    _fields_ = [(n, vp) for n in ("mod_bias", "wqkv", "bqkv", "gq", "gk", "wo", "bo", "ln3_w", "ln3_b", "wcq",
                                  "bcq", "wco", "bco", "w1", "b1", "w2", "b2")] + [("e4m3", C.POINTER(BlockWeightsE4M3))]


class CrossKV(C.Structure):
    _fields_ = [(n, vp) for n in ("k_txt", "vt_txt", "k_img", "vt_img")]


class CrossKVWeights(C.Structure):
    _fields_ = [(n, vp) for n in ("wkv_txt", "bkv_txt", "wkv_img", "bkv_img")]


class TimeWeights(C.Structure):
    _fields_ = [(n, vp) for n in ("wt1", "bt1", "wt2", "bt2", "wtp", "btp")]


class HeadWeights(C.Structure):
    _fields_ = [(n, vp) for n in ("head_mod", "wh", "bh")]


_SIGS = {
    "wan_build_i2v_input": ([vp, vp, vp, LatentShape, vp, vp], C.c_int),
    "wan_patchify": ([vp, LatentShape, vp, vp], C.c_int),
    "wan_unpatchify": ([vp, LatentShape, vp, vp], C.c_int),
    "wan_patch_embed_workspace_bytes": ([C.POINTER(BlockCfg), C.c_int64, C.c_int32], C.c_size_t),
    "wan_patch_embed": ([C.POINTER(BlockCfg), vp, C.c_int64, C.c_int32, vp, vp, vp, vp, C.c_size_t, vp], C.c_int),
    "wan_time_embed": ([C.POINTER(BlockCfg), C.c_int32, C.POINTER(TimeWeights), C.POINTER(C.c_float), C.c_int32,
                        vp, vp, vp], C.c_int),
    "wan_context_embed_workspace_bytes": ([C.POINTER(BlockCfg), C.c_int64], C.c_size_t),
    "wan_context_embed": ([C.POINTER(BlockCfg), vp, C.c_int64, C.c_int32, vp, vp, vp, vp, vp, vp, C.c_size_t, vp],
                          C.c_int),
    "wan_cross_kv_buffer_bytes": ([C.POINTER(BlockCfg), C.c_int32, C.c_int32], C.c_size_t),
    "wan_cross_kv_workspace_bytes": ([C.POINTER(BlockCfg), C.c_int32], C.c_size_t),
    "wan_cross_kv_fwd": ([C.POINTER(BlockCfg), C.POINTER(CrossKVWeights), vp, vp, C.c_int32, C.POINTER(CrossKV), vp,
                          C.c_size_t, vp], C.c_int),
    "wan_dit_block_workspace_bytes": ([C.POINTER(BlockCfg), Grid, C.c_int32], C.c_size_t),
    "wan_dit_block_fwd": ([C.POINTER(BlockCfg), C.POINTER(BlockWeights), Grid, C.c_int32, vp, vp, C.POINTER(CrossKV),
                           vp, C.c_size_t, vp], C.c_int),
    "wan_dit_block_fwd_cached": ([C.POINTER(BlockCfg), C.POINTER(BlockWeights), Grid, C.c_int32, vp, vp,
                                  C.POINTER(CrossKV), vp, C.c_int32, vp, C.c_size_t, vp], C.c_int),
    "wan_dit_block_fwd_noalloc": ([C.POINTER(BlockCfg), C.POINTER(BlockWeights), Grid, C.c_int32, vp, vp,
                                   C.POINTER(CrossKV), vp], C.c_int),
    "wan_head_workspace_bytes": ([C.POINTER(BlockCfg), C.c_int64], C.c_size_t),
    "wan_head_fwd": ([C.POINTER(BlockCfg), C.POINTER(HeadWeights), C.c_int32, C.c_int32, C.c_int32, vp, vp, vp, vp,
                      C.c_size_t, vp], C.c_int),
    "wan_fm_euler_step": ([vp, vp, vp, C.c_float, C.c_float, C.c_int64, vp], C.c_int),
    "wan_attention_workspace_bytes": ([C.c_int32, Grid, C.c_int32, C.c_int32, C.c_int32], C.c_size_t),
    "wan_attention_fwd": ([C.c_int32, vp, vp, vp, Grid, C.c_int32, C.c_int32, C.c_int32, C.c_float, vp, vp,
                           C.c_size_t, vp], C.c_int),
    "wan_attention_partial_workspace_bytes": ([C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32],
                                              C.c_size_t),
    "wan_attention_partial_fwd": ([C.c_int32, vp, vp, vp, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, vp,
                                   vp, vp, C.c_size_t, vp], C.c_int),
    "wan_attention_lse_merge": ([C.c_int32, C.c_int32, C.POINTER(C.c_void_p), C.POINTER(C.c_void_p), C.c_int32,
                                 C.c_int32, C.c_int32, C.c_int32, vp, vp, vp], C.c_int),
    "wan_attention_q8_quantize_workspace_bytes": ([C.c_int32, C.c_int32, C.c_int32, C.c_int32], C.c_size_t),
    "wan_attention_q8_quantize": ([vp, vp, vp, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, vp, vp, vp, vp,
                                   vp, vp, vp, C.c_size_t, vp], C.c_int),
    "wan_attention_q8_fwd": ([vp, vp, vp, vp, vp, vp, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, vp, vp,
                              vp], C.c_int),
    "wan_quantize_rows_e4m3": ([vp, C.c_int64, C.c_int32, C.c_int32, vp, C.c_int64, vp, vp], C.c_int),
    "wan_quantize_tensor_e4m3": ([vp, C.c_int64, vp, vp, vp, C.c_size_t, vp], C.c_int),
    "wan_gemm_e4m3": ([vp, vp, vp, vp, C.c_int32, C.c_int32, C.c_int32, vp, C.c_int32, vp, C.c_int64, vp],
                      C.c_int),
    "wan_pack_weight_bytes": ([C.c_int32, C.c_int64, C.c_int64], C.c_size_t),
    "wan_pack_weight": ([C.c_int32, vp, C.c_int64, C.c_int64, vp, vp], C.c_int),
    "wan_profile_begin": ([C.POINTER(C.c_void_p), C.POINTER(C.c_void_p), C.POINTER(C.c_int32), C.c_int32,
                           C.c_uint32], C.c_int),
    "wan_profile_end": ([], C.c_int32),
    "wan_device_info": ([C.POINTER(C.c_int32), C.POINTER(C.c_int32)], C.c_int),
    "wan_mfma_peak_probe": ([C.c_int32, C.c_uint32, C.c_uint32, C.c_int32, C.c_int32, vp, vp], C.c_int),
    "wan_status_string": ([C.c_int], C.c_char_p),
    "wan_last_error": ([], C.c_char_p),
}

_lib = None


def lib():
    """Load libwan.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m video_diffusion_transformer_step_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


class WanError(RuntimeError):
    def __init__(self, code, fn):
        L = lib()
        super().__init__(f"{fn}: {L.wan_status_string(code).decode()} ({code}): {L.wan_last_error().decode()}")
        self.code = code


def _check(code, fn):
    if code != WAN_OK:
        raise WanError(code, fn)
    return code


def _p(t):
    """Device address of a tensor (None -> NULL)."""
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def dtype_code(torch_dtype):
    import torch
    if torch_dtype == torch.bfloat16:
        return WAN_BF16
    if torch_dtype == torch.float32:
        return WAN_F32
    raise ValueError(f"unsupported dtype {torch_dtype}")


WAN_FLAG_FP8_ATTN = 1
WAN_FLAG_FP8_GEMM = 2


def block_cfg(dim, heads, head_dim, ffn_dim, text_len, img_len, dtype, ln_eps=1e-6, rms_eps=1e-6,
              rope_theta=10000.0, flags=0):
    return BlockCfg(dim, heads, head_dim, ffn_dim, text_len, img_len, dtype, flags, ln_eps, rms_eps, rope_theta)


def latent_shape(x):
    B, Cc, T, H, W = x.shape
    return LatentShape(B, Cc, T, H, W)


# ------------------------------------------------------------------ entry points
def build_i2v_input(x_t, z_img, x_in, known_pixel_frames=None, stream=None):
    kp = None
    if known_pixel_frames is not None:
        buf = (C.c_uint8 * len(known_pixel_frames))(*[1 if v else 0 for v in known_pixel_frames])
        kp = C.cast(buf, C.c_void_p)
    _check(lib().wan_build_i2v_input(_p(x_t), _p(z_img), kp, latent_shape(x_t), _p(x_in), _stream(stream)),
           "wan_build_i2v_input")


def patchify(x, p, stream=None):
    _check(lib().wan_patchify(_p(x), latent_shape(x), _p(p), _stream(stream)), "wan_patchify")


def unpatchify(p, x, stream=None):
    _check(lib().wan_unpatchify(_p(p), latent_shape(x), _p(x), _stream(stream)), "wan_unpatchify")


def fm_euler_step(x, v_cond, v_uncond, guidance, dt, stream=None):
    _check(lib().wan_fm_euler_step(_p(x), _p(v_cond), _p(v_uncond), float(guidance), float(dt), x.numel(),
                                   _stream(stream)), "wan_fm_euler_step")


def patch_embed_ws_bytes(cfg, tokens, in_channels):
    return lib().wan_patch_embed_workspace_bytes(C.byref(cfg), tokens, in_channels)


def patch_embed(cfg, p, in_channels, w_pe, b_pe, x, ws, stream=None):
    tokens = p.numel() // (4 * in_channels)
    _check(lib().wan_patch_embed(C.byref(cfg), _p(p), tokens, in_channels, _p(w_pe), _p(b_pe), _p(x), _p(ws),
                                 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "wan_patch_embed")


def time_embed(cfg, freq_dim, tw: TimeWeights, t_list, e, e0, stream=None):
    arr = (C.c_float * len(t_list))(*[float(v) for v in t_list])
    _check(lib().wan_time_embed(C.byref(cfg), freq_dim, C.byref(tw), arr, len(t_list), _p(e), _p(e0),
                                _stream(stream)), "wan_time_embed")


def context_embed_ws_bytes(cfg, rows):
    return lib().wan_context_embed_workspace_bytes(C.byref(cfg), rows)


def context_embed(cfg, ctx, w1, b1, w2, b2, out, ws, stream=None):
    rows, in_dim = ctx.numel() // ctx.shape[-1], ctx.shape[-1]
    _check(lib().wan_context_embed(C.byref(cfg), _p(ctx), rows, in_dim, _p(w1), _p(b1), _p(w2), _p(b2), _p(out),
                                   _p(ws), ws.numel() * ws.element_size(), _stream(stream)), "wan_context_embed")


def cross_kv_buffer_bytes(cfg, B, which):
    return lib().wan_cross_kv_buffer_bytes(C.byref(cfg), B, which)


def cross_kv_ws_bytes(cfg, B):
    return lib().wan_cross_kv_workspace_bytes(C.byref(cfg), B)


def cross_kv_fwd(cfg, kvw: CrossKVWeights, txt_emb, img_emb, B, out: CrossKV, ws, stream=None):
    _check(lib().wan_cross_kv_fwd(C.byref(cfg), C.byref(kvw), _p(txt_emb), _p(img_emb), B, C.byref(out), _p(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)), "wan_cross_kv_fwd")


def block_ws_bytes(cfg, grid, B):
    return lib().wan_dit_block_workspace_bytes(C.byref(cfg), Grid(*grid), B)


WAN_ATTN_CACHE_OFF, WAN_ATTN_CACHE_STORE, WAN_ATTN_CACHE_REUSE = 0, 1, 2


def dit_block_fwd(cfg, bw: BlockWeights, grid, B, x, e0, kv: CrossKV, ws, stream=None, attn_y=None,
                  attn_mode=WAN_ATTN_CACHE_OFF):
    if attn_mode == WAN_ATTN_CACHE_OFF:
        _check(lib().wan_dit_block_fwd(C.byref(cfg), C.byref(bw), Grid(*grid), B, _p(x), _p(e0), C.byref(kv),
                                       _p(ws), ws.numel() * ws.element_size(), _stream(stream)), "wan_dit_block_fwd")
    else:
        _check(lib().wan_dit_block_fwd_cached(C.byref(cfg), C.byref(bw), Grid(*grid), B, _p(x), _p(e0), C.byref(kv),
                                              _p(attn_y), attn_mode, _p(ws), ws.numel() * ws.element_size(),
                                              _stream(stream)), "wan_dit_block_fwd_cached")


# size of the static scratch behind wan_dit_block_fwd_noalloc (WAN_NOALLOC_SCRATCH_BYTES in wan.h)
NOALLOC_SCRATCH_BYTES = 64 << 20


def dit_block_fwd_noalloc(cfg, bw: BlockWeights, grid, B, x, e0, kv: CrossKV, stream=None):
    _check(lib().wan_dit_block_fwd_noalloc(C.byref(cfg), C.byref(bw), Grid(*grid), B, _p(x), _p(e0), C.byref(kv),
                                           _stream(stream)), "wan_dit_block_fwd_noalloc")


def head_ws_bytes(cfg, tokens):
    return lib().wan_head_workspace_bytes(C.byref(cfg), tokens)


def head_fwd(cfg, hw: HeadWeights, out_channels, B, S, x, e, out, ws, stream=None):
    _check(lib().wan_head_fwd(C.byref(cfg), C.byref(hw), out_channels, B, S, _p(x), _p(e), _p(out), _p(ws),
                              ws.numel() * ws.element_size(), _stream(stream)), "wan_head_fwd")


def attention_ws_bytes(dtype, grid, B, heads, head_dim):
    return lib().wan_attention_workspace_bytes(dtype, Grid(*grid), B, heads, head_dim)


def attention_fwd(q, k, v, grid, o, ws, rope_theta=10000.0, stream=None):
    B, S, H, hd = q.shape
    _check(lib().wan_attention_fwd(dtype_code(q.dtype), _p(q), _p(k), _p(v), Grid(*grid), B, H, hd,
                                   float(rope_theta), _p(o), _p(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)), "wan_attention_fwd")


def attention_partial_ws_bytes(dtype, B, Sq, Sk, heads, head_dim):
    return lib().wan_attention_partial_workspace_bytes(dtype, B, Sq, Sk, heads, head_dim)


def attention_partial_fwd(q, k, v, o, lse, ws, stream=None):
    """q [B, Sq, H, hd], k/v [B, Sk, H, hd] (rotated already) -> o [B, Sq, H, hd], lse [B, H, Sq] fp32
    (lse may be None)."""
    B, Sq, H, hd = q.shape
    Sk = k.shape[1]
    _check(lib().wan_attention_partial_fwd(dtype_code(q.dtype), _p(q), _p(k), _p(v), B, Sq, Sk, H, hd, _p(o), _p(lse),
                                           _p(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "wan_attention_partial_fwd")


def attention_lse_merge(o_parts, lse_parts, o, lse=None, stream=None):
    """Merge results over disjoint key chunks: o_parts [B, S, H, hd], lse_parts [B, H, S] fp32."""
    n = len(o_parts)
    B, S, H, hd = o.shape
    op = (C.c_void_p * n)(*[t.data_ptr() for t in o_parts])
    lp = (C.c_void_p * n)(*[t.data_ptr() for t in lse_parts])
    _check(lib().wan_attention_lse_merge(dtype_code(o.dtype), n, op, lp, B, S, H, hd, _p(o), _p(lse),
                                         _stream(stream)), "wan_attention_lse_merge")


class Q8Codes:
    """Device buffers of the quantised attention inputs (layouts as in wan.h)."""

    def __init__(self, B, Sq, Sk, H, hd, device="cuda"):
        import torch
        nb = -(-Sk // 64)
        skpad = -(-Sk // 128) * 128
        self.shape = (B, Sq, Sk, H, hd)
        self.q8 = torch.empty((B, Sq, H, hd), dtype=torch.int8, device=device)
        self.sq = torch.empty((B, H, Sq), dtype=torch.float32, device=device)
        self.k8 = torch.empty((B, Sk, H, hd), dtype=torch.int8, device=device)
        self.sk = torch.empty((B, H, nb), dtype=torch.float32, device=device)
        self.v8t = torch.empty((B, H, hd, skpad), dtype=torch.uint8, device=device)
        self.sv = torch.empty((B, H, hd), dtype=torch.float32, device=device)


def attention_q8_quantize(q, k, v, codes: Q8Codes, ws, stream=None):
    B, Sq, H, hd = q.shape
    Sk = k.shape[1]
    c = codes
    _check(lib().wan_attention_q8_quantize(_p(q), _p(k), _p(v), B, Sq, Sk, H, hd, _p(c.q8), _p(c.sq), _p(c.k8),
                                           _p(c.sk), _p(c.v8t), _p(c.sv), _p(ws), ws.numel() * ws.element_size(),
                                           _stream(stream)), "wan_attention_q8_quantize")


def attention_q8_quantize_ws_bytes(B, Sk, H, hd):
    return lib().wan_attention_q8_quantize_workspace_bytes(B, Sk, H, hd)


def attention_q8_fwd(codes: Q8Codes, o, lse=None, stream=None):
    B, Sq, Sk, H, hd = codes.shape
    c = codes
    _check(lib().wan_attention_q8_fwd(_p(c.q8), _p(c.sq), _p(c.k8), _p(c.sk), _p(c.v8t), _p(c.sv), B, Sq, Sk, H, hd,
                                      _p(o), _p(lse), _stream(stream)), "wan_attention_q8_fwd")


def quantize_rows_e4m3(x, codes, scales, stream=None):
    """x [rows, cols] bf16 -> codes uint8 [rows, cols], scales float32 [rows]."""
    rows, cols = x.shape
    _check(lib().wan_quantize_rows_e4m3(_p(x), x.stride(0), rows, cols, _p(codes), codes.stride(0), _p(scales),
                                        _stream(stream)), "wan_quantize_rows_e4m3")


def quantize_tensor_e4m3(x, codes, scale, ws, stream=None):
    """x bf16 (any shape, n % 8 == 0) -> codes uint8 (same shape), scale float32 [1] (device)."""
    _check(lib().wan_quantize_tensor_e4m3(_p(x), x.numel(), _p(codes), _p(scale), _p(ws),
                                          ws.numel() * ws.element_size(), _stream(stream)),
           "wan_quantize_tensor_e4m3")


def gemm_e4m3(a_panels, a_scales, w_panels, w_scale, y, K, bias=None, act=0, stream=None):
    """y [M, N] from A codes and W codes, each in K panels (pack_weight of the [M, K] / [N, K] codes)."""
    M, N = y.shape
    _check(lib().wan_gemm_e4m3(_p(a_panels), _p(a_scales), _p(w_panels), _p(w_scale), M, N, K, _p(bias), act,
                               _p(y), y.stride(0), _stream(stream)),
           "wan_gemm_e4m3")


def pack_weight(w, stream=None):
    """A row-major operand w [R, K] (bf16, float32 or uint8 E4M3 codes, contiguous) in K panels
    (wan_pack_weight): a new flat tensor of w's dtype, wan_pack_weight_bytes(...) bytes."""
    import torch
    N, K = w.shape
    es = w.element_size()
    nbytes = lib().wan_pack_weight_bytes(es, N, K)
    if nbytes == 0 or not w.is_contiguous():
        raise WanError(f"pack_weight: unsupported shape {tuple(w.shape)} / layout")
    out = torch.empty(nbytes // es, dtype=w.dtype, device=w.device)
    _check(lib().wan_pack_weight(es, _p(w), N, K, _p(out), _stream(stream)), "wan_pack_weight")
    return out


def device_info():
    """(compute units, peak engine clock in kHz) of the current device."""
    cus, khz = C.c_int32(), C.c_int32()
    _check(lib().wan_device_info(C.byref(cus), C.byref(khz)), "wan_device_info")
    return cus.value, khz.value


MFMA_PROBE_FLOP = {0: 2 * 32 * 32 * 16, 1: 2 * 32 * 32 * 64, 2: 2 * 32 * 32 * 16}  # per instruction and wave
MFMA_PROBE_K = {0: 16, 1: 64}


def mfma_peak_probe(kind, a_word, b_word, blocks, iters, out, stream=None):
    """Enqueue the register-only MFMA kernel (kind 0 bf16, 1 E4M3, 2 bf16 on hashed operands);
    out [blocks * 256] float32.
    Returns the launch's flop count."""
    assert out.numel() >= blocks * 256
    _check(lib().wan_mfma_peak_probe(kind, a_word, b_word, blocks, iters, _p(out), _stream(stream)),
           "wan_mfma_peak_probe")
    return blocks * 4 * 4 * iters * MFMA_PROBE_FLOP[kind]


KERNEL_IDS = ["ln1", "qkv_gemm", "qk_rms", "attn_prologue", "self_attn", "o_gemm", "ln3", "cross_q_gemm",
              "cross_attn", "cross_o_gemm", "ln2", "ffn1_gemm", "ffn2_gemm", "quant"]


class KernelTimer:
    """Records HIP events around selected kernels of wan_dit_block_fwd (wan_profile_begin/end)."""

    def __init__(self, capacity, kernels=("self_attn",)):
        import torch
        self.capacity = capacity
        self.starts = [torch.cuda.Event(enable_timing=True) for _ in range(capacity)]
        self.stops = [torch.cuda.Event(enable_timing=True) for _ in range(capacity)]
        for e in self.starts + self.stops:
            e.record()  # materialise the underlying hipEvent_t
        self._s = (C.c_void_p * capacity)(*[e.cuda_event for e in self.starts])
        self._e = (C.c_void_p * capacity)(*[e.cuda_event for e in self.stops])
        self._tags = (C.c_int32 * capacity)()
        self.mask = 0
        for k in kernels:
            self.mask |= 1 << KERNEL_IDS.index(k)
        self.n = 0

    def __enter__(self):
        _check(lib().wan_profile_begin(self._s, self._e, self._tags, self.capacity, self.mask), "wan_profile_begin")
        return self

    def __exit__(self, *exc):
        self.n = lib().wan_profile_end()
        return False

    def times_ms(self):
        """{kernel name: [ms per launch]} (synchronises)."""
        import torch
        torch.cuda.synchronize()
        out = {}
        for i in range(self.n):
            out.setdefault(KERNEL_IDS[self._tags[i]], []).append(self.starts[i].elapsed_time(self.stops[i]))
        return out

