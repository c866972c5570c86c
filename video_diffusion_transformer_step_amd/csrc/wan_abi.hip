// C ABI of libwan.so: argument validation, workspace planning and the launch
// sequence of each entry point declared in include/wan.h.  No allocation, no
// synchronisation: every call only enqueues kernels on the caller's stream.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "wan.h"
#include <algorithm>
#include <atomic>
#include <mutex>

#include "wan_internal.h"

using namespace wan;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

#define WAN_TRY(expr)                                                                      \
  do {                                                                                     \
    int rc_ = (expr);                                                                      \
    if (rc_ != WAN_OK) return rc_;                                                         \
  } while (0)

#define HIP_TRY(expr)                                                                      \
  do {                                                                                     \
    hipError_t e_ = (expr);                                                                \
    if (e_ != hipSuccess) return fail(WAN_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

inline hipStream_t hs(wan_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

// Kernel-timing hook (wan_profile_begin / wan_profile_end): caller-owned events recorded on the
// launch stream around the selected kernels of wan_dit_block_fwd.  Process-wide, not thread-safe.
struct Profile {
  hipEvent_t* starts = nullptr;
  hipEvent_t* stops = nullptr;
  int32_t* tags = nullptr;
  int32_t cap = 0, n = 0;
  uint32_t mask = 0;
};
Profile g_prof;

struct ProfScope {
  int slot = -1;
  hipStream_t st;
  ProfScope(int id, hipStream_t s) : st(s) {
    if (g_prof.cap > 0 && (g_prof.mask >> id & 1u) && g_prof.n < g_prof.cap) {
      slot = g_prof.n++;
      g_prof.tags[slot] = id;
      (void)hipEventRecord(g_prof.starts[slot], st);
    }
  }
  ~ProfScope() {
    if (slot >= 0) (void)hipEventRecord(g_prof.stops[slot], st);
  }
};
#define PROF_TRY(id, expr)            \
  do {                                \
    ProfScope prof_(id, st);          \
    HIP_TRY(expr);                    \
  } while (0)

int need_ptr(const void* p, const char* name) {
  if (!p) return fail(WAN_EINVAL, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) & 15u) return fail(WAN_EINVAL, "%s is not 16-byte aligned", name);
  return WAN_OK;
}
int opt_ptr(const void* p, const char* name) { return p ? need_ptr(p, name) : WAN_OK; }
int need_f32(const void* p, const char* name) {
  if (!p || (reinterpret_cast<uintptr_t>(p) & 3)) return fail(WAN_EINVAL, "%s is NULL or not 4-byte aligned", name);
  return WAN_OK;
}

int check_shape(const wan_latent_shape& s) {
  if (s.B <= 0 || s.C <= 0 || s.T <= 0 || s.H <= 0 || s.W <= 0)
    return fail(WAN_EINVAL, "latent shape must be positive (B=%d C=%d T=%d H=%d W=%d)", s.B, s.C, s.T, s.H, s.W);
  if ((s.H & 1) || (s.W & 1)) return fail(WAN_EINVAL, "H (%d) and W (%d) must be even for (1,2,2) patches", s.H, s.W);
  return WAN_OK;
}

int check_grid(const wan_grid& g) {
  if (g.T <= 0 || g.Hp <= 0 || g.Wp <= 0) return fail(WAN_EINVAL, "grid must be positive (%d,%d,%d)", g.T, g.Hp, g.Wp);
  if ((int64_t)g.T * g.Hp * g.Wp > (1ll << 30)) return fail(WAN_EUNSUPPORTED, "too many tokens");
  return WAN_OK;
}

int check_dtype(int32_t dtype) {
  if (dtype != WAN_F32 && dtype != WAN_BF16) return fail(WAN_EINVAL, "unknown dtype %d", dtype);
  return WAN_OK;
}

int check_cfg(const wan_block_cfg* c) {
  if (!c) return fail(WAN_EINVAL, "cfg is NULL");
  WAN_TRY(check_dtype(c->dtype));
  if (c->flags & ~(WAN_FLAG_FP8_ATTN | WAN_FLAG_FP8_GEMM))
    return fail(WAN_EUNSUPPORTED, "unknown cfg->flags bits 0x%x", c->flags);
  if ((c->flags & WAN_FLAG_FP8_ATTN) && (c->dtype != WAN_BF16 || c->head_dim != 128))
    return fail(WAN_EUNSUPPORTED, "WAN_FLAG_FP8_ATTN needs dtype WAN_BF16 and head_dim 128");
  if ((c->flags & WAN_FLAG_FP8_GEMM) && (c->dtype != WAN_BF16 || c->dim % 256 != 0 || c->ffn_dim % 256 != 0))
    return fail(WAN_EUNSUPPORTED, "WAN_FLAG_FP8_GEMM needs dtype WAN_BF16 and dim, ffn_dim multiples of 256");
  if (c->heads <= 0 || c->head_dim <= 0 || c->dim != c->heads * c->head_dim)
    return fail(WAN_EINVAL, "dim (%d) must equal heads (%d) * head_dim (%d)", c->dim, c->heads, c->head_dim);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(WAN_EUNSUPPORTED, "head_dim %d not supported (64 or 128)", c->head_dim);
  if (c->dim % 8 != 0 || c->dim > 6144) return fail(WAN_EUNSUPPORTED, "dim %d must be a multiple of 8 and <= 6144", c->dim);
  if (c->ffn_dim <= 0 || c->ffn_dim % 32 != 0)
    return fail(WAN_EINVAL, "ffn_dim %d must be a positive multiple of 32", c->ffn_dim);
  if (c->text_len <= 0 || c->img_len < 0) return fail(WAN_EINVAL, "text_len must be > 0 and img_len >= 0");
  if (!(c->ln_eps >= 0.f) || !(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f))
    return fail(WAN_EINVAL, "eps must be >= 0 and rope_theta > 0");
  return WAN_OK;
}

inline size_t esize(int32_t dtype) { return dtype == WAN_BF16 ? 2 : 4; }
inline size_t a256(size_t x) { return (x + 255) & ~size_t(255); }
inline int64_t pad64(int64_t L) { return round_up(L, 64); }

// Bump allocator over the caller's workspace.
struct Carve {
  char* base;
  size_t off = 0;
  template <typename T>
  T* take(size_t count) {
    T* p = reinterpret_cast<T*>(base ? base + off : nullptr);
    off += a256(count * sizeof(T));
    return p;
  }
};

// ---------------------------------------------------------------- block plan
template <typename T>
struct BlockWs {
  T *u, *qkv, *vt, *o, *h;
  float* mod;  // [B, 6, dim]: e0 + the block's modulation bias
  // Q/K RMSNorm: the Q/K/V epilogue's sums of squares [2 dim / 32, B S] and the q rows' factors [B S]
  float *ssq, *rq;
  float2* rope;  // 3D RoPE (cos, sin) table of the grid (launch_attn_prologue)
  // quantised self-attention (WAN_FLAG_FP8_ATTN only): codes and scales of q, k, v
  uint8_t *q8, *k8, *v8t;
  float *sq, *sk, *sv;
  // E4M3 products (WAN_FLAG_FP8_GEMM only): per-token codes of the current product's input
  uint8_t* a8;
  float* sa;
};
template <typename T>
size_t block_plan(const wan_block_cfg& c, const wan_grid& g, int B, char* base, BlockWs<T>* out) {
  const int64_t S = (int64_t)g.T * g.Hp * g.Wp, BS = (int64_t)B * S, dim = c.dim;
  Carve cv{base};
  BlockWs<T> w;
  // u, o, h (and the E4M3 codes a8) are the products' A operands, held in K panels of Mp rows
  const int64_t Mp = panel_rows(BS);
  w.u = cv.take<T>(Mp * dim);
  w.qkv = cv.take<T>(BS * 2 * dim);  // q | k per token (v goes to vt)
  w.vt = cv.take<T>((size_t)B * dim * pad64(S));
  w.o = cv.take<T>(Mp * dim);
  w.h = cv.take<T>(Mp * c.ffn_dim);
  w.mod = cv.take<float>((size_t)B * 6 * dim);
  w.ssq = cv.take<float>((size_t)(2 * dim / 32) * BS);
  w.rq = cv.take<float>((size_t)BS);
  w.rope = cv.take<float2>((size_t)rope_table_entries(g.T, g.Hp, g.Wp, c.head_dim));
  w.q8 = w.k8 = w.v8t = nullptr;
  w.sq = w.sk = w.sv = nullptr;
  if (c.flags & WAN_FLAG_FP8_ATTN) {
    w.q8 = cv.take<uint8_t>(BS * dim);
    w.k8 = cv.take<uint8_t>(BS * dim);
    w.v8t = cv.take<uint8_t>((size_t)B * dim * round_up(S, 128));
    w.sq = cv.take<float>((size_t)B * c.heads * S);
    w.sk = cv.take<float>((size_t)B * c.heads * (pad64(S) / 64));
    w.sv = cv.take<float>((size_t)B * dim);
  }
  w.a8 = nullptr;
  w.sa = nullptr;
  if (c.flags & WAN_FLAG_FP8_GEMM) {
    w.a8 = cv.take<uint8_t>(Mp * std::max<int64_t>(dim, c.ffn_dim));
    w.sa = cv.take<float>(BS);
  }
  if (out) *out = w;
  return cv.off;
}

template <typename T>
int block_fwd_t(const wan_block_cfg& c, const wan_block_weights& W, const wan_grid& g, int B, float* x,
                const float* e0, const wan_cross_kv& kv, void* ws, hipStream_t st, float* attn_y = nullptr,
                int attn_mode = WAN_ATTN_CACHE_OFF) {
  BlockWs<T> w;
  block_plan<T>(c, g, B, reinterpret_cast<char*>(ws), &w);
  const int S = g.T * g.Hp * g.Wp, BS = B * S, dim = c.dim, H = c.heads, hd = c.head_dim;
  const int Spad = (int)pad64(S);
  const float scale = 1.f / sqrtf((float)hd);
  // The products' A operands (u, o, h and their E4M3 codes) live in K panels (see KMat / ActLayout).
  const ActLayout pan = act_panels(BS);
  const int64_t o_cs = pan.bs;  // attention output: channel block stride of the panels (row stride 32)
  // self-attention branch
  // the block's six modulation vectors e0 + mod_bias ("Wan 技术深度解析" §2.5), formed once
  HIP_TRY(launch_mod_combine(e0, W.mod_bias, B, dim, w.mod, st));
  const bool f8g = (c.flags & WAN_FLAG_FP8_GEMM) != 0;
  const wan_block_weights_e4m3* Q8 = W.e4m3;
  if (attn_mode == WAN_ATTN_CACHE_REUSE) {
    // attention cache ("Wan 技术深度解析" §5.3): the layer output y recorded at an earlier step, gated now
    PROF_TRY(WAN_K_O_GEMM, launch_gated_add(x, attn_y, w.mod, 2, (int64_t)BS, dim, S, st));
  } else {
    float* ystore = attn_mode == WAN_ATTN_CACHE_STORE ? attn_y : nullptr;
    PROF_TRY(WAN_K_LN1, launch_ln_mod<T>(x, BS, dim, S, 0, w.mod, nullptr, 0, 1, c.ln_eps, w.u, pan, st));
    // q, k -> qkv[:, 0 .. 2 dim) (row stride 2 dim), with the RMSNorm gains and the 3D RoPE applied
    // ("图解 Wan2.1 I2V" §5.3 ①②) and the rows' sums of squares in ssq; v -> V^T directly.  The
    // prologue clears V^T's padded keys and writes the rotation table the epilogue reads.
    PROF_TRY(WAN_K_ATTN_PROLOGUE, launch_attn_prologue<T>(w.vt, (int64_t)B * dim, S, Spad, w.rope, g.T, g.Hp, g.Wp,
                                                          hd, c.rope_theta, st));
    const QKNormRope nr{W.gq, W.gk, w.ssq, w.rope, g.T, g.Hp, g.Wp};
    if (f8g) {  // E4M3 products ("Wan 技术深度解析" §5.3): per-token codes of u, then the product
      PROF_TRY(WAN_K_QUANT, launch_quant_rows_e4m3((const bf16*)w.u, pan, BS, dim, w.a8, pan, w.sa, st));
      PROF_TRY(WAN_K_QKV_GEMM, gemm_qkv_e4m3(k_panels<uint8_t>(w.a8, BS), w.sa, k_panels<uint8_t>(Q8->wqkv, 3 * dim), Q8->s_wqkv, BS, dim, dim,
                                             W.bqkv, (bf16*)w.qkv, 2 * dim, (bf16*)w.vt, S, H, hd, Spad, nr, st));
    } else {
      PROF_TRY(WAN_K_QKV_GEMM, gemm_qkv<T>(k_panels<T>(w.u, BS), k_panels<T>(W.wqkv, 3 * dim), BS, dim, dim, W.bqkv, w.qkv, 2 * dim, w.vt,
                                           S, H, hd, Spad, nr, st));
    }
    // the RMS factors: k rows scaled in place, r_q kept for the attention's score scale
    PROF_TRY(WAN_K_QK_RMS, launch_qk_rms<T>(w.ssq, BS, dim, c.rms_eps, w.qkv + dim, 2 * dim, w.rq, st));
    if constexpr (sizeof(T) == 2) {
      if (c.flags & WAN_FLAG_FP8_ATTN) {  // quantised self-attention ("Wan 技术深度解析" §5.3)
        // q codes of the rows before r_q, which the attention applies with the codes' scales
        PROF_TRY(WAN_K_QUANT, launch_quant_q(w.qkv, 2 * dim, B, S, H, hd, (int8_t*)w.q8, w.sq, st));
        PROF_TRY(WAN_K_QUANT, launch_quant_k(w.qkv + dim, 2 * dim, B, S, H, hd, (int8_t*)w.k8, w.sk, st));
        PROF_TRY(WAN_K_QUANT, launch_quant_vt(w.vt, (int64_t)B * dim, Spad, (int)round_up(S, 128), w.v8t, w.sv, st));
        PROF_TRY(WAN_K_SELF_ATTN, launch_attention_q8(w.q8, w.sq, w.k8, w.sk, w.v8t, w.sv, B, S, S, H, hd, w.o, pan, nullptr,
                                                      st, w.rq));
      }
    }
    if (!(c.flags & WAN_FLAG_FP8_ATTN)) {
      KVStream self{w.qkv + dim, (int64_t)S * 2 * dim, 2 * dim, w.vt, S, Spad};
      PROF_TRY(WAN_K_SELF_ATTN, launch_attention<T>(w.qkv, (int64_t)S * 2 * dim, 2 * dim, self, B, S, H, hd,
                                                    scale, w.o, (int64_t)S * pan.ld, pan.ld, 0, st, nullptr,
                                                    KeySplit{}, false, w.rq, o_cs));
    }
    if (f8g) {
      PROF_TRY(WAN_K_QUANT, launch_quant_rows_e4m3((const bf16*)w.o, pan, BS, dim, w.a8, pan, w.sa, st));
      PROF_TRY(WAN_K_O_GEMM, gemm_e4m3_residual(k_panels<uint8_t>(w.a8, BS), w.sa, k_panels<uint8_t>(Q8->wo, dim), Q8->s_wo, BS, dim, dim, W.bo,
                                                w.mod, 2, S, x, dim, st, ystore));
    } else {
      PROF_TRY(WAN_K_O_GEMM, gemm_residual<T>(k_panels<T>(w.o, BS), k_panels<T>(W.wo, dim), BS, dim, dim, W.bo, w.mod, 2, S, x,
                                              dim, st, ystore));
    }
  }  // self-attention branch
  // cross-attention branch (no adaLN, no RoPE)
  PROF_TRY(WAN_K_LN3, launch_ln_mod<T>(x, BS, dim, S, 1, W.ln3_w, W.ln3_b, 0, 0, c.ln_eps, w.u, pan, st));
  T* qc = w.qkv;  // reuse: [BS, dim]
  PROF_TRY(WAN_K_CROSS_Q_GEMM, (gemm_store<T, T>(k_panels<T>(w.u, BS), k_panels<T>(W.wcq, dim), BS, dim, dim, W.bcq, ACT_NONE,
                                                qc, act_rows(dim), st)));
  const int Lt = c.text_len, Li = c.img_len;
  KVStream st_txt{kv.k_txt, (int64_t)Lt * dim, dim, kv.vt_txt, Lt, (int)pad64(Lt)};
  KVStream st_img{kv.k_img, (int64_t)Li * dim, dim, kv.vt_img, Li, (int)pad64(Li > 0 ? Li : 1)};
  // text, then (I2V) image: two launches, the second adding its softmax's result to the first's (one
  // launch holding both streams' state would spill registers)
  PROF_TRY(WAN_K_CROSS_ATTN, launch_attention<T>(qc, (int64_t)S * dim, dim, st_txt, B, S, H, hd, scale, w.o,
                                                 (int64_t)S * pan.ld, pan.ld, 1, st, nullptr, KeySplit{}, false,
                                                 nullptr, o_cs));
  if (Li > 0)
    PROF_TRY(WAN_K_CROSS_ATTN, launch_attention<T>(qc, (int64_t)S * dim, dim, st_img, B, S, H, hd, scale,
                                                   w.o, (int64_t)S * pan.ld, pan.ld, 1, st, nullptr, KeySplit{}, true,
                                                   nullptr, o_cs));
  PROF_TRY(WAN_K_CROSS_O_GEMM, gemm_residual<T>(k_panels<T>(w.o, BS), k_panels<T>(W.wco, dim), BS, dim, dim, W.bco, nullptr, 0, S, x, dim, st));
  // FFN branch
  PROF_TRY(WAN_K_LN2, launch_ln_mod<T>(x, BS, dim, S, 0, w.mod, nullptr, 3, 4, c.ln_eps, w.u, pan, st));
  if (f8g) {
    const int F = c.ffn_dim;
    PROF_TRY(WAN_K_QUANT, launch_quant_rows_e4m3((const bf16*)w.u, pan, BS, dim, w.a8, pan, w.sa, st));
    PROF_TRY(WAN_K_FFN1_GEMM, gemm_e4m3_store(k_panels<uint8_t>(w.a8, BS), w.sa, k_panels<uint8_t>(Q8->w1, F), Q8->s_w1,
                                              BS, F, dim, W.b1, ACT_GELU, (bf16*)w.h, pan, st));
    PROF_TRY(WAN_K_QUANT, launch_quant_rows_e4m3((const bf16*)w.h, pan, BS, F, w.a8, pan, w.sa, st));
    PROF_TRY(WAN_K_FFN2_GEMM, gemm_e4m3_residual(k_panels<uint8_t>(w.a8, BS), w.sa, k_panels<uint8_t>(Q8->w2, dim), Q8->s_w2, BS, dim, F, W.b2,
                                                 w.mod, 5, S, x, dim, st));
  } else {
    PROF_TRY(WAN_K_FFN1_GEMM, (gemm_store<T, T>(k_panels<T>(w.u, BS), k_panels<T>(W.w1, c.ffn_dim), BS, c.ffn_dim, dim, W.b1,
                                                ACT_GELU, w.h, pan, st)));
    PROF_TRY(WAN_K_FFN2_GEMM, gemm_residual<T>(k_panels<T>(w.h, BS), k_panels<T>(W.w2, dim), BS, dim, c.ffn_dim, W.b2, w.mod,
                                               5, S, x, dim, st));
  }
  return WAN_OK;
}

int check_block_weights(const wan_block_cfg& c, const wan_block_weights* w) {
  if (!w) return fail(WAN_EINVAL, "weights is NULL");
  WAN_TRY(need_ptr(w->mod_bias, "mod_bias"));
  WAN_TRY(need_ptr(w->wqkv, "wqkv"));
  WAN_TRY(opt_ptr(w->bqkv, "bqkv"));
  WAN_TRY(need_ptr(w->gq, "gq"));
  WAN_TRY(need_ptr(w->gk, "gk"));
  WAN_TRY(need_ptr(w->wo, "wo"));
  WAN_TRY(opt_ptr(w->bo, "bo"));
  WAN_TRY(need_ptr(w->ln3_w, "ln3_w"));
  WAN_TRY(need_ptr(w->ln3_b, "ln3_b"));
  WAN_TRY(need_ptr(w->wcq, "wcq"));
  WAN_TRY(opt_ptr(w->bcq, "bcq"));
  WAN_TRY(need_ptr(w->wco, "wco"));
  WAN_TRY(opt_ptr(w->bco, "bco"));
  WAN_TRY(need_ptr(w->w1, "w1"));
  WAN_TRY(opt_ptr(w->b1, "b1"));
  WAN_TRY(need_ptr(w->w2, "w2"));
  WAN_TRY(opt_ptr(w->b2, "b2"));
  if (c.flags & WAN_FLAG_FP8_GEMM) {
    const wan_block_weights_e4m3* q = w->e4m3;
    if (!q) return fail(WAN_EINVAL, "WAN_FLAG_FP8_GEMM needs weights->e4m3");
    WAN_TRY(need_ptr(q->wqkv, "e4m3->wqkv"));
    WAN_TRY(need_ptr(q->wo, "e4m3->wo"));
    WAN_TRY(need_ptr(q->w1, "e4m3->w1"));
    WAN_TRY(need_ptr(q->w2, "e4m3->w2"));
    WAN_TRY(need_f32(q->s_wqkv, "e4m3->s_wqkv"));
    WAN_TRY(need_f32(q->s_wo, "e4m3->s_wo"));
    WAN_TRY(need_f32(q->s_w1, "e4m3->s_w1"));
    WAN_TRY(need_f32(q->s_w2, "e4m3->s_w2"));
  }
  return WAN_OK;
}

int check_kv(const wan_block_cfg& c, const wan_cross_kv* kv, bool is_output) {
  if (!kv) return fail(WAN_EINVAL, "cross kv is NULL");
  WAN_TRY(need_ptr(kv->k_txt, "k_txt"));
  WAN_TRY(need_ptr(kv->vt_txt, "vt_txt"));
  if (c.img_len > 0) {
    WAN_TRY(need_ptr(kv->k_img, "k_img"));
    WAN_TRY(need_ptr(kv->vt_img, "vt_img"));
  }
  (void)is_output;
  return WAN_OK;
}

}  // namespace

// Definitions below take their C linkage from the declarations in wan.h.

const char* wan_status_string(int status) {
  switch (status) {
    case WAN_OK: return "WAN_OK";
    case WAN_EINVAL: return "WAN_EINVAL";
    case WAN_EUNSUPPORTED: return "WAN_EUNSUPPORTED";
    case WAN_EWORKSPACE: return "WAN_EWORKSPACE";
    case WAN_EHIP: return "WAN_EHIP";
    default: return "WAN_E?";
  }
}

const char* wan_last_error(void) { return g_err; }

int wan_build_i2v_input(const float* x_t, const float* z_img, const uint8_t* known_pixel_frames_host,
                        wan_latent_shape s, float* x_in, wan_stream_t stream) {
  WAN_TRY(check_shape(s));
  if (s.T > 64) return fail(WAN_EUNSUPPORTED, "T = %d > 64 latent frames", s.T);
  WAN_TRY(need_ptr(x_t, "x_t"));
  WAN_TRY(need_ptr(z_img, "z_img"));
  WAN_TRY(need_ptr(x_in, "x_in"));
  const int F = 4 * (s.T - 1) + 1;
  uint64_t bits[4] = {0, 0, 0, 0};
  for (int e = 0; e < 4 * s.T; ++e) {
    const int frame = e < 4 ? 0 : e - 3;  // entries 0..3 repeat frame 0; entry e >= 4 is frame e - 3
    const bool known = known_pixel_frames_host ? known_pixel_frames_host[frame] != 0 : frame == 0;
    if (known) bits[e >> 6] |= 1ull << (e & 63);
  }
  (void)F;
  HIP_TRY(launch_i2v_input(x_t, z_img, bits, s.B, s.C, s.T, s.H, s.W, x_in, hs(stream)));
  return WAN_OK;
}

int wan_patchify(const float* x, wan_latent_shape s, float* p, wan_stream_t stream) {
  WAN_TRY(check_shape(s));
  WAN_TRY(need_ptr(x, "x"));
  WAN_TRY(need_ptr(p, "p"));
  HIP_TRY(launch_patchify(x, s.B, s.C, s.T, s.H, s.W, p, hs(stream)));
  return WAN_OK;
}

int wan_unpatchify(const float* p, wan_latent_shape s, float* x, wan_stream_t stream) {
  WAN_TRY(check_shape(s));
  WAN_TRY(need_ptr(p, "p"));
  WAN_TRY(need_ptr(x, "x"));
  HIP_TRY(launch_unpatchify(p, s.B, s.C, s.T, s.H, s.W, x, hs(stream)));
  return WAN_OK;
}

size_t wan_patch_embed_workspace_bytes(const wan_block_cfg* cfg, int64_t tokens, int32_t in_channels) {
  if (!cfg || tokens <= 0 || in_channels <= 0) return 0;
  return cfg->dtype == WAN_BF16 ? a256((size_t)tokens * 4 * in_channels * 2) : 0;
}

int wan_patch_embed(const wan_block_cfg* cfg, const float* p, int64_t tokens, int32_t in_channels, const void* w_pe,
                    const float* b_pe, float* x, void* ws, size_t ws_bytes, wan_stream_t stream) {
  WAN_TRY(check_cfg(cfg));
  if (tokens <= 0 || tokens > (1ll << 30) || in_channels <= 0) return fail(WAN_EINVAL, "tokens / in_channels must be positive");
  const int K = 4 * in_channels;
  if (K % 8 != 0) return fail(WAN_EUNSUPPORTED, "4*in_channels = %d must be a multiple of 8", K);
  WAN_TRY(need_ptr(p, "p"));
  WAN_TRY(need_ptr(w_pe, "w_pe"));
  WAN_TRY(opt_ptr(b_pe, "b_pe"));
  WAN_TRY(need_ptr(x, "x"));
  const size_t need = wan_patch_embed_workspace_bytes(cfg, tokens, in_channels);
  if (ws_bytes < need) return fail(WAN_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if (need) WAN_TRY(need_ptr(ws, "ws"));
  const int M = (int)tokens;
  if (cfg->dtype == WAN_BF16) {
    bf16* pb = reinterpret_cast<bf16*>(ws);
    HIP_TRY(launch_convert<bf16>(p, pb, (int64_t)M * K, hs(stream)));
    HIP_TRY((gemm_store<bf16, float>(k_rows<bf16>(pb, K), k_rows<bf16>(w_pe, K), M, cfg->dim, K, b_pe, ACT_NONE, x,
                                     act_rows(cfg->dim), hs(stream))));
  } else {
    HIP_TRY((gemm_store<float, float>(k_rows<float>(p, K), k_rows<float>(w_pe, K), M, cfg->dim, K, b_pe, ACT_NONE, x,
                                      act_rows(cfg->dim), hs(stream))));
  }
  return WAN_OK;
}

int wan_time_embed(const wan_block_cfg* cfg, int32_t freq_dim, const wan_time_weights* w, const float* t_host,
                   int32_t B, float* e, float* e0, wan_stream_t stream) {
  WAN_TRY(check_cfg(cfg));
  if (B < 1 || B > 4) return fail(WAN_EUNSUPPORTED, "time embedding batch %d not in [1, 4]", B);
  if (freq_dim <= 0 || freq_dim % 8 != 0 || freq_dim > 2 * cfg->dim)
    return fail(WAN_EINVAL, "freq_dim %d must be a positive multiple of 8 and <= 2*dim", freq_dim);
  if (!w || !t_host) return fail(WAN_EINVAL, "weights / t_host is NULL");
  WAN_TRY(need_ptr(w->wt1, "wt1"));
  WAN_TRY(need_ptr(w->wt2, "wt2"));
  WAN_TRY(need_ptr(w->wtp, "wtp"));
  WAN_TRY(opt_ptr(w->bt1, "bt1"));
  WAN_TRY(opt_ptr(w->bt2, "bt2"));
  WAN_TRY(opt_ptr(w->btp, "btp"));
  WAN_TRY(need_ptr(e, "e"));
  WAN_TRY(need_ptr(e0, "e0"));
  const int dim = cfg->dim;
  float* h = e0;                          // scratch [B, dim]
  float* emb = e0 + (int64_t)4 * B * dim;  // scratch [B, freq_dim]
  hipStream_t st = hs(stream);
  HIP_TRY(launch_sinusoid(t_host, B, freq_dim, emb, st));
  if (cfg->dtype == WAN_BF16) {
    HIP_TRY(gemv<bf16>((const bf16*)w->wt1, dim, freq_dim, emb, B, w->bt1, ACT_NONE, ACT_SILU, h, st));
    HIP_TRY(gemv<bf16>((const bf16*)w->wt2, dim, dim, h, B, w->bt2, ACT_NONE, ACT_NONE, e, st));
    HIP_TRY(gemv<bf16>((const bf16*)w->wtp, 6 * dim, dim, e, B, w->btp, ACT_SILU, ACT_NONE, e0, st));
  } else {
    HIP_TRY(gemv<float>((const float*)w->wt1, dim, freq_dim, emb, B, w->bt1, ACT_NONE, ACT_SILU, h, st));
    HIP_TRY(gemv<float>((const float*)w->wt2, dim, dim, h, B, w->bt2, ACT_NONE, ACT_NONE, e, st));
    HIP_TRY(gemv<float>((const float*)w->wtp, 6 * dim, dim, e, B, w->btp, ACT_SILU, ACT_NONE, e0, st));
  }
  return WAN_OK;
}

size_t wan_context_embed_workspace_bytes(const wan_block_cfg* cfg, int64_t rows) {
  if (!cfg || rows <= 0) return 0;
  return a256((size_t)rows * cfg->dim * esize(cfg->dtype));
}

template <typename T>
static int context_embed_t(const wan_block_cfg& c, const void* ctx, int rows, int in_dim, const void* w1,
                           const float* b1, const void* w2, const float* b2, void* out, void* ws, hipStream_t st) {
  T* hid = reinterpret_cast<T*>(ws);
  HIP_TRY((gemm_store<T, T>(k_rows<T>(ctx, in_dim), k_rows<T>(w1, in_dim), rows, c.dim, in_dim, b1, ACT_GELU, hid,
                            act_rows(c.dim), st)));
  HIP_TRY((gemm_store<T, T>(k_rows<T>(hid, c.dim), k_rows<T>(w2, c.dim), rows, c.dim, c.dim, b2, ACT_NONE, (T*)out,
                            act_rows(c.dim), st)));
  return WAN_OK;
}

int wan_context_embed(const wan_block_cfg* cfg, const void* ctx, int64_t rows, int32_t in_dim, const void* w1,
                      const float* b1, const void* w2, const float* b2, void* out, void* ws, size_t ws_bytes,
                      wan_stream_t stream) {
  WAN_TRY(check_cfg(cfg));
  if (rows <= 0 || rows > (1 << 24) || in_dim <= 0 || in_dim % 8 != 0)
    return fail(WAN_EINVAL, "rows must be positive and in_dim a positive multiple of 8");
  WAN_TRY(need_ptr(ctx, "ctx"));
  WAN_TRY(need_ptr(w1, "w1"));
  WAN_TRY(need_ptr(w2, "w2"));
  WAN_TRY(opt_ptr(b1, "b1"));
  WAN_TRY(opt_ptr(b2, "b2"));
  WAN_TRY(need_ptr(out, "out"));
  const size_t need = wan_context_embed_workspace_bytes(cfg, rows);
  if (ws_bytes < need) return fail(WAN_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  WAN_TRY(need_ptr(ws, "ws"));
  if (cfg->dtype == WAN_BF16)
    return context_embed_t<bf16>(*cfg, ctx, (int)rows, in_dim, w1, b1, w2, b2, out, ws, hs(stream));
  return context_embed_t<float>(*cfg, ctx, (int)rows, in_dim, w1, b1, w2, b2, out, ws, hs(stream));
}

size_t wan_cross_kv_buffer_bytes(const wan_block_cfg* cfg, int32_t B, int32_t which) {
  if (!cfg || B <= 0) return 0;
  const size_t es = esize(cfg->dtype);
  const int64_t L = (which < 2) ? cfg->text_len : cfg->img_len;
  if (L <= 0) return 0;
  if (which == 0 || which == 2) return (size_t)B * L * cfg->dim * es;
  if (which == 1 || which == 3) return (size_t)B * cfg->dim * pad64(L) * es;
  return 0;
}

size_t wan_cross_kv_workspace_bytes(const wan_block_cfg* cfg, int32_t B) {
  if (!cfg || B <= 0) return 0;
  const int64_t L = cfg->text_len > cfg->img_len ? cfg->text_len : cfg->img_len;
  return a256((size_t)B * L * cfg->dim * esize(cfg->dtype));
}

template <typename T>
static int cross_kv_t(const wan_block_cfg& c, const wan_cross_kv_weights& w, const void* txt, const void* img, int B,
                      const wan_cross_kv& out, void* ws, hipStream_t st) {
  const int dim = c.dim;
  T* tmp = reinterpret_cast<T*>(ws);
  for (int which = 0; which < 2; ++which) {
    const int L = which == 0 ? c.text_len : c.img_len;
    if (L <= 0) continue;
    const T* ctx = (const T*)(which == 0 ? txt : img);
    const T* wkv = (const T*)(which == 0 ? w.wkv_txt : w.wkv_img);
    const float* bkv = which == 0 ? w.bkv_txt : w.bkv_img;
    T* k = (T*)(which == 0 ? out.k_txt : out.k_img);
    T* vt = (T*)(which == 0 ? out.vt_txt : out.vt_img);
    const int M = B * L;
    HIP_TRY((gemm_store<T, T>(k_rows<T>(ctx, dim), k_rows<T>(wkv, dim), M, dim, dim, bkv, ACT_NONE, k, act_rows(dim), st)));
    HIP_TRY((gemm_store<T, T>(k_rows<T>(ctx, dim), k_rows<T>(wkv + (int64_t)dim * dim, dim), M, dim, dim,
                              bkv ? bkv + dim : nullptr, ACT_NONE, tmp, act_rows(dim), st)));
    HIP_TRY(launch_transpose_heads<T>(tmp, dim, 0, B, L, c.heads, c.head_dim, (int)pad64(L), vt, st));
  }
  return WAN_OK;
}

int wan_cross_kv_fwd(const wan_block_cfg* cfg, const wan_cross_kv_weights* w, const void* txt_emb, const void* img_emb,
                     int32_t B, const wan_cross_kv* out, void* ws, size_t ws_bytes, wan_stream_t stream) {
  WAN_TRY(check_cfg(cfg));
  if (B <= 0) return fail(WAN_EINVAL, "B must be positive");
  if (!w) return fail(WAN_EINVAL, "weights is NULL");
  WAN_TRY(need_ptr(w->wkv_txt, "wkv_txt"));
  WAN_TRY(opt_ptr(w->bkv_txt, "bkv_txt"));
  WAN_TRY(need_ptr(txt_emb, "txt_emb"));
  if (cfg->img_len > 0) {
    WAN_TRY(need_ptr(w->wkv_img, "wkv_img"));
    WAN_TRY(opt_ptr(w->bkv_img, "bkv_img"));
    WAN_TRY(need_ptr(img_emb, "img_emb"));
  }
  WAN_TRY(check_kv(*cfg, out, true));
  const size_t need = wan_cross_kv_workspace_bytes(cfg, B);
  if (ws_bytes < need) return fail(WAN_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  WAN_TRY(need_ptr(ws, "ws"));
  if (cfg->dtype == WAN_BF16) return cross_kv_t<bf16>(*cfg, *w, txt_emb, img_emb, B, *out, ws, hs(stream));
  return cross_kv_t<float>(*cfg, *w, txt_emb, img_emb, B, *out, ws, hs(stream));
}

size_t wan_dit_block_workspace_bytes(const wan_block_cfg* cfg, wan_grid grid, int32_t B) {
  if (!cfg || B <= 0 || grid.T <= 0 || grid.Hp <= 0 || grid.Wp <= 0) return 0;
  if (cfg->dtype == WAN_BF16) return block_plan<bf16>(*cfg, grid, B, nullptr, nullptr);
  return block_plan<float>(*cfg, grid, B, nullptr, nullptr);
}

int wan_dit_block_fwd(const wan_block_cfg* cfg, const wan_block_weights* w, wan_grid grid, int32_t B, float* x,
                      const float* e0, const wan_cross_kv* kv, void* ws, size_t ws_bytes, wan_stream_t stream) {
  return wan_dit_block_fwd_cached(cfg, w, grid, B, x, e0, kv, nullptr, WAN_ATTN_CACHE_OFF, ws, ws_bytes, stream);
}

int wan_dit_block_fwd_cached(const wan_block_cfg* cfg, const wan_block_weights* w, wan_grid grid, int32_t B, float* x,
                             const float* e0, const wan_cross_kv* kv, float* attn_y, int32_t attn_mode, void* ws,
                             size_t ws_bytes, wan_stream_t stream) {
  if (attn_mode != WAN_ATTN_CACHE_OFF && attn_mode != WAN_ATTN_CACHE_STORE && attn_mode != WAN_ATTN_CACHE_REUSE)
    return fail(WAN_EINVAL, "attn_mode %d not in 0..2", attn_mode);
  if (attn_mode != WAN_ATTN_CACHE_OFF) WAN_TRY(need_ptr(attn_y, "attn_y"));
  WAN_TRY(check_cfg(cfg));
  WAN_TRY(check_grid(grid));
  if (B <= 0) return fail(WAN_EINVAL, "B must be positive");
  if ((int64_t)B * grid.T * grid.Hp * grid.Wp > (1ll << 30)) return fail(WAN_EUNSUPPORTED, "too many rows");
  WAN_TRY(check_block_weights(*cfg, w));
  WAN_TRY(need_ptr(x, "x"));
  WAN_TRY(need_ptr(e0, "e0"));
  WAN_TRY(check_kv(*cfg, kv, false));
  const size_t need = wan_dit_block_workspace_bytes(cfg, grid, B);
  if (ws_bytes < need) return fail(WAN_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  WAN_TRY(need_ptr(ws, "ws"));
  if (cfg->dtype == WAN_BF16)
    return block_fwd_t<bf16>(*cfg, *w, grid, B, x, e0, *kv, ws, hs(stream), attn_y, attn_mode);
  return block_fwd_t<float>(*cfg, *w, grid, B, x, e0, *kv, ws, hs(stream), attn_y, attn_mode);
}

// ---- the block without a caller workspace: the scratch lives in a static device array ----------------
// One array per device the library runs on, held until the process ends.  In host code `scratch` names
// a host-side stand-in: its device address comes from hipGetSymbolAddress, taken once per device (with
// that device current) and kept in g_scratch_dev; only that address is ever passed to kernels.
static __device__ __align__(256) unsigned char scratch[WAN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[SCRATCH_MAX_DEVICES];

// Device address of the current device's scratch array (looked up on the first call on that device).
int scratch_address(void** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return fail(WAN_EUNSUPPORTED, "device %d has no scratch slot", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (p == nullptr) return fail(WAN_EHIP, "hipGetSymbolAddress returned no address for the scratch array");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return WAN_OK;
}

}  // namespace

int wan_dit_block_fwd_noalloc(const wan_block_cfg* cfg, const wan_block_weights* w, wan_grid grid, int32_t B,
                              float* x, const float* e0, const wan_cross_kv* kv, wan_stream_t stream) {
  WAN_TRY(check_cfg(cfg));
  WAN_TRY(check_grid(grid));
  if (B <= 0) return fail(WAN_EINVAL, "B must be positive");
  const size_t need = wan_dit_block_workspace_bytes(cfg, grid, B);
  if (need > WAN_NOALLOC_SCRATCH_BYTES)
    return fail(WAN_EWORKSPACE,
                "block needs %zu bytes of scratch; wan_dit_block_fwd_noalloc holds %zu (use wan_dit_block_fwd with "
                "a caller workspace)", need, (size_t)WAN_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  WAN_TRY(scratch_address(&ws));
  return wan_dit_block_fwd(cfg, w, grid, B, x, e0, kv, ws, WAN_NOALLOC_SCRATCH_BYTES, stream);
}

size_t wan_head_workspace_bytes(const wan_block_cfg* cfg, int64_t tokens) {
  if (!cfg || tokens <= 0) return 0;
  return a256((size_t)tokens * cfg->dim * esize(cfg->dtype));
}

int wan_head_fwd(const wan_block_cfg* cfg, const wan_head_weights* w, int32_t out_channels, int32_t B, int32_t S,
                 const float* x, const float* e, float* out, void* ws, size_t ws_bytes, wan_stream_t stream) {
  WAN_TRY(check_cfg(cfg));
  if (B <= 0 || S <= 0 || out_channels <= 0) return fail(WAN_EINVAL, "B, S, out_channels must be positive");
  if ((4 * out_channels) % 8 != 0) return fail(WAN_EUNSUPPORTED, "4*out_channels must be a multiple of 8");
  if (!w) return fail(WAN_EINVAL, "weights is NULL");
  WAN_TRY(need_ptr(w->head_mod, "head_mod"));
  WAN_TRY(need_ptr(w->wh, "wh"));
  WAN_TRY(opt_ptr(w->bh, "bh"));
  WAN_TRY(need_ptr(x, "x"));
  WAN_TRY(need_ptr(e, "e"));
  WAN_TRY(need_ptr(out, "out"));
  const int64_t rows = (int64_t)B * S;
  const size_t need = wan_head_workspace_bytes(cfg, rows);
  if (ws_bytes < need) return fail(WAN_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  WAN_TRY(need_ptr(ws, "ws"));
  const int N = 4 * out_channels, dim = cfg->dim;
  hipStream_t st = hs(stream);
  if (cfg->dtype == WAN_BF16) {
    bf16* u = reinterpret_cast<bf16*>(ws);
    HIP_TRY(launch_ln_mod<bf16>(x, rows, dim, S, 2, w->head_mod, e, 0, 1, cfg->ln_eps, u, act_rows(dim), st));
    HIP_TRY((gemm_store<bf16, float>(k_rows<bf16>(u, dim), k_rows<bf16>(w->wh, dim), (int)rows, N, dim, w->bh, ACT_NONE,
                                     out, act_rows(N), st)));
  } else {
    float* u = reinterpret_cast<float*>(ws);
    HIP_TRY(launch_ln_mod<float>(x, rows, dim, S, 2, w->head_mod, e, 0, 1, cfg->ln_eps, u, act_rows(dim), st));
    HIP_TRY((gemm_store<float, float>(k_rows<float>(u, dim), k_rows<float>(w->wh, dim), (int)rows, N, dim, w->bh,
                                      ACT_NONE, out, act_rows(N), st)));
  }
  return WAN_OK;
}

int wan_fm_euler_step(float* x, const float* v_cond, const float* v_uncond, float guidance, float dt, int64_t n,
                      wan_stream_t stream) {
  if (n < 0) return fail(WAN_EINVAL, "n must be >= 0");
  WAN_TRY(need_ptr(x, "x"));
  WAN_TRY(need_ptr(v_cond, "v_cond"));
  WAN_TRY(opt_ptr(v_uncond, "v_uncond"));
  HIP_TRY(launch_euler(x, v_cond, v_uncond, guidance, dt, n, hs(stream)));
  return WAN_OK;
}

size_t wan_attention_workspace_bytes(int32_t dtype, wan_grid g, int32_t B, int32_t heads, int32_t head_dim) {
  if ((dtype != WAN_F32 && dtype != WAN_BF16) || B <= 0 || heads <= 0 || head_dim <= 0) return 0;
  if (g.T <= 0 || g.Hp <= 0 || g.Wp <= 0) return 0;
  const int64_t S = (int64_t)g.T * g.Hp * g.Wp, dim = (int64_t)heads * head_dim;
  const size_t es = esize(dtype);
  return 2 * a256((size_t)B * S * dim * es) + a256((size_t)B * dim * pad64(S) * es);
}

template <typename T>
static int attention_t(const T* q, const T* k, const T* v, const wan_grid& g, int B, int H, int hd, float theta, T* o,
                       void* ws, hipStream_t st) {
  const int S = g.T * g.Hp * g.Wp, dim = H * hd, Spad = (int)pad64(S);
  Carve cv{reinterpret_cast<char*>(ws)};
  T* qr = cv.take<T>((size_t)B * S * dim);
  T* kr = cv.take<T>((size_t)B * S * dim);
  T* vt = cv.take<T>((size_t)B * dim * Spad);
  HIP_TRY(launch_rope_qk<T>(q, k, dim, qr, kr, dim, B, g.T, g.Hp, g.Wp, H, hd, theta, st));
  HIP_TRY(launch_transpose_heads<T>(v, dim, 0, B, S, H, hd, Spad, vt, st));
  KVStream s0{kr, (int64_t)S * dim, dim, vt, S, Spad};
  HIP_TRY(launch_attention<T>(qr, (int64_t)S * dim, dim, s0, B, S, H, hd, 1.f / sqrtf((float)hd), o,
                              (int64_t)S * dim, dim, 0, st));
  return WAN_OK;
}

int wan_attention_fwd(int32_t dtype, const void* q, const void* k, const void* v, wan_grid grid, int32_t B,
                      int32_t heads, int32_t head_dim, float rope_theta, void* o, void* ws, size_t ws_bytes,
                      wan_stream_t stream) {
  WAN_TRY(check_dtype(dtype));
  WAN_TRY(check_grid(grid));
  if (B <= 0 || heads <= 0) return fail(WAN_EINVAL, "B and heads must be positive");
  if (head_dim != 64 && head_dim != 128) return fail(WAN_EUNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (heads * head_dim > 6144) return fail(WAN_EUNSUPPORTED, "heads*head_dim > 6144");
  if (!(rope_theta > 0.f)) return fail(WAN_EINVAL, "rope_theta must be > 0");
  if ((int64_t)B * grid.T * grid.Hp * grid.Wp > (1ll << 30)) return fail(WAN_EUNSUPPORTED, "too many rows");
  WAN_TRY(need_ptr(q, "q"));
  WAN_TRY(need_ptr(k, "k"));
  WAN_TRY(need_ptr(v, "v"));
  WAN_TRY(need_ptr(o, "o"));
  const size_t need = wan_attention_workspace_bytes(dtype, grid, B, heads, head_dim);
  if (ws_bytes < need) return fail(WAN_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  WAN_TRY(need_ptr(ws, "ws"));
  if (dtype == WAN_BF16)
    return attention_t<bf16>((const bf16*)q, (const bf16*)k, (const bf16*)v, grid, B, heads, head_dim, rope_theta,
                             (bf16*)o, ws, hs(stream));
  return attention_t<float>((const float*)q, (const float*)k, (const float*)v, grid, B, heads, head_dim, rope_theta,
                            (float*)o, ws, hs(stream));
}

namespace {

// Key split of a partial attention whose grid would leave compute units idle: n parts of `chunk` keys
// (a multiple of 64, at least 256).  Cost in units of one workgroup's 64-key tile:
//   rounds(n) * (tiles(n) + SPLIT_FIXED_TILES) + merge(n),
// rounds = ceil(nwg * n / resident slots), tiles = chunk / 64, SPLIT_FIXED_TILES the per-workgroup
// start and finish (Q load, first tiles, normalisation, store), and merge = the (n + 1) o-part passes
// of the merge at HBM speed over the time of one tile.  Workspace layout: V^T, then n o-parts
// [B, Sq, H, hd] and n lse-parts [B, H, Sq], each 256-byte aligned.
constexpr double SPLIT_FIXED_TILES = 8.0;
constexpr double SPLIT_CU_FLOPS = 4.9e12;   // one compute unit's bf16 attention rate (flop/s)
constexpr double SPLIT_MERGE_BW = 4.5e12;   // the merge's bandwidth (B/s)
struct PartialPlan {
  int n = 1, chunk = 0;
  size_t vt_bytes = 0, o_part_bytes = 0, lse_part_bytes = 0, bytes = 0;
};

PartialPlan partial_plan(int32_t dtype, int B, int Sq, int Sk, int H, int hd) {
  PartialPlan p;
  const size_t es = esize(dtype);
  p.vt_bytes = a256((size_t)B * H * hd * pad64(Sk) * es);
  p.bytes = p.vt_bytes;
  p.chunk = (int)pad64(Sk);
  int rows = 0, per_cu = 0;
  if (dtype == WAN_BF16)
    attention_tile<bf16>(0, rows, per_cu);
  else
    attention_tile<float>(0, rows, per_cu);
  const int64_t nwg = ceil_div((int64_t)Sq, (int64_t)rows) * H * B;
  const int64_t slots = (int64_t)device_compute_units() * per_cu;
  const double tile_s = (double)rows * 64 * hd * 4 / SPLIT_CU_FLOPS;
  const double part_tiles = (double)B * Sq * H * hd * es / SPLIT_MERGE_BW / tile_s;
  double best = (double)ceil_div(nwg, slots) * ((double)ceil_div((int64_t)Sk, (int64_t)64) + SPLIT_FIXED_TILES);
  for (int n = 2; n <= MERGE_MAX_PARTS && (int64_t)B * n <= 65535; ++n) {
    const int chunk = (int)pad64(ceil_div((int64_t)Sk, (int64_t)n));
    if (chunk < 256 || (int64_t)(n - 1) * chunk >= Sk) continue;
    const double cost = (double)ceil_div(nwg * n, slots) * (chunk / 64 + SPLIT_FIXED_TILES) + (n + 1) * part_tiles;
    if (cost < best - 1e-9) {
      best = cost;
      p.n = n;
      p.chunk = chunk;
    }
  }
  if (p.n > 1) {
    p.o_part_bytes = a256((size_t)B * Sq * H * hd * es);
    p.lse_part_bytes = a256((size_t)B * H * Sq * 4);
    p.bytes += (size_t)p.n * (p.o_part_bytes + p.lse_part_bytes);
  }
  return p;
}

}  // namespace

size_t wan_attention_partial_workspace_bytes(int32_t dtype, int32_t B, int32_t Sq, int32_t Sk, int32_t heads,
                                             int32_t head_dim) {
  if ((dtype != WAN_F32 && dtype != WAN_BF16) || B <= 0 || Sq <= 0 || Sk <= 0 || heads <= 0 || head_dim <= 0) return 0;
  return partial_plan(dtype, B, Sq, Sk, heads, head_dim).bytes;
}

namespace {

template <typename T>
int attention_partial_t(const T* q, const T* k, const T* v, int B, int Sq, int Sk, int H, int hd, T* o, float* lse,
                        void* ws, size_t ws_bytes, hipStream_t st) {
  const int64_t dim = (int64_t)H * hd;
  const int Skpad = (int)pad64(Sk);
  T* vt = reinterpret_cast<T*>(ws);
  HIP_TRY(launch_transpose_heads<T>(v, dim, 0, B, Sk, H, hd, Skpad, vt, st));
  KVStream s0{k, (int64_t)Sk * dim, dim, vt, Sk, Skpad};
  const float scale = 1.f / sqrtf((float)hd);
  const PartialPlan p = partial_plan(sizeof(T) == 2 ? WAN_BF16 : WAN_F32, B, Sq, Sk, H, hd);
  if (p.n == 1 || ws_bytes < p.bytes) {  // unsplit (also when the workspace holds only V^T)
    HIP_TRY(launch_attention<T>(q, (int64_t)Sq * dim, dim, s0, B, Sq, H, hd, scale, o, (int64_t)Sq * dim, dim,
                                0, st, lse));
    return WAN_OK;
  }
  char* base = reinterpret_cast<char*>(ws) + p.vt_bytes;
  T* o_parts = reinterpret_cast<T*>(base);
  float* l_parts = reinterpret_cast<float*>(base + (size_t)p.n * p.o_part_bytes);
  KeySplit ks;
  ks.n = p.n;
  ks.chunk = p.chunk;
  ks.o_stride = (int64_t)(p.o_part_bytes / sizeof(T));
  ks.lse_stride = (int64_t)(p.lse_part_bytes / 4);
  HIP_TRY(launch_attention<T>(q, (int64_t)Sq * dim, dim, s0, B, Sq, H, hd, scale, o_parts, (int64_t)Sq * dim,
                              dim, 0, st, l_parts, ks));
  const void* op[MERGE_MAX_PARTS];
  const float* lp[MERGE_MAX_PARTS];
  for (int i = 0; i < p.n; ++i) {
    op[i] = o_parts + i * ks.o_stride;
    lp[i] = l_parts + i * ks.lse_stride;
  }
  HIP_TRY(launch_lse_merge<T>(op, lp, p.n, B, Sq, H, hd, o, lse, st));
  return WAN_OK;
}

}  // namespace

int wan_attention_partial_fwd(int32_t dtype, const void* q, const void* k, const void* v, int32_t B, int32_t Sq,
                              int32_t Sk, int32_t heads, int32_t head_dim, void* o, float* lse, void* ws,
                              size_t ws_bytes, wan_stream_t stream) {
  WAN_TRY(check_dtype(dtype));
  if (B <= 0 || Sq <= 0 || Sk <= 0 || heads <= 0) return fail(WAN_EINVAL, "B, Sq, Sk and heads must be positive");
  if (head_dim != 64 && head_dim != 128) return fail(WAN_EUNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (heads * head_dim > 6144) return fail(WAN_EUNSUPPORTED, "heads*head_dim > 6144");
  if ((int64_t)B * Sq > (1ll << 30) || (int64_t)B * Sk > (1ll << 30)) return fail(WAN_EUNSUPPORTED, "too many rows");
  WAN_TRY(need_ptr(q, "q"));
  WAN_TRY(need_ptr(k, "k"));
  WAN_TRY(need_ptr(v, "v"));
  WAN_TRY(need_ptr(o, "o"));
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3)) return fail(WAN_EINVAL, "lse is not 4-byte aligned");
  const size_t need = a256((size_t)B * heads * head_dim * pad64(Sk) * esize(dtype));  // V^T: the unsplit minimum
  if (ws_bytes < need) return fail(WAN_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  WAN_TRY(need_ptr(ws, "ws"));
  if (dtype == WAN_BF16)
    return attention_partial_t<bf16>((const bf16*)q, (const bf16*)k, (const bf16*)v, B, Sq, Sk, heads, head_dim,
                                     (bf16*)o, lse, ws, ws_bytes, hs(stream));
  return attention_partial_t<float>((const float*)q, (const float*)k, (const float*)v, B, Sq, Sk, heads, head_dim,
                                    (float*)o, lse, ws, ws_bytes, hs(stream));
}

int wan_attention_lse_merge(int32_t dtype, int32_t n_parts, const void* const* o_parts, const float* const* lse_parts,
                            int32_t B, int32_t S, int32_t heads, int32_t head_dim, void* o, float* lse,
                            wan_stream_t stream) {
  WAN_TRY(check_dtype(dtype));
  if (n_parts < 1 || n_parts > MERGE_MAX_PARTS) return fail(WAN_EINVAL, "n_parts %d not in 1..%d", n_parts, MERGE_MAX_PARTS);
  if (B <= 0 || S <= 0 || heads <= 0) return fail(WAN_EINVAL, "B, S and heads must be positive");
  if (head_dim != 64 && head_dim != 128) return fail(WAN_EUNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if ((int64_t)B * S * heads * head_dim > (1ll << 40)) return fail(WAN_EUNSUPPORTED, "too many elements");
  if (!o_parts || !lse_parts) return fail(WAN_EINVAL, "o_parts / lse_parts are NULL");
  for (int i = 0; i < n_parts; ++i) {
    WAN_TRY(need_ptr(o_parts[i], "o_parts[i]"));
    if (!lse_parts[i] || (reinterpret_cast<uintptr_t>(lse_parts[i]) & 3))
      return fail(WAN_EINVAL, "lse_parts[%d] is NULL or not 4-byte aligned", i);
  }
  WAN_TRY(need_ptr(o, "o"));
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3)) return fail(WAN_EINVAL, "lse is not 4-byte aligned");
  if (dtype == WAN_BF16)
    HIP_TRY(launch_lse_merge<bf16>(o_parts, lse_parts, n_parts, B, S, heads, head_dim, (bf16*)o, lse, hs(stream)));
  else
    HIP_TRY(launch_lse_merge<float>(o_parts, lse_parts, n_parts, B, S, heads, head_dim, (float*)o, lse, hs(stream)));
  return WAN_OK;
}

size_t wan_attention_q8_quantize_workspace_bytes(int32_t B, int32_t Sk, int32_t heads, int32_t head_dim) {
  if (B <= 0 || Sk <= 0 || heads <= 0 || head_dim <= 0) return 0;
  return a256((size_t)B * heads * head_dim * pad64(Sk) * 2);
}

static int check_q8_shape(int32_t B, int32_t Sq, int32_t Sk, int32_t heads, int32_t head_dim) {
  if (B <= 0 || Sq <= 0 || Sk <= 0 || heads <= 0) return fail(WAN_EINVAL, "B, Sq, Sk and heads must be positive");
  if (head_dim != 128) return fail(WAN_EUNSUPPORTED, "head_dim %d not supported by the quantised path (128)", head_dim);
  if (heads * head_dim > 6144) return fail(WAN_EUNSUPPORTED, "heads*head_dim > 6144");
  if ((int64_t)B * Sq > (1ll << 30) || (int64_t)B * Sk > (1ll << 30)) return fail(WAN_EUNSUPPORTED, "too many rows");
  return WAN_OK;
}

int wan_attention_q8_quantize(const void* q, const void* k, const void* v, int32_t B, int32_t Sq, int32_t Sk,
                              int32_t heads, int32_t head_dim, void* q8, float* sq, void* k8, float* sk, void* v8t,
                              float* sv, void* ws, size_t ws_bytes, wan_stream_t stream) {
  WAN_TRY(check_q8_shape(B, Sq, Sk, heads, head_dim));
  WAN_TRY(need_ptr(q, "q"));
  WAN_TRY(need_ptr(k, "k"));
  WAN_TRY(need_ptr(v, "v"));
  WAN_TRY(need_ptr(q8, "q8"));
  WAN_TRY(need_ptr(k8, "k8"));
  WAN_TRY(need_ptr(v8t, "v8t"));
  WAN_TRY(need_f32(sq, "sq"));
  WAN_TRY(need_f32(sk, "sk"));
  WAN_TRY(need_ptr(sv, "sv"));
  const size_t need = wan_attention_q8_quantize_workspace_bytes(B, Sk, heads, head_dim);
  if (ws_bytes < need) return fail(WAN_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  WAN_TRY(need_ptr(ws, "ws"));
  const int dim = heads * head_dim, Skpad = (int)pad64(Sk);
  const hipStream_t st = hs(stream);
  bf16* vt = reinterpret_cast<bf16*>(ws);
  HIP_TRY(launch_quant_q((const bf16*)q, dim, B, Sq, heads, head_dim, (int8_t*)q8, sq, st));
  HIP_TRY(launch_quant_k((const bf16*)k, dim, B, Sk, heads, head_dim, (int8_t*)k8, sk, st));
  HIP_TRY(launch_transpose_heads<bf16>((const bf16*)v, dim, 0, B, Sk, heads, head_dim, Skpad, vt, st));
  HIP_TRY(launch_quant_vt(vt, (int64_t)B * dim, Skpad, (int)round_up(Sk, 128), (uint8_t*)v8t, sv, st));
  return WAN_OK;
}

int wan_attention_q8_fwd(const void* q8, const float* sq, const void* k8, const float* sk, const void* v8t,
                         const float* sv, int32_t B, int32_t Sq, int32_t Sk, int32_t heads, int32_t head_dim, void* o,
                         float* lse, wan_stream_t stream) {
  WAN_TRY(check_q8_shape(B, Sq, Sk, heads, head_dim));
  WAN_TRY(need_ptr(q8, "q8"));
  WAN_TRY(need_ptr(k8, "k8"));
  WAN_TRY(need_ptr(v8t, "v8t"));
  WAN_TRY(need_f32(sq, "sq"));
  WAN_TRY(need_f32(sk, "sk"));
  WAN_TRY(need_ptr(sv, "sv"));
  WAN_TRY(need_ptr(o, "o"));
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3)) return fail(WAN_EINVAL, "lse is not 4-byte aligned");
  HIP_TRY(launch_attention_q8((const uint8_t*)q8, sq, (const uint8_t*)k8, sk, (const uint8_t*)v8t, sv, B, Sq, Sk,
                              heads, head_dim, (bf16*)o, act_rows((int64_t)heads * head_dim), lse, hs(stream)));
  return WAN_OK;
}

int wan_quantize_rows_e4m3(const void* x, int64_t ld, int32_t rows, int32_t cols, void* codes, int64_t ldc,
                           float* scales, wan_stream_t stream) {
  if (rows <= 0 || cols <= 0 || cols % 8 != 0) return fail(WAN_EINVAL, "rows > 0 and cols a positive multiple of 8");
  if (ld < cols || ld % 8 != 0 || ldc < cols || ldc % 16 != 0) return fail(WAN_EINVAL, "bad row strides");
  WAN_TRY(need_ptr(x, "x"));
  WAN_TRY(need_ptr(codes, "codes"));
  WAN_TRY(need_f32(scales, "scales"));
  HIP_TRY(launch_quant_rows_e4m3((const bf16*)x, act_rows(ld), rows, cols, (uint8_t*)codes, act_rows(ldc), scales,
                                 hs(stream)));
  return WAN_OK;
}

int wan_quantize_tensor_e4m3(const void* x, int64_t n, void* codes, float* scale, void* ws, size_t ws_bytes,
                             wan_stream_t stream) {
  if (n <= 0 || n % 8 != 0) return fail(WAN_EINVAL, "n must be a positive multiple of 8");
  WAN_TRY(need_ptr(x, "x"));
  WAN_TRY(need_ptr(codes, "codes"));
  WAN_TRY(need_f32(scale, "scale"));
  if (ws_bytes < 256) return fail(WAN_EWORKSPACE, "workspace %zu < 256 bytes", ws_bytes);
  WAN_TRY(need_ptr(ws, "ws"));
  HIP_TRY(launch_quant_tensor_e4m3((const bf16*)x, n, (uint8_t*)codes, scale, (uint32_t*)ws, hs(stream)));
  return WAN_OK;
}

size_t wan_pack_weight_bytes(int32_t elem_bytes, int64_t N, int64_t K) {
  if ((elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4) || N <= 0 || K <= 0 || K % 32 != 0) return 0;
  return (size_t)panel_rows(N) * (size_t)K * (size_t)elem_bytes;
}

int wan_pack_weight(int32_t elem_bytes, const void* w, int64_t N, int64_t K, void* packed, wan_stream_t stream) {
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4) return fail(WAN_EINVAL, "elem_bytes must be 1, 2 or 4");
  if (N <= 0 || K <= 0 || K % 32 != 0) return fail(WAN_EINVAL, "N > 0 and K a positive multiple of 32");
  WAN_TRY(need_ptr(w, "w"));
  WAN_TRY(need_ptr(packed, "packed"));
  HIP_TRY(launch_pack_panels(w, N, K, K, elem_bytes, packed, hs(stream)));
  return WAN_OK;
}

int wan_gemm_e4m3(const void* a, const float* a_scales, const void* w, const float* w_scale, int32_t M, int32_t N,
                  int32_t K, const float* bias, int32_t act, void* y, int64_t ldy, wan_stream_t stream) {
  if (M <= 0 || N <= 0 || N % 4 != 0) return fail(WAN_EINVAL, "M > 0 and N a positive multiple of 4");
  if (K <= 0 || K % 256 != 0) return fail(WAN_EUNSUPPORTED, "K %d must be a positive multiple of 256", K);
  if (ldy < N || ldy % 4 != 0) return fail(WAN_EINVAL, "bad row stride ldy");
  if ((int64_t)K * panel_rows(N) >= ((int64_t)1 << 31) || (int64_t)K * panel_rows(M) >= ((int64_t)1 << 31))
    return fail(WAN_EUNSUPPORTED, "operand panels of 2 GiB or more");
  if (act != ACT_NONE && act != ACT_GELU) return fail(WAN_EINVAL, "act must be 0 or 1");
  WAN_TRY(need_ptr(a, "a"));
  WAN_TRY(need_ptr(w, "w"));
  WAN_TRY(need_f32(a_scales, "a_scales"));
  WAN_TRY(need_f32(w_scale, "w_scale"));
  WAN_TRY(opt_ptr(bias, "bias"));
  WAN_TRY(need_ptr(y, "y"));
  HIP_TRY(gemm_e4m3_store(k_panels<uint8_t>(a, M), a_scales, k_panels<uint8_t>(w, N), w_scale, M, N, K, bias, act,
                          (bf16*)y, act_rows(ldy), hs(stream)));
  return WAN_OK;
}

int wan_device_info(int32_t* compute_units, int32_t* clock_khz) {
  if (!compute_units || !clock_khz) return fail(WAN_EINVAL, "compute_units / clock_khz is NULL");
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  HIP_TRY(hipDeviceGetAttribute(compute_units, hipDeviceAttributeMultiprocessorCount, dev));
  HIP_TRY(hipDeviceGetAttribute(clock_khz, hipDeviceAttributeClockRate, dev));
  return WAN_OK;
}

int wan_mfma_peak_probe(int32_t kind, uint32_t a_word, uint32_t b_word, int32_t blocks, int32_t iters, float* out,
                        wan_stream_t stream) {
  if (kind < 0 || kind > 2)
    return fail(WAN_EINVAL, "kind must be 0 (bf16), 1 (E4M3) or 2 (bf16, hashed operands), got %d", kind);
  if (blocks < 1 || blocks > (1 << 20)) return fail(WAN_EINVAL, "blocks must be in 1..2^20, got %d", blocks);
  if (iters < 1 || iters > (1 << 20)) return fail(WAN_EINVAL, "iters must be in 1..2^20, got %d", iters);
  WAN_TRY(need_f32(out, "out"));
  HIP_TRY(launch_mfma_peak(kind, a_word, b_word, blocks, iters, out, hs(stream)));
  return WAN_OK;
}

int wan_profile_begin(void* const* start_events, void* const* stop_events, int32_t* tags, int32_t capacity,
                      uint32_t kernel_mask) {
  if (capacity < 0) return fail(WAN_EINVAL, "capacity must be >= 0");
  if (capacity > 0 && (!start_events || !stop_events || !tags))
    return fail(WAN_EINVAL, "event / tag arrays are NULL");
  g_prof.starts = reinterpret_cast<hipEvent_t*>(const_cast<void**>(start_events));
  g_prof.stops = reinterpret_cast<hipEvent_t*>(const_cast<void**>(stop_events));
  g_prof.tags = tags;
  g_prof.cap = capacity;
  g_prof.n = 0;
  g_prof.mask = kernel_mask;
  return WAN_OK;
}

int32_t wan_profile_end(void) {
  const int32_t n = g_prof.n;
  g_prof = Profile{};
  return n;
}
