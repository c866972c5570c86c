// Internal launchers shared by the kernel files and the C-ABI layer.
// Every launcher enqueues on `stream` and returns hipGetLastError() of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wan_common.h"

namespace wan {

// Compute units of the current device, queried once per device (256 when no device answers).
int device_compute_units();

// Activation applied in a GEMM / GEMV epilogue.
enum Act { ACT_NONE = 0, ACT_GELU = 1, ACT_SILU = 2 };

// ---- layout (layout.hip) ----------------------------------------------------
hipError_t launch_i2v_input(const float* x_t, const float* z_img, const uint64_t mask_bits[4], int B, int C,
                            int T, int H, int W, float* x_in, hipStream_t s);
hipError_t launch_patchify(const float* x, int B, int C, int T, int H, int W, float* p, hipStream_t s);
hipError_t launch_unpatchify(const float* p, int B, int C, int T, int H, int W, float* x, hipStream_t s);
hipError_t launch_euler(float* x, const float* v_c, const float* v_u, float guidance, float dt, int64_t n,
                        hipStream_t s);
template <typename T>
hipError_t launch_convert(const float* in, T* out, int64_t n, hipStream_t s);
// V [B, S, *] rows (row stride ld elements, head h at column col0 + h*hd) -> V^T [B, H, hd, Spad],
// zero-filled for tokens S..Spad-1.
template <typename T>
hipError_t launch_transpose_heads(const T* v, int64_t ld, int64_t col0, int B, int S, int H, int hd, int Spad,
                                  T* vt, hipStream_t s);

// x[m, n] += mod[m / S][chunk][n] * y[m, n] for m < rows, n < dim (all float32; dim % 4 == 0): the
// gated residual of a cached branch output y.
hipError_t launch_gated_add(float* x, const float* y, const float* mod, int chunk, int64_t rows, int dim, int S,
                            hipStream_t s);

// mod[b, c, n] = e0[b, c, n] + mb[c, n] for b < B, c < 6, n < dim: a block's six modulation vectors
// (e0 [B, 6, dim] from the shared timestep MLP, mb [6, dim] the block's own bias).
hipError_t launch_mod_combine(const float* e0, const float* mb, int B, int dim, float* mod, hipStream_t s);

// The block's launch before its Q/K/V product, two jobs in one grid:
//  * zero V^T[r, S16 .. Spad) for rows r < rows (row stride Spad), S16 = S rounded down to 16: every
//    position that can hold a padded key of the last tile (bf16 V^T permutes keys within 16-key
//    groups); runs before the keys < S are written;
//  * write the 3D RoPE table of a T_ x Hp x Wp grid and head dim hd (rope_table_entries float2 of
//    (cos, sin); layout at QKNormRope) for the product's epilogue.
template <typename T>
hipError_t launch_attn_prologue(T* vt, int64_t rows, int S, int Spad, float2* rope, int T_, int Hp, int Wp, int hd,
                                float theta, hipStream_t s);
inline int64_t rope_table_entries(int T_, int Hp, int Wp, int hd) {
  return (int64_t)T_ * rope_pairs_time(hd) + (int64_t)(Hp + Wp) * rope_pairs_space(hd);
}

// ---- norms (norm.hip) -------------------------------------------------------
// Row-wise LayerNorm of fp32 x [rows, dim] followed by one of:
//  mode 0 (adaLN):   u = LN(x) * (1 + (e0[b][c_scale] + mb[c_scale])) + (e0[b][c_shift] + mb[c_shift])
//                    with e0 = p0 [B, 6, dim], mb = p1 per-block modulation bias [6, dim] (null: p0
//                    already holds the sums), b = row / S;
//  mode 1 (affine):  u = LN(x) * w + bias (w = p0, bias = p1, each [dim]);
//  mode 2 (head):    u = LN(x) * (1 + (hm[1] + e[b])) + (hm[0] + e[b]) with hm = p0 [2, dim], e = p1 [B, dim].
// Where a kernel writes (or reads) an activation [M, N]: element (m, n) at m * ld + (n / 32) * bs + n % 32.
// Row-major with row stride ld: bs = 32.  K panels of the products' A operand (KMat): ld = 32,
// bs = 32 * panel_rows(M), N % 32 == 0.
struct ActLayout {
  int64_t ld, bs;
};
inline ActLayout act_rows(int64_t ld) { return ActLayout{ld, 32}; }
inline ActLayout act_panels(int64_t M) { return ActLayout{32, 32 * ((M + 255) / 256 * 256)}; }
// u in the layout lu (see ActLayout; panels need dim % 32 == 0).
template <typename T>
hipError_t launch_ln_mod(const float* x, int64_t rows, int dim, int S, int mode, const float* p0, const float* p1,
                         int c_shift, int c_scale, float eps, T* u, ActLayout lu, hipStream_t s);
// 3D RoPE (no norm) on the q and k rows of B * T_ * Hp * Wp tokens (row strides ld_in / ld_out; in place
// allowed); hd % 8 == 0.
template <typename T>
hipError_t launch_rope_qk(const T* q_in, const T* k_in, int64_t ld_in, T* q_out, T* k_out, int64_t ld_out, int B,
                          int T_, int Hp, int Wp, int heads, int hd, float theta, hipStream_t s);
// The block's Q/K RMSNorm factors from the Q/K/V epilogue's partial sums of squares ssq [2 dim / 32, rows]
// (see QKNormRope): rq[row] = (sum_q / dim + eps)^-1/2, and the k rows (row stride ldk) scaled in place
// by (sum_k / dim + eps)^-1/2.  dim % 32 == 0, dim <= 6144.
template <typename T>
hipError_t launch_qk_rms(const float* ssq, int64_t rows, int dim, float eps, T* k, int64_t ldk, float* rq,
                         hipStream_t s);

// ---- GEMM (gemm.hip) --------------------------------------------------------
// A product operand X [R, K] (the activations A [M, K] or the weights W [N, K]): row-major with row
// stride ld (panel == 0), or in K panels of 32 elements (panel > 0, the rows of each panel: R rounded
// up to a multiple of 256): element (r, k) at ((k / 32) * panel + r) * 32 + k % 32.  Weight panels hold
// zeros in rows N .. panel - 1 (launch_pack_panels); activation panels hold whatever the workspace
// held there, which only reaches outputs that are not stored.  In panels, the 32-deep K step of a
// 256-row tile is one contiguous run of whole cache lines.
template <typename T>
struct KMat {
  const T* p;
  int64_t ld;
  int64_t panel;
};
inline int64_t panel_rows(int64_t R) { return (R + 255) / 256 * 256; }
template <typename T>
inline KMat<T> k_rows(const void* p, int64_t ld) {
  return KMat<T>{static_cast<const T*>(p), ld, 0};
}
template <typename T>
inline KMat<T> k_panels(const void* p, int64_t R) {
  return KMat<T>{static_cast<const T*>(p), 0, panel_rows(R)};
}
template <typename T>
inline bool k_panels_ok(const KMat<T>& x, int64_t R, int64_t K) {
  return x.panel >= R && x.panel % 256 == 0 && K % 32 == 0;
}
// Row-major [rows, cols] of elem_bytes-byte elements (row stride ld elements) -> K panels of 32
// ([cols / 32][panel_rows(rows)][32], zero rows past `rows`).  cols % 32 == 0, ld * elem_bytes % 16 == 0.
hipError_t launch_pack_panels(const void* src, int64_t rows, int64_t cols, int64_t ld, int elem_bytes, void* dst,
                              hipStream_t s);

// C[m, n] = sum_k A[m, k] * W[n, k]   (A [M, K] and W [N, K], each a KMat)
// Epilogues:
//   store:      out[m, n] = act(C + bias[n])  (OutT = T or float)
//   residual:   x[m, n] += g(m, n) * (C + bias[n]), g = gate[m / S][chunk][n] from a [B, 6, N] table
//               (the block's e0 + modulation bias), or 1 if gate is null; ystore (optional, row stride N)
//               also receives C + bias.
template <typename T, typename OutT>
hipError_t gemm_store(KMat<T> A, KMat<T> W, int M, int N, int K, const float* bias, int act, OutT* out, ActLayout lo,
                      hipStream_t s);
// Q/K/V projection (N = 3 dim): q, k columns to qk[m, 0 .. 2 dim) (row stride ldo), v columns to
// V^T [B, H, hd, Spad] (keys permuted within 16-key groups for bf16; see launch_transpose_heads);
// m = b * S + pos.  Only keys pos < S are written: the positions of keys S .. Spad - 1 are left as they
// were (launch_attn_prologue clears them first).
// The q and k columns leave the epilogue as RoPE(g * (C + bias)) with the RMSNorm gains g (gq for q,
// gk for k) and the 3D rotation of token m's position (frame, row, column) in the T x Hp x Wp grid of
// its batch row (m % S); the per-row RMS factor comes later (launch_qk_rms): the epilogue writes the
// sums of squares of C + bias over each 32-column block, ssq[(n / 32) * M + m] for n < 2 dim.
// The rotation reads (cos, sin) from rope (launch_attn_prologue writes it): with npT =
// rope_pairs_time(hd), npH = rope_pairs_space(hd), pair p of a head at frame f, row i, column j is
// entry f npT + p (p < npT), T npT + i npH + (p - npT) (p < npT + npH), else
// T npT + Hp npH + j npH + (p - npT - npH).  dim % 32 == 0, hd a power of 2 (>= 4).
struct QKNormRope {
  const float* gq;
  const float* gk;
  float* ssq;  // [2 dim / 32, M]
  const float2* rope;
  int T, Hp, Wp;
};
template <typename T>
hipError_t gemm_qkv(KMat<T> A, KMat<T> W, int M, int dim, int K, const float* bias,
                    T* qk, int64_t ldo, T* vt, int S, int H, int hd, int Spad, const QKNormRope& nr,
                    hipStream_t s);
template <typename T>
hipError_t gemm_residual(KMat<T> A, KMat<T> W, int M, int N, int K, const float* bias,
                         const float* gate, int chunk, int S, float* x, int64_t ldx, hipStream_t s,
                         float* ystore = nullptr);
// E4M3 products: C = (sum_k A[m, k] W[n, k]) * a_scales[m] * w_scale[0] over E4M3 codes (A and W in K
// panels; K % 256 == 0), then the store (bf16 out, act NONE or GELU) or residual epilogue.
hipError_t gemm_e4m3_store(KMat<uint8_t> A, const float* a_scales, KMat<uint8_t> W,
                           const float* w_scale, int M, int N, int K, const float* bias, int act, bf16* out,
                           ActLayout lo, hipStream_t s);
hipError_t gemm_e4m3_residual(KMat<uint8_t> A, const float* a_scales, KMat<uint8_t> W,
                              const float* w_scale, int M, int N, int K, const float* bias, const float* gate,
                              int chunk, int S, float* x, int64_t ldx, hipStream_t s, float* ystore = nullptr);
hipError_t gemm_qkv_e4m3(KMat<uint8_t> A, const float* a_scales, KMat<uint8_t> W,
                         const float* w_scale, int M, int dim, int K, const float* bias, bf16* qk, int64_t ldo, bf16* vt,
                         int S, int H, int hd, int Spad, const QKNormRope& nr, hipStream_t s);
// y[b, n] = out_act(sum_k W[n, k] * in_act(x[b, k]) + bias[n]) for b < B (fp32 x, y).
template <typename T>
hipError_t gemv(const T* W, int N, int K, const float* x, int B, const float* bias, int in_act, int out_act,
                float* y, hipStream_t s);
hipError_t launch_sinusoid(const float* t_host, int B, int freq_dim, float* emb, hipStream_t s);

// ---- attention (attention.hip) ----------------------------------------------
// Flash attention, non-causal, over one key/value stream (a second stream adds to the first's output).
// q:  element (b, s, h, d) at q[b*q_bs + s*q_ss + h*hd + d]
// k:  element (b, j, h, d) at k[b*k_bs + j*k_ss + h*hd + d]
// vt: element (b, h, d, j) at vt[((b*H + h)*hd + d)*Lpad + j]  (zero beyond L)
// o:  element (b, s, h, d) at o[b*o_bs + s*o_ss + h*hd + d]
struct KVStream {
  const void* k;
  int64_t k_bs, k_ss;
  const void* vt;
  int L, Lpad;
};
// Key split (one stream only): the grid runs B * n batch entries; entry b * n + i attends the queries
// of batch row b to keys [i * chunk, min((i + 1) * chunk, L)) and writes its o at o + i * o_stride and
// its lse at lse + i * lse_stride, to be combined by launch_lse_merge.  chunk is a multiple of 64 and
// (n - 1) * chunk < L.  n == 1 (the default) is the plain attention.
struct KeySplit {
  int n = 1, chunk = 0;
  int64_t o_stride = 0, lse_stride = 0;
};
// Query rows per workgroup of the kernel launch_attention picks for (T, kind), and how many such
// workgroups one compute unit holds at once.
template <typename T>
void attention_tile(int kind, int& rows, int& per_cu);
// kind: 0 self-attention, 1 cross-attention (separate kernel symbols).  lse (NULL = not written):
// [B, H, S] float32, the natural log of each query row's softmax normaliser.  accumulate: the result is
// added to what o holds (a second key/value stream after a first launch; not with key splits, and not
// for bf16 kind 0, which runs the ping-pong kernel).  qscale (NULL = 1): [B, S] float32, a per-query
// factor of the score scale (the block's RMSNorm factor r_q of a query whose row is not yet normalised).
// o_cs: channel n of a row at (n / 32) o_cs + n % 32 from the row's start (32: row-major; the products'
// K panels: o_ss = 32 and o_cs = 32 * rows per panel, see ActLayout).
template <typename T>
hipError_t launch_attention(const T* q, int64_t q_bs, int64_t q_ss, KVStream kv, int B, int S, int H, int hd,
                            float scale, T* o, int64_t o_bs, int64_t o_ss, int kind, hipStream_t s,
                            float* lse = nullptr, KeySplit ks = KeySplit{}, bool accumulate = false,
                            const float* qscale = nullptr, int64_t o_cs = 32);

// Quantised attention (INT8 Q.K, FP8 P.V): q8 [B, S, H, hd] INT8 codes with sq [B, H, S]; k8 [B, L, H, hd]
// INT8 codes with sk [B, H, ceil(L / 64)]; v8t [B, H, hd, round_up(L, 128)] E4M3 codes (keys in P.V
// order, zero past L) with sv [B, H, hd]; o [B, S, H, hd] bf16; lse [B, H, S] or NULL; qscale [B, S] or
// NULL, as for launch_attention; o row (b, s) = row b S + s of the layout lo.
hipError_t launch_attention_q8(const uint8_t* q8, const float* sq, const uint8_t* k8, const float* sk,
                               const uint8_t* v8t, const float* sv, int B, int S, int L, int H, int hd, bf16* o,
                               ActLayout lo, float* lse, hipStream_t s, const float* qscale = nullptr);

// ---- quantisers (quant.hip) --------------------------------------------------
// x rows [B*S, *] bf16 with head h at columns h*hd (row stride ld elements).
hipError_t launch_quant_q(const bf16* x, int64_t ld, int B, int S, int H, int hd, int8_t* codes, float* scales,
                          hipStream_t s);  // codes [B*S, H*hd], scales [B, H, S]
hipError_t launch_quant_k(const bf16* x, int64_t ld, int B, int S, int H, int hd, int8_t* codes, float* scales,
                          hipStream_t s);  // codes [B*S, H*hd], scales [B, H, ceil(S / 64)]
// bf16 V^T rows of Lpad_in keys (the bf16 attention's order, Lpad_in a multiple of 64) -> E4M3 V^T rows of
// Lpad_out >= Lpad_in keys (multiple of 64, zero past Lpad_in) in the quantised attention's order,
// scales [rows].
hipError_t launch_quant_vt(const bf16* vt, int64_t rows, int Lpad_in, int Lpad_out, uint8_t* out, float* scales,
                           hipStream_t s);

// E4M3 codes of activations per row (scale = amax / 448 per row) and of a whole tensor (one scale,
// written to *scale on the device; amax_word is a 4-byte device scratch word).
// (x and the codes in the layouts lx, lc: element (row, n) as in ActLayout, the codes in bytes)
hipError_t launch_quant_rows_e4m3(const bf16* x, ActLayout lx, int rows, int cols, uint8_t* codes, ActLayout lc,
                                  float* scales, hipStream_t s);
hipError_t launch_quant_tensor_e4m3(const bf16* x, int64_t n, uint8_t* codes, float* scale, uint32_t* amax_word,
                                    hipStream_t s);

// Combine n (1..MERGE_MAX_PARTS) attention results of the same queries over disjoint key chunks:
// o_parts[i] [B, S, H, hd] T, lse_parts[i] [B, H, S] float32 (host arrays of device pointers);
// lse = log sum_i exp(lse_i), o = sum_i exp(lse_i - lse) o_i; lse may be NULL.
constexpr int MERGE_MAX_PARTS = 16;
template <typename T>
hipError_t launch_lse_merge(const void* const* o_parts, const float* const* lse_parts, int n, int B, int S, int H,
                            int hd, T* o, float* lse, hipStream_t s);

// ---- device ceilings (probe.hip) --------------------------------------------
// `blocks` workgroups of 256 threads, each wave issuing 4 * iters MFMAs (kind 0 bf16 32x32x16,
// kind 1 E4M3 32x32x64) on register operands built from a_word / b_word; out [blocks * 256] float32
// receives each lane's accumulator sum, 64 * K * iters * a * b.
hipError_t launch_mfma_peak(int kind, uint32_t a_word, uint32_t b_word, int blocks, int iters, float* out,
                            hipStream_t s);

}  // namespace wan
