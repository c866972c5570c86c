/*
 * wan.h -- C ABI of libwan.so: one Wan-style video DiT denoise step on an
 * AMD Instinct MI355X (gfx950), built from hand-written HIP kernels.
 *
 * Pages cited (titles as they appear on them):
 *   [I2V]  "图解 Wan2.1 I2V：从一张图到一段视频，模型到底发生了什么" (liyongzhi.xyz)
 *   [DEEP] "Wan（通义万相）：大规模视频生成基础模型 — 技术深度解析 & Wan2.1 vs Wan2.2对比"
 *          (devpress.csdn.net)
 *   [TI2V] "Wan2.2 TI2V-5B" (lnwmold.com)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are caller-owned DEVICE pointers, dense and row-major in the
 *    layouts stated, 16-byte aligned.  Host pointers are named *_host.
 *  - Every call is asynchronous on `stream` (NULL = the default stream).  The
 *    library never allocates, frees or synchronises and keeps no pointer after
 *    it returns; buffers must stay alive until the stream has consumed them.
 *  - Return value: WAN_OK (0) or a negative wan_status.  Argument errors are
 *    detected on the host before anything is enqueued.  A failed launch
 *    returns WAN_EHIP; device faults surface at the caller's next
 *    synchronisation.  wan_last_error() gives a thread-local message.
 *  - Linear weights are stored [out, in] (y = x W^T + b).  "dtype" tensors are
 *    float (WAN_F32) or bf16 (WAN_BF16, raw 16-bit storage); biases, gains,
 *    modulation, latents and the residual stream are always float32.
 *  - Outputs never alias inputs, except the in-place x of wan_dit_block_fwd
 *    and wan_fm_euler_step.
 */
#ifndef WAN_H
#define WAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The same type as HIP's hipStream_t. */
typedef struct ihipStream_t* wan_stream_t;

typedef enum {
  WAN_OK = 0,
  WAN_EINVAL = -1,       /* bad argument: null/misaligned pointer, inconsistent or non-positive size */
  WAN_EUNSUPPORTED = -2, /* valid but not built: head_dim not 64/128, dim > 6144, flags != 0, ... */
  WAN_EWORKSPACE = -3,   /* ws_bytes below the size the matching *_workspace_bytes() returns */
  WAN_EHIP = -4          /* a HIP launch failed */
} wan_status;

typedef enum { WAN_F32 = 0, WAN_BF16 = 1 } wan_dtype;

/* Latent [B, C, T, H, W] float32; H and W even.  Tokens S = T * (H/2) * (W/2) ([I2V] §5.1). */
typedef struct {
  int32_t B, C, T, H, W;
} wan_latent_shape;

/* Token grid (frames, rows, columns) = (T, H/2, W/2): the 3D RoPE positions ([I2V] §5.3). */
typedef struct {
  int32_t T, Hp, Wp;
} wan_grid;

/* Block hyper-parameters.  dim = heads * head_dim; head_dim 64 or 128; dim <= 6144; ffn_dim % 32 == 0;
 * text_len > 0 text keys; img_len >= 0 image keys (0 = single-stream cross-attention).
 * Proposed eps 1e-6 for both norms and rope_theta 10000.  flags: 0 or WAN_FLAG_FP8_ATTN | WAN_FLAG_FP8_GEMM. */
/* WAN_FLAG_FP8_ATTN: the block's self-attention runs the quantised path of wan_attention_q8_fwd (INT8
 * Q.K, E4M3 P.V; [DEEP] §5.3) on the rotated q, k and v it computes; requires dtype WAN_BF16 and
 * head_dim 128.  Everything else in the block is unchanged. */
#define WAN_FLAG_FP8_ATTN 1u
/* WAN_FLAG_FP8_GEMM: the Q/K/V, O, FFN1 and FFN2 products run in E4M3 as in wan_gemm_e4m3 (activations
 * quantised per token inside the block, weights taken from w->e4m3); requires dtype WAN_BF16 and dim
 * and ffn_dim multiples of 256.  The cross-attention products stay bf16. */
#define WAN_FLAG_FP8_GEMM 2u

typedef struct {
  int32_t dim, heads, head_dim, ffn_dim;
  int32_t text_len, img_len;
  int32_t dtype; /* wan_dtype */
  uint32_t flags;
  float ln_eps, rms_eps, rope_theta;
} wan_block_cfg;

/* K panels: the operand layout of the block's products.  A matrix W [N, K] (y = x W^T) is stored as
 * K / 32 panels, each holding 32 consecutive k of every row n: element (n, k) at
 * ((k / 32) * Np + n) * 32 + k % 32, where Np = N rounded up to a multiple of 256 and rows N .. Np - 1
 * are zero.  wan_pack_weight_bytes(elem_bytes, N, K) = Np * K * elem_bytes (0 for invalid sizes:
 * elem_bytes not 1, 2 or 4, N or K not positive, K % 32 != 0); wan_pack_weight writes the panels of
 * a row-major W [N, K] (row stride K) with elem_bytes-byte elements (2 for bf16, 4 for float32, 1 for
 * E4M3 codes) into `packed`.  Errors: WAN_EINVAL for those sizes or a NULL / misaligned pointer.
 * Why: the products copy 32-deep K steps of 256-row weight tiles, and in panels each such step is one
 * contiguous run of whole cache lines instead of 256 half-line segments. */
size_t wan_pack_weight_bytes(int32_t elem_bytes, int64_t N, int64_t K);
int wan_pack_weight(int32_t elem_bytes, const void* w, int64_t N, int64_t K, void* packed, wan_stream_t stream);

/* Weights of one DiT block ([I2V] §5.2-§5.5; per-block modulation bias [DEEP] §2.5).
 * dtype matrices, each in K panels (wan_pack_weight): wqkv [3*dim, dim] = rows [W_q; W_k; W_v];
 * wo, wcq, wco [dim, dim]; w1 [ffn_dim, dim]; w2 [dim, ffn_dim].  float32 vectors: mod_bias [6, dim]
 * (chunks shift1, scale1, gate1, shift2, scale2, gate2); bqkv [3*dim]; gq, gk [dim] RMSNorm gains; bo;
 * ln3_w, ln3_b [dim] (affine LayerNorm before cross-attention); bcq, bco [dim]; b1 [ffn_dim]; b2 [dim].
 * Bias pointers may be NULL (zero bias); all others are required.  e4m3: NULL, or (required under
 * WAN_FLAG_FP8_GEMM) the E4M3 codes of wqkv, wo, w1, w2 in K panels with one float32 device scale
 * each: wan_quantize_tensor_e4m3 of the packed bf16 matrices (codes are per element, so the codes of
 * packed values are packed codes). */
typedef struct {
  const void *wqkv, *wo, *w1, *w2;
  const float *s_wqkv, *s_wo, *s_w1, *s_w2;
} wan_block_weights_e4m3;

typedef struct {
  const float* mod_bias;
  const void* wqkv;
  const float* bqkv;
  const float *gq, *gk;
  const void* wo;
  const float* bo;
  const float *ln3_w, *ln3_b;
  const void* wcq;
  const float* bcq;
  const void* wco;
  const float* bco;
  const void* w1;
  const float* b1;
  const void* w2;
  const float* b2;
  const wan_block_weights_e4m3* e4m3;
} wan_block_weights;

/* Cross-attention keys/values of one block, computed once per generation by wan_cross_kv_fwd
 * (context and weights do not change across sampling steps, [I2V] §7).
 *   k_txt  [B, text_len, dim] dtype;   vt_txt [B, heads, head_dim, Lpad_txt] dtype: V transposed
 *   per head, zero for keys >= text_len, Lpad = text_len rounded up to a multiple of 64.  In bf16
 *   the key axis is stored permuted within each 16-key group (position p holds key p with bits 2
 *   and 3 swapped: keys 0-3, 8-11, 4-7, 12-15), the order the attention kernel's MFMA operands use.
 *   k_img / vt_img likewise with img_len (NULL when img_len == 0). */
typedef struct {
  const void *k_txt, *vt_txt, *k_img, *vt_img;
} wan_cross_kv;

/* Cross-attention K/V projection weights of one block: text [W_k; W_v] = wkv_txt [2*dim, dim]
 * (+ bkv_txt [2*dim]); image (img_len > 0) wkv_img [2*dim, dim] (+ bkv_img). */
typedef struct {
  const void* wkv_txt;
  const float* bkv_txt;
  const void* wkv_img;
  const float* bkv_img;
} wan_cross_kv_weights;

/* Timestep MLP shared by all blocks ([I2V] §5.2; [DEEP] §2.5): wt1 [dim, freq_dim], wt2 [dim, dim],
 * wtp [6*dim, dim] dtype; biases float32 (may be NULL). */
typedef struct {
  const void* wt1;
  const float* bt1;
  const void* wt2;
  const float* bt2;
  const void* wtp;
  const float* btp;
} wan_time_weights;

/* Head ([I2V] §5.5): head_mod [2, dim] float32 (shift, scale biases); wh [4*C_out, dim] dtype;
 * bh [4*C_out] float32 (may be NULL). */
typedef struct {
  const float* head_mod;
  const void* wh;
  const float* bh;
} wan_head_weights;

/* ---------------------------------------------------------------------------------------------- */

/* a1 -- image-to-video input ([I2V] §4.1 steps 3-4, §4.2; layout of the mask per §10 Q3/Q6).
 * x_in [B, 2C+4, T, H, W] = [x_t, mask, z_img] along channels; mask channel c of latent frame t is
 * entry 4t+c of the pixel-frame flag sequence (frame 0's flag repeated 4 times, then frames 1..F-1,
 * F = 4(T-1)+1).  known_pixel_frames_host: F host bytes (nonzero = known), or NULL for "frame 0
 * only".  x_t, z_img [B, C, T, H, W] float32.  T <= 64.  Bit-exact copy. */
int wan_build_i2v_input(const float* x_t, const float* z_img, const uint8_t* known_pixel_frames_host,
                        wan_latent_shape shape, float* x_in, wan_stream_t stream);

/* a2 -- (1,2,2) patchify ([I2V] §5.1): p[b, (f*Hp+i)*Wp+j, c*4+kh*2+kw] = x[b, c, f, 2i+kh, 2j+kw].
 * x [B, C, T, H, W] float32 -> p [B, S, 4C] float32.  Bit-exact copy. */
int wan_patchify(const float* x, wan_latent_shape shape, float* p, wan_stream_t stream);

/* a11 (layout part) -- inverse of wan_patchify: p [B, S, 4C] -> x [B, C, T, H, W] float32. */
int wan_unpatchify(const float* p, wan_latent_shape shape, float* x, wan_stream_t stream);

/* a3 -- patch embedding ([I2V] §5.1, the Conv3d with kernel = stride = (1,2,2) as a matrix
 * product): x [B*S, dim] float32 = p [B*S, 4*C_in] float32 @ w_pe^T + b_pe; w_pe [dim, 4*C_in]
 * dtype (the Conv3d weight [dim, C_in, 1, 2, 2] flattened), b_pe [dim] float32 or NULL.
 * 4*C_in % 8 == 0.  Workspace: wan_patch_embed_workspace_bytes(). */
size_t wan_patch_embed_workspace_bytes(const wan_block_cfg* cfg, int64_t tokens, int32_t in_channels);
int wan_patch_embed(const wan_block_cfg* cfg, const float* p, int64_t tokens, int32_t in_channels,
                    const void* w_pe, const float* b_pe, float* x, void* ws, size_t ws_bytes, wan_stream_t stream);

/* a4 -- timestep embedding ([I2V] §5.2; [DEEP] §2.5): for each row b, with tau = 1000 * t[b],
 * emb = [cos(tau f_i) | sin(tau f_i)], f_i = 10000^(-i/(freq_dim/2));
 * e[b] = wt2 SiLU(wt1 emb + bt1) + bt2  -> e [B, dim] float32;
 * e0[b] = wtp SiLU(e[b]) + btp          -> e0 [B, 6, dim] float32 (e0 doubles as scratch).
 * t_host: B host floats; 1 <= B <= 4; freq_dim even, freq_dim % 8 == 0. */
int wan_time_embed(const wan_block_cfg* cfg, int32_t freq_dim, const wan_time_weights* w, const float* t_host,
                   int32_t B, float* e, float* e0, wan_stream_t stream);

/* Context embedding, once per generation ([I2V] §7 steps 1-2: umT5 [512, 4096] -> MLP -> [512, dim];
 * CLIP [257, 1280] -> MLPProj -> [257, dim]): out = GELU(ctx w1^T + b1) w2^T + b2.
 * ctx [rows, in_dim] dtype; w1 [dim, in_dim], w2 [dim, dim] dtype; out [rows, dim] dtype.
 * in_dim % 8 == 0.  Workspace: wan_context_embed_workspace_bytes(). */
size_t wan_context_embed_workspace_bytes(const wan_block_cfg* cfg, int64_t rows);
int wan_context_embed(const wan_block_cfg* cfg, const void* ctx, int64_t rows, int32_t in_dim, const void* w1,
                      const float* b1, const void* w2, const float* b2, void* out, void* ws, size_t ws_bytes,
                      wan_stream_t stream);

/* Cross-attention keys/values of one block ([I2V] §5.4: k = Linear_k(context), v = Linear_v(context);
 * separate image projections for the CLIP tokens).  txt_emb [B, text_len, dim] dtype; img_emb
 * [B, img_len, dim] dtype (ignored when img_len == 0).  Writes the buffers named in `out` (layouts as
 * in wan_cross_kv; the caller allocates them: wan_cross_kv_buffer_bytes gives each size).
 * Workspace: wan_cross_kv_workspace_bytes(). */
size_t wan_cross_kv_buffer_bytes(const wan_block_cfg* cfg, int32_t B, int32_t which /*0 k_txt,1 vt_txt,2 k_img,3 vt_img*/);
size_t wan_cross_kv_workspace_bytes(const wan_block_cfg* cfg, int32_t B);
int wan_cross_kv_fwd(const wan_block_cfg* cfg, const wan_cross_kv_weights* w, const void* txt_emb,
                     const void* img_emb, int32_t B, const wan_cross_kv* out, void* ws, size_t ws_bytes,
                     wan_stream_t stream);

/* a5-a10 -- one DiT block, in place on x [B, S, dim] float32 (S = grid.T * grid.Hp * grid.Wp),
 * in the order of [I2V] §5.3-§5.5:
 *   mod = e0[b] + mod_bias -> (shift1, scale1, gate1, shift2, scale2, gate2)   ([I2V] §5.2)
 *   u = LN(x)(1 + scale1) + shift1;  q, k = RoPE3D(RMSNorm(u W_{q,k}^T + b) * g);  v = u W_v^T + b
 *   x += gate1 * (Attn(q, k, v) W_o^T + b_o)                    (full, non-causal, [DEEP] §2.5)
 *   x += CrossAttn(LN_affine(x)) W_co^T + b_co                   (text, or image + text, [I2V] §5.4)
 *   x += gate2 * FFN(LN(x)(1 + scale2) + shift2),  FFN = Linear -> GELU -> Linear
 * e0 [B, 6, dim] float32 from wan_time_embed; kv from wan_cross_kv_fwd.  LN has no affine (except the
 * cross-attention pre-norm), eps = cfg->ln_eps; attention scale 1/sqrt(head_dim).
 * Workspace: wan_dit_block_workspace_bytes() (about B*S*(5*dim + ffn_dim) dtype elements, the
 * products' inputs (LayerNorm outputs, attention outputs, FFN hidden state) held in K panels of
 * B*S rounded up to 256 rows; plus B*S*(dim/16 + 1) float32 of Q/K sums of squares and query
 * scales, 6*B*dim float32 of modulation and the RoPE table's (T + Hp + Wp) * head_dim/2 or fewer
 * float2). */
size_t wan_dit_block_workspace_bytes(const wan_block_cfg* cfg, wan_grid grid, int32_t B);
int wan_dit_block_fwd(const wan_block_cfg* cfg, const wan_block_weights* w, wan_grid grid, int32_t B, float* x,
                      const float* e0, const wan_cross_kv* kv, void* ws, size_t ws_bytes, wan_stream_t stream);

/* Attention cache ([DEEP] §5.3: attention outputs reused across sampling steps).  Same as
 * wan_dit_block_fwd, with the self-attention layer's output y = o W_o^T + b_o (before the gate) kept in
 * attn_y [B, S, dim] float32 (caller-owned, one per block and batch row set):
 *   WAN_ATTN_CACHE_OFF    attn_y unused (this is wan_dit_block_fwd);
 *   WAN_ATTN_CACHE_STORE  the block computes as usual and writes y to attn_y;
 *   WAN_ATTN_CACHE_REUSE  the block skips LN1, the Q/K/V product, the norms and RoPE, the attention
 *                         and the O product, and adds gate1 * attn_y (gate1 of this call's e0) to x.
 * The other branches always run.  Which steps reuse is the caller's schedule.  REUSE reads attn_y as an
 * earlier STORE with the same cfg, grid and B left it; the library cannot check that.  Errors: as
 * wan_dit_block_fwd, plus WAN_EINVAL for attn_mode outside 0..2 or a NULL / misaligned attn_y in a
 * cache mode (nothing is enqueued). */
typedef enum { WAN_ATTN_CACHE_OFF = 0, WAN_ATTN_CACHE_STORE = 1, WAN_ATTN_CACHE_REUSE = 2 } wan_attn_cache_mode;
int wan_dit_block_fwd_cached(const wan_block_cfg* cfg, const wan_block_weights* w, wan_grid grid, int32_t B, float* x,
                             const float* e0, const wan_cross_kv* kv, float* attn_y, int32_t attn_mode, void* ws,
                             size_t ws_bytes, wan_stream_t stream);

/* The block for callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): wan_dit_block_fwd without ws / ws_bytes.  Its scratch is a
 * static device array of WAN_NOALLOC_SCRATCH_BYTES in the library, one per device, held until the process
 * ends; the call allocates nothing (no hipMalloc / hipFree / allocating library routine).  The caller
 * still passes x, e0, the weights and kv as for wan_dit_block_fwd, and the result is the same.
 * Errors: as wan_dit_block_fwd, and WAN_EWORKSPACE (nothing enqueued) when
 * wan_dit_block_workspace_bytes(cfg, grid, B) exceeds WAN_NOALLOC_SCRATCH_BYTES.
 * Every call on one device shares that device's array: calls that overlap on one device (two streams,
 * two threads) race and must be serialised by the caller.  The block never reads scratch it has not
 * written in the same call, so what an earlier call left there does not matter. */
#define WAN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int wan_dit_block_fwd_noalloc(const wan_block_cfg* cfg, const wan_block_weights* w, wan_grid grid, int32_t B,
                              float* x, const float* e0, const wan_cross_kv* kv, wan_stream_t stream);

/* a11 -- head ([I2V] §5.5): (shift, scale) = head_mod + e[b];
 * out [B*S, 4*C_out] float32 = (LN(x)(1 + scale) + shift) wh^T + bh, x [B, S, dim] float32,
 * e [B, dim] float32.  Follow with wan_unpatchify.  Workspace: wan_head_workspace_bytes(). */
size_t wan_head_workspace_bytes(const wan_block_cfg* cfg, int64_t tokens);
int wan_head_fwd(const wan_block_cfg* cfg, const wan_head_weights* w, int32_t out_channels, int32_t B, int32_t S,
                 const float* x, const float* e, float* out, void* ws, size_t ws_bytes, wan_stream_t stream);

/* a12 -- classifier-free guidance + flow-matching Euler step ([I2V] §7; [DEEP] §2.7), in place:
 * v = v_uncond + guidance * (v_cond - v_uncond)   (v = v_cond when v_uncond is NULL);
 * x <- x + dt * v, dt signed (t runs 1 -> 0, so dt < 0).  x, v_cond, v_uncond: n float32 each.
 * Computed as fma(dt, fma(guidance, v_c - v_u, v_u), x). */
int wan_fm_euler_step(float* x, const float* v_cond, const float* v_uncond, float guidance, float dt, int64_t n,
                      wan_stream_t stream);

/* a7 on its own -- full non-causal self-attention with 3D RoPE on q and k ([I2V] §5.3 ②) and no
 * projections or norms: q, k, v [B, S, heads, head_dim] dtype -> o [B, S, heads, head_dim] dtype,
 * S = grid.T * grid.Hp * grid.Wp.  Workspace: wan_attention_workspace_bytes(). */
size_t wan_attention_workspace_bytes(int32_t dtype, wan_grid grid, int32_t B, int32_t heads, int32_t head_dim);
int wan_attention_fwd(int32_t dtype, const void* q, const void* k, const void* v, wan_grid grid, int32_t B,
                      int32_t heads, int32_t head_dim, float rope_theta, void* o, void* ws, size_t ws_bytes,
                      wan_stream_t stream);

/* Sequence-sharded (ring) attention pieces.  [DEEP] §5.2 runs the DiT's attention with 2D context
 * parallelism whose outer level, RingAttention, shards the sequence: each GPU attends its own queries
 * to one key/value shard at a time and combines the partial results.  These two calls are that
 * per-shard step and that combination, on one GPU.
 *
 * wan_attention_partial_fwd: q [B, Sq, heads, head_dim] attends to one key/value chunk
 * k, v [B, Sk, heads, head_dim] (all dtype; no RoPE or norm is applied here, so pass rotated q and k):
 *   o   [B, Sq, heads, head_dim] dtype = softmax(q k^T / sqrt(head_dim)) v over the chunk's keys;
 *   lse [B, heads, Sq] float32 (NULL = not written) = ln sum_j exp(q k_j / sqrt(head_dim)).
 * head_dim 64 or 128.  Workspace: wan_attention_partial_workspace_bytes() for the device current at the
 * call.  It holds the chunk's V^T and, when B * heads query tiles would leave compute units idle, room
 * for up to 16 key splits.  The call then attends each split in its own workgroups and merges them as
 * wan_attention_lse_merge does (every split holds >= 256 keys).  A workspace holding only V^T
 * (B * heads * head_dim * round_up(Sk, 64) dtype elements) runs unsplit; smaller is WAN_EWORKSPACE.
 *
 * wan_attention_lse_merge: combines n_parts (1..16) results for the same queries over disjoint key
 * chunks: lse = ln sum_n exp(lse_parts[n]); o = sum_n exp(lse_parts[n] - lse) * o_parts[n], which is
 * attention over the union of the chunks.  o_parts and lse_parts are HOST arrays of n_parts device
 * pointers ([B, S, heads, head_dim] dtype and [B, heads, S] float32); o has o_parts' layout; lse
 * (NULL = not written) has lse_parts' layout.  Outputs must not alias the inputs. */
size_t wan_attention_partial_workspace_bytes(int32_t dtype, int32_t B, int32_t Sq, int32_t Sk, int32_t heads,
                                             int32_t head_dim);
int wan_attention_partial_fwd(int32_t dtype, const void* q, const void* k, const void* v, int32_t B, int32_t Sq,
                              int32_t Sk, int32_t heads, int32_t head_dim, void* o, float* lse, void* ws,
                              size_t ws_bytes, wan_stream_t stream);
int wan_attention_lse_merge(int32_t dtype, int32_t n_parts, const void* const* o_parts, const float* const* lse_parts,
                            int32_t B, int32_t S, int32_t heads, int32_t head_dim, void* o, float* lse,
                            wan_stream_t stream);

/* Quantised (FP8) attention.  [DEEP] §5.3 lists an FP8 FlashAttention-3 among the inference
 * optimisations: Q.K inner products in INT8, O = P.V in FP8, FP32 accumulation across key blocks.
 * Codes (readings of the page, which names only the formats):
 *   q8  int8 [B, Sq, heads, head_dim], sq float32 [B, heads, Sq]: one symmetric group per (token, head),
 *       scale = amax / 127, code = round-half-even(x * (127 / amax)) clamped to +-127;
 *   k8  int8 [B, Sk, heads, head_dim], sk float32 [B, heads, ceil(Sk / 64)]: one group per (head, block
 *       of 64 consecutive keys), same rule;
 *   v8t uint8 OCP E4M3 [B, heads, head_dim, Skpad], Skpad = Sk rounded up to 128, zero past Sk;
 *       sv float32 [B, heads, head_dim]: one group per (head, channel) over all keys,
 *       scale = amax / 448, code = e4m3(clamp(x * (448 / amax), -448, 448)) rounded to nearest even.
 *       Within each 64-key tile, byte h*32 + kb*16 + r holds key kb*32 + (r/4)*8 + h*4 + r%4
 *       (h, kb in {0, 1}, r < 16): the order in which the P.V product reads the keys.
 *   A group whose amax is 0 has scale 0 and zero codes.  Quotients and products are float32, IEEE
 *   rounded, so the codes are a fixed function of the inputs.
 * wan_attention_q8_quantize: q [B, Sq, heads, head_dim] and k, v [B, Sk, heads, head_dim] bf16 (rotated
 *   already) -> the codes above.  Workspace: wan_attention_q8_quantize_workspace_bytes() (a bf16 V^T).
 * wan_attention_q8_fwd: codes -> o [B, Sq, heads, head_dim] bf16 = softmax(q k^T / sqrt(head_dim)) v
 *   computed from the codes (exact int32 Q.K, P rounded to E4M3 after a shift that keeps it in
 *   [0, 256], fp32 accumulation), and lse [B, heads, Sq] float32 (NULL = not written) as for
 *   wan_attention_partial_fwd.  head_dim 128.  sv must be 16-byte aligned. */
size_t wan_attention_q8_quantize_workspace_bytes(int32_t B, int32_t Sk, int32_t heads, int32_t head_dim);
int wan_attention_q8_quantize(const void* q, const void* k, const void* v, int32_t B, int32_t Sq, int32_t Sk,
                              int32_t heads, int32_t head_dim, void* q8, float* sq, void* k8, float* sk, void* v8t,
                              float* sv, void* ws, size_t ws_bytes, wan_stream_t stream);
int wan_attention_q8_fwd(const void* q8, const float* sq, const void* k8, const float* sk, const void* v8t,
                         const float* sv, int32_t B, int32_t Sq, int32_t Sk, int32_t heads, int32_t head_dim, void* o,
                         float* lse, wan_stream_t stream);

/* FP8 GEMMs.  [DEEP] §5.3 also lists FP8 GEMMs with weights quantised per tensor and activations per
 * token.  Codes are OCP E4M3 as above, scale = amax / 448, code = e4m3(clamp(x * (448 / amax))).
 * wan_quantize_rows_e4m3: x [rows, cols] bf16 (row stride ld elements, cols % 8 == 0) -> codes uint8
 *   [rows, cols] (row stride ldc bytes, % 16 == 0) and scales float32 [rows], one per row.
 * wan_quantize_tensor_e4m3: x [n] bf16 (n % 8 == 0) -> codes [n] and one float32 scale, both on the
 *   device; ws: at least 256 bytes of device scratch.
 * wan_gemm_e4m3: y [M, N] bf16 (row stride ldy elements) = act((A W^T) * a_scales[m] * w_scale[0] + bias[n])
 *   from codes A [M, K] and W [N, K], both in K panels (wan_pack_weight with elem_bytes 1: rows M and
 *   N rounded up to 256); K % 256 == 0, N % 4 == 0, ldy % 4 == 0; act 0 = none, 1 = GELU (erf); bias
 *   may be NULL.  WAN_EUNSUPPORTED when either operand's panels reach 2 GiB. */
int wan_quantize_rows_e4m3(const void* x, int64_t ld, int32_t rows, int32_t cols, void* codes, int64_t ldc,
                           float* scales, wan_stream_t stream);
int wan_quantize_tensor_e4m3(const void* x, int64_t n, void* codes, float* scale, void* ws, size_t ws_bytes,
                             wan_stream_t stream);
int wan_gemm_e4m3(const void* a, const float* a_scales, const void* w, const float* w_scale, int32_t M, int32_t N,
                  int32_t K, const float* bias, int32_t act, void* y, int64_t ldy, wan_stream_t stream);

/* Kernel timing (measurement only).  wan_profile_begin hands the library `capacity` caller-created
 * HIP events (hipEvent_t, passed as void*) for starts and stops plus an int32 tag array; until
 * wan_profile_end, each launch inside wan_dit_block_fwd whose id bit is set in kernel_mask is
 * bracketed by hipEventRecord(start[i]) / hipEventRecord(stop[i]) on the launch stream, and tags[i]
 * receives its wan_kernel_id, until capacity pairs are used.  The arrays must stay valid until
 * wan_profile_end, which returns the number of pairs recorded and disables recording.  Process-wide
 * state, not thread-safe; calls that overlap on several threads must not use it.
 * Ids name the block's launches in order.  WAN_K_ATTN_PROLOGUE precedes the Q/K/V GEMM: it zero-fills
 * the padded keys of V^T (the GEMM writes V^T itself) and writes the 3D RoPE table the GEMM's epilogue
 * reads.  WAN_K_QK_RMS is the Q/K RMSNorm pass after the Q/K/V GEMM (whose epilogue applies the gains
 * and the RoPE): it scales the k rows and keeps the q rows' factors for the attention's score scale.
 * WAN_K_QUANT marks the three quantiser launches that precede the self-attention under
 * WAN_FLAG_FP8_ATTN. */
typedef enum {
  WAN_K_LN1 = 0, WAN_K_QKV_GEMM = 1, WAN_K_QK_RMS = 2, WAN_K_ATTN_PROLOGUE = 3, WAN_K_SELF_ATTN = 4,
  WAN_K_O_GEMM = 5, WAN_K_LN3 = 6, WAN_K_CROSS_Q_GEMM = 7, WAN_K_CROSS_ATTN = 8, WAN_K_CROSS_O_GEMM = 9,
  WAN_K_LN2 = 10, WAN_K_FFN1_GEMM = 11, WAN_K_FFN2_GEMM = 12, WAN_K_QUANT = 13
} wan_kernel_id;
int wan_profile_begin(void* const* start_events, void* const* stop_events, int32_t* tags, int32_t capacity,
                      uint32_t kernel_mask);
int32_t wan_profile_end(void);

/* Device ceilings (measurement only): what the roofline fractions of the kernels above are quoted
 * against, measured on the device at hand beside the nominal figures.
 * wan_device_info: compute units and peak engine clock (kHz) of the current device, as the HIP
 *   runtime reports them (hipDeviceAttributeMultiprocessorCount, hipDeviceAttributeClockRate).
 * wan_mfma_peak_probe: launches `blocks` workgroups of 256 threads (4 waves); each wave issues
 *   4 * iters matrix-core instructions on register operands only:
 *     kind 0: v_mfma_f32_32x32x16_bf16, every A element = the bf16 in each half of a_word, B likewise
 *             from b_word; 32768 flop per instruction and wave;
 *     kind 1: v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 with unit block scales, every element = the
 *             code in each byte of a_word / b_word; 131072 flop per instruction and wave;
 *     kind 2: v_mfma_f32_32x32x16_bf16 on operands that differ per lane and per instruction (hashed
 *             sign and mantissa, magnitude in [0.5, 2); a_word and b_word seed the hash): the rate
 *             under the operand bit toggling of real data, which costs matrix-core power.
 *   out [blocks * 256] float32 (caller-owned device memory) receives each lane's sum of its four
 *   accumulators: for kinds 0 and 1, 64 * K * iters * a * b (K = 16, resp. 64), so a caller can check
 *   the work was done; for kind 2, a finite value.
 *   Time it with events on `stream`; flop per launch = blocks * 4 * 4 * iters * (flop per instruction).
 *   Errors: WAN_EINVAL for kind outside 0..2, blocks or iters outside 1..2^20, or a NULL / misaligned
 *   out (nothing is enqueued). */
int wan_device_info(int32_t* compute_units, int32_t* clock_khz);
int wan_mfma_peak_probe(int32_t kind, uint32_t a_word, uint32_t b_word, int32_t blocks, int32_t iters, float* out,
                        wan_stream_t stream);

/* Human-readable name of a wan_status; message of the last failed call on this thread. */
const char* wan_status_string(int status);
const char* wan_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* WAN_H */
