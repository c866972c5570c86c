// MFMA GEMMs for the DiT block's linear layers (patch embedding, Q/K/V, O,
// cross-attention q/o and K/V, FFN, head, context MLPs) and a small GEMV for the
// timestep MLP.
//
// Every linear layer computes y = x W^T + b with W stored [out, in] ("图解 Wan2.1
// I2V" §5.3-§5.5 and the Conv3d patch embedding of §5.1), so both operands are
// contiguous along K (an "NT" product).
//
// Two kernels share the tile order and the epilogues:
//  * gemm_lds_kernel (bf16, K a multiple of 128; the block's large products):
//    256 x 256 tiles, 8 waves of 64 x 128, K steps of 32 copied global -> LDS by
//    asynchronous global_load_lds_dwordx4 into a ring of four stages, two steps
//    ahead of their use (no staging registers);
//  * gemm_nt_kernel (everything else): K steps of 128 bytes staged through
//    double-buffered, row-padded LDS with register prefetch of the next step;
//    loads are predicate-free (out-of-range rows clamped, a final partial K step
//    zero-filled).
// Common to both:
//  * the MFMA is issued as C^T = W A^T (A-operand = weight rows), so a lane's
//    accumulator holds 4 consecutive output columns of one row: the epilogue
//    reads bias / gate / residual and writes results 4 columns (8 or 16 bytes)
//    at a time;
//  * the 1D grid is remapped so each XCD (blockIdx % 8) receives a contiguous run
//    of tiles, grouped a few row-tiles at a time (group_m), so concurrent tiles
//    share A rows and W columns in that XCD's L2;
//  * k is accumulated in increasing order in every configuration, so all tile
//    shapes give bitwise-identical results;
//  * epilogues fuse the bias, GELU / SiLU, the output cast and the adaLN-gated
//    residual update x += gate * (.) ("图解 Wan2.1 I2V" §5.2).
#include "wan_internal.h"

namespace wan {

namespace {


// Exact GELU x * Phi(x) = x/2 (1 + erf(x / sqrt 2)), with erf from Abramowitz & Stegun, Handbook of
// Mathematical Functions, formula 7.1.26 (absolute error <= 1.5e-7): for z >= 0,
// erf(z) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2), t = 1 / (1 + p z).
__device__ __forceinline__ float gelu_erf(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.f));
  const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f),
                                      -0.284496736f), 0.254829592f);
  const float e = __builtin_amdgcn_exp2f(-z * z * 1.4426950408889634f);  // exp(-z^2); 0 for large z
  const float erf_abs = 1.f - poly * e;
  return 0.5f * x * (1.f + copysignf(erf_abs, x));
}

__device__ __forceinline__ float apply_act(float v, int act) {
  if (act == ACT_GELU) return gelu_erf(v);
  if (act == ACT_SILU) return v / (1.f + __expf(-v));
  return v;
}

// Epilogues receive four consecutive columns n..n+3 of row m.
template <typename OutT, int ACT>
struct EpiStore {
  OutT* out;
  int64_t ldo;
  const float* bias;
  __device__ __forceinline__ void operator()(int m, int n, float4 v) const {
    if (bias) {
      const float4 b = *reinterpret_cast<const float4*>(bias + n);
      v.x += b.x; v.y += b.y; v.z += b.z; v.w += b.w;
    }
    if constexpr (ACT != ACT_NONE) {
      v.x = apply_act(v.x, ACT); v.y = apply_act(v.y, ACT);
      v.z = apply_act(v.z, ACT); v.w = apply_act(v.w, ACT);
    }
    OutT* p = out + (int64_t)m * ldo + n;
    if constexpr (sizeof(OutT) == 2) {
      bf16x4 o;
      o[0] = (bf16)v.x; o[1] = (bf16)v.y; o[2] = (bf16)v.z; o[3] = (bf16)v.w;
      *reinterpret_cast<bf16x4*>(p) = o;
    } else {
      *reinterpret_cast<float4*>(p) = v;
    }
  }
};

// Q/K/V projection: columns [0, vcol0) (q, k) are stored row-major like EpiStore; columns >= vcol0
// (v) go straight to the per-head transposed layout V^T[b, h, d, pos] the attention kernels read
// (pos = token within its batch row, bf16 keys permuted within 16-key groups: position p holds key
// p with bits 2 and 3 swapped).
template <typename T>
struct EpiQKV {
  T* out;
  int64_t ldo;
  const float* bias;
  T* vt;
  int vcol0, S, H, hd, Spad;
  __device__ __forceinline__ void operator()(int m, int n, float4 v) const {
    if (bias) {
      const float4 b = *reinterpret_cast<const float4*>(bias + n);
      v.x += b.x; v.y += b.y; v.z += b.z; v.w += b.w;
    }
    if (n < vcol0) {
      T* p = out + (int64_t)m * ldo + n;
      if constexpr (sizeof(T) == 2) {
        bf16x4 o;
        o[0] = (bf16)v.x; o[1] = (bf16)v.y; o[2] = (bf16)v.z; o[3] = (bf16)v.w;
        *reinterpret_cast<bf16x4*>(p) = o;
      } else {
        *reinterpret_cast<float4*>(p) = v;
      }
    } else {
      const int nn = n - vcol0, h = nn / hd, d = nn - h * hd;  // 4 channels d..d+3 of head h
      const int b = m / S, pos = m - b * S;
      const int pp = sizeof(T) == 2 ? ((pos & ~12) | ((pos & 4) << 1) | ((pos & 8) >> 1)) : pos;
      T* p = vt + (((int64_t)b * H + h) * hd + d) * Spad + pp;
      p[0] = from_f32<T>(v.x);
      p[Spad] = from_f32<T>(v.y);
      p[2 * (int64_t)Spad] = from_f32<T>(v.z);
      p[3 * (int64_t)Spad] = from_f32<T>(v.w);
    }
  }
};

struct EpiResidual {
  float* x;
  int64_t ldx;
  const float* bias;
  const float* e0;  // [B, 6, N] or null (gate 1)
  const float* mb;  // [6, N]
  int chunk, S, N;
  float* y = nullptr;  // optional: also record the branch output C + bias (row stride N)
  __device__ __forceinline__ void operator()(int m, int n, float4 v) const {
    if (bias) {
      const float4 b = *reinterpret_cast<const float4*>(bias + n);
      v.x += b.x; v.y += b.y; v.z += b.z; v.w += b.w;
    }
    if (y) *reinterpret_cast<float4*>(y + (int64_t)m * N + n) = v;
    float* p = x + (int64_t)m * ldx + n;
    float4 r = *reinterpret_cast<const float4*>(p);
    if (e0) {
      const int b = m / S;
      float4 g = *reinterpret_cast<const float4*>(e0 + ((int64_t)b * 6 + chunk) * N + n);
      if (mb) {
        const float4 h = *reinterpret_cast<const float4*>(mb + (int64_t)chunk * N + n);
        g.x += h.x; g.y += h.y; g.z += h.z; g.w += h.w;
      }
      r.x = fmaf(g.x, v.x, r.x); r.y = fmaf(g.y, v.y, r.y);
      r.z = fmaf(g.z, v.z, r.z); r.w = fmaf(g.w, v.w, r.w);
    } else {
      r.x += v.x; r.y += v.y; r.z += v.z; r.w += v.w;
    }
    *reinterpret_cast<float4*>(p) = r;
  }
};

// Map a linear block id to (tile_m, tile_n): XCD-contiguous runs, then groups of gm row-tiles
// (column tiles vary slowest inside a group).
__device__ __forceinline__ void tile_coords(int id, int tiles_m, int tiles_n, int gm, int& tm, int& tn) {
  const int n = tiles_m * tiles_n;
  const int q = n >> 3, r = n & 7;
  const int xcd = id & 7, k = id >> 3;
  const int t = xcd * q + min(xcd, r) + k;  // bijection on [0, n)
  const int per_group = gm * tiles_n;
  const int g = t / per_group;
  const int first_m = g * gm;
  const int gsz = min(tiles_m - first_m, gm);
  const int w = t - g * per_group;
  tm = first_m + w % gsz;
  tn = w / gsz;
}

// Row-group size of the tile order (measured on the block's shapes): wide products (>= 32 column
// tiles) share weights best in groups of 4, long-K products in groups of 2, the rest in groups of 8.
inline int group_m(int tiles_n, int K) { return (K >= 4096 && tiles_n < 32) ? 2 : 4; }

template <typename T, int BM, int BN, int WM, int WN, class Epi>
__global__ __launch_bounds__(WM* WN * 64) void gemm_nt_kernel(const T* __restrict__ A, int64_t lda,
                                                               const T* __restrict__ W, int64_t ldw, int M,
                                                               int N, int K, int tiles_m, int tiles_n, int gm,
                                                               Epi epi) {
  constexpr int NT = WM * WN * 64;
  constexpr int E16 = dtype_traits<T>::per16;  // elements per 16 bytes
  constexpr int BK = 8 * E16;                  // 128 bytes of K per step
  constexpr int ROW = BK + E16;                // padded LDS row (144 bytes): conflict-free 16-byte reads
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int AC = BM * 8 / NT, BC = BN * 8 / NT;  // 16-byte chunks per thread per step
  constexpr int STAGE = (BM + BN) * ROW;
  static_assert(AC * NT == BM * 8 && BC * NT == BN * 8, "tile / thread mismatch");
  __shared__ u32x4 smem_raw[2 * STAGE * sizeof(T) / 16];
  T* smem = reinterpret_cast<T*>(smem_raw);

  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, gm, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // Per-thread global source rows (clamped into range) and LDS destinations.
  const T* pa[AC];
  const T* pb[BC];
  int la[AC], lb[BC];
#pragma unroll
  for (int i = 0; i < AC; ++i) {
    const int c = tid + i * NT, r = c >> 3, kc = (c & 7) * E16;
    pa[i] = A + (int64_t)min(m0 + r, M - 1) * lda + kc;
    la[i] = r * ROW + kc;
  }
#pragma unroll
  for (int i = 0; i < BC; ++i) {
    const int c = tid + i * NT, r = c >> 3, kc = (c & 7) * E16;
    pb[i] = W + (int64_t)min(n0 + r, N - 1) * ldw + kc;
    lb[i] = BM * ROW + r * ROW + kc;
  }

  u32x4 ra[AC], rb[BC];
  auto load_full = [&](int k0) {
#pragma unroll
    for (int i = 0; i < AC; ++i) ra[i] = *reinterpret_cast<const u32x4*>(pa[i] + k0);
#pragma unroll
    for (int i = 0; i < BC; ++i) rb[i] = *reinterpret_cast<const u32x4*>(pb[i] + k0);
  };
  auto load_tail = [&](int k0) {  // last, partial K step: zero-fill k >= K
#pragma unroll
    for (int i = 0; i < AC; ++i) {
      const int kk = k0 + ((tid + i * NT) & 7) * E16;
      ra[i] = kk < K ? *reinterpret_cast<const u32x4*>(pa[i] + k0) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < BC; ++i) {
      const int kk = k0 + ((tid + i * NT) & 7) * E16;
      rb[i] = kk < K ? *reinterpret_cast<const u32x4*>(pb[i] + k0) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_stage = [&](int buf) {
    T* st = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < AC; ++i) *reinterpret_cast<u32x4*>(st + la[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < BC; ++i) *reinterpret_cast<u32x4*>(st + lb[i]) = rb[i];
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = zero16();

  const int nk = (K + BK - 1) / BK;
  const int nfull = K / BK;
  if (nfull > 0) load_full(0); else load_tail(0);
  store_stage(0);
  __syncthreads();
  const int lrow = lane & 31, lhalf = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nfull) load_full((kt + 1) * BK);
    else if (kt + 1 < nk) load_tail((kt + 1) * BK);
    const T* sa = smem + buf * STAGE + (wm * TM + lrow) * ROW + lhalf * E16;
    const T* sb = smem + buf * STAGE + BM * ROW + (wn * TN + lrow) * ROW + lhalf * E16;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      u32x4 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const u32x4*>(sa + i * 32 * ROW + kc * 2 * E16);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = *reinterpret_cast<const u32x4*>(sb + j * 32 * ROW + kc * 2 * E16);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mfma_chunk(bfr[j], af[i], acc[i][j], T());  // C^T = W A^T
    }
    if (kt + 1 < nk) store_stage(buf ^ 1);
    __syncthreads();
  }

  // acc[i][j]: lane holds row m = m0 + wm*TM + i*32 + lrow and columns
  // n = n0 + wn*TN + j*32 + g*8 + lhalf*4 + (0..3) in elements 4g..4g+3.
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * TM + i * 32 + lrow;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * TN + j * 32 + g * 8 + lhalf * 4;
        if (n < N)
          epi(m, n, make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]));
      }
  }
}

// ---------------------------------------------------------------------------
// bf16 GEMM with asynchronous global -> LDS copies and a ring of ST LDS stages.
//
// One workgroup = WM x WN waves owning a BM x BN tile; a wave owns (BM/WM) x (BN/WN) (128 x 128:
// 16 MFMA blocks, 256 accumulator registers, so one wave per SIMD).  Each K step of BK elements
// is copied by global_load_lds_dwordx4 straight into LDS, ST - 1 steps ahead of its use, so the
// copies need no staging registers and have ST - 1 steps of MFMA work to land.  Row r of a stage
// holds BK * 2 bytes; its 16-byte chunk c sits at slot c ^ ((r / RPB) % CH) (RPB rows share one
// 256-byte bank window), which makes the 16 rows one ds_read_b128 phase reads hit 16 distinct
// bank groups.  The copy instead permutes which global chunk each lane fetches: lanes still write
// LDS linearly.  Requires K % BK == 0 (callers fall back to gemm_nt_kernel otherwise).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// s_waitcnt with only the vector-memory counter constrained to <= n (gfx9 encoding).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int BM, int BN, int BK, int NW>
struct LdsGemmCfg {
  static constexpr int CH = BK / 8;        // 16-byte chunks per row
  static constexpr int RPB = 16 / CH;      // rows per 256-byte bank window
  static constexpr int ROWB = BK * 2;      // bytes per row
  static constexpr int ABYTES = BM * ROWB, BBYTES = BN * ROWB;
  static constexpr int LA = ABYTES / 1024 / NW, LB = BBYTES / 1024 / NW;  // copies per wave per stage
  static_assert(CH >= 1 && CH <= 16 && LA * NW * 1024 == ABYTES && LB * NW * 1024 == BBYTES, "shape");
  __device__ static __forceinline__ int off(int r, int c) { return r * ROWB + ((c ^ ((r / RPB) & (CH - 1))) << 4); }
};

template <int BM, int BN, int BK, int NW>
struct LdsCopyPlan {
  using C = LdsGemmCfg<BM, BN, BK, NW>;
  const bf16* ga[C::LA];
  const bf16* gb[C::LB];
  __device__ __forceinline__ LdsCopyPlan(const bf16* A, int64_t lda, const bf16* W, int64_t ldw, int m0, int n0,
                                         int M, int N) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < C::LA; ++i) {
      const int p = (i * NW + wave) * 64 + lane, r = p / C::CH, s = p % C::CH;
      const int c = s ^ ((r / C::RPB) & (C::CH - 1));
      ga[i] = A + (int64_t)min(m0 + r, M - 1) * lda + c * 8;
    }
#pragma unroll
    for (int i = 0; i < C::LB; ++i) {
      const int p = (i * NW + wave) * 64 + lane, r = p / C::CH, s = p % C::CH;
      const int c = s ^ ((r / C::RPB) & (C::CH - 1));
      gb[i] = W + (int64_t)min(n0 + r, N - 1) * ldw + c * 8;
    }
  }
  __device__ __forceinline__ void issue(int k0, char* sa, char* sb) const {
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < C::LA; ++i)
      __builtin_amdgcn_global_load_lds((glb_void*)(ga[i] + k0), (lds_void*)(sa + (i * NW + wave) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < C::LB; ++i)
      __builtin_amdgcn_global_load_lds((glb_void*)(gb[i] + k0), (lds_void*)(sb + (i * NW + wave) * 1024), 16, 0, 0);
  }
};

template <int BM, int BN, int BK, int ST, int WM, int WN>
struct LdsSlots {
  char* a[4];
  char* b[4];
};

// One K step kt with static ring slot P = kt % ST.  The K loop runs a multiple of ST steps and
// always refills the freed slot (past the last stage it re-copies stage 0, which is never read), so
// the body is straight-line code with a constant wait count: at the start of step kt exactly
// ST - 2 later stages are in flight.
//
// F8: the operands are E4M3 codes.  A row of 2 BK codes occupies the bytes of BK bf16 elements, so
// the copies and the LDS layout are unchanged; each K step is then one
// v_mfma_scale_f32_32x32x64_f8f6f4 per output block (unit block scales) on 32-byte fragments
// (lane half h reads 16-byte chunks 2h and 2h + 1 of its row, the same k for A and W).
template <int BM, int BN, int BK, int ST, int WM, int WN, int P, bool F8 = false>
__device__ __forceinline__ void lds_gemm_step(const LdsCopyPlan<BM, BN, BK, WM * WN>& cp,
                                              const LdsSlots<BM, BN, BK, ST, WM, WN>& sl, int kt, int nk,
                                              f32x16 (&acc)[BM / WM / 32][BN / WN / 32]) {
  using C = LdsGemmCfg<BM, BN, BK, WM * WN>;
  constexpr int FM = BM / WM / 32, FN = BN / WN / 32, PER = C::LA + C::LB;
  wait_vmcnt<(ST - 2) * PER>();  // this wave's copies of stage kt have landed
  // Every wave's copies of stage kt are visible and slot (kt - 1) % ST is free after this barrier.
  // A bare s_barrier: __syncthreads()'s workgroup fence would also wait for the copies of the later
  // stages still in flight.  The wavefront-scope fences only keep the compiler from moving LDS
  // accesses across the barrier; they emit no instructions.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // Refill the slot freed by the barrier with stage kt + ST - 1: with two slots right away (the copy
  // then has this whole step to land), with more slots after this step's LDS reads.
  constexpr int Q = (P + ST - 1) % ST;
  const int kn = kt + ST - 1;
  if constexpr (ST == 2) cp.issue((kn < nk ? kn : 0) * BK, sl.a[Q], sl.b[Q]);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, lrow = lane & 31, lhalf = lane >> 5;
  const int wm = wave / WN, wn = wave % WN;
  const char* sa = sl.a[P];
  const char* sb = sl.b[P];
  if constexpr (F8) {
    static_assert(BK == 32, "one 64-code step per E4M3 product");
    u32x4 af[FM][2], bfr[FN][2];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int x = 0; x < 2; ++x)
        af[i][x] = *reinterpret_cast<const u32x4*>(sa + C::off(wm * (BM / WM) + i * 32 + lrow, 2 * lhalf + x));
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int x = 0; x < 2; ++x)
        bfr[j][x] = *reinterpret_cast<const u32x4*>(sb + C::off(wn * (BN / WN) + j * 32 + lrow, 2 * lhalf + x));
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        typedef int v8i_t __attribute__((ext_vector_type(8)));
        const v8i_t a = {(int)bfr[j][0].x, (int)bfr[j][0].y, (int)bfr[j][0].z, (int)bfr[j][0].w,
                         (int)bfr[j][1].x, (int)bfr[j][1].y, (int)bfr[j][1].z, (int)bfr[j][1].w};
        const v8i_t b = {(int)af[i][0].x, (int)af[i][0].y, (int)af[i][0].z, (int)af[i][0].w,
                         (int)af[i][1].x, (int)af[i][1].y, (int)af[i][1].z, (int)af[i][1].w};
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], 0, 0, 0, 127, 0, 127);
      }
    if constexpr (ST > 2) cp.issue((kn < nk ? kn : 0) * BK, sl.a[Q], sl.b[Q]);
    return;
  }
#pragma unroll
  for (int kc = 0; kc < BK / 16; ++kc) {
    u32x4 af[FM], bfr[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
      af[i] = *reinterpret_cast<const u32x4*>(sa + C::off(wm * (BM / WM) + i * 32 + lrow, kc * 2 + lhalf));
#pragma unroll
    for (int j = 0; j < FN; ++j)
      bfr[j] = *reinterpret_cast<const u32x4*>(sb + C::off(wn * (BN / WN) + j * 32 + lrow, kc * 2 + lhalf));
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) mfma_chunk(bfr[j], af[i], acc[i][j], bf16());  // C^T = W A^T
  }
  if constexpr (ST > 2) cp.issue((kn < nk ? kn : 0) * BK, sl.a[Q], sl.b[Q]);
}

template <int BM, int BN, int BK, int ST, int WM, int WN, class Epi, bool F8 = false>
__global__ __launch_bounds__(WM* WN * 64) void gemm_lds_kernel(const bf16* __restrict__ A, int64_t lda,
                                                                const bf16* __restrict__ W, int64_t ldw, int M,
                                                                int N, int K, int tiles_m, int tiles_n, int gm,
                                                               Epi epi) {
  constexpr int NW = WM * WN;
  using C = LdsGemmCfg<BM, BN, BK, NW>;
  constexpr int FM = BM / WM / 32, FN = BN / WN / 32;
  static_assert(ST >= 2 && ST <= 4, "stages");
  // One __shared__ object per ring slot, so the compiler can tell a slot being read from the slots
  // with copies in flight (it then needs no vmcnt wait before the reads).
  __shared__ u32x4 a0[C::ABYTES / 16], a1[C::ABYTES / 16], a2[ST > 2 ? C::ABYTES / 16 : 1],
      a3[ST > 3 ? C::ABYTES / 16 : 1];
  __shared__ u32x4 b0[C::BBYTES / 16], b1[C::BBYTES / 16], b2[ST > 2 ? C::BBYTES / 16 : 1],
      b3[ST > 3 ? C::BBYTES / 16 : 1];
  const LdsSlots<BM, BN, BK, ST, WM, WN> sl{{(char*)a0, (char*)a1, (char*)a2, (char*)a3},
                                            {(char*)b0, (char*)b1, (char*)b2, (char*)b3}};
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, gm, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const LdsCopyPlan<BM, BN, BK, NW> cp(A, lda, W, ldw, m0, n0, M, N);

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = zero16();

  const int nk = K / BK;  // a multiple of ST
#pragma unroll
  for (int s = 0; s < ST - 1; ++s) cp.issue(s * BK, sl.a[s], sl.b[s]);
  for (int kt = 0; kt < nk; kt += ST) {
    lds_gemm_step<BM, BN, BK, ST, WM, WN, 0, F8>(cp, sl, kt, nk, acc);
    lds_gemm_step<BM, BN, BK, ST, WM, WN, 1, F8>(cp, sl, kt + 1, nk, acc);
    if constexpr (ST > 2) lds_gemm_step<BM, BN, BK, ST, WM, WN, 2 % ST, F8>(cp, sl, kt + 2, nk, acc);
    if constexpr (ST > 3) lds_gemm_step<BM, BN, BK, ST, WM, WN, 3 % ST, F8>(cp, sl, kt + 3, nk, acc);
  }
  wait_vmcnt<0>();  // the surplus copies past the last stage land before the LDS is released

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, lrow = lane & 31, lhalf = lane >> 5;
  const int wm = wave / WN, wn = wave % WN;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * (BM / WM) + i * 32 + lrow;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * (BN / WN) + j * 32 + g * 8 + lhalf * 4;
        if (n < N)
          epi(m, n, make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]));
      }
  }
}

template <int BM, int BN, int BK, int ST, int WM, int WN, class Epi, bool F8 = false>
hipError_t launch_lds(const bf16* A, int64_t lda, const bf16* W, int64_t ldw, int M, int N, int K, const Epi& epi,
                      hipStream_t s) {
  const int tm = (int)ceil_div(M, BM), tn = (int)ceil_div(N, BN);
  hipLaunchKernelGGL((gemm_lds_kernel<BM, BN, BK, ST, WM, WN, Epi, F8>), dim3((unsigned)(tm * tn)),
                     dim3(WM * WN * 64), 0, s, A, lda, W, ldw, M, N, K, tm, tn, group_m(tn, K), epi);
  return hipGetLastError();
}

// Epilogue wrapper of the E4M3 products: the accumulator times (row scale * tensor scale), then the
// wrapped epilogue.
template <class Epi>
struct EpiScaled {
  const float* row_scale;
  const float* w_scale;  // one value, on the device
  Epi inner;
  __device__ __forceinline__ void operator()(int m, int n, float4 v) const {
    const float sc = row_scale[m] * *w_scale;
    v.x *= sc; v.y *= sc; v.z *= sc; v.w *= sc;
    inner(m, n, v);
  }
};

// E4M3 product ("Wan 技术深度解析" §5.3: per-token activation, per-tensor weight scales): A codes [M, K]
// (row stride lda bytes) with per-row scales, W codes [N, K] (row stride ldw bytes) with one tensor scale.  K a multiple of 256, strides multiples of 16 bytes.
template <class Epi>
hipError_t run_gemm_e4m3(const uint8_t* A, int64_t lda, const float* a_scales, const uint8_t* W, int64_t ldw,
                         const float* w_scale, int M, int N, int K, const Epi& epi, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (N % 4 != 0 || K % 256 != 0 || lda % 16 != 0 || ldw % 16 != 0) return hipErrorInvalidValue;
  return launch_lds<256, 256, 32, 4, 4, 2, EpiScaled<Epi>, true>(
      reinterpret_cast<const bf16*>(A), lda / 2, reinterpret_cast<const bf16*>(W), ldw / 2, M, N, K / 2,
      EpiScaled<Epi>{a_scales, w_scale, epi}, s);
}

template <typename T, int BM, int BN, int WM, int WN, class Epi>
hipError_t launch_cfg(const T* A, int64_t lda, const T* W, int64_t ldw, int M, int N, int K, const Epi& epi,
                      hipStream_t s) {
  const int tm = (int)ceil_div(M, BM), tn = (int)ceil_div(N, BN);
  hipLaunchKernelGGL((gemm_nt_kernel<T, BM, BN, WM, WN, Epi>), dim3((unsigned)(tm * tn)), dim3(WM * WN * 64), 0,
                     s, A, lda, W, ldw, M, N, K, tm, tn, group_m(tn, K), epi);
  return hipGetLastError();
}

#ifndef WAN_GEMM_FORCE
#define WAN_GEMM_FORCE 0
#endif

// Tile choice.  bf16 products with many rows and K a multiple of 128 use the asynchronous-copy
// kernel (256 x 256 tiles, 8 waves of 64 x 128, BK 32, four LDS stages); other bf16 products with
// many rows use the register-staged kernel with 256-row tiles; small products and fp32 use 128 x 128.
template <typename T, class Epi>
hipError_t run_gemm(const T* A, int64_t lda, const T* W, int64_t ldw, int M, int N, int K, const Epi& epi,
                    hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (N % 4 != 0 || K % dtype_traits<T>::per16 != 0) return hipErrorInvalidValue;
  if constexpr (sizeof(T) == 2) {
    int cfg = 0;
    if (M >= 4096 && N >= 1024 && K % 128 == 0 && lda % 8 == 0 && ldw % 8 == 0) cfg = 1;
    else if (M >= 4096 && N % 256 == 0 && N >= 1024) cfg = 2;
    else if (M >= 4096 && N % 128 == 0 && N >= 1024) cfg = 3;
    if (WAN_GEMM_FORCE) cfg = WAN_GEMM_FORCE;
    if (cfg == 1) return launch_lds<256, 256, 32, 4, 4, 2>(A, lda, W, ldw, M, N, K, epi, s);
    if (cfg == 2) return launch_cfg<T, 256, 256, 4, 2>(A, lda, W, ldw, M, N, K, epi, s);
    if (cfg == 3) return launch_cfg<T, 256, 128, 4, 2>(A, lda, W, ldw, M, N, K, epi, s);
  }
  return launch_cfg<T, 128, 128, 2, 2>(A, lda, W, ldw, M, N, K, epi, s);
}

// ---------------------------------------------------------------------------
// GEMV for the timestep MLP (M = batch, at most a few rows): one wave per output.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void gemv_kernel(const T* __restrict__ W, int N, int K, const float* __restrict__ x,
                                                    int B, const float* __restrict__ bias, int in_act, int out_act,
                                                    float* __restrict__ y) {
  constexpr int E16 = dtype_traits<T>::per16;
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const T* wr = W + (int64_t)n * K;
  for (int k0 = lane * E16; k0 < K; k0 += 64 * E16) {
    u32x4 raw = *reinterpret_cast<const u32x4*>(wr + k0);
    const T* wv = reinterpret_cast<const T*>(&raw);
#pragma unroll
    for (int e = 0; e < E16; ++e) {
      const float w = to_f32(wv[e]);
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (b < B) acc[b] += w * apply_act(x[(int64_t)b * K + k0 + e], in_act);
    }
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (b >= B) break;
    float v = wave_sum(acc[b]);
    if (lane == 0) {
      if (bias) v += bias[n];
      y[(int64_t)b * N + n] = apply_act(v, out_act);
    }
  }
}

struct SinArgs {
  float t[8];
};
// Sinusoidal timestep embedding [cos(tau f_i) | sin(tau f_i)], tau = 1000 t, f_i = 10000^(-i/half).
__global__ void sinusoid_kernel(SinArgs a, int B, int freq_dim, float* __restrict__ emb) {
  const int half = freq_dim / 2;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * half) return;
  const int b = i / half, f = i % half;
  // double precision: tau * f_i reaches 1000 rad, where fp32 phase error would be ~1e-4.
  const double freq = exp(-(double)f / (double)half * 9.210340371976184);  // ln(10000)
  const double arg = 1000.0 * (double)a.t[b] * freq;
  emb[(int64_t)b * freq_dim + f] = (float)cos(arg);
  emb[(int64_t)b * freq_dim + half + f] = (float)sin(arg);
}

}  // namespace

template <typename T, typename OutT>
hipError_t gemm_store(const T* A, int64_t lda, const T* W, int64_t ldw, int M, int N, int K, const float* bias,
                      int act, OutT* out, int64_t ldo, hipStream_t s) {
  if (act == ACT_GELU) return run_gemm<T>(A, lda, W, ldw, M, N, K, EpiStore<OutT, ACT_GELU>{out, ldo, bias}, s);
  if (act == ACT_SILU) return run_gemm<T>(A, lda, W, ldw, M, N, K, EpiStore<OutT, ACT_SILU>{out, ldo, bias}, s);
  return run_gemm<T>(A, lda, W, ldw, M, N, K, EpiStore<OutT, ACT_NONE>{out, ldo, bias}, s);
}

template <typename T>
hipError_t gemm_qkv(const T* A, int64_t lda, const T* W, int64_t ldw, int M, int dim, int K, const float* bias,
                    T* qk, int64_t ldo, T* vt, int S, int H, int hd, int Spad, hipStream_t s) {
  if (hd % 4 != 0) return hipErrorInvalidValue;
  return run_gemm<T>(A, lda, W, ldw, M, 3 * dim, K, EpiQKV<T>{qk, ldo, bias, vt, 2 * dim, S, H, hd, Spad}, s);
}

template <typename T>
hipError_t gemm_residual(const T* A, int64_t lda, const T* W, int64_t ldw, int M, int N, int K, const float* bias,
                         const float* e0, const float* mb, int chunk, int S, float* x, int64_t ldx, hipStream_t s,
                         float* ystore) {
  EpiResidual epi{x, ldx, bias, e0, mb, chunk, S, N, ystore};
  return run_gemm<T>(A, lda, W, ldw, M, N, K, epi, s);
}

hipError_t gemm_e4m3_store(const uint8_t* A, int64_t lda, const float* a_scales, const uint8_t* W, int64_t ldw,
                           const float* w_scale, int M, int N, int K, const float* bias, int act, bf16* out, int64_t ldo,
                           hipStream_t s) {
  if (act == ACT_GELU)
    return run_gemm_e4m3(A, lda, a_scales, W, ldw, w_scale, M, N, K, EpiStore<bf16, ACT_GELU>{out, ldo, bias}, s);
  return run_gemm_e4m3(A, lda, a_scales, W, ldw, w_scale, M, N, K, EpiStore<bf16, ACT_NONE>{out, ldo, bias}, s);
}

hipError_t gemm_qkv_e4m3(const uint8_t* A, int64_t lda, const float* a_scales, const uint8_t* W, int64_t ldw,
                         const float* w_scale, int M, int dim, int K, const float* bias, bf16* qk, int64_t ldo, bf16* vt,
                         int S, int H, int hd, int Spad, hipStream_t s) {
  if (hd % 4 != 0) return hipErrorInvalidValue;
  return run_gemm_e4m3(A, lda, a_scales, W, ldw, w_scale, M, 3 * dim, K,
                       EpiQKV<bf16>{qk, ldo, bias, vt, 2 * dim, S, H, hd, Spad}, s);
}

hipError_t gemm_e4m3_residual(const uint8_t* A, int64_t lda, const float* a_scales, const uint8_t* W, int64_t ldw,
                              const float* w_scale, int M, int N, int K, const float* bias, const float* e0, const float* mb,
                              int chunk, int S, float* x, int64_t ldx, hipStream_t s, float* ystore) {
  return run_gemm_e4m3(A, lda, a_scales, W, ldw, w_scale, M, N, K,
                       EpiResidual{x, ldx, bias, e0, mb, chunk, S, N, ystore}, s);
}

template <typename T>
hipError_t gemv(const T* W, int N, int K, const float* x, int B, const float* bias, int in_act, int out_act,
                float* y, hipStream_t s) {
  if (B > 4 || (K % dtype_traits<T>::per16) != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemv_kernel<T>, dim3((unsigned)ceil_div(N, 4)), dim3(256), 0, s, W, N, K, x, B, bias, in_act,
                     out_act, y);
  return hipGetLastError();
}

hipError_t launch_sinusoid(const float* t_host, int B, int freq_dim, float* emb, hipStream_t s) {
  if (B > 8) return hipErrorInvalidValue;
  SinArgs a{};
  for (int b = 0; b < B; ++b) a.t[b] = t_host[b];
  const int n = B * (freq_dim / 2);
  hipLaunchKernelGGL(sinusoid_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, a, B, freq_dim, emb);
  return hipGetLastError();
}

template hipError_t gemm_store<float, float>(const float*, int64_t, const float*, int64_t, int, int, int,
                                             const float*, int, float*, int64_t, hipStream_t);
template hipError_t gemm_store<bf16, bf16>(const bf16*, int64_t, const bf16*, int64_t, int, int, int, const float*,
                                           int, bf16*, int64_t, hipStream_t);
template hipError_t gemm_store<bf16, float>(const bf16*, int64_t, const bf16*, int64_t, int, int, int,
                                            const float*, int, float*, int64_t, hipStream_t);
template hipError_t gemm_qkv<float>(const float*, int64_t, const float*, int64_t, int, int, int, const float*, float*,
                                    int64_t, float*, int, int, int, int, hipStream_t);
template hipError_t gemm_qkv<bf16>(const bf16*, int64_t, const bf16*, int64_t, int, int, int, const float*, bf16*,
                                   int64_t, bf16*, int, int, int, int, hipStream_t);
template hipError_t gemm_residual<float>(const float*, int64_t, const float*, int64_t, int, int, int, const float*,
                                         const float*, const float*, int, int, float*, int64_t, hipStream_t, float*);
template hipError_t gemm_residual<bf16>(const bf16*, int64_t, const bf16*, int64_t, int, int, int, const float*,
                                        const float*, const float*, int, int, float*, int64_t, hipStream_t, float*);
template hipError_t gemv<float>(const float*, int, int, const float*, int, const float*, int, int, float*,
                                hipStream_t);
template hipError_t gemv<bf16>(const bf16*, int, int, const float*, int, const float*, int, int, float*,
                               hipStream_t);

}  // namespace wan
