// MFMA GEMMs for the DiT block's linear layers (patch embedding, Q/K/V, O,
// cross-attention q/o and K/V, FFN, head, context MLPs) and a small GEMV for the
// timestep MLP.
//
// Every linear layer computes y = x W^T + b with W stored [out, in] ("图解 Wan2.1
// I2V" §5.3-§5.5 and the Conv3d patch embedding of §5.1), so both operands are
// contiguous along K (an "NT" product).  The block's products take both operands in
// K panels of 32 (KMat: each 32-deep K step of a 256-row tile is one contiguous run);
// the other linear layers take them row-major.
//
// Two kernels share the tile order and the epilogues:
//  * gemm_lds_kernel (bf16 / E4M3, K a multiple of 128, both operands in panels; the
//    block's large products): 256 x 256 tiles, 8 waves of 64 x 128, K steps of 32
//    copied global -> LDS by asynchronous direct-to-LDS buffer loads (16 bytes a lane)
//    into a ring of four stages, three steps ahead of their use (no staging
//    registers); the plain-store products run one workgroup per CU walking several
//    tiles, the next tile's first stages copied during the current tile's last steps;
//  * gemm_nt_kernel (everything else): K steps of 128 bytes staged through
//    double-buffered, row-padded LDS with register prefetch of the next step, either
//    operand row-major or in panels; loads are predicate-free (out-of-range rows
//    clamped, a final partial K step zero-filled).
// Common to both:
//  * the MFMA is issued as C^T = W A^T (A-operand = weight rows), so a lane's
//    accumulator holds 4 consecutive output columns of one row: the epilogue
//    reads bias / gate / residual and writes results 4 columns (8 or 16 bytes)
//    at a time;
//  * the 1D grid is remapped so each XCD (blockIdx % 8) receives a contiguous run
//    of tiles, grouped a few row-tiles at a time (group_m), so concurrent tiles
//    share A rows and W columns in that XCD's L2;
//  * k is accumulated in increasing order in every configuration; a configuration's results
//    are bitwise repeatable, and configurations on different MFMA shapes (16 x 16 x 32 for the
//    store and residual products, 32 x 32 x 16 elsewhere) may differ in the last bits;
//  * epilogues fuse the bias, GELU / SiLU, the output cast, the adaLN-gated
//    residual update x += gate * (.) ("图解 Wan2.1 I2V" §5.2), and for the Q/K/V
//    projection the q/k RMSNorm gains, the 3D RoPE and the row sums of squares of
//    the RMSNorm, plus the transposed V layout (§5.3).
#include "wan_internal.h"

#include <atomic>
#include <type_traits>

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

// Whether an epilogue reports per-row block sums (its kBlockSums member; false if it has none).
template <class E, class = void>
struct BlockSums : std::false_type {};
template <class E>
struct BlockSums<E, std::void_t<decltype(E::kBlockSums)>> : std::integral_constant<bool, E::kBlockSums> {};

// Epilogues receive four consecutive columns n..n+3 of row m, in two phases: pre(m, n) issues every
// load the group needs (bias, residual, gate, scales) and returns them; post(m, n, v, pre) does the
// arithmetic and the stores.  run_epilogue issues the loads of four groups before any of their stores,
// so a lane waits about one memory latency per four groups rather than one per group.
// Loads through the constant address space (memory the kernel only reads).
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float4 load_const4(const float* p) {
  const f32x4 v = *(const __attribute__((address_space(4))) f32x4*)p;
  return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ float2 load_const2(const float2* p) {
  const f32x2 v = *(const __attribute__((address_space(4))) f32x2*)p;
  return make_float2(v[0], v[1]);
}

__device__ __forceinline__ float4 load_bias4(const float* bias, int n) {
  return bias ? *reinterpret_cast<const float4*>(bias + n) : make_float4(0.f, 0.f, 0.f, 0.f);
}

template <typename OutT, int ACT>
struct EpiStore {
  OutT* out;
  int64_t ldo, obs;  // element (m, n) at out + m ldo + (n / 32) obs + n % 32 (see ActLayout)
  const float* bias;
  struct Pre {
    float4 b;
  };
  __device__ __forceinline__ Pre pre(int, int n) const { return Pre{load_bias4(bias, n)}; }
  __device__ __forceinline__ void post(int m, int n, float4 v, const Pre& p) const {
    v.x += p.b.x; v.y += p.b.y; v.z += p.b.z; v.w += p.b.w;
    if constexpr (ACT != ACT_NONE) {
      v.x = apply_act(v.x, ACT); v.y = apply_act(v.y, ACT);
      v.z = apply_act(v.z, ACT); v.w = apply_act(v.w, ACT);
    }
    OutT* q = out + (int64_t)m * ldo + (n >> 5) * obs + (n & 31);
    if constexpr (sizeof(OutT) == 2) {
      bf16x4 o;
      o[0] = (bf16)v.x; o[1] = (bf16)v.y; o[2] = (bf16)v.z; o[3] = (bf16)v.w;
      *reinterpret_cast<bf16x4*>(q) = o;
    } else {
      *reinterpret_cast<float4*>(q) = v;
    }
  }
};

// Q/K/V projection ("图解 Wan2.1 I2V" §5.3): columns [0, vcol0) hold q, then k (dim = vcol0 / 2 each);
// columns >= vcol0 hold v.
//  * q, k are stored row-major as RoPE(g * (C + bias)): the RMSNorm gains g (gq, gk), then the 3D
//    rotation of the token's (frame, row, column) position.  The RMS factor itself needs the whole
//    row, which spans several column tiles, so post returns the group's sum of squares of C + bias;
//    run_epilogue adds these up over each 32-column block and passes the block's sum to ssq_store.
//    The factor is applied later: to the k rows by launch_qk_rms, and to the q rows inside the
//    attention's score scale (both the gains and the rotation are linear, so it commutes with them).
//  * v goes straight to the per-head transposed layout V^T[b, h, d, pos] the attention kernels read
//    (pos = token within its batch row, bf16 keys permuted within 16-key groups: position p holds
//    key p with bits 2 and 3 swapped).
template <typename T>
struct EpiQKV {
  static constexpr bool kBlockSums = true;
  T* out;
  int64_t ldo;
  const float* bias;
  T* vt;
  int vcol0, S, H, hd, Spad;
  const float* gq;
  const float* gk;
  float* ssq;          // [vcol0 / 32, ldp]
  int64_t ldp;         // the product's M
  const float2* rope;  // (cos, sin) table, layout at QKNormRope
  int Hp, Wp, npT, npH, baseH, baseW;
  struct Pre {
    float4 b, g;      // bias, gains
    float2 cs0, cs1;  // (cos, sin) of the pairs (n, n+1), (n+2, n+3)
  };
  __device__ __forceinline__ int rope_entry(int p, const RopePos& t) const {
    return p < npT         ? t.f * npT + p
           : p < npT + npH ? baseH + t.i * npH + (p - npT)
                           : baseW + t.j * npH + (p - npT - npH);
  }
  // Bias, gains and table are read through the constant address space: the compiler then knows the
  // epilogue's stores cannot change them, so a lane's loads of the same column for its two rows (and
  // the row's position decode, outside the region test) merge into one.
  __device__ __forceinline__ Pre pre(int m, int n) const {
    const int dim = vcol0 >> 1;
    Pre p;
    p.b = make_float4(0.f, 0.f, 0.f, 0.f);
    if (bias) p.b = load_const4(bias + n);
    const int c = n < dim ? n : min(n - dim, dim - 4);
    p.g = load_const4((n < dim ? gq : gk) + c);
    const RopePos t = rope_pos(m % S, Hp, Wp);
    const int p0 = (c & (hd - 1)) >> 1;  // channels 2 p0 .. 2 p0 + 3 of one head
    if (n < vcol0) {
      p.cs0 = load_const2(rope + rope_entry(p0, t));
      p.cs1 = load_const2(rope + rope_entry(p0 + 1, t));
    } else {
      p.cs0 = p.cs1 = make_float2(1.f, 0.f);
    }
    return p;
  }
  __device__ __forceinline__ float post(int m, int n, float4 v, const Pre& p) const {
    v.x += p.b.x; v.y += p.b.y; v.z += p.b.z; v.w += p.b.w;
    if (n < vcol0) {
      const float ss = (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
      const float a0 = v.x * p.g.x, b0 = v.y * p.g.y, a1 = v.z * p.g.z, b1 = v.w * p.g.w;
      const float r0 = a0 * p.cs0.x - b0 * p.cs0.y, r1 = a0 * p.cs0.y + b0 * p.cs0.x;
      const float r2 = a1 * p.cs1.x - b1 * p.cs1.y, r3 = a1 * p.cs1.y + b1 * p.cs1.x;
      T* q = out + (int64_t)m * ldo + n;
      if constexpr (sizeof(T) == 2) {
        bf16x4 o;
        o[0] = (bf16)r0; o[1] = (bf16)r1; o[2] = (bf16)r2; o[3] = (bf16)r3;
        *reinterpret_cast<bf16x4*>(q) = o;
      } else {
        *reinterpret_cast<float4*>(q) = make_float4(r0, r1, r2, r3);
      }
      return ss;
    }
    const int nn = n - vcol0, h = nn / hd, d = nn - h * hd;  // 4 channels d..d+3 of head h
    const int b = m / S, pos = m - b * S;
    const int pp = sizeof(T) == 2 ? ((pos & ~12) | ((pos & 4) << 1) | ((pos & 8) >> 1)) : pos;
    T* q = vt + (((int64_t)b * H + h) * hd + d) * Spad + pp;
    q[0] = from_f32<T>(v.x);
    q[Spad] = from_f32<T>(v.y);
    q[2 * (int64_t)Spad] = from_f32<T>(v.z);
    q[3 * (int64_t)Spad] = from_f32<T>(v.w);
    return 0.f;
  }
  // Row m's sum of squares over the 32 columns n0 .. n0 + 31 (n0 a multiple of 32).
  __device__ __forceinline__ void ssq_store(int m, int n0, float sum) const {
    if (n0 < vcol0) ssq[(int64_t)(n0 >> 5) * ldp + m] = sum;
  }
};

struct EpiResidual {
  float* x;
  int64_t ldx;
  const float* bias;
  const float* gate;  // [B, 6, N] or null (gate 1)
  int chunk, S, N;
  float* y = nullptr;  // optional: also record the branch output C + bias (row stride N)
  struct Pre {
    float4 b, r, g;  // bias, residual x, gate
  };
  __device__ __forceinline__ Pre pre(int m, int n) const {
    Pre p;
    p.b = load_bias4(bias, n);
    p.r = *reinterpret_cast<const float4*>(x + (int64_t)m * ldx + n);
    p.g = gate ? *reinterpret_cast<const float4*>(gate + ((int64_t)(m / S) * 6 + chunk) * N + n)
               : make_float4(1.f, 1.f, 1.f, 1.f);
    return p;
  }
  __device__ __forceinline__ void post(int m, int n, float4 v, const Pre& p) const {
    v.x += p.b.x; v.y += p.b.y; v.z += p.b.z; v.w += p.b.w;
    if (y) *reinterpret_cast<float4*>(y + (int64_t)m * N + n) = v;
    float4 r = p.r;
    r.x = fmaf(p.g.x, v.x, r.x); r.y = fmaf(p.g.y, v.y, r.y);
    r.z = fmaf(p.g.z, v.z, r.z); r.w = fmaf(p.g.w, v.w, r.w);
    *reinterpret_cast<float4*>(x + (int64_t)m * ldx + n) = r;
  }
};

// The epilogue of a lane's FM x FN 32 x 32 accumulator blocks: lane row mrow + 32 i, columns
// ncol + 32 j + 8 g + 0..3 (g < 4) in elements 4g..4g+3 of block (i, j).  A block's four groups issue
// all their loads together (clamped coordinates: in range, their values unused where a group is out of
// range), then do their arithmetic and guarded stores, so a lane waits about one memory latency per
// block rather than one per group.  (Issuing the next block's loads before this block's stores as well
// needs a second set of registers and spills.)
// An epilogue with kBlockSums set (the Q/K/V one) returns a float from post and receives, through
// ssq_store, the sum of those values over each 32-column block of a row: lanes l and l + 32 hold the
// row's 32 columns.
template <int FM, int FN, class Epi>
__device__ __forceinline__ void run_epilogue(const Epi& epi, const f32x16 (&acc)[FM][FN], int mrow, int ncol, int M,
                                             int N) {
  constexpr bool kBlockSums = BlockSums<Epi>::value;
#pragma unroll
  for (int q = 0; q < FM * FN; ++q) {
    const int i = q / FN, j = q % FN, m = mrow + i * 32, mc = min(m, M - 1);
    typename Epi::Pre pre[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) pre[g] = epi.pre(mc, min(ncol + j * 32 + g * 8, N - 4));
    float sum = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int n = ncol + j * 32 + g * 8;
      if (m < M && n < N) {
        const float4 v =
            make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
        if constexpr (kBlockSums)
          sum += epi.post(m, n, v, pre[g]);
        else
          epi.post(m, n, v, pre[g]);
      }
    }
    if constexpr (kBlockSums) {
      sum = half_sum(sum);  // every lane of the wave takes part
      if ((threadIdx.x & 32) == 0 && m < M) epi.ssq_store(m, (ncol + j * 32) & ~31, sum);
    }
  }
}

// The epilogue of a lane's FM x FN 16 x 16 accumulator blocks: lane row mrow + 16 i, columns
// ncol + 16 j + 0..3 in block (i, j).  Four blocks of a row issue their loads together, then do their
// arithmetic and guarded stores.
template <int FM, int FN, class Epi>
__device__ __forceinline__ void run_epilogue16(const Epi& epi, const f32x4 (&acc)[FM][FN], int mrow, int ncol, int M,
                                               int N) {
  static_assert(FN % 4 == 0, "groups of four blocks");
#pragma unroll
  for (int q = 0; q < FM * FN / 4; ++q) {
    const int i = q / (FN / 4), j0 = (q % (FN / 4)) * 4, m = mrow + i * 16, mc = min(m, M - 1);
    typename Epi::Pre pre[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) pre[g] = epi.pre(mc, min(ncol + (j0 + g) * 16, N - 4));
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int n = ncol + (j0 + g) * 16;
      const f32x4& a = acc[i][j0 + g];
      if (m < M && n < N) epi.post(m, n, make_float4(a[0], a[1], a[2], a[3]), pre[g]);
    }
  }
}

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

// Row-group size of the tile order (measured on the block's shapes with both operands in K panels):
// long-K products with few column tiles (FFN2) share weights best in groups of 2, products of 16 to
// 31 column tiles (Q/K/V) in groups of 8, the rest (O, cross-q, cross-O; FFN1's 35 column tiles) in
// groups of 4.
inline int group_m(int tiles_n, int K) {
  if (K >= 4096 && tiles_n < 32) return 2;
  return tiles_n >= 16 && tiles_n < 32 ? 8 : 4;
}

template <typename T, int BM, int BN, int WM, int WN, class Epi>
__global__ __launch_bounds__(WM* WN * 64) void gemm_nt_kernel(const T* __restrict__ A, int64_t lda, int64_t apr,
                                                               const T* __restrict__ W, int64_t ldw, int64_t wpr,
                                                               int M, int N, int K, int tiles_m, int tiles_n, int gm,
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
    const int64_t m = min(m0 + r, M - 1);
    pa[i] = apr ? A + ((kc / 32) * apr + m) * 32 + kc % 32 : A + m * lda + kc;  // K step k0 adds k0 * astep
    la[i] = r * ROW + kc;
  }
  const int64_t astep = apr ? apr : 1;
#pragma unroll
  for (int i = 0; i < BC; ++i) {
    const int c = tid + i * NT, r = c >> 3, kc = (c & 7) * E16;
    const int64_t n = min(n0 + r, N - 1);
    pb[i] = wpr ? W + ((kc / 32) * wpr + n) * 32 + kc % 32 : W + n * ldw + kc;  // K step k0 adds k0 * wstep
    lb[i] = BM * ROW + r * ROW + kc;
  }
  const int64_t wstep = wpr ? wpr : 1;

  u32x4 ra[AC], rb[BC];
  auto load_full = [&](int k0) {
#pragma unroll
    for (int i = 0; i < AC; ++i) ra[i] = *reinterpret_cast<const u32x4*>(pa[i] + k0 * astep);
#pragma unroll
    for (int i = 0; i < BC; ++i) rb[i] = *reinterpret_cast<const u32x4*>(pb[i] + k0 * wstep);
  };
  auto load_tail = [&](int k0) {  // last, partial K step: zero-fill k >= K
#pragma unroll
    for (int i = 0; i < AC; ++i) {
      const int kk = k0 + ((tid + i * NT) & 7) * E16;
      ra[i] = kk < K ? *reinterpret_cast<const u32x4*>(pa[i] + k0 * astep) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < BC; ++i) {
      const int kk = k0 + ((tid + i * NT) & 7) * E16;
      rb[i] = kk < K ? *reinterpret_cast<const u32x4*>(pb[i] + k0 * wstep) : u32x4{0, 0, 0, 0};
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
  run_epilogue<FM, FN>(epi, acc, m0 + wm * TM + lrow, n0 + wn * TN + lhalf * 4, M, N);
}

// ---------------------------------------------------------------------------
// bf16 GEMM with asynchronous global -> LDS copies and a ring of ST LDS stages.
//
// One workgroup = WM x WN waves owning a BM x BN tile; a wave owns (BM/WM) x (BN/WN) (the block's
// products use 8 waves of 64 x 128: 8 blocks of 32 x 32 or 32 of 16 x 16, 128 accumulator registers
// either way, two waves per SIMD).
// Each K step of BK elements is copied by direct-to-LDS loads straight into LDS, ST - 1 steps ahead
// of its use, so the copies need no staging registers and have ST - 1 steps of MFMA work to land.
// Row r of a stage holds BK * 2 bytes; its 16-byte chunk c sits at slot c ^ ((r / RPB) % CH) (RPB
// rows share one 256-byte bank window), which makes the 16 rows one ds_read_b128 phase reads hit 16
// distinct bank groups.  The copy instead permutes which global chunk each lane fetches: lanes still
// write LDS linearly.  Requires K % BK == 0 (callers fall back to gemm_nt_kernel otherwise).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt with only the vector-memory counter constrained to <= n (gfx9 encoding).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// M16: the stage is read by 16 x 16 x 32 fragments (lane l: row l % 16 of a 16-row block, chunk l / 16)
// instead of 32 x 32 x 16 ones (lane l: row l % 32, chunk 2 kc + l / 32).  The two read patterns need
// different row swizzles: measured in a read-only loop of each pattern, the 32 x 32
// pattern is conflict-free under slot = c ^ ((r / RPB) % CH) (221 B per clock and CU) where the 16 x 16
// pattern runs 2-way conflicted (121 B); for the 16 x 16 pattern, slot = c ^ (2 bit3(r) + bit1(r)) reads
// 202 B per clock (K steps of 32: four chunks per row).
template <int BM, int BN, int BK, int NW, bool M16 = false>
struct LdsGemmCfg {
  static constexpr int CH = BK / 8;        // 16-byte chunks per row
  static constexpr int RPB = 16 / CH;      // rows per 256-byte bank window
  static constexpr int ROWB = BK * 2;      // bytes per row
  static constexpr int ABYTES = BM * ROWB, BBYTES = BN * ROWB;
  static constexpr int LA = ABYTES / 1024 / NW, LB = BBYTES / 1024 / NW;  // copies per wave per stage
  static_assert(CH >= 1 && CH <= 16 && LA * NW * 1024 == ABYTES && LB * NW * 1024 == BBYTES, "shape");
  static_assert(!M16 || CH == 4, "the 16 x 16 swizzle is for K steps of 32");
  __device__ static __forceinline__ int swz(int r) {
    if constexpr (M16) return ((r >> 2) & 2) | ((r >> 1) & 1);
    return (r / RPB) & (CH - 1);
  }
  __device__ static __forceinline__ int off(int r, int c) { return r * ROWB + ((c ^ swz(r)) << 4); }
};

// The copies go through buffer resources (the MUBUF form of the direct-to-LDS load: lane i writes its
// 16 bytes at lds + 16 i).  The compiler counts them as plain vector-memory loads, so the fragment
// reads of a step wait only for their own results; with the FLAT form in flight every LDS read would
// wait for all outstanding LDS accesses.  Each operand tile has one wave-uniform base (its first row)
// and a record count (the bytes from there to the end of its panels); each lane a 32-bit byte offset
// (row, permuted chunk) that is the same for every tile; the K step sets the scalar offset.  Both
// operands are in K panels of 32 elements (see KMat): the stage of a 256-row tile is one contiguous
// run, 16 KB of bf16 or two runs of 8 KB of E4M3 codes (the two panels of a 64-code step), so every
// copy instruction reads whole 128-byte lines.  In a lab loop on the block's shapes this made the
// products 6-12 % faster than 64-byte segments of row-major operands.  The panels hold the rows
// rounded up to 256 (weights: zero past N; activations: unstored rows past M), so a tile's rows all
// exist.
__device__ __forceinline__ void buffer_copy16(const void* base, uint32_t records, uint32_t voff, uint32_t soff,
                                              char* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)records, 0x00020000),
      (lds_void*)lds, 16, voff, soff, 0, 0);
}

// Where one output tile's operands start: A's row m0 and W's row n0, with their record counts.
struct LdsTileSrc {
  const bf16* ba;
  const bf16* bb;
  uint32_t na, nb;
};

// F8: the operands are E4M3 codes (a K step of BK bf16 units = 2 BK codes = two W panels).
template <int BM, int BN, int BK, int NW, bool M16, bool F8>
struct LdsCopyPlan {
  using C = LdsGemmCfg<BM, BN, BK, NW, M16>;
  static_assert(BK == 32, "one W panel (bf16) or two (E4M3) per K step");
  uint32_t oa[C::LA];
  uint32_t ob[C::LB];
  uint32_t astage, wstage;  // bytes between consecutive K steps of A and W: 64 * panel rows
  __device__ static __forceinline__ const bf16* uniform(const bf16* p) {
    const uint64_t a = (uint64_t)p;
    return (const bf16*)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a));
  }
  // Byte offset of LDS chunk p's source in a tile's panels (pr rows each): row r = p / CH, global chunk
  // c = slot ^ swizzle; bf16: chunk c of row r's 64-byte panel row; E4M3: chunk c % 2 of row r's
  // 32-byte row in panel c / 2.
  __device__ static __forceinline__ uint32_t chunk_offset(int p, int64_t pr) {
    const int r = p / C::CH, c = (p % C::CH) ^ C::swz(r);
    return F8 ? (uint32_t)((c >> 1) * 32 * pr + r * 32 + (c & 1) * 16) : (uint32_t)(r * 64 + c * 16);
  }
  // apr, wpr: rows per A and W panel (M and N rounded up to 256); the panels of each operand stay below
  // 2^31 bytes.
  __device__ __forceinline__ LdsCopyPlan(int64_t apr, int64_t wpr)
      : astage((uint32_t)(64 * apr)), wstage((uint32_t)(64 * wpr)) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < C::LA; ++i) oa[i] = chunk_offset((i * NW + wave) * 64 + lane, apr);
#pragma unroll
    for (int i = 0; i < C::LB; ++i) ob[i] = chunk_offset((i * NW + wave) * 64 + lane, wpr);
  }
  // Records of the bytes from a tile's first row r0 of panel 0 to the end of the panels (2 K pr bytes
  // with K in bf16 units).
  __device__ static __forceinline__ uint32_t records(int K, int64_t pr, int r0) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(2 * (int64_t)K * pr - (int64_t)r0 * (F8 ? 32 : 64)));
  }
  // K: the product depth in bf16 units.  Row r0 of panel 0 sits r0 * (F8 ? 32 : 64) bytes in.
  __device__ static __forceinline__ LdsTileSrc tile(const bf16* A, int64_t apr, const bf16* W, int64_t wpr, int K,
                                                    int m0, int n0) {
    return LdsTileSrc{uniform(A + (int64_t)m0 * (F8 ? 16 : 32)), uniform(W + (int64_t)n0 * (F8 ? 16 : 32)),
                      records(K, apr, m0), records(K, wpr, n0)};
  }
  __device__ __forceinline__ void issue(const LdsTileSrc& t, int k0, char* sa, char* sb) const {
    const int wave = threadIdx.x >> 6;
    const uint32_t as = (uint32_t)(k0 / BK) * astage;
#pragma unroll
    for (int i = 0; i < C::LA; ++i) buffer_copy16(t.ba, t.na, oa[i], as, sa + (i * NW + wave) * 1024);
    const uint32_t ws = (uint32_t)(k0 / BK) * wstage;
#pragma unroll
    for (int i = 0; i < C::LB; ++i) buffer_copy16(t.bb, t.nb, ob[i], ws, sb + (i * NW + wave) * 1024);
  }
};

// Accumulators of one wave: 32 x 32 blocks (v_mfma_f32_32x32x16_bf16, or the E4M3
// v_mfma_scale_f32_32x32x64_f8f6f4), or 16 x 16 blocks (v_mfma_f32_16x16x32_bf16, which sustains ~12 %
// more than the 32 x 32 x 16 form on gfx950 in a register-only loop).
template <int TM, int TN, bool M16>
struct LdsAcc {
  using type = f32x16[TM / 32][TN / 32];
};
template <int TM, int TN>
struct LdsAcc<TM, TN, true> {
  using type = f32x4[TM / 16][TN / 16];
};

template <int BM, int BN, int BK, int ST, int WM, int WN>
struct LdsSlots {
  char* a[4];
  char* b[4];
};

// One K step kt with static ring slot P = kt % ST.  The K loop runs a multiple of ST steps and
// always refills the freed slot: past the last stage with the next tile's first stages (tile source
// nxt), or, after a workgroup's last tile, with this tile's first stages again (never read).  So the
// body is straight-line code with a constant wait count: at the start of step kt at least ST - 2
// later stages' copies were issued after stage kt's (other vector-memory operations issued in
// between only make the wait stricter).
//
// F8: the operands are E4M3 codes.  A row of 2 BK codes occupies the bytes of BK bf16 elements, so
// the copies and the LDS layout are unchanged; each K step is then one
// v_mfma_scale_f32_32x32x64_f8f6f4 per output block (unit block scales) on 32-byte fragments
// (lane half h reads 16-byte chunks 2h and 2h + 1 of its row, the same k for A and W).
// M16 (bf16 only): 16 x 16 x 32 products on 16 x 16 accumulator blocks instead of 32 x 32 x 16 ones.
template <int BM, int BN, int BK, int ST, int WM, int WN, int P, bool F8, bool M16>
__device__ __forceinline__ void lds_gemm_step(const LdsCopyPlan<BM, BN, BK, WM * WN, M16, F8>& cp, const LdsTileSrc& cur,
                                              const LdsTileSrc& nxt, const LdsSlots<BM, BN, BK, ST, WM, WN>& sl,
                                              int kt, int nk,
                                              typename LdsAcc<BM / WM, BN / WN, M16>::type& acc) {
  using C = LdsGemmCfg<BM, BN, BK, WM * WN, M16>;
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
  auto refill = [&]() {
    if (kn < nk)
      cp.issue(cur, kn * BK, sl.a[Q], sl.b[Q]);
    else
      cp.issue(nxt, (kn - nk) * BK, sl.a[Q], sl.b[Q]);
  };
  if constexpr (ST == 2) refill();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, lrow = lane & 31, lhalf = lane >> 5;
  const int wm = wave / WN, wn = wave % WN;
  const char* sa = sl.a[P];
  const char* sb = sl.b[P];
  static_assert(!(F8 && M16), "E4M3 products use 32 x 32 blocks");
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
    if constexpr (ST > 2) refill();
    return;
  }
  if constexpr (M16) {
    // 16 x 16 x 32 products: lane l reads row l % 16 of a 16-row block, 16-byte chunk l / 16 of the
    // 32-deep k-chunk (k = 8 (l / 16) .. +7), for both operands; 16 rows of one chunk fill the 64
    // banks once under the row swizzle.
    constexpr int FM16 = BM / WM / 16, FN16 = BN / WN / 16;
    const int l16 = lane & 15, lq = lane >> 4;
#pragma unroll
    for (int kc = 0; kc < BK / 32; ++kc) {
      u32x4 af[FM16], bfr[FN16];
#pragma unroll
      for (int i = 0; i < FM16; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(sa + C::off(wm * (BM / WM) + i * 16 + l16, kc * 4 + lq));
#pragma unroll
      for (int j = 0; j < FN16; ++j)
        bfr[j] = *reinterpret_cast<const u32x4*>(sb + C::off(wn * (BN / WN) + j * 16 + l16, kc * 4 + lq));
#pragma unroll
      for (int i = 0; i < FM16; ++i)
#pragma unroll
        for (int j = 0; j < FN16; ++j)  // C^T = W A^T
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bfr[j]),
                                                              __builtin_bit_cast(bf16x8, af[i]), acc[i][j], 0, 0, 0);
    }
  } else {
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
  }
  if constexpr (ST > 2) refill();
}

template <int BM, int BN, int BK, int ST, int WM, int WN, class Epi, bool F8, bool M16, bool PERSIST>
__global__ __launch_bounds__(WM* WN * 64) void gemm_lds_kernel(const bf16* __restrict__ A, int64_t apr,
                                                                const bf16* __restrict__ W, int64_t wpr, int M,
                                                                int N, int K, int tiles_m, int tiles_n, int gm,
                                                               Epi epi) {
  constexpr int NW = WM * WN;
  using C = LdsGemmCfg<BM, BN, BK, NW, M16>;
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
  // A fixed grid walks the tiles blockIdx.x, blockIdx.x + gridDim.x, ...  The last ST - 1 refills of a
  // tile's K loop copy the first stages of the next tile (slot s for stage s, as nk is a multiple of
  // ST), so those copies land while this tile's epilogue runs.  The epilogue touches no LDS.
  const int ntiles = tiles_m * tiles_n;
  int id = blockIdx.x, tm, tn;
  tile_coords(id, tiles_m, tiles_n, gm, tm, tn);
  using Plan = LdsCopyPlan<BM, BN, BK, NW, M16, F8>;
  const Plan cp(apr, wpr);
  LdsTileSrc cur = Plan::tile(A, apr, W, wpr, K, tm * BM, tn * BN);
  const int nk = K / BK;  // a multiple of ST
#pragma unroll
  for (int s = 0; s < ST - 1; ++s) cp.issue(cur, s * BK, sl.a[s], sl.b[s]);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, lrow = lane & 31, lhalf = lane >> 5;
  const int wm = wave / WN, wn = wave % WN;

  for (;;) {
    const int m0 = tm * BM, n0 = tn * BN, next = PERSIST ? id + (int)gridDim.x : ntiles;
    int tm2 = tm, tn2 = tn;
    LdsTileSrc nxt = cur;  // past the last tile the surplus refills re-copy this tile's stages (never read)
    if (next < ntiles) {
      tile_coords(next, tiles_m, tiles_n, gm, tm2, tn2);
      nxt = Plan::tile(A, apr, W, wpr, K, tm2 * BM, tn2 * BN);
    }

    typename LdsAcc<BM / WM, BN / WN, M16>::type acc;
    if constexpr (M16) {
#pragma unroll
      for (int i = 0; i < FM * 2; ++i)
#pragma unroll
        for (int j = 0; j < FN * 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = zero16();
    }
    for (int kt = 0; kt < nk; kt += ST) {
      lds_gemm_step<BM, BN, BK, ST, WM, WN, 0, F8, M16>(cp, cur, nxt, sl, kt, nk, acc);
      lds_gemm_step<BM, BN, BK, ST, WM, WN, 1, F8, M16>(cp, cur, nxt, sl, kt + 1, nk, acc);
      if constexpr (ST > 2) lds_gemm_step<BM, BN, BK, ST, WM, WN, 2 % ST, F8, M16>(cp, cur, nxt, sl, kt + 2, nk, acc);
      if constexpr (ST > 3) lds_gemm_step<BM, BN, BK, ST, WM, WN, 3 % ST, F8, M16>(cp, cur, nxt, sl, kt + 3, nk, acc);
    }
    if constexpr (M16)
      run_epilogue16<FM * 2, FN * 2>(epi, acc, m0 + wm * (BM / WM) + (lane & 15),
                                     n0 + wn * (BN / WN) + (lane >> 4) * 4, M, N);
    else
      run_epilogue<FM, FN>(epi, acc, m0 + wm * (BM / WM) + lrow, n0 + wn * (BN / WN) + lhalf * 4, M, N);
    if (next >= ntiles) break;
    id = next;
    tm = tm2;
    tn = tn2;
    cur = nxt;
  }
  wait_vmcnt<0>();  // the surplus copies past the last stage land before the LDS is released
}

// Which bf16 products take 16 x 16 x 32 MFMAs: the store and residual epilogues.  The Q/K/V epilogue keeps
// 32 x 32 blocks, whose 32 consecutive tokens per lane group write 64-byte runs of the transposed V.
template <class Epi>
struct UseMfma16 {
  static constexpr bool value = true;
};
template <typename OutT>
struct UseMfma16<EpiQKV<OutT>> {
  static constexpr bool value = false;
};

// Which products walk their tiles with a fixed grid: the plain-store ones (bf16 and E4M3).  Measured
// in the block against one workgroup per tile: FFN1 2 % and the cross-attention q product 1.5 % faster;
// the residual products gained nothing (FFN2 1 % slower) and the Q/K/V epilogue has no registers to
// spare for a second tile's state.
template <class Epi>
struct EpiScaled;
template <class Epi>
struct UsePersistent {
  static constexpr bool value = false;
};
template <typename OutT, int ACT>
struct UsePersistent<EpiStore<OutT, ACT>> {
  static constexpr bool value = true;
};
template <typename OutT, int ACT>
struct UsePersistent<EpiScaled<EpiStore<OutT, ACT>>> {
  static constexpr bool value = true;
};

template <int BM, int BN, int BK, int ST, int WM, int WN, class Epi, bool F8 = false>
hipError_t launch_lds(const bf16* A, int64_t apr, const bf16* W, int64_t wpr, int M, int N, int K, const Epi& epi,
                      hipStream_t s) {
  const int tm = (int)ceil_div(M, BM), tn = (int)ceil_div(N, BN);
  constexpr bool M16 = !F8 && UseMfma16<Epi>::value;
  constexpr bool PERSIST = UsePersistent<Epi>::value;
  // One workgroup per compute unit: the ring takes ST * (BM + BN) * BK * 2 bytes of LDS.
  static_assert(2 * ST * (BM + BN) * BK * 2 > 160 * 1024, "the persistent grid assumes one workgroup per CU");
  const int64_t ntiles = (int64_t)tm * tn;
  const int grid = PERSIST ? (int)std::min<int64_t>(ntiles, device_compute_units()) : (int)ntiles;
  hipLaunchKernelGGL((gemm_lds_kernel<BM, BN, BK, ST, WM, WN, Epi, F8, M16, PERSIST>), dim3((unsigned)grid),
                     dim3(WM * WN * 64), 0, s, A, apr, W, wpr, M, N, K, tm, tn, group_m(tn, K), epi);
  return hipGetLastError();
}

// Epilogue wrapper of the E4M3 products: the accumulator times (row scale * tensor scale), then the
// wrapped epilogue.
template <class Epi>
struct EpiScaled {
  static constexpr bool kBlockSums = BlockSums<Epi>::value;
  const float* row_scale;
  const float* w_scale;  // one value, on the device
  Epi inner;
  struct Pre {
    float sc;
    typename Epi::Pre in;
  };
  __device__ __forceinline__ Pre pre(int m, int n) const { return Pre{row_scale[m] * *w_scale, inner.pre(m, n)}; }
  __device__ __forceinline__ auto post(int m, int n, float4 v, const Pre& p) const {
    v.x *= p.sc; v.y *= p.sc; v.z *= p.sc; v.w *= p.sc;
    return inner.post(m, n, v, p.in);
  }
  __device__ __forceinline__ void ssq_store(int m, int n0, float sum) const { inner.ssq_store(m, n0, sum); }
};

// E4M3 product ("Wan 技术深度解析" §5.3: per-token activation, per-tensor weight scales): A codes [M, K]
// with per-row scales and W codes [N, K] with one tensor scale, both in K panels (see KMat).  K a
// multiple of 256; each operand's panels below 2^31 bytes.
template <class Epi>
hipError_t run_gemm_e4m3(KMat<uint8_t> A, const float* a_scales, KMat<uint8_t> W, const float* w_scale, int M, int N,
                         int K, const Epi& epi, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (N % 4 != 0 || K % 256 != 0 || !k_panels_ok(A, M, K) || !k_panels_ok(W, N, K) ||
      (int64_t)K * A.panel >= ((int64_t)1 << 31) || (int64_t)K * W.panel >= ((int64_t)1 << 31))
    return hipErrorInvalidValue;
  return launch_lds<256, 256, 32, 4, 4, 2, EpiScaled<Epi>, true>(
      reinterpret_cast<const bf16*>(A.p), A.panel, reinterpret_cast<const bf16*>(W.p), W.panel, M, N, K / 2,
      EpiScaled<Epi>{a_scales, w_scale, epi}, s);
}

template <typename T, int BM, int BN, int WM, int WN, class Epi>
hipError_t launch_cfg(KMat<T> A, KMat<T> W, int M, int N, int K, const Epi& epi, hipStream_t s) {
  const int tm = (int)ceil_div(M, BM), tn = (int)ceil_div(N, BN);
  hipLaunchKernelGGL((gemm_nt_kernel<T, BM, BN, WM, WN, Epi>), dim3((unsigned)(tm * tn)), dim3(WM * WN * 64), 0,
                     s, A.p, A.ld, A.panel, W.p, W.ld, W.panel, M, N, K, tm, tn, group_m(tn, K), epi);
  return hipGetLastError();
}

// Tile choice.  bf16 products with many rows, K a multiple of 128 and both operands in K panels use
// the asynchronous-copy kernel (256 x 256 tiles, 8 waves of 64 x 128, BK 32, four LDS stages); other
// bf16 products with many rows use the register-staged kernel with 256-row tiles; small products and
// fp32 use 128 x 128.  The register-staged kernel reads either layout.
template <typename T, class Epi>
hipError_t run_gemm(KMat<T> A, KMat<T> W, int M, int N, int K, const Epi& epi, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (N % 4 != 0 || K % dtype_traits<T>::per16 != 0) return hipErrorInvalidValue;
  if (A.panel ? !k_panels_ok(A, M, K) : A.ld % dtype_traits<T>::per16 != 0) return hipErrorInvalidValue;
  if (W.panel ? !k_panels_ok(W, N, K) : W.ld % dtype_traits<T>::per16 != 0) return hipErrorInvalidValue;
  if constexpr (sizeof(T) == 2) {
    int cfg = 0;
    // (the asynchronous-copy kernel addresses the panels with 32-bit byte offsets)
    if (A.panel && W.panel && M >= 4096 && N >= 1024 && K % 128 == 0 &&
        (int64_t)2 * K * A.panel < ((int64_t)1 << 31) && (int64_t)2 * K * W.panel < ((int64_t)1 << 31))
      cfg = 1;
    else if (M >= 4096 && N % 256 == 0 && N >= 1024) cfg = 2;
    else if (M >= 4096 && N % 128 == 0 && N >= 1024) cfg = 3;
    if (cfg == 1) return launch_lds<256, 256, 32, 4, 4, 2>(A.p, A.panel, W.p, W.panel, M, N, K, epi, s);
    if (cfg == 2) return launch_cfg<T, 256, 256, 4, 2>(A, W, M, N, K, epi, s);
    if (cfg == 3) return launch_cfg<T, 256, 128, 4, 2>(A, W, M, N, K, epi, s);
  }
  return launch_cfg<T, 128, 128, 2, 2>(A, W, M, N, K, epi, s);
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

int device_compute_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

template <typename T, typename OutT>
hipError_t gemm_store(KMat<T> A, KMat<T> W, int M, int N, int K, const float* bias, int act, OutT* out, ActLayout lo,
                      hipStream_t s) {
  if (lo.bs != 32 && N % 32 != 0) return hipErrorInvalidValue;
  if (act == ACT_GELU) return run_gemm<T>(A, W, M, N, K, EpiStore<OutT, ACT_GELU>{out, lo.ld, lo.bs, bias}, s);
  if (act == ACT_SILU) return run_gemm<T>(A, W, M, N, K, EpiStore<OutT, ACT_SILU>{out, lo.ld, lo.bs, bias}, s);
  return run_gemm<T>(A, W, M, N, K, EpiStore<OutT, ACT_NONE>{out, lo.ld, lo.bs, bias}, s);
}

namespace {

template <typename T>
EpiQKV<T> make_epi_qkv(T* qk, int64_t ldo, const float* bias, T* vt, int M, int dim, int S, int H, int hd, int Spad,
                       const QKNormRope& nr) {
  const int npT = rope_pairs_time(hd), npH = rope_pairs_space(hd);
  const int baseH = nr.T * npT, baseW = baseH + nr.Hp * npH;
  return EpiQKV<T>{qk, ldo, bias, vt, 2 * dim, S, H, hd, Spad, nr.gq, nr.gk, nr.ssq, M, nr.rope, nr.Hp, nr.Wp, npT,
                   npH, baseH, baseW};
}

bool qkv_args_ok(int M, int dim, int S, int hd, const QKNormRope& nr) {
  return hd >= 4 && (hd & (hd - 1)) == 0 && dim % 32 == 0 && dim % hd == 0 && nr.gq && nr.gk && nr.ssq && nr.rope &&
         nr.T > 0 && nr.Hp > 0 && nr.Wp > 0 && (int64_t)nr.T * nr.Hp * nr.Wp == S && M % S == 0;
}

}  // namespace

template <typename T>
hipError_t gemm_qkv(KMat<T> A, KMat<T> W, int M, int dim, int K, const float* bias,
                    T* qk, int64_t ldo, T* vt, int S, int H, int hd, int Spad, const QKNormRope& nr, hipStream_t s) {
  if (!qkv_args_ok(M, dim, S, hd, nr)) return hipErrorInvalidValue;
  return run_gemm<T>(A, W, M, 3 * dim, K, make_epi_qkv<T>(qk, ldo, bias, vt, M, dim, S, H, hd, Spad, nr), s);
}

template <typename T>
hipError_t gemm_residual(KMat<T> A, KMat<T> W, int M, int N, int K, const float* bias,
                         const float* gate, int chunk, int S, float* x, int64_t ldx, hipStream_t s, float* ystore) {
  EpiResidual epi{x, ldx, bias, gate, chunk, S, N, ystore};
  return run_gemm<T>(A, W, M, N, K, epi, s);
}

hipError_t gemm_e4m3_store(KMat<uint8_t> A, const float* a_scales, KMat<uint8_t> W, const float* w_scale, int M,
                           int N, int K, const float* bias, int act, bf16* out, ActLayout lo, hipStream_t s) {
  if (lo.bs != 32 && N % 32 != 0) return hipErrorInvalidValue;
  if (act == ACT_GELU)
    return run_gemm_e4m3(A, a_scales, W, w_scale, M, N, K, EpiStore<bf16, ACT_GELU>{out, lo.ld, lo.bs, bias}, s);
  return run_gemm_e4m3(A, a_scales, W, w_scale, M, N, K, EpiStore<bf16, ACT_NONE>{out, lo.ld, lo.bs, bias}, s);
}

hipError_t gemm_qkv_e4m3(KMat<uint8_t> A, const float* a_scales, KMat<uint8_t> W,
                         const float* w_scale, int M, int dim, int K, const float* bias, bf16* qk, int64_t ldo, bf16* vt,
                         int S, int H, int hd, int Spad, const QKNormRope& nr, hipStream_t s) {
  if (!qkv_args_ok(M, dim, S, hd, nr)) return hipErrorInvalidValue;
  return run_gemm_e4m3(A, a_scales, W, w_scale, M, 3 * dim, K,
                       make_epi_qkv<bf16>(qk, ldo, bias, vt, M, dim, S, H, hd, Spad, nr), s);
}

hipError_t gemm_e4m3_residual(KMat<uint8_t> A, const float* a_scales, KMat<uint8_t> W,
                              const float* w_scale, int M, int N, int K, const float* bias, const float* gate,
                              int chunk, int S, float* x, int64_t ldx, hipStream_t s, float* ystore) {
  return run_gemm_e4m3(A, a_scales, W, w_scale, M, N, K, EpiResidual{x, ldx, bias, gate, chunk, S, N, ystore},
                       s);
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

template hipError_t gemm_store<float, float>(KMat<float>, KMat<float>, int, int, int, const float*, int, float*,
                                             ActLayout, hipStream_t);
template hipError_t gemm_store<bf16, bf16>(KMat<bf16>, KMat<bf16>, int, int, int, const float*, int, bf16*, ActLayout,
                                           hipStream_t);
template hipError_t gemm_store<bf16, float>(KMat<bf16>, KMat<bf16>, int, int, int, const float*, int, float*,
                                            ActLayout, hipStream_t);
template hipError_t gemm_qkv<float>(KMat<float>, KMat<float>, int, int, int, const float*, float*, int64_t, float*,
                                    int, int, int, int, const QKNormRope&, hipStream_t);
template hipError_t gemm_qkv<bf16>(KMat<bf16>, KMat<bf16>, int, int, int, const float*, bf16*, int64_t, bf16*, int,
                                   int, int, int, const QKNormRope&, hipStream_t);
template hipError_t gemm_residual<float>(KMat<float>, KMat<float>, int, int, int, const float*, const float*, int,
                                         int, float*, int64_t, hipStream_t, float*);
template hipError_t gemm_residual<bf16>(KMat<bf16>, KMat<bf16>, int, int, int, const float*, const float*, int, int,
                                        float*, int64_t, hipStream_t, float*);
template hipError_t gemv<float>(const float*, int, int, const float*, int, const float*, int, int, float*,
                                hipStream_t);
template hipError_t gemv<bf16>(const bf16*, int, int, const float*, int, const float*, int, int, float*,
                               hipStream_t);

}  // namespace wan
