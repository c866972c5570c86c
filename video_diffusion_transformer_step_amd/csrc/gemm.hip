// MFMA GEMMs for the DiT block's linear layers (patch embedding, Q/K/V, O,
// cross-attention q/o and K/V, FFN, head, context MLPs) and a small GEMV for the
// timestep MLP.
//
// Every linear layer computes y = x W^T + b with W stored [out, in] ("图解 Wan2.1
// I2V" §5.3-§5.5 and the Conv3d patch embedding of §5.1), so both operands are
// contiguous along K (an "NT" product).  One workgroup owns a BM x BN output tile;
// K advances 128 bytes at a time (64 bf16 or 32 fp32), staged through
// double-buffered LDS with register prefetch of the next K tile.  Each wave
// computes a (BM/WM) x (BN/WN) sub-tile with 32x32 MFMA blocks.  Epilogues fuse
// the bias, GELU / SiLU, the fp32 store and the adaLN-gated residual update
// x += gate * (.) ("图解 Wan2.1 I2V" §5.2).
#include "wan_internal.h"

namespace wan {

namespace {

__device__ __forceinline__ float apply_act(float v, int act) {
  if (act == ACT_GELU) return 0.5f * v * (1.f + erff(v * 0.70710678118654752f));
  if (act == ACT_SILU) return v / (1.f + __expf(-v));
  return v;
}

template <typename OutT>
struct EpiStore {
  OutT* out;
  int64_t ldo;
  const float* bias;
  int act;
  __device__ __forceinline__ void operator()(int m, int n, float v) const {
    if (bias) v += bias[n];
    v = apply_act(v, act);
    out[(int64_t)m * ldo + n] = from_f32<OutT>(v);
  }
};

struct EpiResidual {
  float* x;
  int64_t ldx;
  const float* bias;
  const float* e0;  // [B, 6, N] or null (gate 1)
  const float* mb;  // [6, N]
  int chunk, S, N;
  __device__ __forceinline__ void operator()(int m, int n, float v) const {
    if (bias) v += bias[n];
    float g = 1.f;
    if (e0) {
      const int b = m / S;
      g = e0[((int64_t)b * 6 + chunk) * N + n] + mb[(int64_t)chunk * N + n];
    }
    float* p = x + (int64_t)m * ldx + n;
    *p = *p + g * v;
  }
};

// BM x BN tile, WM x WN waves.  BK = 128 bytes of K.
template <typename T, int BM, int BN, int WM, int WN, class Epi>
__global__ __launch_bounds__(WM* WN * 64) void gemm_nt_kernel(const T* __restrict__ A, int64_t lda,
                                                               const T* __restrict__ W, int64_t ldw, int M,
                                                               int N, int K, Epi epi) {
  constexpr int NT = WM * WN * 64;
  constexpr int E16 = dtype_traits<T>::per16;  // elements per 16 bytes
  constexpr int BK = 8 * E16;                  // 128 bytes
  constexpr int ROW = BK + E16;                // padded LDS row (144 bytes): conflict-free 16 B reads
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int AC = BM * 8 / NT, BC = BN * 8 / NT;  // 16-byte chunks per thread
  static_assert(AC * NT == BM * 8 && BC * NT == BN * 8, "tile / thread mismatch");
  __shared__ u32x4 smem_raw[2 * (BM + BN) * ROW * sizeof(T) / 16];
  T* smem = reinterpret_cast<T*>(smem_raw);

  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  u32x4 ra[AC], rb[BC];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < AC; ++i) {
      const int c = tid + i * NT, r = c >> 3, kk = k0 + (c & 7) * E16;
      const int gm = m0 + r;
      if (gm < M && kk < K)
        ra[i] = *reinterpret_cast<const u32x4*>(A + (int64_t)gm * lda + kk);
      else
        ra[i] = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < BC; ++i) {
      const int c = tid + i * NT, r = c >> 3, kk = k0 + (c & 7) * E16;
      const int gn = n0 + r;
      if (gn < N && kk < K)
        rb[i] = *reinterpret_cast<const u32x4*>(W + (int64_t)gn * ldw + kk);
      else
        rb[i] = u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int buf) {
    T* sa = smem + buf * (BM + BN) * ROW;
    T* sb = sa + BM * ROW;
#pragma unroll
    for (int i = 0; i < AC; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<u32x4*>(sa + (c >> 3) * ROW + (c & 7) * E16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < BC; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<u32x4*>(sb + (c >> 3) * ROW + (c & 7) * E16) = rb[i];
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = zero16();

  const int nk = (K + BK - 1) / BK;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  const int lrow = lane & 31, lhalf = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tile((kt + 1) * BK);
    const T* sa = smem + buf * (BM + BN) * ROW + (wm * TM + lrow) * ROW + lhalf * E16;
    const T* sb = smem + buf * (BM + BN) * ROW + BM * ROW + (wn * TN + lrow) * ROW + lhalf * E16;
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
        for (int j = 0; j < FN; ++j) mfma_chunk(af[i], bfr[j], acc[i][j], T());
    }
    if (kt + 1 < nk) store_tile(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * TM + i * 32 + (r >> 2) * 8 + lhalf * 4 + (r & 3);
        const int n = n0 + wn * TN + j * 32 + lrow;
        if (m < M && n < N) epi(m, n, acc[i][j][r]);
      }
}

template <typename T, class Epi>
hipError_t run_gemm(const T* A, int64_t lda, const T* W, int64_t ldw, int M, int N, int K, const Epi& epi,
                    hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  constexpr int BM = 128, BN = 128;
  dim3 grid((unsigned)ceil_div(N, BN), (unsigned)ceil_div(M, BM));
  hipLaunchKernelGGL((gemm_nt_kernel<T, BM, BN, 2, 2, Epi>), grid, dim3(256), 0, s, A, lda, W, ldw, M, N, K, epi);
  return hipGetLastError();
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
  EpiStore<OutT> epi{out, ldo, bias, act};
  return run_gemm<T>(A, lda, W, ldw, M, N, K, epi, s);
}

template <typename T>
hipError_t gemm_residual(const T* A, int64_t lda, const T* W, int64_t ldw, int M, int N, int K, const float* bias,
                         const float* e0, const float* mb, int chunk, int S, float* x, int64_t ldx, hipStream_t s) {
  EpiResidual epi{x, ldx, bias, e0, mb, chunk, S, N};
  return run_gemm<T>(A, lda, W, ldw, M, N, K, epi, s);
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
template hipError_t gemm_residual<float>(const float*, int64_t, const float*, int64_t, int, int, int, const float*,
                                         const float*, const float*, int, int, float*, int64_t, hipStream_t);
template hipError_t gemm_residual<bf16>(const bf16*, int64_t, const bf16*, int64_t, int, int, int, const float*,
                                        const float*, const float*, int, int, float*, int64_t, hipStream_t);
template hipError_t gemv<float>(const float*, int, int, const float*, int, const float*, int, int, float*,
                                hipStream_t);
template hipError_t gemv<bf16>(const bf16*, int, int, const float*, int, const float*, int, int, float*,
                               hipStream_t);

}  // namespace wan
