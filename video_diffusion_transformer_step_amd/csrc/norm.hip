// Row-wise normalisation kernels (HBM-bound): LayerNorm + adaLN modulation,
// affine LayerNorm, the head's modulated LayerNorm, and the Q/K RMSNorm + gain +
// 3D RoPE pass.  One 64-lane wave owns one token row; the row stays in registers
// between the statistics and the write.
#include "wan_internal.h"

namespace wan {

namespace {

constexpr int LN_MAX4 = 24;  // float4 chunks per lane: dim <= 24 * 256 = 6144

template <typename T> __device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
template <> __device__ __forceinline__ void store4<bf16>(bf16* p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (bf16)a;
  v[1] = (bf16)b;
  v[2] = (bf16)c;
  v[3] = (bf16)d;
  *reinterpret_cast<bf16x4*>(p) = v;
}

// LayerNorm (biased variance, no affine) then modulation; see launch_ln_mod in wan_internal.h.
// "图解 Wan2.1 I2V" §5.2: x' = norm(x) * (1 + scale) + shift; the cross-attention pre-norm (mode 1)
// and the head (mode 2, §5.5) reuse the same row statistics.
template <typename T>
__global__ __launch_bounds__(256) void ln_mod_kernel(const float* __restrict__ x, int64_t rows, int dim, int S,
                                                      int mode, const float* __restrict__ p0,
                                                      const float* __restrict__ p1, int c_shift, int c_scale,
                                                      float eps, T* __restrict__ u) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int n4 = dim >> 2;
  const float4* xr = reinterpret_cast<const float4*>(x + row * dim);
  float4 v[LN_MAX4];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < LN_MAX4; ++i) {
    const int idx = i * 64 + lane;
    if (idx < n4) {
      v[i] = xr[idx];
      sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    }
  }
  const float mean = wave_sum(sum) / (float)dim;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < LN_MAX4; ++i) {
    const int idx = i * 64 + lane;
    if (idx < n4) {
      const float a = v[i].x - mean, b = v[i].y - mean, c = v[i].z - mean, d = v[i].w - mean;
      sq += (a * a + b * b) + (c * c + d * d);
    }
  }
  const float rstd = 1.f / sqrtf(wave_sum(sq) / (float)dim + eps);
  const int64_t b = row / S;
  T* ur = u + row * dim;
#pragma unroll
  for (int i = 0; i < LN_MAX4; ++i) {
    const int idx = i * 64 + lane;
    if (idx < n4) {
      const int c = idx * 4;
      float n0 = (v[i].x - mean) * rstd, n1 = (v[i].y - mean) * rstd;
      float n2 = (v[i].z - mean) * rstd, n3 = (v[i].w - mean) * rstd;
      float4 sh, sc;
      if (mode == 0) {
        const float4 es = *reinterpret_cast<const float4*>(p0 + (b * 6 + c_shift) * dim + c);
        const float4 ms = *reinterpret_cast<const float4*>(p1 + (int64_t)c_shift * dim + c);
        const float4 ec = *reinterpret_cast<const float4*>(p0 + (b * 6 + c_scale) * dim + c);
        const float4 mc = *reinterpret_cast<const float4*>(p1 + (int64_t)c_scale * dim + c);
        sh = make_float4(es.x + ms.x, es.y + ms.y, es.z + ms.z, es.w + ms.w);
        sc = make_float4(1.f + (ec.x + mc.x), 1.f + (ec.y + mc.y), 1.f + (ec.z + mc.z), 1.f + (ec.w + mc.w));
      } else if (mode == 1) {
        sc = *reinterpret_cast<const float4*>(p0 + c);
        sh = *reinterpret_cast<const float4*>(p1 + c);
      } else {
        const float4 h0 = *reinterpret_cast<const float4*>(p0 + c);
        const float4 h1 = *reinterpret_cast<const float4*>(p0 + dim + c);
        const float4 e = *reinterpret_cast<const float4*>(p1 + b * dim + c);
        sh = make_float4(h0.x + e.x, h0.y + e.y, h0.z + e.z, h0.w + e.w);
        sc = make_float4(1.f + (h1.x + e.x), 1.f + (h1.y + e.y), 1.f + (h1.z + e.z), 1.f + (h1.w + e.w));
      }
      store4<T>(ur + c, fmaf(n0, sc.x, sh.x), fmaf(n1, sc.y, sh.y), fmaf(n2, sc.z, sh.z), fmaf(n3, sc.w, sh.w));
    }
  }
}

// 8 consecutive elements of a row as fp32.
template <typename T> __device__ __forceinline__ void load8(const T* p, float (&o)[8]);
template <> __device__ __forceinline__ void load8<bf16>(const bf16* p, float (&o)[8]) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (float)v[i];
}
template <> __device__ __forceinline__ void load8<float>(const float* p, float (&o)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
template <typename T> __device__ __forceinline__ void store8(T* p, const float (&o)[8]);
template <> __device__ __forceinline__ void store8<bf16>(bf16* p, const float (&o)[8]) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (bf16)o[i];
  *reinterpret_cast<bf16x8*>(p) = v;
}
template <> __device__ __forceinline__ void store8<float>(float* p, const float (&o)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(o[0], o[1], o[2], o[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(o[4], o[5], o[6], o[7]);
}

constexpr int QK_MAX8 = 12;  // 8-element chunks per lane: dim <= 12 * 512 = 6144

// One row of q or k: optional RMSNorm over the full row ("图解 Wan2.1 I2V" §5.3 ①), gain, then
// 3D RoPE per head (§5.3 ②): head channels split into time / height / width segments of
// sizes hd - 4*(hd/6), 2*(hd/6), 2*(hd/6); pair (2m, 2m+1) of a segment of width n rotates by
// pos * theta^(-2m/n), pos being the token's frame / row / column index.
template <typename T>
__device__ __forceinline__ void norm_rope_row(const T* __restrict__ in, T* __restrict__ out, int dim, int hd,
                                              const float* __restrict__ g, int do_norm, float eps,
                                              float log2_theta, int f, int i, int j, int lane) {
  float v[QK_MAX8][8];
  float sq = 0.f;
#pragma unroll
  for (int c = 0; c < QK_MAX8; ++c) {
    const int c0 = c * 512 + lane * 8;
    if (c0 < dim) {
      load8<T>(in + c0, v[c]);
#pragma unroll
      for (int e = 0; e < 8; ++e) sq += v[c][e] * v[c][e];
    }
  }
  float r = 1.f;
  if (do_norm) r = 1.f / sqrtf(wave_sum(sq) / (float)dim + eps);
  const int q6 = hd / 6;
  const int dT = hd - 4 * q6, dH = 2 * q6;
#pragma unroll
  for (int c = 0; c < QK_MAX8; ++c) {
    const int c0 = c * 512 + lane * 8;
    if (c0 < dim) {
      float o[8];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int ch = c0 + 2 * p;
        const int d = ch % hd;
        int m, n, pos;
        if (d < dT) {
          m = d >> 1; n = dT; pos = f;
        } else if (d < dT + dH) {
          m = (d - dT) >> 1; n = dH; pos = i;
        } else {
          m = (d - dT - dH) >> 1; n = dH; pos = j;
        }
        float a = v[c][2 * p] * r, b = v[c][2 * p + 1] * r;
        if (g) {
          a *= g[ch];
          b *= g[ch + 1];
        }
        const float freq = exp2f(-(float)(2 * m) / (float)n * log2_theta);
        float sn, cs;
        sincosf((float)pos * freq, &sn, &cs);
        o[2 * p] = a * cs - b * sn;
        o[2 * p + 1] = a * sn + b * cs;
      }
      store8<T>(out + c0, o);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(const T* q_in, const T* k_in, int64_t ld_in, T* q_out,
                                                            T* k_out, int64_t ld_out, int64_t rows, int S, int Hp,
                                                            int Wp, int dim, int hd, const float* __restrict__ gq,
                                                            const float* __restrict__ gk, int do_norm, float eps,
                                                            float log2_theta) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int s = (int)(row % S);
  const int jj = s % Wp, ii = (s / Wp) % Hp, ff = s / (Wp * Hp);
  norm_rope_row<T>(q_in + row * ld_in, q_out + row * ld_out, dim, hd, gq, do_norm, eps, log2_theta, ff, ii, jj,
                   lane);
  norm_rope_row<T>(k_in + row * ld_in, k_out + row * ld_out, dim, hd, gk, do_norm, eps, log2_theta, ff, ii, jj,
                   lane);
}

}  // namespace

template <typename T>
hipError_t launch_ln_mod(const float* x, int64_t rows, int dim, int S, int mode, const float* p0, const float* p1,
                         int c_shift, int c_scale, float eps, T* u, hipStream_t s) {
  if (dim % 4 != 0 || dim > LN_MAX4 * 256) return hipErrorInvalidValue;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(ln_mod_kernel<T>, dim3((unsigned)ceil_div(rows, 4)), dim3(256), 0, s, x, rows, dim, S, mode,
                     p0, p1, c_shift, c_scale, eps, u);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_qk_norm_rope(const T* q_in, const T* k_in, int64_t ld_in, T* q_out, T* k_out, int64_t ld_out,
                               int B, int T_, int Hp, int Wp, int heads, int hd, const float* gq, const float* gk,
                               int do_norm, float eps, float theta, hipStream_t s) {
  const int dim = heads * hd;
  if (dim % 8 != 0 || dim > QK_MAX8 * 512 || hd % 8 != 0) return hipErrorInvalidValue;
  const int S = T_ * Hp * Wp;
  const int64_t rows = (int64_t)B * S;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(qk_norm_rope_kernel<T>, dim3((unsigned)ceil_div(rows, 4)), dim3(256), 0, s, q_in, k_in, ld_in,
                     q_out, k_out, ld_out, rows, S, Hp, Wp, dim, hd, gq, gk, do_norm, eps, log2f(theta));
  return hipGetLastError();
}

template hipError_t launch_ln_mod<float>(const float*, int64_t, int, int, int, const float*, const float*, int, int,
                                         float, float*, hipStream_t);
template hipError_t launch_ln_mod<bf16>(const float*, int64_t, int, int, int, const float*, const float*, int, int,
                                        float, bf16*, hipStream_t);
template hipError_t launch_qk_norm_rope<float>(const float*, const float*, int64_t, float*, float*, int64_t, int, int,
                                               int, int, int, int, const float*, const float*, int, float, float,
                                               hipStream_t);
template hipError_t launch_qk_norm_rope<bf16>(const bf16*, const bf16*, int64_t, bf16*, bf16*, int64_t, int, int,
                                              int, int, int, int, const float*, const float*, int, float, float,
                                              hipStream_t);

}  // namespace wan
