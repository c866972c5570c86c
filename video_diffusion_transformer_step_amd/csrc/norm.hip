// Row-wise normalisation kernels (HBM-bound): LayerNorm + adaLN modulation,
// affine LayerNorm, the head's modulated LayerNorm, and the Q/K RMSNorm + gain +
// 3D RoPE pass.  A 64-lane wave owns a few consecutive token rows, one at a time; a
// row stays in registers between the statistics and the write, and per-channel
// parameters are kept in registers across the wave's rows.
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

constexpr int LN_ROWS = 4;  // rows per wave: the per-channel modulation is loaded once per wave (dim <= 3072)

// (shift, 1 + scale) of the four channels c..c+3 for batch row b.  mode 0: adaLN, from e0 [B, 6, dim]
// (p0; chunks c_shift, c_scale) plus the block's bias [6, dim] (p1, or NULL when p0 already holds the
// sum); mode 1: affine LN, weight p0 and bias p1; mode 2: the head, biases p0 [2, dim] plus e [B, dim] (p1).
__device__ __forceinline__ void ln_modulation(int mode, const float* __restrict__ p0, const float* __restrict__ p1,
                                              int c_shift, int c_scale, int dim, int64_t b, int c, float4& vsh,
                                              float4& vsc) {
  if (mode == 0) {
    const float4 es = *reinterpret_cast<const float4*>(p0 + (b * 6 + c_shift) * dim + c);
    const float4 ec = *reinterpret_cast<const float4*>(p0 + (b * 6 + c_scale) * dim + c);
    if (p1) {
      const float4 ms = *reinterpret_cast<const float4*>(p1 + (int64_t)c_shift * dim + c);
      const float4 mc = *reinterpret_cast<const float4*>(p1 + (int64_t)c_scale * dim + c);
      vsh = make_float4(es.x + ms.x, es.y + ms.y, es.z + ms.z, es.w + ms.w);
      vsc = make_float4(1.f + (ec.x + mc.x), 1.f + (ec.y + mc.y), 1.f + (ec.z + mc.z), 1.f + (ec.w + mc.w));
    } else {
      vsh = es;
      vsc = make_float4(1.f + ec.x, 1.f + ec.y, 1.f + ec.z, 1.f + ec.w);
    }
  } else if (mode == 1) {
    vsc = *reinterpret_cast<const float4*>(p0 + c);
    vsh = *reinterpret_cast<const float4*>(p1 + c);
  } else {
    const float4 h0 = *reinterpret_cast<const float4*>(p0 + c);
    const float4 h1 = *reinterpret_cast<const float4*>(p0 + dim + c);
    const float4 e = *reinterpret_cast<const float4*>(p1 + b * dim + c);
    vsh = make_float4(h0.x + e.x, h0.y + e.y, h0.z + e.z, h0.w + e.w);
    vsc = make_float4(1.f + (h1.x + e.x), 1.f + (h1.y + e.y), 1.f + (h1.z + e.z), 1.f + (h1.w + e.w));
  }
}

// LayerNorm (biased variance, no affine) then modulation; see launch_ln_mod in wan_internal.h.
// "图解 Wan2.1 I2V" §5.2: x' = norm(x) * (1 + scale) + shift; the cross-attention pre-norm (mode 1)
// and the head (mode 2, §5.5) reuse the same row statistics.  A wave normalises LN_ROWS
// consecutive rows; for rows of up to 3072 channels the (shift, 1 + scale) vectors of its lanes'
// channels are formed once and re-formed only when the batch row changes.  NC = float4 chunks per
// lane (dim <= 256 NC).
template <typename T, int NC>
__global__ __launch_bounds__(256) void ln_mod_kernel(const float* __restrict__ x, int64_t rows, int dim, int S,
                                                      int mode, const float* __restrict__ p0,
                                                      const float* __restrict__ p1, int c_shift, int c_scale,
                                                      float eps, T* __restrict__ u) {
  constexpr bool CACHE = NC <= 12;
  const int lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * LN_ROWS;
  const int n4 = dim >> 2;
  float4 sh[CACHE ? NC : 1], sc[CACHE ? NC : 1];
  // (shift, 1 + scale) of float4 chunk idx (channels 4 idx ..) for batch row b
  auto modulation = [&](int64_t b, int idx, float4& vsh, float4& vsc) {
    ln_modulation(mode, p0, p1, c_shift, c_scale, dim, b, idx * 4, vsh, vsc);
  };
  // rows are software-pipelined: the next row's loads are issued before this row's reductions
  float4 vn[NC];
  auto load_row = [&](int64_t row) {
    const float4* xr = reinterpret_cast<const float4*>(x + row * dim);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int idx = i * 64 + lane;
      if (idx < n4) vn[i] = xr[idx];
    }
  };
  if (row0 >= rows) return;
  if constexpr (CACHE) load_row(row0);  // (wide rows: no registers to spare for the next row)
  int64_t bcur = -1;
  for (int rr = 0; rr < LN_ROWS; ++rr) {
    const int64_t row = row0 + rr;
    if (row >= rows) return;
    if constexpr (!CACHE) load_row(row);
    float4 v[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) v[i] = vn[i];
    if (CACHE && rr + 1 < LN_ROWS && row + 1 < rows) load_row(row + 1);
    const int64_t b = row / S;
    if (CACHE && b != bcur) {  // modulation of this batch row (uniform branch)
      bcur = b;
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int idx = i * 64 + lane;
        if (idx < n4) modulation(b, idx, sh[CACHE ? i : 0], sc[CACHE ? i : 0]);
      }
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int idx = i * 64 + lane;
      if (idx < n4) sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    }
    const float mean = wave_sum(sum) / (float)dim;
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int idx = i * 64 + lane;
      if (idx < n4) {
        const float a = v[i].x - mean, bb = v[i].y - mean, c = v[i].z - mean, d = v[i].w - mean;
        sq += (a * a + bb * bb) + (c * c + d * d);
      }
    }
    const float rstd = 1.f / sqrtf(wave_sum(sq) / (float)dim + eps);
    T* ur = u + row * dim;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int idx = i * 64 + lane;
      if (idx < n4) {
        float4 vsh, vsc;
        if constexpr (CACHE) {
          vsh = sh[i];
          vsc = sc[i];
        } else {
          modulation(b, idx, vsh, vsc);
        }
        const float n0 = (v[i].x - mean) * rstd, n1 = (v[i].y - mean) * rstd;
        const float n2 = (v[i].z - mean) * rstd, n3 = (v[i].w - mean) * rstd;
        store4<T>(ur + idx * 4, fmaf(n0, vsc.x, vsh.x), fmaf(n1, vsc.y, vsh.y), fmaf(n2, vsc.z, vsh.z),
                  fmaf(n3, vsc.w, vsh.w));
      }
    }
  }
}

// 8 consecutive elements of a row as fp32.
// Rows wider than 1536 channels (ln_mod_kernel's per-lane arrays would cost the occupancy that hides
// the loads): one workgroup of NT threads per row (256 up to 3072 channels, 512 up to 6144),
// LNW_ROWS consecutive rows per workgroup.  Thread t holds float4 chunks t, t + NT, t + 2 NT; the next
// row's chunks are loaded before this row's reductions, the (shift, 1 + scale) vectors are formed once
// per batch row, and each of the two row sums crosses the waves through LDS (one slot per sum, so two
// barriers per row suffice).
constexpr int LNW_ROWS = 8;
constexpr int LNW_CH = 3;  // float4 chunks per thread

template <typename T, int NT>
__global__ __launch_bounds__(NT) void ln_mod_wide_kernel(const float* __restrict__ x, int64_t rows, int dim, int S,
                                                          int mode, const float* __restrict__ p0,
                                                          const float* __restrict__ p1, int c_shift, int c_scale,
                                                          float eps, T* __restrict__ u) {
  constexpr int NWV = NT / 64;
  __shared__ float part[2][NWV];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * LNW_ROWS;
  const int n4 = dim >> 2;
  float4 sh[LNW_CH], sc[LNW_CH], vn[LNW_CH];
  auto load_row = [&](int64_t row) {
    const float4* xr = reinterpret_cast<const float4*>(x + row * dim);
#pragma unroll
    for (int i = 0; i < LNW_CH; ++i) {
      const int idx = i * NT + tid;
      if (idx < n4) vn[i] = xr[idx];
    }
  };
  auto block_sum = [&](float v, int slot) {
    v = wave_sum(v);
    if (lane == 0) part[slot][wave] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) t += part[slot][w];
    return t;
  };
  load_row(row0);  // the grid holds no workgroup past the last row
  int64_t bcur = -1;
  for (int rr = 0; rr < LNW_ROWS; ++rr) {
    const int64_t row = row0 + rr;
    if (row >= rows) return;  // uniform in the workgroup
    float4 v[LNW_CH];
#pragma unroll
    for (int i = 0; i < LNW_CH; ++i) v[i] = vn[i];
    if (rr + 1 < LNW_ROWS && row + 1 < rows) load_row(row + 1);
    const int64_t b = row / S;
    if (b != bcur) {  // uniform in the workgroup
      bcur = b;
#pragma unroll
      for (int i = 0; i < LNW_CH; ++i) {
        const int idx = i * NT + tid;
        if (idx < n4) ln_modulation(mode, p0, p1, c_shift, c_scale, dim, b, idx * 4, sh[i], sc[i]);
      }
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < LNW_CH; ++i)
      if (i * NT + tid < n4) sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    const float mean = block_sum(sum, 0) / (float)dim;
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < LNW_CH; ++i)
      if (i * NT + tid < n4) {
        const float a = v[i].x - mean, bb = v[i].y - mean, c = v[i].z - mean, d = v[i].w - mean;
        sq += (a * a + bb * bb) + (c * c + d * d);
      }
    const float rstd = 1.f / sqrtf(block_sum(sq, 1) / (float)dim + eps);
    T* ur = u + row * dim;
#pragma unroll
    for (int i = 0; i < LNW_CH; ++i) {
      const int idx = i * NT + tid;
      if (idx < n4) {
        const float n0 = (v[i].x - mean) * rstd, n1 = (v[i].y - mean) * rstd;
        const float n2 = (v[i].z - mean) * rstd, n3 = (v[i].w - mean) * rstd;
        store4<T>(ur + idx * 4, fmaf(n0, sc[i].x, sh[i].x), fmaf(n1, sc[i].y, sh[i].y), fmaf(n2, sc[i].z, sh[i].z),
                  fmaf(n3, sc[i].w, sh[i].w));
      }
    }
  }
}

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
constexpr int QK_ROWS = 4;   // token rows per wave

// 3D RoPE ("图解 Wan2.1 I2V" §5.3 ②): head channels split into time / height / width segments of
// sizes hd - 4*(hd/6), 2*(hd/6), 2*(hd/6); pair (2m, 2m+1) of a segment of width n rotates by
// pos * theta^(-2m/n), pos being the token's frame / row / column index.  A lane's 8-channel
// chunks all sit at the same offset within their heads (hd divides 512), so its 4 pairs' frequencies
// (fixed per lane) and angles (per token) serve every chunk of the row and both q and k.
struct RopeLane {
  float freq[4];
  int axis[4];  // 0 frame, 1 row, 2 column
};

__device__ __forceinline__ RopeLane rope_lane(int d0, int hd, float log2_theta) {
  const int q6 = hd / 6;
  const int dT = hd - 4 * q6, dH = 2 * q6;
  RopeLane r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int d = d0 + 2 * p;
    int m, n;
    if (d < dT) {
      m = d >> 1; n = dT; r.axis[p] = 0;
    } else if (d < dT + dH) {
      m = (d - dT) >> 1; n = dH; r.axis[p] = 1;
    } else {
      m = (d - dT - dH) >> 1; n = dH; r.axis[p] = 2;
    }
    r.freq[p] = exp2f(-(float)(2 * m) / (float)n * log2_theta);
  }
  return r;
}

// The lane's pair angles at token position (f, i, j), by the hardware sine / cosine (angles here are
// at most a few hundred radians, where their error stays near 1e-6).
__device__ __forceinline__ void rope_angles(const RopeLane& r, int f, int i, int j, float (&cs)[4], float (&sn)[4]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int pos = r.axis[p] == 0 ? f : (r.axis[p] == 1 ? i : j);
    const float a = (float)pos * r.freq[p];
    sn[p] = __sinf(a);
    cs[p] = __cosf(a);
  }
}

// One 8-channel chunk: scale by the row's RMS factor r and the gains g, rotate the lane's 4 pairs by
// their angles, store.
template <typename T>
__device__ __forceinline__ void rotate_store8(const float (&v)[8], float r, const float (&g)[8], const float (&cs)[4],
                                              const float (&sn)[4], T* __restrict__ out) {
  float o[8];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float a = v[2 * p] * r * g[2 * p], b = v[2 * p + 1] * r * g[2 * p + 1];
    o[2 * p] = a * cs[p] - b * sn[p];
    o[2 * p + 1] = a * sn[p] + b * cs[p];
  }
  store8<T>(out, o);
}

// The q and k rows of one token: RMSNorm over the full row ("图解 Wan2.1 I2V" §5.3 ①, optional), the
// gains (this lane's in gq / gk), then the rotation by the lane's pair angles.  Both rows are loaded
// before either reduction so their loads are in flight together.
template <typename T, int NC8>
__device__ __forceinline__ void norm_rope_qk(const T* __restrict__ qi, const T* __restrict__ ki, T* __restrict__ qo,
                                             T* __restrict__ ko, int dim, const float (&gq)[NC8][8],
                                             const float (&gk)[NC8][8], int do_norm, float eps, const float (&cs)[4],
                                             const float (&sn)[4], int lane) {
  float vq[NC8][8], vk[NC8][8];
#pragma unroll
  for (int c = 0; c < NC8; ++c) {
    const int c0 = c * 512 + lane * 8;
    if (c0 < dim) {
      load8<T>(qi + c0, vq[c]);
      load8<T>(ki + c0, vk[c]);
    }
  }
  float sq = 0.f, sk = 0.f;
#pragma unroll
  for (int c = 0; c < NC8; ++c) {
    const int c0 = c * 512 + lane * 8;
    if (c0 < dim) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sq += vq[c][e] * vq[c][e];
        sk += vk[c][e] * vk[c][e];
      }
    }
  }
  float rq = 1.f, rk = 1.f;
  if (do_norm) {
    rq = 1.f / sqrtf(wave_sum(sq) / (float)dim + eps);
    rk = 1.f / sqrtf(wave_sum(sk) / (float)dim + eps);
  }
#pragma unroll
  for (int c = 0; c < NC8; ++c) {
    const int c0 = c * 512 + lane * 8;
    if (c0 < dim) {
      rotate_store8<T>(vq[c], rq, gq[c], cs, sn, qo + c0);
      rotate_store8<T>(vk[c], rk, gk[c], cs, sn, ko + c0);
    }
  }
}

// NC8 = 8-channel chunks per lane (dim <= 512 NC8).
template <typename T, int NC8>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(const T* q_in, const T* k_in, int64_t ld_in, T* q_out,
                                                            T* k_out, int64_t ld_out, int64_t rows, int S, int Hp,
                                                            int Wp, int dim, int hd, const float* __restrict__ gq,
                                                            const float* __restrict__ gk, int do_norm, float eps,
                                                            float log2_theta) {
  const int lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * QK_ROWS;
  if (row0 >= rows) return;
  float gql[NC8][8], gkl[NC8][8];
#pragma unroll
  for (int c = 0; c < NC8; ++c) {
    const int c0 = c * 512 + lane * 8;
    if (c0 < dim && gq) {
      load8<float>(gq + c0, gql[c]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) gql[c][e] = 1.f;
    }
    if (c0 < dim && gk) {
      load8<float>(gk + c0, gkl[c]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) gkl[c][e] = 1.f;
    }
  }
  const RopeLane rl = rope_lane((lane * 8) % hd, hd, log2_theta);
  for (int rr = 0; rr < QK_ROWS; ++rr) {
    const int64_t row = row0 + rr;
    if (row >= rows) return;
    const int s = (int)(row % S);
    const int jj = s % Wp, ii = (s / Wp) % Hp, ff = s / (Wp * Hp);
    float cs[4], sn[4];
    rope_angles(rl, ff, ii, jj, cs, sn);
    norm_rope_qk<T, NC8>(q_in + row * ld_in, k_in + row * ld_in, q_out + row * ld_out, k_out + row * ld_out, dim,
                         gql, gkl, do_norm, eps, cs, sn, lane);
  }
}

// Rows wider than 1536 channels: one workgroup of NT threads per token row (256 up to 4096 channels,
// 512 up to 6144), QKW_ROWS consecutive rows per workgroup.  Thread t holds the 8-channel chunks at
// t * 8 + c * 8 NT of q and of k; hd divides 8 NT, so they sit at one offset within their heads and the
// thread's pair frequencies are fixed.  The next row is loaded before this row's sums, which cross the
// waves through LDS (slots alternate by row, so one barrier per row suffices).
constexpr int QKW_ROWS = 8;
constexpr int QKW_CH = 2;  // 8-channel chunks per thread, of q and of k

template <typename T, int NT>
__global__ __launch_bounds__(NT) void qk_norm_rope_wide_kernel(const T* q_in, const T* k_in, int64_t ld_in,
                                                                T* q_out, T* k_out, int64_t ld_out, int64_t rows,
                                                                int S, int Hp, int Wp, int dim, int hd,
                                                                const float* __restrict__ gq,
                                                                const float* __restrict__ gk, int do_norm, float eps,
                                                                float log2_theta) {
  constexpr int NWV = NT / 64;
  __shared__ float part[2][NWV][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * QKW_ROWS;
  float gql[QKW_CH][8], gkl[QKW_CH][8];
#pragma unroll
  for (int c = 0; c < QKW_CH; ++c) {
    const int c0 = c * NT * 8 + tid * 8;
    if (c0 < dim && gq) {
      load8<float>(gq + c0, gql[c]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) gql[c][e] = 1.f;
    }
    if (c0 < dim && gk) {
      load8<float>(gk + c0, gkl[c]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) gkl[c][e] = 1.f;
    }
  }
  const RopeLane rl = rope_lane((tid * 8) % hd, hd, log2_theta);
  float nq[QKW_CH][8], nk[QKW_CH][8];
  auto load_row = [&](int64_t row) {
#pragma unroll
    for (int c = 0; c < QKW_CH; ++c) {
      const int c0 = c * NT * 8 + tid * 8;
      if (c0 < dim) {
        load8<T>(q_in + row * ld_in + c0, nq[c]);
        load8<T>(k_in + row * ld_in + c0, nk[c]);
      }
    }
  };
  load_row(row0);  // the grid holds no workgroup past the last row
  for (int rr = 0; rr < QKW_ROWS; ++rr) {
    const int64_t row = row0 + rr;
    if (row >= rows) return;  // uniform in the workgroup
    float vq[QKW_CH][8], vk[QKW_CH][8];
#pragma unroll
    for (int c = 0; c < QKW_CH; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        vq[c][e] = nq[c][e];
        vk[c][e] = nk[c][e];
      }
    if (rr + 1 < QKW_ROWS && row + 1 < rows) load_row(row + 1);
    const int s = (int)(row % S);
    const int jj = s % Wp, ii = (s / Wp) % Hp, ff = s / (Wp * Hp);
    float cs[4], sn[4];
    rope_angles(rl, ff, ii, jj, cs, sn);
    float rq = 1.f, rk = 1.f;
    if (do_norm) {  // uniform
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int c = 0; c < QKW_CH; ++c)
        if (c * NT * 8 + tid * 8 < dim) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            sq += vq[c][e] * vq[c][e];
            sk += vk[c][e] * vk[c][e];
          }
        }
      sq = wave_sum(sq);
      sk = wave_sum(sk);
      const int slot = rr & 1;
      if (lane == 0) {
        part[slot][wave][0] = sq;
        part[slot][wave][1] = sk;
      }
      __syncthreads();
      float tq = 0.f, tk = 0.f;
#pragma unroll
      for (int w = 0; w < NWV; ++w) {
        tq += part[slot][w][0];
        tk += part[slot][w][1];
      }
      rq = 1.f / sqrtf(tq / (float)dim + eps);
      rk = 1.f / sqrtf(tk / (float)dim + eps);
    }
#pragma unroll
    for (int c = 0; c < QKW_CH; ++c) {
      const int c0 = c * NT * 8 + tid * 8;
      if (c0 < dim) {
        rotate_store8<T>(vq[c], rq, gql[c], cs, sn, q_out + row * ld_out + c0);
        rotate_store8<T>(vk[c], rk, gkl[c], cs, sn, k_out + row * ld_out + c0);
      }
    }
  }
}

}  // namespace

template <typename T>
hipError_t launch_ln_mod(const float* x, int64_t rows, int dim, int S, int mode, const float* p0, const float* p1,
                         int c_shift, int c_scale, float eps, T* u, hipStream_t s) {
  if (dim % 4 != 0 || dim > LN_MAX4 * 256) return hipErrorInvalidValue;
  if (rows <= 0) return hipSuccess;
  if (dim <= 6 * 256) {
    const dim3 grid((unsigned)ceil_div(rows, 4 * LN_ROWS));
    hipLaunchKernelGGL((ln_mod_kernel<T, 6>), grid, dim3(256), 0, s, x, rows, dim, S, mode, p0, p1, c_shift, c_scale,
                       eps, u);
  } else {
    const dim3 grid((unsigned)ceil_div(rows, (int64_t)LNW_ROWS));
    if (dim <= 4 * LNW_CH * 256)
      hipLaunchKernelGGL((ln_mod_wide_kernel<T, 256>), grid, dim3(256), 0, s, x, rows, dim, S, mode, p0, p1, c_shift,
                         c_scale, eps, u);
    else
      hipLaunchKernelGGL((ln_mod_wide_kernel<T, 512>), grid, dim3(512), 0, s, x, rows, dim, S, mode, p0, p1, c_shift,
                         c_scale, eps, u);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_qk_norm_rope(const T* q_in, const T* k_in, int64_t ld_in, T* q_out, T* k_out, int64_t ld_out,
                               int B, int T_, int Hp, int Wp, int heads, int hd, const float* gq, const float* gk,
                               int do_norm, float eps, float theta, hipStream_t s) {
  const int dim = heads * hd;
  if (dim % 8 != 0 || dim > QK_MAX8 * 512 || hd % 8 != 0 || 512 % hd != 0) return hipErrorInvalidValue;
  const int S = T_ * Hp * Wp;
  const int64_t rows = (int64_t)B * S;
  if (rows <= 0) return hipSuccess;
  const float l2t = log2f(theta);
  if (dim <= 3 * 512) {
    const dim3 grid((unsigned)ceil_div(rows, 4 * QK_ROWS));
    hipLaunchKernelGGL((qk_norm_rope_kernel<T, 3>), grid, dim3(256), 0, s, q_in, k_in, ld_in, q_out, k_out, ld_out,
                       rows, S, Hp, Wp, dim, hd, gq, gk, do_norm, eps, l2t);
  } else {
    const dim3 grid((unsigned)ceil_div(rows, (int64_t)QKW_ROWS));
    if (dim <= QKW_CH * 8 * 256)
      hipLaunchKernelGGL((qk_norm_rope_wide_kernel<T, 256>), grid, dim3(256), 0, s, q_in, k_in, ld_in, q_out, k_out,
                         ld_out, rows, S, Hp, Wp, dim, hd, gq, gk, do_norm, eps, l2t);
    else
      hipLaunchKernelGGL((qk_norm_rope_wide_kernel<T, 512>), grid, dim3(512), 0, s, q_in, k_in, ld_in, q_out, k_out,
                         ld_out, rows, S, Hp, Wp, dim, hd, gq, gk, do_norm, eps, l2t);
  }
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
