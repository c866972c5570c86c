// Row-wise normalisation kernels (HBM-bound): LayerNorm + adaLN modulation,
// affine LayerNorm, the head's modulated LayerNorm, the block's Q/K RMSNorm factors
// (finished from the Q/K/V projection epilogue's sums of squares), and the standalone
// attention's 3D RoPE pass.  For the LayerNorms a 64-lane wave owns a few consecutive
// token rows, one at a time; a row stays in registers between the statistics and the
// write, and per-channel parameters are kept in registers across the wave's rows.
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
                                                      float eps, T* __restrict__ u, int64_t ldu, int64_t ubs) {
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
  uint2 held[sizeof(T) == 2 ? NC : 1];  // K panels, bf16: the even row of a pair (see below)
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
    T* ur = u + row * ldu;  // channel c at ur + (c / 32) ubs + c % 32
    if constexpr (sizeof(T) == 2) {
      if (ldu == 32) {
        // K panels: a bf16 row's 32 channels of a panel are 64 bytes, half a line whose other half is
        // the next row.  Rows pair up: the even row's packed outputs wait for the odd row's, then one
        // v_permlane32_swap per dword gives the lower 32 lanes the even row's chunks i 64 + 32 .. + 63
        // and the upper lanes the odd row's chunks i 64 .. + 31, so each store instruction writes both
        // rows of the same panels: whole 128-byte lines.
        uint2 w[NC];
#pragma unroll
        for (int i = 0; i < NC; ++i) {
          const int idx = i * 64 + lane;
          float4 vsh, vsc;
          if constexpr (CACHE) {
            vsh = sh[i];
            vsc = sc[i];
          } else if (idx < n4) {
            modulation(b, idx, vsh, vsc);
          }
          bf16x4 o;
          o[0] = (bf16)fmaf((v[i].x - mean) * rstd, vsc.x, vsh.x);
          o[1] = (bf16)fmaf((v[i].y - mean) * rstd, vsc.y, vsh.y);
          o[2] = (bf16)fmaf((v[i].z - mean) * rstd, vsc.z, vsh.z);
          o[3] = (bf16)fmaf((v[i].w - mean) * rstd, vsc.w, vsh.w);
          w[i] = __builtin_bit_cast(uint2, o);  // lanes past n4 hold values that are never stored
        }
        if ((rr & 1) == 0 && rr + 1 < LN_ROWS && row + 1 < rows) {  // even row of a pair: wait
#pragma unroll
          for (int i = 0; i < NC; ++i) held[i] = w[i];
          continue;
        }
        if (rr & 1) {  // odd row: rows row - 1 (held) and row, one line per panel and store
          const int64_t prow = row - 1 + (lane >> 5);
          T* pr = u + prow * 32;
#pragma unroll
          for (int i = 0; i < NC; ++i) {
            const auto x = __builtin_amdgcn_permlane32_swap(held[i].x, w[i].x, false, false);
            const auto y = __builtin_amdgcn_permlane32_swap(held[i].y, w[i].y, false, false);
            const int c1 = i * 64 + (lane & 31), c2 = c1 + 32;  // chunks of row prow
            if (c1 < n4) *reinterpret_cast<uint2*>(pr + (c1 >> 3) * ubs + (c1 & 7) * 4) = make_uint2(x[0], y[0]);
            if (c2 < n4) *reinterpret_cast<uint2*>(pr + (c2 >> 3) * ubs + (c2 & 7) * 4) = make_uint2(x[1], y[1]);
          }
        } else {  // a row without a partner
#pragma unroll
          for (int i = 0; i < NC; ++i) {
            const int idx = i * 64 + lane;
            if (idx < n4) *reinterpret_cast<uint2*>(ur + (idx >> 3) * ubs + (idx & 7) * 4) = w[i];
          }
        }
        continue;
      }
    }
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
        store4<T>(ur + (idx >> 3) * ubs + (idx & 7) * 4, fmaf(n0, vsc.x, vsh.x), fmaf(n1, vsc.y, vsh.y), fmaf(n2, vsc.z, vsh.z),
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
                                                          float eps, T* __restrict__ u, int64_t ldu, int64_t ubs) {
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
    T* ur = u + row * ldu;  // channel c at ur + (c / 32) ubs + c % 32
#pragma unroll
    for (int i = 0; i < LNW_CH; ++i) {
      const int idx = i * NT + tid;
      if (idx < n4) {
        const float n0 = (v[i].x - mean) * rstd, n1 = (v[i].y - mean) * rstd;
        const float n2 = (v[i].z - mean) * rstd, n3 = (v[i].w - mean) * rstd;
        store4<T>(ur + (idx >> 3) * ubs + (idx & 7) * 4, fmaf(n0, sc[i].x, sh[i].x), fmaf(n1, sc[i].y, sh[i].y), fmaf(n2, sc[i].z, sh[i].z),
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

// ---------------------------------------------------------------------------
// Q/K rotation for the standalone attention, and the block's Q/K RMSNorm factors.
// ---------------------------------------------------------------------------

// 3D RoPE of q and k rows, without norm: one thread per 8-channel chunk of one token row (hd is a
// multiple of 8, so the chunk's four pairs sit in one head).  In place is allowed (a thread reads its
// chunks before writing them).
template <typename T>
__global__ __launch_bounds__(256) void rope_qk_kernel(const T* q_in, const T* k_in, int64_t ld_in, T* q_out, T* k_out,
                                                      int64_t ld_out, int64_t rows, int S, int Hp, int Wp, int dim,
                                                      int hd, float log2_theta) {
  const int nc = dim / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = idx / nc;
  if (row >= rows) return;
  const int c0 = (int)(idx - row * nc) * 8, d0 = c0 % hd;
  float vq[8], vk[8];
  load8<T>(q_in + row * ld_in + c0, vq);
  load8<T>(k_in + row * ld_in + c0, vk);
  const RopePos t = rope_pos((int)(row % S), Hp, Wp);
  float oq[8], ok[8];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    float c, s;
    rope_cs(rope_pair(d0 + 2 * p, hd, log2_theta), t, c, s);
    oq[2 * p] = vq[2 * p] * c - vq[2 * p + 1] * s;
    oq[2 * p + 1] = vq[2 * p] * s + vq[2 * p + 1] * c;
    ok[2 * p] = vk[2 * p] * c - vk[2 * p + 1] * s;
    ok[2 * p + 1] = vk[2 * p] * s + vk[2 * p + 1] * c;
  }
  store8<T>(q_out + row * ld_out + c0, oq);
  store8<T>(k_out + row * ld_out + c0, ok);
}

// The block's Q/K RMSNorm ("图解 Wan2.1 I2V" §5.3 ①), finished from the Q/K/V projection epilogue's
// partial sums of squares: ssq[nb * rows + row] is the sum of squares of the row's projected q
// channels 32 nb .. 32 nb + 31 (nb < dim/32), then of its k channels (the next dim/32 blocks), taken
// before the gains and the rotation.  With r = (sum / dim + eps)^-1/2 per row, this writes r_q to rq
// (the attention multiplies its score scale by it) and scales the k row in place by r_k (the epilogue
// already applied the gains and the rotation, both linear, so r commutes with them).
// QKR_ROWS rows per wave: their sums with lane = (part, row), then the k rows RB at a time, NC8
// 8-channel chunks per lane and row (dim <= 512 NC8), all of a batch's loads before its stores.
constexpr int QKR_ROWS = 8;

template <typename T, int NC8, int RB>
__global__ __launch_bounds__(256) void qk_rms_kernel(const float* __restrict__ ssq, int64_t rows, int dim, float eps,
                                                     T* __restrict__ k, int64_t ldk, float* __restrict__ rq) {
  static_assert(QKR_ROWS % RB == 0, "whole batches of rows");
  const int lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * QKR_ROWS;
  if (row0 >= rows) return;  // uniform in the wave
  const int np = dim / 32, part = lane >> 3, r = lane & 7;
  const int64_t myrow = row0 + r < rows ? row0 + r : rows - 1;
  float sq = 0.f, sk = 0.f;
  for (int nb = part; nb < 2 * np; nb += 8) {
    const float v = ssq[(int64_t)nb * rows + myrow];
    if (nb < np)
      sq += v;
    else
      sk += v;
  }
  // the eight parts of row r sit in lanes r, r + 8, ..., r + 56
  sq += __shfl_xor(sq, 8);
  sq += __shfl_xor(sq, 16);
  sq += __shfl_xor(sq, 32);
  sk += __shfl_xor(sk, 8);
  sk += __shfl_xor(sk, 16);
  sk += __shfl_xor(sk, 32);
  const float fq = 1.f / sqrtf(sq / (float)dim + eps);
  const float fk = 1.f / sqrtf(sk / (float)dim + eps);
  if (part == 0 && row0 + r < rows) rq[row0 + r] = fq;
  const int nr = rows - row0 < QKR_ROWS ? (int)(rows - row0) : QKR_ROWS;
#pragma unroll
  for (int r0 = 0; r0 < QKR_ROWS; r0 += RB) {
    float v[RB][NC8][8];
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int c = 0; c < NC8; ++c) {
        const int c0 = c * 512 + lane * 8;
        if (r0 + b < nr && c0 < dim) load8<T>(k + (row0 + r0 + b) * ldk + c0, v[b][c]);
      }
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const float f = __shfl(fk, r0 + b);  // lane r0 + b (part 0) holds row r0 + b's factor
#pragma unroll
      for (int c = 0; c < NC8; ++c) {
        const int c0 = c * 512 + lane * 8;
        if (r0 + b < nr && c0 < dim) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[b][c][e] *= f;
          store8<T>(k + (row0 + r0 + b) * ldk + c0, v[b][c]);
        }
      }
    }
  }
}

}  // namespace

template <typename T>
hipError_t launch_ln_mod(const float* x, int64_t rows, int dim, int S, int mode, const float* p0, const float* p1,
                         int c_shift, int c_scale, float eps, T* u, ActLayout lu, hipStream_t s) {
  if (dim % 4 != 0 || dim > LN_MAX4 * 256) return hipErrorInvalidValue;
  if (lu.bs != 32 && dim % 32 != 0) return hipErrorInvalidValue;
  if (rows <= 0) return hipSuccess;
  if (dim <= 6 * 256) {
    const dim3 grid((unsigned)ceil_div(rows, 4 * LN_ROWS));
    hipLaunchKernelGGL((ln_mod_kernel<T, 6>), grid, dim3(256), 0, s, x, rows, dim, S, mode, p0, p1, c_shift, c_scale,
                       eps, u, lu.ld, lu.bs);
  } else {
    const dim3 grid((unsigned)ceil_div(rows, (int64_t)LNW_ROWS));
    if (dim <= 4 * LNW_CH * 256)
      hipLaunchKernelGGL((ln_mod_wide_kernel<T, 256>), grid, dim3(256), 0, s, x, rows, dim, S, mode, p0, p1, c_shift,
                         c_scale, eps, u, lu.ld, lu.bs);
    else
      hipLaunchKernelGGL((ln_mod_wide_kernel<T, 512>), grid, dim3(512), 0, s, x, rows, dim, S, mode, p0, p1, c_shift,
                         c_scale, eps, u, lu.ld, lu.bs);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_rope_qk(const T* q_in, const T* k_in, int64_t ld_in, T* q_out, T* k_out, int64_t ld_out, int B,
                          int T_, int Hp, int Wp, int heads, int hd, float theta, hipStream_t s) {
  if (hd % 8 != 0 || !(theta > 0.f)) return hipErrorInvalidValue;
  const int dim = heads * hd, S = T_ * Hp * Wp;
  const int64_t rows = (int64_t)B * S;
  if (rows <= 0 || dim <= 0) return hipSuccess;
  const int64_t n = rows * (dim / 8);
  hipLaunchKernelGGL((rope_qk_kernel<T>), dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, q_in, k_in, ld_in, q_out,
                     k_out, ld_out, rows, S, Hp, Wp, dim, hd, log2f(theta));
  return hipGetLastError();
}

template <typename T>
hipError_t launch_qk_rms(const float* ssq, int64_t rows, int dim, float eps, T* k, int64_t ldk, float* rq,
                         hipStream_t s) {
  if (dim % 32 != 0 || dim > 12 * 512 || ldk % 8 != 0) return hipErrorInvalidValue;
  if (rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(rows, 4 * QKR_ROWS));
  if (dim <= 3 * 512)
    hipLaunchKernelGGL((qk_rms_kernel<T, 3, 4>), grid, dim3(256), 0, s, ssq, rows, dim, eps, k, ldk, rq);
  else if (dim <= 6 * 512)
    hipLaunchKernelGGL((qk_rms_kernel<T, 6, 2>), grid, dim3(256), 0, s, ssq, rows, dim, eps, k, ldk, rq);
  else
    hipLaunchKernelGGL((qk_rms_kernel<T, 12, 1>), grid, dim3(256), 0, s, ssq, rows, dim, eps, k, ldk, rq);
  return hipGetLastError();
}

template hipError_t launch_ln_mod<float>(const float*, int64_t, int, int, int, const float*, const float*, int, int,
                                         float, float*, ActLayout, hipStream_t);
template hipError_t launch_ln_mod<bf16>(const float*, int64_t, int, int, int, const float*, const float*, int, int,
                                        float, bf16*, ActLayout, hipStream_t);
template hipError_t launch_rope_qk<float>(const float*, const float*, int64_t, float*, float*, int64_t, int, int, int,
                                          int, int, int, float, hipStream_t);
template hipError_t launch_rope_qk<bf16>(const bf16*, const bf16*, int64_t, bf16*, bf16*, int64_t, int, int, int,
                                         int, int, int, float, hipStream_t);
template hipError_t launch_qk_rms<float>(const float*, int64_t, int, float, float*, int64_t, float*, hipStream_t);
template hipError_t launch_qk_rms<bf16>(const float*, int64_t, int, float, bf16*, int64_t, float*, hipStream_t);

}  // namespace wan
