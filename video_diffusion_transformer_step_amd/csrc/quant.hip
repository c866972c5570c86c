// Quantisation of attention inputs for the FP8 attention path ("Wan 技术深度解析" §5.3: Q.K inner
// products in INT8, O = P.V in FP8 with FP32 accumulation across key blocks).
//
//  * Q -> INT8 per (token, head): scale = amax / 127, code = rne(x * (127 / amax)), clamped to
//    +-127 (float32 quotients and product, IEEE-rounded, so codes are a fixed function of x);
//  * K -> INT8 per (head, block of 64 consecutive keys), same rule;
//  * V -> FP8 E4M3 (OCP) per (head, channel) over all keys: scale = amax / 448,
//    code = e4m3(clamp(x * (448 / amax), -448, 448)), written as V^T [B, H, hd, Lpad] (Lpad a multiple
//    of 128, zero past the keys) with the keys of each 64-key tile in the order the FP8 P.V product
//    reads them (wan.h documents it).
// A group whose amax is 0 gets scale 0 and zero codes.
#include <algorithm>

#include "wan_internal.h"

namespace wan {

namespace {

// Max over each aligned group of 16 (W16) or 8 lanes; every lane of the group gets the result.
template <int W>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror: 8-lane groups
  if constexpr (W == 16) v = fmaxf(v, dpp_f32<0x140>(v));  // row_mirror: 16-lane rows
  return v;
}

__device__ __forceinline__ int8_t i8_code(float x, float inv) {
  return (int8_t)fminf(fmaxf(rintf(x * inv), -127.f), 127.f);
}

// One thread = 8 consecutive channels of one token; a (token, head) group is HD / 8 lanes.
template <typename T, int HD>
__global__ __launch_bounds__(256) void quant_q_kernel(const T* __restrict__ x, int64_t ld, int64_t rows, int S,
                                                      int H, int8_t* __restrict__ codes, float* __restrict__ scales) {
  constexpr int G = HD / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_row = (int64_t)H * G;
  const bool live = t < rows * per_row;
  const int64_t tt = live ? t : 0;
  const int64_t row = tt / per_row;
  const int c8 = (int)(tt - row * per_row);  // 8-channel chunk within the row
  const int h = c8 / G;
  float v[8];
  const u32x4 raw = *reinterpret_cast<const u32x4*>(x + row * ld + c8 * 8);
  const bf16* e = reinterpret_cast<const bf16*>(&raw);
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = (float)e[i];
    m = fmaxf(m, fabsf(v[i]));
  }
  m = group_max<G>(m);  // groups never straddle a wave; dead lanes only see dead lanes' zeros
  if (!live) return;
  const float inv = m > 0.f ? 127.f / m : 0.f;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= (uint32_t)(uint8_t)i8_code(v[i], inv) << (8 * i);
    hi |= (uint32_t)(uint8_t)i8_code(v[4 + i], inv) << (8 * i);
  }
  *reinterpret_cast<uint2*>(codes + row * (int64_t)H * HD + c8 * 8) = make_uint2(lo, hi);
  if (c8 % G == 0) {
    const int64_t b = row / S, s = row - b * S;
    scales[(b * H + h) * S + s] = m > 0.f ? m / 127.f : 0.f;
  }
}

// One workgroup = one (batch row, head, 64-key block).
template <typename T, int HD>
__global__ __launch_bounds__(256) void quant_k_kernel(const T* __restrict__ x, int64_t ld, int S, int H,
                                                      int8_t* __restrict__ codes, float* __restrict__ scales) {
  constexpr int G = HD / 8, PER = 64 * G / 256;  // 8-channel chunks per thread
  __shared__ float red[4];
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int nb = (int)ceil_div(S, 64);
  float v[PER][8];
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = i * 256 + threadIdx.x;
    const int key = blk * 64 + idx / G, c8 = idx % G;
    if (key < S) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(x + ((int64_t)b * S + key) * ld + h * HD + c8 * 8);
      const bf16* e = reinterpret_cast<const bf16*>(&raw);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[i][j] = (float)e[j];
        m = fmaxf(m, fabsf(v[i][j]));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[i][j] = 0.f;
    }
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = m > 0.f ? 127.f / m : 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = i * 256 + threadIdx.x;
    const int key = blk * 64 + idx / G, c8 = idx % G;
    if (key >= S) continue;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo |= (uint32_t)(uint8_t)i8_code(v[i][j], inv) << (8 * j);
      hi |= (uint32_t)(uint8_t)i8_code(v[i][4 + j], inv) << (8 * j);
    }
    *reinterpret_cast<uint2*>(codes + ((int64_t)b * S + key) * H * HD + h * HD + c8 * 8) = make_uint2(lo, hi);
  }
  if (threadIdx.x == 0) scales[((int64_t)b * H + h) * nb + blk] = m > 0.f ? m / 127.f : 0.f;
}

// Four fp32 values -> four E4M3 codes (round to nearest even; |y| <= 448 so no NaN).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// One workgroup = one V^T row (batch row, head, channel d).  Input: bf16 V^T rows of Lpad_in keys whose keys
// are permuted within 16-key groups (position p holds key p with bits 2 and 3 swapped, the layout of
// the bf16 attention); output: E4M3 V^T whose 64-key tiles hold at position h*32 + kb*16 + r the key
// kb*32 + (r/4)*8 + h*4 + r%4, i.e. the 32 keys one lane half of the P.V product consumes are
// contiguous.  Position r of an output 16-byte group reads input position kb*32 + h*8 + (r%8) +
// 16 (r/8).  Output rows have Lpad_out >= Lpad_in keys; positions past Lpad_in are zero.
__global__ __launch_bounds__(256) void quant_vt_kernel(const bf16* __restrict__ vt, int Lpad_in, int Lpad_out,
                                                       uint8_t* __restrict__ out, float* __restrict__ scales) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const bf16* src = vt + row * Lpad_in;
  float m = 0.f;
  for (int c = threadIdx.x; c < Lpad_in / 8; c += 256) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(src + c * 8);
    const bf16* e = reinterpret_cast<const bf16*>(&raw);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf((float)e[j]));
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = m > 0.f ? 448.f / m : 0.f;
  uint8_t* dst = out + row * Lpad_out;
  for (int g = threadIdx.x; g < Lpad_out / 16; g += 256) {  // output group g: 16 positions
    const int tile = g >> 2, hh = (g >> 1) & 1, kb = g & 1;
    if (tile * 64 >= Lpad_in) {
      *reinterpret_cast<u32x4*>(dst + g * 16) = u32x4{0u, 0u, 0u, 0u};
      continue;
    }
    const bf16* s0 = src + tile * 64 + kb * 32 + hh * 8;
    const u32x4 r0 = *reinterpret_cast<const u32x4*>(s0);
    const u32x4 r1 = *reinterpret_cast<const u32x4*>(s0 + 16);
    const bf16* e0 = reinterpret_cast<const bf16*>(&r0);
    const bf16* e1 = reinterpret_cast<const bf16*>(&r1);
    float y[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      y[j] = fminf(fmaxf((float)e0[j] * inv, -448.f), 448.f);
      y[8 + j] = fminf(fmaxf((float)e1[j] * inv, -448.f), 448.f);
    }
    u32x4 o;
    o.x = e4m3x4(y[0], y[1], y[2], y[3]);
    o.y = e4m3x4(y[4], y[5], y[6], y[7]);
    o.z = e4m3x4(y[8], y[9], y[10], y[11]);
    o.w = e4m3x4(y[12], y[13], y[14], y[15]);
    // output positions of group g: tile*64 + hh*32 + kb*16 + r
    *reinterpret_cast<u32x4*>(dst + tile * 64 + hh * 32 + kb * 16) = o;
  }
  if (threadIdx.x == 0) scales[row] = m > 0.f ? m / 448.f : 0.f;
}

// Per-row E4M3 codes (scale = amax / 448): one workgroup per row of `cols` bf16 values (cols % 8 == 0).
// Element (row, n) of x at x + row ld + (n / 32) xbs + n % 32, its code at codes + row ldc + (n / 32) cbs +
// n % 32 (row-major: xbs = cbs = 32; K panels: see ActLayout).
__global__ __launch_bounds__(256) void quant_rows_kernel(const bf16* __restrict__ x, int64_t ld, int64_t xbs, int cols,
                                                         uint8_t* __restrict__ codes, int64_t ldc, int64_t cbs,
                                                         float* __restrict__ scales) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const bf16* src = x + row * ld;
  float m = 0.f;
  for (int c = threadIdx.x; c < cols / 8; c += 256) {  // chunk c: elements 8c .. 8c + 7
    const u32x4 raw = *reinterpret_cast<const u32x4*>(src + (c >> 2) * xbs + (c & 3) * 8);
    const bf16* e = reinterpret_cast<const bf16*>(&raw);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf((float)e[j]));
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = m > 0.f ? 448.f / m : 0.f;
  uint8_t* dst = codes + row * ldc;
  for (int c = threadIdx.x; c < cols / 8; c += 256) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(src + (c >> 2) * xbs + (c & 3) * 8);
    const bf16* e = reinterpret_cast<const bf16*>(&raw);
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = fminf(fmaxf((float)e[j] * inv, -448.f), 448.f);
    *reinterpret_cast<uint2*>(dst + (c >> 2) * cbs + (c & 3) * 8) = make_uint2(e4m3x4(y[0], y[1], y[2], y[3]), e4m3x4(y[4], y[5], y[6], y[7]));
  }
  if (threadIdx.x == 0) scales[row] = m > 0.f ? m / 448.f : 0.f;
}

// The same codes for x and codes in K panels (ActLayout ld = 32; xbs, cbs = 32 * rows per panel): a wave
// takes 8 consecutive rows.  Lane l reads the 8 values (16 bytes) of row r0 + (l % 32) / 4 at chunk l % 4
// of panel 2 j + l / 32, so each load covers the 512-byte runs of two panels, and the codes leave as
// 256-byte runs.  Rows past `rows` (up to the panels' padded row count) are read and coded but get no
// scale.
__global__ __launch_bounds__(256) void quant_rows_panels_kernel(const bf16* __restrict__ x, int64_t xbs, int rows,
                                                                int npanel, uint8_t* __restrict__ codes, int64_t cbs,
                                                                float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t r0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 8;
  if (r0 >= rows) return;  // uniform in the wave
  const int half = lane >> 5, ch = lane & 3;
  const int64_t row = r0 + ((lane & 31) >> 2);
  const bf16* src = x + row * 32 + ch * 8;  // panel p at src + p xbs
  float m = 0.f;
  for (int p = half; p < npanel; p += 2) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(src + p * xbs);
    const bf16* e = reinterpret_cast<const bf16*>(&raw);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf((float)e[j]));
  }
  // the row's 8 lanes: chunk (lane bits 0, 1) and panel parity (bit 5)
  m = fmaxf(m, __shfl_xor(m, 1, 64));
  m = fmaxf(m, __shfl_xor(m, 2, 64));
  m = fmaxf(m, __shfl_xor(m, 32, 64));
  const float inv = m > 0.f ? 448.f / m : 0.f;
  uint8_t* dst = codes + row * 32 + ch * 8;
  for (int p = half; p < npanel; p += 2) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(src + p * xbs);
    const bf16* e = reinterpret_cast<const bf16*>(&raw);
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = fminf(fmaxf((float)e[j] * inv, -448.f), 448.f);
    *reinterpret_cast<uint2*>(dst + p * cbs) = make_uint2(e4m3x4(y[0], y[1], y[2], y[3]), e4m3x4(y[4], y[5], y[6], y[7]));
  }
  if (half == 0 && ch == 0 && row < rows) scales[row] = m > 0.f ? m / 448.f : 0.f;
}

// Per-tensor E4M3 codes: amax over the whole tensor (non-negative floats order like their bits, so an
// unsigned atomic max collects it), then the codes.
__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* p, uint32_t v) { *p = v; }

__global__ __launch_bounds__(256) void amax_kernel(const bf16* __restrict__ x, int64_t n8, uint32_t* amax_bits) {
  __shared__ float red[4];
  float m = 0.f;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n8; c += (int64_t)gridDim.x * 256) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(x + c * 8);
    const bf16* e = reinterpret_cast<const bf16*>(&raw);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf((float)e[j]));
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(amax_bits, __float_as_uint(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))));
}

__global__ __launch_bounds__(256) void quant_tensor_kernel(const bf16* __restrict__ x, int64_t n8,
                                                           const uint32_t* __restrict__ amax_bits,
                                                           uint8_t* __restrict__ codes, float* __restrict__ scale) {
  const float m = __uint_as_float(*amax_bits);
  const float inv = m > 0.f ? 448.f / m : 0.f;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n8; c += (int64_t)gridDim.x * 256) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(x + c * 8);
    const bf16* e = reinterpret_cast<const bf16*>(&raw);
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = fminf(fmaxf((float)e[j] * inv, -448.f), 448.f);
    *reinterpret_cast<uint2*>(codes + c * 8) = make_uint2(e4m3x4(y[0], y[1], y[2], y[3]), e4m3x4(y[4], y[5], y[6], y[7]));
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale = m > 0.f ? m / 448.f : 0.f;
}

}  // namespace

hipError_t launch_quant_rows_e4m3(const bf16* x, ActLayout lx, int rows, int cols, uint8_t* codes, ActLayout lc,
                                  float* scales, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (cols <= 0 || cols % 8 != 0 || ((lx.bs != 32 || lc.bs != 32) && cols % 32 != 0)) return hipErrorInvalidValue;
  const int64_t pbs = 32 * panel_rows(rows);
  if (lx.ld == 32 && lc.ld == 32 && lx.bs == pbs && lc.bs == pbs) {  // both in K panels
    hipLaunchKernelGGL(quant_rows_panels_kernel, dim3((unsigned)ceil_div((int64_t)rows, (int64_t)32)), dim3(256), 0, s,
                       x, lx.bs, rows, cols / 32, codes, lc.bs, scales);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)rows), dim3(256), 0, s, x, lx.ld, lx.bs, cols, codes, lc.ld,
                     lc.bs, scales);
  return hipGetLastError();
}

hipError_t launch_quant_tensor_e4m3(const bf16* x, int64_t n, uint8_t* codes, float* scale, uint32_t* amax_word,
                                    hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n % 8 != 0) return hipErrorInvalidValue;
  const int64_t n8 = n / 8;
  const unsigned blocks = (unsigned)std::min<int64_t>(ceil_div(n8, 256), 2048);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(1), 0, s, amax_word, 0u);
  hipLaunchKernelGGL(amax_kernel, dim3(blocks), dim3(256), 0, s, x, n8, amax_word);
  hipLaunchKernelGGL(quant_tensor_kernel, dim3(blocks), dim3(256), 0, s, x, n8, amax_word, codes, scale);
  return hipGetLastError();
}

hipError_t launch_quant_q(const bf16* x, int64_t ld, int B, int S, int H, int hd, int8_t* codes, float* scales,
                          hipStream_t s) {
  const int64_t rows = (int64_t)B * S, threads = rows * H * (hd / 8);
  if (rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(threads, 256));
  if (hd == 128)
    hipLaunchKernelGGL((quant_q_kernel<bf16, 128>), grid, dim3(256), 0, s, x, ld, rows, S, H, codes, scales);
  else if (hd == 64)
    hipLaunchKernelGGL((quant_q_kernel<bf16, 64>), grid, dim3(256), 0, s, x, ld, rows, S, H, codes, scales);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_quant_k(const bf16* x, int64_t ld, int B, int S, int H, int hd, int8_t* codes, float* scales,
                          hipStream_t s) {
  if (B <= 0 || S <= 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(S, 64), (unsigned)H, (unsigned)B);
  if (hd == 128)
    hipLaunchKernelGGL((quant_k_kernel<bf16, 128>), grid, dim3(256), 0, s, x, ld, S, H, codes, scales);
  else if (hd == 64)
    hipLaunchKernelGGL((quant_k_kernel<bf16, 64>), grid, dim3(256), 0, s, x, ld, S, H, codes, scales);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_quant_vt(const bf16* vt, int64_t rows, int Lpad_in, int Lpad_out, uint8_t* out, float* scales,
                           hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (Lpad_in % 64 != 0 || Lpad_out % 64 != 0 || Lpad_out < Lpad_in) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_vt_kernel, dim3((unsigned)rows), dim3(256), 0, s, vt, Lpad_in, Lpad_out, out, scales);
  return hipGetLastError();
}

}  // namespace wan
