// Shared device helpers for the gfx950 (CDNA4) kernels of the Wan DiT step.
//
// Storage types: float (f32 mode) and bf16 (__bf16, bf16 mode).  GEMM and
// attention operands are one of the two; accumulation, norms, statistics,
// modulation, the residual stream and latents are always fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wan {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// 16-byte load/store unit used for every global <-> LDS move.
struct alignas(16) u32x4 {
  uint32_t x, y, z, w;
};

template <typename T> struct dtype_traits;
template <> struct dtype_traits<float> {
  static constexpr int per16 = 4;  // elements per 16 bytes
};
template <> struct dtype_traits<bf16> {
  static constexpr int per16 = 8;
};
template <> struct dtype_traits<uint8_t> {  // INT8 / FP8 codes
  static constexpr int per16 = 16;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

// Wave-wide (64 lanes) reductions without LDS traffic.  The first four butterfly steps stay inside
// 16-lane rows and use DPP lane permutes (quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror); the last two exchange 16-lane rows and 32-lane halves with
// v_permlane16_swap / v_permlane32_swap.  Every step pairs lanes symmetrically, so all lanes end
// with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// (a, b) = (v of this lane, v of lane ^ 16) or (v, v of lane ^ 32), in some order per lane.
__device__ __forceinline__ void swap16(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
// v + (v of lane ^ 32), v max (v of lane ^ 32)
__device__ __forceinline__ float half_sum(float v) {
  float a, b;
  swap32(v, a, b);
  return a + b;
}
__device__ __forceinline__ float half_max(float v) {
  float a, b;
  swap32(v, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float wave_sum(float v) {
  float a, b;
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  swap16(v, a, b);
  v = a + b;
  return half_sum(v);
}
__device__ __forceinline__ float wave_max(float v) {
  float a, b;
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  swap16(v, a, b);
  v = fmaxf(a, b);
  return half_max(v);
}

// ---------------------------------------------------------------------------
// MFMA 32x32 helpers.  One "k-chunk" is 32 bytes of K per operand row: lane l
// supplies row (l % 32) and the 16 bytes at byte offset (l / 32) * 16 of the
// chunk.  For bf16 that is one v_mfma_f32_32x32x16_bf16 (8 elements per lane);
// for f32 it is four v_mfma_f32_32x32x2_f32, instruction i taking element i of
// the lane's 4 (lane half h then holds k = 4h + i, so A and B agree on k).
// Output layout (both): lane l holds column (l % 32) and rows
// (j / 4) * 8 + (l / 32) * 4 + (j % 4), j = 0..15.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void mfma_chunk(const u32x4& a, const u32x4& b, f32x16& acc, bf16) {
  bf16x8 av = __builtin_bit_cast(bf16x8, a);
  bf16x8 bv = __builtin_bit_cast(bf16x8, b);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma_chunk(const u32x4& a, const u32x4& b, f32x16& acc, float) {
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// ---------------------------------------------------------------------------
// 3D RoPE ("图解 Wan2.1 I2V" §5.3 ②), shared by the Q/K/V projection epilogue and the standalone
// rotation pass.  A head's channels split into time / height / width segments of sizes
// hd - 4*(hd/6), 2*(hd/6), 2*(hd/6); pair (2m, 2m+1) of a segment of width n rotates by
// pos * theta^(-2m/n), pos being the token's frame / row / column index.
// ---------------------------------------------------------------------------
// Pairs per head in the time segment, and in each of the two spatial segments.
__host__ __device__ __forceinline__ int rope_pairs_time(int hd) { return (hd - 4 * (hd / 6)) / 2; }
__host__ __device__ __forceinline__ int rope_pairs_space(int hd) { return hd / 6; }
struct RopePair {
  float freq;
  int axis;  // 0 frame, 1 row, 2 column
};
// The pair starting at head channel d (even).
__device__ __forceinline__ RopePair rope_pair(int d, int hd, float log2_theta) {
  const int q6 = hd / 6;
  const int dT = hd - 4 * q6, dH = 2 * q6;
  int m, n, axis;
  if (d < dT) {
    m = d >> 1; n = dT; axis = 0;
  } else if (d < dT + dH) {
    m = (d - dT) >> 1; n = dH; axis = 1;
  } else {
    m = (d - dT - dH) >> 1; n = dH; axis = 2;
  }
  return RopePair{exp2f(-(float)(2 * m) / (float)n * log2_theta), axis};
}
// (frame, row, column) of position s in a frames x Hp x Wp token grid (row-major).
struct RopePos {
  int f, i, j;
};
__device__ __forceinline__ RopePos rope_pos(int s, int Hp, int Wp) {
  return RopePos{s / (Wp * Hp), (s / Wp) % Hp, s % Wp};
}
// The pair's cosine and sine at a token position, by the hardware sine / cosine (angles here are at
// most a few hundred radians, where their error stays near 1e-6).
__device__ __forceinline__ void rope_cs(const RopePair& p, const RopePos& t, float& c, float& s) {
  const int pos = p.axis == 0 ? t.f : (p.axis == 1 ? t.i : t.j);
  const float a = (float)pos * p.freq;
  s = __sinf(a);
  c = __cosf(a);
}

__host__ __device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ __forceinline__ int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

}  // namespace wan
