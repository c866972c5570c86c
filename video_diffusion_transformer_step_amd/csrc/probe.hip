// Device ceilings for the roofline figures: a kernel that issues nothing but matrix-core
// instructions on register operands (no LDS, no global loads apart from one store per lane at the
// end), so its rate is what the MFMA units sustain at the clock the chip holds under that load.
// The step's kernels are quoted against the nominal peak; this gives the measured one beside it.
#include "wan_internal.h"

namespace wan {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int PROBE_THREADS = 256;

// KIND 0: v_mfma_f32_32x32x16_bf16 (a_word, b_word = two equal bf16 halves each);
// KIND 1: v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 with unit block scales (four equal code bytes);
// KIND 2: v_mfma_f32_32x32x16_bf16 on operands that differ per lane and per instruction: four A and
//   four B register quads per lane, each bf16 with a hashed sign and mantissa and exponent 2^-1 or
//   2^0 (hash seeded by a_word).  The matrix core's power draw depends on how many operand bits
//   toggle; constant operands (kind 0) toggle none, data like a real product's toggle about half.
// Four independent accumulators per wave, so an MFMA's result is needed again only four instructions
// later.  Every lane ends with the sum of its 64 accumulator elements:
//   64 * K * iters * a * b   (K = 16 for bf16, 64 for E4M3),
// which the caller can check, so the instruction stream is known to have run in full.
// Lowbias32 integer hash (C. Wellons), used only to draw the kind-2 operands.
__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

template <int KIND>
__global__ __launch_bounds__(PROBE_THREADS) void mfma_peak_kernel(uint32_t a_word, uint32_t b_word, int iters,
                                                                  float* out) {
  f32x16 acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
  if constexpr (KIND == 2) {
    const uint32_t tid = blockIdx.x * PROBE_THREADS + threadIdx.x;
    bf16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t aw[4], bw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t h = probe_hash(a_word ^ (tid * 16u + (uint32_t)(i * 4 + j)));
        aw[j] = (h & 0x807f807fu) | 0x3f003f00u;  // sign, mantissa hashed; exponent 126 or 127
        bw[j] = (probe_hash(h ^ b_word) & 0x807f807fu) | 0x3f003f00u;
      }
      a[i] = __builtin_bit_cast(bf16x8, aw);
      b[i] = __builtin_bit_cast(bf16x8, bw);
    }
    for (int i = 0; i < iters; ++i) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[1], acc1, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[2], acc2, 0, 0, 0);
      acc3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[3], b[3], acc3, 0, 0, 0);
    }
  } else if constexpr (KIND == 0) {
    const u32x4 aw = {a_word, a_word, a_word, a_word}, bw = {b_word, b_word, b_word, b_word};
    const bf16x8 a = __builtin_bit_cast(bf16x8, aw), b = __builtin_bit_cast(bf16x8, bw);
    for (int i = 0; i < iters; ++i) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc1, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc2, 0, 0, 0);
      acc3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc3, 0, 0, 0);
    }
  } else {
    const int ai = (int)a_word, bi = (int)b_word;
    const v8i a = {ai, ai, ai, ai, ai, ai, ai, ai}, b = {bi, bi, bi, bi, bi, bi, bi, bi};
    for (int i = 0; i < iters; ++i) {
      acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc0, 0, 0, 0, 127, 0, 127);
      acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc1, 0, 0, 0, 127, 0, 127);
      acc2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc2, 0, 0, 0, 127, 0, 127);
      acc3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc3, 0, 0, 0, 127, 0, 127);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += (acc0[j] + acc1[j]) + (acc2[j] + acc3[j]);
  out[(int64_t)blockIdx.x * PROBE_THREADS + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_peak(int kind, uint32_t a_word, uint32_t b_word, int blocks, int iters, float* out,
                            hipStream_t s) {
  if (kind == 0)
    hipLaunchKernelGGL(mfma_peak_kernel<0>, dim3(blocks), dim3(PROBE_THREADS), 0, s, a_word, b_word, iters, out);
  else if (kind == 1)
    hipLaunchKernelGGL(mfma_peak_kernel<1>, dim3(blocks), dim3(PROBE_THREADS), 0, s, a_word, b_word, iters, out);
  else
    hipLaunchKernelGGL(mfma_peak_kernel<2>, dim3(blocks), dim3(PROBE_THREADS), 0, s, a_word, b_word, iters, out);
  return hipGetLastError();
}

}  // namespace wan
