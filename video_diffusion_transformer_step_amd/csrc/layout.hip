// Bandwidth-bound layout kernels: image-to-video input build, (1,2,2) patchify /
// unpatchify, the CFG + flow-matching Euler update, dtype conversion and the
// per-head transpose of V used by the attention kernels.
#include "wan_internal.h"

#include <cmath>

namespace wan {

namespace {

struct MaskBits {
  uint64_t w[4];  // bit i = entry i of the 4T-entry frame sequence (T <= 64)
};

// x_in[b, c, t, h, w] = x_t (c < C) | mask (C <= c < C + 4) | z_img (c >= C + 4).
// "图解 Wan2.1 I2V" §4.1-§4.2: y = [mask (4), image latent (16)], x = [x_t, y]; the
// mask channel c of latent frame t is entry 4t + c of the frame sequence.
__global__ __launch_bounds__(256) void i2v_input_kernel(const float* __restrict__ x_t, const float* __restrict__ z,
                                                         MaskBits bits, int B, int C, int T, int HW,
                                                         float* __restrict__ x_in) {
  const int64_t per_b = (int64_t)(2 * C + 4) * T * HW;
  const int64_t n = (int64_t)B * per_b;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = i / per_b;
    const int64_t r = i - b * per_b;
    const int c = (int)(r / ((int64_t)T * HW));
    const int64_t thw = r - (int64_t)c * T * HW;
    float v;
    if (c < C) {
      v = x_t[(b * C + c) * (int64_t)T * HW + thw];
    } else if (c < C + 4) {
      const int t = (int)(thw / HW);
      const int e = 4 * t + (c - C);
      v = ((bits.w[e >> 6] >> (e & 63)) & 1ull) ? 1.f : 0.f;
    } else {
      v = z[(b * C + (c - C - 4)) * (int64_t)T * HW + thw];
    }
    x_in[i] = v;
  }
}

// p[b, (f*Hp + i)*Wp + j, c*4 + kh*2 + kw] = x[b, c, f, 2i + kh, 2j + kw]   ("图解 Wan2.1 I2V" §5.1)
// One thread per (b, token, c): reads two 8-byte pairs, writes 16 bytes.
__global__ __launch_bounds__(256) void patchify_kernel(const float* __restrict__ x, int B, int C, int T, int H,
                                                        int W, float* __restrict__ p) {
  const int Hp = H / 2, Wp = W / 2;
  const int64_t S = (int64_t)T * Hp * Wp;
  const int64_t n = (int64_t)B * S * C;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % C);
    const int64_t bs = i / C;
    const int64_t s = bs % S;
    const int64_t b = bs / S;
    const int j = (int)(s % Wp);
    const int ii = (int)((s / Wp) % Hp);
    const int f = (int)(s / ((int64_t)Wp * Hp));
    const float* src = x + (((b * C + c) * T + f) * H + 2 * ii) * (int64_t)W + 2 * j;
    const float2 top = *reinterpret_cast<const float2*>(src);
    const float2 bot = *reinterpret_cast<const float2*>(src + W);
    *reinterpret_cast<float4*>(p + i * 4) = make_float4(top.x, top.y, bot.x, bot.y);
  }
}

__global__ __launch_bounds__(256) void unpatchify_kernel(const float* __restrict__ p, int B, int C, int T, int H,
                                                          int W, float* __restrict__ x) {
  const int Hp = H / 2, Wp = W / 2;
  const int64_t S = (int64_t)T * Hp * Wp;
  const int64_t n = (int64_t)B * S * C;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % C);
    const int64_t bs = i / C;
    const int64_t s = bs % S;
    const int64_t b = bs / S;
    const int j = (int)(s % Wp);
    const int ii = (int)((s / Wp) % Hp);
    const int f = (int)(s / ((int64_t)Wp * Hp));
    const float4 v = *reinterpret_cast<const float4*>(p + i * 4);
    float* dst = x + (((b * C + c) * T + f) * H + 2 * ii) * (int64_t)W + 2 * j;
    *reinterpret_cast<float2*>(dst) = make_float2(v.x, v.y);
    *reinterpret_cast<float2*>(dst + W) = make_float2(v.z, v.w);
  }
}

// x <- x + dt * v,  v = v_u + s (v_c - v_u)  (or v = v_c without guidance).
// "图解 Wan2.1 I2V" §7 (CFG and the Euler step, t from 1 to 0 so dt < 0).
__device__ __forceinline__ float euler1(float x, float vc, float vu, float s, float dt, bool cfg) {
  const float v = cfg ? fmaf(s, vc - vu, vu) : vc;
  return fmaf(dt, v, x);
}

__global__ __launch_bounds__(256) void euler_kernel(float* __restrict__ x, const float* __restrict__ vc,
                                                     const float* __restrict__ vu, float s, float dt, int64_t n) {
  const bool cfg = vu != nullptr;
  const int64_t n4 = n / 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    float4 xv = reinterpret_cast<float4*>(x)[i];
    const float4 c = reinterpret_cast<const float4*>(vc)[i];
    const float4 u = cfg ? reinterpret_cast<const float4*>(vu)[i] : c;
    xv.x = euler1(xv.x, c.x, u.x, s, dt, cfg);
    xv.y = euler1(xv.y, c.y, u.y, s, dt, cfg);
    xv.z = euler1(xv.z, c.z, u.z, s, dt, cfg);
    xv.w = euler1(xv.w, c.w, u.w, s, dt, cfg);
    reinterpret_cast<float4*>(x)[i] = xv;
  }
  // tail (n % 4 elements), handled by the first threads
  const int64_t t = n4 * 4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) x[t] = euler1(x[t], vc[t], cfg ? vu[t] : 0.f, s, dt, cfg);
}

template <typename T>
__global__ __launch_bounds__(256) void convert_kernel(const float* __restrict__ in, T* __restrict__ out, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = from_f32<T>(in[i]);
}

// V^T[b, h, d, pos] = V[b, key(pos), h*hd + d] (+col0) for key < S, 0 for S <= key < Spad.
// In bf16 the keys are permuted within each 16-key group, key(pos) = pos with bits 2 and 3 swapped
// ([0-3, 8-11, 4-7, 12-15]), so that the 8 keys one attention MFMA lane-half consumes are one
// contiguous 16-byte chunk; fp32 keeps the natural order.  One workgroup per (64-token tile, head,
// batch row); LDS tile [64][hd + 1] elements.
template <typename T>
__global__ __launch_bounds__(256) void transpose_heads_kernel(const T* __restrict__ v, int64_t ld, int64_t col0,
                                                               int S, int H, int hd, int Spad, T* __restrict__ vt) {
  __shared__ T tile[64 * (128 + 1)];
  const int j0 = blockIdx.x * 64, h = blockIdx.y, b = blockIdx.z;
  const int P = hd + 1;
  for (int e = threadIdx.x; e < 64 * hd; e += 256) {
    const int r = e / hd, d = e % hd;
    const int j = j0 + r;
    tile[r * P + d] = (j < S) ? v[((int64_t)b * S + j) * ld + col0 + (int64_t)h * hd + d] : from_f32<T>(0.f);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * hd; e += 256) {
    const int d = e / 64, pos = e % 64;
    const int r = (sizeof(T) == 2) ? ((pos & ~12) | ((pos & 4) << 1) | ((pos & 8) >> 1)) : pos;
    const int j = j0 + pos;
    if (j < Spad) vt[(((int64_t)b * H + h) * hd + d) * Spad + j] = tile[r * P + d];
  }
}

// x += g * y over float4 groups: row m = i / d4, channels 4 (i % d4) ..; g from the row's batch entry.
__global__ __launch_bounds__(256) void gated_add_kernel(float* __restrict__ x, const float* __restrict__ y,
                                                        const float* __restrict__ mod, int chunk, int64_t n4, int d4,
                                                        int S) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / d4;
    const int c4 = (int)(i - m * d4);
    const int64_t b = m / S;
    const float4 g = reinterpret_cast<const float4*>(mod + (b * 6 + chunk) * (int64_t)d4 * 4)[c4];
    const float4 v = reinterpret_cast<const float4*>(y)[i];
    float4 r = reinterpret_cast<float4*>(x)[i];
    r.x = fmaf(g.x, v.x, r.x);
    r.y = fmaf(g.y, v.y, r.y);
    r.z = fmaf(g.z, v.z, r.z);
    r.w = fmaf(g.w, v.w, r.w);
    reinterpret_cast<float4*>(x)[i] = r;
  }
}

__global__ __launch_bounds__(256) void mod_combine_kernel(const float* __restrict__ e0, const float* __restrict__ mb,
                                                          int B, int dim, float* __restrict__ mod) {
  const int64_t n = (int64_t)B * 6 * dim;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    mod[i] = e0[i] + mb[i % (6 * (int64_t)dim)];
}

// The launch before the block's Q/K/V product (see launch_attn_prologue): entries [0, nrope) write the
// 3D RoPE table ("图解 Wan2.1 I2V" §5.3 ②) the product's epilogue reads, the rest clear the padded key
// positions S .. Spad - 1 of each V^T row.  Table entry (pos, m) of a segment of width n holds the
// cosine and sine of pos * theta^(-2m/n), computed in double precision: frame rows (nT x npT pairs),
// then height rows (nH x npH), then width rows (nW x npH).
template <typename T>
__global__ __launch_bounds__(256) void attn_prologue_kernel(T* __restrict__ vt, int64_t rows, int S, int Spad,
                                                            float2* __restrict__ rope, int nT, int nH, int nW,
                                                            int npT, int npH, double log2_theta) {
  const int w = Spad - S;
  const int64_t eT = (int64_t)nT * npT, eH = (int64_t)nH * npH;
  const int64_t nrope = eT + eH + (int64_t)nW * npH;
  const int64_t n = nrope + rows * w;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    if (i < nrope) {
      int64_t k = i;
      int np = npT;
      if (k >= eT) {
        k -= eT;
        np = npH;
        if (k >= eH) k -= eH;
      }
      const int pos = (int)(k / np), m = (int)(k % np);
      const double a = (double)pos * exp2(-(double)(2 * m) / (double)(2 * np) * log2_theta);
      rope[i] = make_float2((float)cos(a), (float)sin(a));
    } else {
      const int64_t t = i - nrope, r = t / w;
      vt[r * Spad + S + (t - r * w)] = from_f32<T>(0.f);
    }
  }
}

inline unsigned grid_for(int64_t n, int per_thread = 1) {
  int64_t blocks = ceil_div(ceil_div(n, per_thread), 256);
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  return (unsigned)blocks;
}

}  // namespace

hipError_t launch_i2v_input(const float* x_t, const float* z_img, const uint64_t mask_bits[4], int B, int C, int T,
                            int H, int W, float* x_in, hipStream_t s) {
  MaskBits bits{{mask_bits[0], mask_bits[1], mask_bits[2], mask_bits[3]}};
  const int64_t n = (int64_t)B * (2 * C + 4) * T * H * W;
  hipLaunchKernelGGL(i2v_input_kernel, dim3(grid_for(n)), dim3(256), 0, s, x_t, z_img, bits, B, C, T, H * W, x_in);
  return hipGetLastError();
}

hipError_t launch_patchify(const float* x, int B, int C, int T, int H, int W, float* p, hipStream_t s) {
  const int64_t n = (int64_t)B * T * (H / 2) * (W / 2) * C;
  hipLaunchKernelGGL(patchify_kernel, dim3(grid_for(n)), dim3(256), 0, s, x, B, C, T, H, W, p);
  return hipGetLastError();
}

hipError_t launch_unpatchify(const float* p, int B, int C, int T, int H, int W, float* x, hipStream_t s) {
  const int64_t n = (int64_t)B * T * (H / 2) * (W / 2) * C;
  hipLaunchKernelGGL(unpatchify_kernel, dim3(grid_for(n)), dim3(256), 0, s, p, B, C, T, H, W, x);
  return hipGetLastError();
}

hipError_t launch_euler(float* x, const float* v_c, const float* v_u, float guidance, float dt, int64_t n,
                        hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(euler_kernel, dim3(grid_for(n, 4)), dim3(256), 0, s, x, v_c, v_u, guidance, dt, n);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_convert(const float* in, T* out, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(convert_kernel<T>, dim3(grid_for(n)), dim3(256), 0, s, in, out, n);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_transpose_heads(const T* v, int64_t ld, int64_t col0, int B, int S, int H, int hd, int Spad,
                                  T* vt, hipStream_t s) {
  if (hd > 128) return hipErrorInvalidValue;
  dim3 grid((unsigned)ceil_div(Spad, 64), (unsigned)H, (unsigned)B);
  hipLaunchKernelGGL(transpose_heads_kernel<T>, grid, dim3(256), 0, s, v, ld, col0, S, H, hd, Spad, vt);
  return hipGetLastError();
}

hipError_t launch_gated_add(float* x, const float* y, const float* mod, int chunk, int64_t rows, int dim, int S,
                            hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (dim % 4 != 0) return hipErrorInvalidValue;
  const int64_t n4 = rows * (dim / 4);
  hipLaunchKernelGGL(gated_add_kernel, dim3(grid_for(n4)), dim3(256), 0, s, x, y, mod, chunk, n4, dim / 4, S);
  return hipGetLastError();
}

hipError_t launch_mod_combine(const float* e0, const float* mb, int B, int dim, float* mod, hipStream_t s) {
  const int64_t n = (int64_t)B * 6 * dim;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(mod_combine_kernel, dim3(grid_for(n)), dim3(256), 0, s, e0, mb, B, dim, mod);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_attn_prologue(T* vt, int64_t rows, int S, int Spad, float2* rope, int T_, int Hp, int Wp, int hd,
                                float theta, hipStream_t s) {
  if (hd < 4 || !(theta > 0.f)) return hipErrorInvalidValue;
  // bf16 V^T permutes keys within 16-key groups, so a padded key of the last group can sit at a
  // position below S: clear from the start of that group (the real keys are written afterwards).
  const int S16 = S & ~15;
  const int npT = rope_pairs_time(hd), npH = rope_pairs_space(hd);
  const int64_t nrope = (int64_t)T_ * npT + (int64_t)(Hp + Wp) * npH;
  const int64_t ntail = Spad > S16 && rows > 0 ? rows * (Spad - S16) : 0;
  hipLaunchKernelGGL(attn_prologue_kernel<T>, dim3(grid_for(nrope + ntail)), dim3(256), 0, s, vt, ntail ? rows : 0,
                     S16, Spad, rope, T_, Hp, Wp, npT, npH, std::log2((double)theta));
  return hipGetLastError();
}

// Row-major [rows, cols] -> K panels of 32 elements ([cols / 32][prow][32], rows past `rows` zero): one
// thread per 16-byte chunk of the destination, which is written in order.
__global__ __launch_bounds__(256) void pack_panels_kernel(const uint8_t* __restrict__ src, int64_t rows,
                                                           int64_t ld_bytes, int64_t prow, int pb, int64_t nchunks,
                                                           uint8_t* __restrict__ dst) {
  const int cpr = pb / 16;  // chunks per panel row
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < nchunks; q += (int64_t)gridDim.x * blockDim.x) {
    const int j = (int)(q % cpr);
    const int64_t t = q / cpr, n = t % prow, p = t / prow;
    u32x4 v{0u, 0u, 0u, 0u};
    if (n < rows) v = *reinterpret_cast<const u32x4*>(src + n * ld_bytes + p * pb + j * 16);
    *reinterpret_cast<u32x4*>(dst + q * 16) = v;
  }
}

hipError_t launch_pack_panels(const void* src, int64_t rows, int64_t cols, int64_t ld, int elem_bytes, void* dst,
                              hipStream_t s) {
  if (rows < 0 || cols < 0 || cols % 32 != 0 || (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4) ||
      (ld * elem_bytes) % 16 != 0 || ld < cols)
    return hipErrorInvalidValue;
  const int64_t prow = panel_rows(rows), pb = 32 * elem_bytes;
  const int64_t nchunks = cols / 32 * prow * (pb / 16);
  if (nchunks == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_panels_kernel, dim3(grid_for(nchunks)), dim3(256), 0, s,
                     static_cast<const uint8_t*>(src), rows, ld * elem_bytes, prow, (int)pb, nchunks,
                     static_cast<uint8_t*>(dst));
  return hipGetLastError();
}

template hipError_t launch_attn_prologue<float>(float*, int64_t, int, int, float2*, int, int, int, int, float,
                                                hipStream_t);
template hipError_t launch_attn_prologue<bf16>(bf16*, int64_t, int, int, float2*, int, int, int, int, float,
                                               hipStream_t);
template hipError_t launch_convert<float>(const float*, float*, int64_t, hipStream_t);
template hipError_t launch_convert<bf16>(const float*, bf16*, int64_t, hipStream_t);
template hipError_t launch_transpose_heads<float>(const float*, int64_t, int64_t, int, int, int, int, int, float*,
                                                  hipStream_t);
template hipError_t launch_transpose_heads<bf16>(const bf16*, int64_t, int64_t, int, int, int, int, int, bf16*,
                                                 hipStream_t);

}  // namespace wan
