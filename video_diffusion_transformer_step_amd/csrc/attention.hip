// Flash-style attention on 32x32 MFMA for the DiT's full 3D self-attention and
// its (single- or dual-stream) cross-attention.
//
// What it computes: o = softmax(q k^T / sqrt(hd)) v per (batch row, head), over
// all keys, no mask ("图解 Wan2.1 I2V" §5.3; "Wan 技术深度解析" §2.5: global,
// non-causal attention).  With two key/value streams it returns the sum of the
// two separately normalised attentions ("图解 Wan2.1 I2V" §5.4: image and text
// branches share q, each has its own softmax, outputs are added).
//
// How (gfx950): one workgroup = 4 waves = 128 queries of one (b, head); each
// wave owns 32 queries.  Scores are formed transposed, S^T = K Q^T, so MFMA lane l
// holds query (l % 32) and 16 keys per 32-key block: the row max and row sum are
// in-lane plus a single exchange with lane l ^ 32.  The same register layout is
// the B operand of O^T = V^T P^T, so P never leaves registers.  K tiles
// [64 keys][hd] and V^T tiles [hd][64 keys] (V is pre-transposed per head in HBM)
// are double-buffered in LDS with register prefetch.  The running maximum is only
// moved when a new score exceeds it by more than 2^8 (in exp2 units), so the O
// rescale (hd/32 x 16 multiplies per lane) is rare; p <= 256 keeps fp32 and bf16
// safe.  log2(e)/sqrt(hd) is folded into one fma before exp2.
#include "wan_internal.h"

namespace wan {

namespace {

constexpr int KT = 64;   // keys per tile
constexpr float RESCALE_THRESHOLD = 8.f;

template <typename T, int HD>
struct AttnCfg {
  static constexpr int E16 = dtype_traits<T>::per16;
  static constexpr int ROWB = HD * (int)sizeof(T);      // bytes per K row
  static constexpr int KROW = HD + E16;                 // padded K row (elements)
  static constexpr int VROWB = KT * (int)sizeof(T);     // bytes per V^T row
  static constexpr int VROW = KT + 4;                   // padded V^T row (+4 elements)
  static constexpr int NCH = ROWB / 32;                 // 32-byte k-chunks along hd
  static constexpr int KCH = KT * ROWB / 16 / 256;      // 16-byte K chunks per thread
  static constexpr int VCH = HD * VROWB / 16 / 256;     // 16-byte V^T chunks per thread
  static constexpr int KBUF = KT * KROW;                // elements
  static constexpr int VBUF = HD * VROW;
  static constexpr int BUF = KBUF + VBUF;
  static constexpr int ND = HD / 32;                    // 32-wide d blocks of O^T
};

template <typename T, int HD, int QB>
struct StreamState {
  f32x16 o[QB][AttnCfg<T, HD>::ND];
  float m[QB], l[QB];
};

template <typename T, int HD>
__device__ __forceinline__ void load_kv_tile(const T* __restrict__ kbase, int64_t k_ss, const T* __restrict__ vtb,
                                             int Lpad, int L, int j0, int tid, u32x4* rk, u32x4* rv) {
  using C = AttnCfg<T, HD>;
  constexpr int KC_ROW = C::ROWB / 16;
#pragma unroll
  for (int i = 0; i < C::KCH; ++i) {
    const int c = tid + i * 256, r = c / KC_ROW, cc = c % KC_ROW;
    const int j = j0 + r;
    rk[i] = (j < L) ? *reinterpret_cast<const u32x4*>(kbase + (int64_t)j * k_ss + cc * C::E16) : u32x4{0, 0, 0, 0};
  }
  constexpr int VC_ROW = C::VROWB / 16;
#pragma unroll
  for (int i = 0; i < C::VCH; ++i) {
    const int c = tid + i * 256, d = c / VC_ROW, cc = c % VC_ROW;
    rv[i] = *reinterpret_cast<const u32x4*>(vtb + (int64_t)d * Lpad + j0 + cc * C::E16);
  }
}

template <typename T, int HD>
__device__ __forceinline__ void store_kv_tile(T* buf, int tid, const u32x4* rk, const u32x4* rv) {
  using C = AttnCfg<T, HD>;
  constexpr int KC_ROW = C::ROWB / 16;
#pragma unroll
  for (int i = 0; i < C::KCH; ++i) {
    const int c = tid + i * 256, r = c / KC_ROW, cc = c % KC_ROW;
    *reinterpret_cast<u32x4*>(buf + r * C::KROW + cc * C::E16) = rk[i];
  }
  T* vb = buf + C::KBUF;
  constexpr int VC_ROW = C::VROWB / 16;
#pragma unroll
  for (int i = 0; i < C::VCH; ++i) {
    const int c = tid + i * 256, d = c / VC_ROW, cc = c % VC_ROW;
    uint2* p = reinterpret_cast<uint2*>(vb + d * C::VROW + cc * C::E16);
    p[0] = make_uint2(rv[i].x, rv[i].y);
    p[1] = make_uint2(rv[i].z, rv[i].w);
  }
}

// One key/value stream for the wave's QB x 32 queries; accumulates into st.  Every K / V^T
// fragment read from LDS feeds QB MFMAs (one per 32-query block).
template <typename T, int HD, int QB>
__device__ __forceinline__ void attend_stream(const u32x4 (&qf)[QB][AttnCfg<T, HD>::NCH], const KVStream& kv, int b,
                                              int h, int H, float c_log2, T* smem, StreamState<T, HD, QB>& st) {
  using C = AttnCfg<T, HD>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int lrow = lane & 31, lhalf = lane >> 5;
  const T* kbase = reinterpret_cast<const T*>(kv.k) + (int64_t)b * kv.k_bs + (int64_t)h * HD;
  const T* vtb = reinterpret_cast<const T*>(kv.vt) + ((int64_t)b * H + h) * HD * (int64_t)kv.Lpad;
  const int ntiles = (kv.L + KT - 1) / KT;

  u32x4 rk[C::KCH], rv[C::VCH];
  load_kv_tile<T, HD>(kbase, kv.k_ss, vtb, kv.Lpad, kv.L, 0, tid, rk, rv);
  __syncthreads();  // previous users of the LDS buffers are done
  store_kv_tile<T, HD>(smem, tid, rk, rv);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int j0 = t * KT;
    if (t + 1 < ntiles) load_kv_tile<T, HD>(kbase, kv.k_ss, vtb, kv.Lpad, kv.L, j0 + KT, tid, rk, rv);
    const T* kb_lds = smem + buf * C::BUF;
    const T* vb_lds = kb_lds + C::KBUF;

    // S^T for two 32-key blocks and QB query blocks.
    f32x16 s[QB][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int q = 0; q < QB; ++q) s[q][kb] = zero16();
      const T* kr = kb_lds + (kb * 32 + lrow) * C::KROW + lhalf * C::E16;
#pragma unroll
      for (int c = 0; c < C::NCH; ++c) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kr + c * 2 * C::E16);
#pragma unroll
        for (int q = 0; q < QB; ++q) mfma_chunk(a, qf[q][c], s[q][kb], T());
      }
    }
    // mask keys beyond L (only the last tile can hold any)
    if (j0 + KT > kv.L) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + kb * 32 + (r >> 2) * 8 + lhalf * 4 + (r & 3);
          if (key >= kv.L) {
#pragma unroll
            for (int q = 0; q < QB; ++q) s[q][kb][r] = (-__builtin_inff());
          }
        }
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      float mx = (-__builtin_inff());
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[q][kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = mx * c_log2;
      const bool need = mnew > st.m[q] + RESCALE_THRESHOLD;
      if (__ballot(need) != 0ull) {
        const float mm = need ? mnew : st.m[q];
        const float alpha = __builtin_amdgcn_exp2f(st.m[q] - mm);  // 0 on the first tile (m = -inf)
        st.m[q] = mm;
        st.l[q] *= alpha;
#pragma unroll
        for (int d = 0; d < C::ND; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) st.o[q][d][r] *= alpha;
      }
      const float negm = -st.m[q];
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // raw v_exp_f32: the argument is <= RESCALE_THRESHOLD or -inf, so no range fix-up is needed
          const float p = __builtin_amdgcn_exp2f(fmaf(s[q][kb][r], c_log2, negm));
          s[q][kb][r] = p;
          lsum += p;
        }
      st.l[q] += lsum;
    }

    // O^T += V^T P^T
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {  // 16-key chunks
        const int kb = c >> 1, r0 = (c & 1) * 8;
        u32x4 pb[QB];
#pragma unroll
        for (int q = 0; q < QB; ++q) {
          bf16x8 pk;
#pragma unroll
          for (int i = 0; i < 8; ++i) pk[i] = (bf16)s[q][kb][r0 + i];
          pb[q] = __builtin_bit_cast(u32x4, pk);
        }
#pragma unroll
        for (int d = 0; d < C::ND; ++d) {
          const T* vr = vb_lds + (d * 32 + lrow) * C::VROW + c * 16 + lhalf * 4;
          const uint2 lo = *reinterpret_cast<const uint2*>(vr);
          const uint2 hi = *reinterpret_cast<const uint2*>(vr + 8);
          const u32x4 a{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
          for (int q = 0; q < QB; ++q) mfma_chunk(a, pb[q], st.o[q][d], T());
        }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
#pragma unroll
          for (int d = 0; d < C::ND; ++d) {
            const T* vr = vb_lds + (d * 32 + lrow) * C::VROW + kb * 32 + g * 8 + lhalf * 4;
            const u32x4 a = *reinterpret_cast<const u32x4*>(vr);
#pragma unroll
            for (int q = 0; q < QB; ++q) {
              const u32x4 pb{__float_as_uint(s[q][kb][4 * g]), __float_as_uint(s[q][kb][4 * g + 1]),
                             __float_as_uint(s[q][kb][4 * g + 2]), __float_as_uint(s[q][kb][4 * g + 3])};
              mfma_chunk(a, pb, st.o[q][d], T());
            }
          }
        }
    }
    if (t + 1 < ntiles) store_kv_tile<T, HD>(smem + (buf ^ 1) * C::BUF, tid, rk, rv);
    __syncthreads();
  }
}

template <typename T, int HD, int NS, int QB>
__global__ __launch_bounds__(256, QB == 1 ? 2 : 1) void attention_kernel(
    const T* __restrict__ q, int64_t q_bs, int64_t q_ss, KVStream s0, KVStream s1, int S, int H, float c_log2,
    T* __restrict__ o, int64_t o_bs, int64_t o_ss) {
  using C = AttnCfg<T, HD>;
  __shared__ u32x4 smem_raw[2 * C::BUF * sizeof(T) / 16];
  T* smem = reinterpret_cast<T*>(smem_raw);
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int qrow0 = blockIdx.x * (4 * QB * 32) + wave * (QB * 32) + lrow;

  // Q^T as the B operand: lane holds query qrow, 16 bytes per 32-byte chunk of hd.
  u32x4 qf[QB][C::NCH];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = qrow0 + qb * 32;
    const T* qp = q + (int64_t)b * q_bs + (int64_t)qrow * q_ss + (int64_t)h * HD + lhalf * C::E16;
#pragma unroll
    for (int c = 0; c < C::NCH; ++c)
      qf[qb][c] = (qrow < S) ? *reinterpret_cast<const u32x4*>(qp + c * 2 * C::E16) : u32x4{0, 0, 0, 0};
  }

  StreamState<T, HD, QB> st;
  f32x16 acc[QB][C::ND];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int d = 0; d < C::ND; ++d) {
      st.o[qb][d] = zero16();
      if (NS > 1) acc[qb][d] = zero16();
    }
#pragma unroll
  for (int si = 0; si < NS; ++si) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      st.m[qb] = (-__builtin_inff());
      st.l[qb] = 0.f;
      if (si > 0) {
#pragma unroll
        for (int d = 0; d < C::ND; ++d) st.o[qb][d] = zero16();
      }
    }
    attend_stream<T, HD, QB>(qf, si == 0 ? s0 : s1, b, h, H, c_log2, smem, st);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float inv = 1.f / (st.l[qb] + __shfl_xor(st.l[qb], 32, 64));
#pragma unroll
      for (int d = 0; d < C::ND; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (NS > 1) acc[qb][d][r] += st.o[qb][d][r] * inv;
          else acc[qb][d][r] = st.o[qb][d][r] * inv;
        }
    }
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = qrow0 + qb * 32;
    if (qrow >= S) continue;
    T* op = o + (int64_t)b * o_bs + (int64_t)qrow * o_ss + (int64_t)h * HD;
#pragma unroll
    for (int d = 0; d < C::ND; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = d * 32 + g * 8 + lhalf * 4;
        if constexpr (sizeof(T) == 2) {
          bf16x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = (bf16)acc[qb][d][4 * g + i];
          *reinterpret_cast<bf16x4*>(op + dd) = v;
        } else {
          *reinterpret_cast<float4*>(op + dd) =
              make_float4(acc[qb][d][4 * g], acc[qb][d][4 * g + 1], acc[qb][d][4 * g + 2], acc[qb][d][4 * g + 3]);
        }
      }
  }
}

#ifndef WAN_ATTN_QB
#define WAN_ATTN_QB 1
#endif

template <typename T, int HD>
hipError_t launch_hd(const T* q, int64_t q_bs, int64_t q_ss, KVStream s0, KVStream s1, int nstreams, int B, int S,
                     int H, float c_log2, T* o, int64_t o_bs, int64_t o_ss, hipStream_t s) {
  constexpr int QB = (sizeof(T) == 2 && HD == 128) ? WAN_ATTN_QB : 1;
  dim3 grid((unsigned)ceil_div(S, 4 * QB * 32), (unsigned)H, (unsigned)B);
  if (nstreams == 2)
    hipLaunchKernelGGL((attention_kernel<T, HD, 2, 1>), dim3((unsigned)ceil_div(S, 128), H, B), dim3(256), 0, s, q,
                       q_bs, q_ss, s0, s1, S, H, c_log2, o, o_bs, o_ss);
  else
    hipLaunchKernelGGL((attention_kernel<T, HD, 1, QB>), grid, dim3(256), 0, s, q, q_bs, q_ss, s0, s1, S, H, c_log2,
                       o, o_bs, o_ss);
  return hipGetLastError();
}

}  // namespace

template <typename T>
hipError_t launch_attention(const T* q, int64_t q_bs, int64_t q_ss, KVStream s0, KVStream s1, int nstreams, int B,
                            int S, int H, int hd, float scale, T* o, int64_t o_bs, int64_t o_ss, hipStream_t s) {
  if (S <= 0 || B <= 0 || H <= 0) return hipSuccess;
  if (nstreams < 1 || nstreams > 2) return hipErrorInvalidValue;
  if (s0.L <= 0 || s0.Lpad % KT != 0 || s0.Lpad < s0.L) return hipErrorInvalidValue;
  if (nstreams == 2 && (s1.L <= 0 || s1.Lpad % KT != 0 || s1.Lpad < s1.L)) return hipErrorInvalidValue;
  const float c_log2 = scale * 1.4426950408889634f;
  if (hd == 128) return launch_hd<T, 128>(q, q_bs, q_ss, s0, s1, nstreams, B, S, H, c_log2, o, o_bs, o_ss, s);
  if (hd == 64) return launch_hd<T, 64>(q, q_bs, q_ss, s0, s1, nstreams, B, S, H, c_log2, o, o_bs, o_ss, s);
  return hipErrorInvalidValue;
}

template hipError_t launch_attention<float>(const float*, int64_t, int64_t, KVStream, KVStream, int, int, int, int,
                                            int, float, float*, int64_t, int64_t, hipStream_t);
template hipError_t launch_attention<bf16>(const bf16*, int64_t, int64_t, KVStream, KVStream, int, int, int, int,
                                           int, float, bf16*, int64_t, int64_t, hipStream_t);

}  // namespace wan
