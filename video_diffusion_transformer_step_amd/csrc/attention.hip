// Flash-style attention on 32x32 MFMA for the DiT's full 3D self-attention and
// its (single- or dual-stream) cross-attention.
//
// What it computes: o = softmax(q k^T / sqrt(hd)) v per (batch row, head), over
// all keys, no mask ("图解 Wan2.1 I2V" §5.3; "Wan 技术深度解析" §2.5: global,
// non-causal attention).  With two key/value streams it returns the sum of the
// two separately normalised attentions ("图解 Wan2.1 I2V" §5.4: image and text
// branches share q, each has its own softmax, outputs are added).
//
// How (gfx950):
//  * one workgroup = 4 waves = 128 queries of one (b, head); each wave owns 32
//    queries, held in registers as the B operand of S^T = K Q^T.  MFMA lane l then
//    holds query (l % 32) and 16 keys per 32-key block, so the row max / sum are
//    in-lane plus one exchange with lane l ^ 32, and the same registers (as bf16)
//    are the B operand of O^T = V^T P^T: P never leaves registers;
//  * K tiles [64 keys][hd] and V^T tiles [hd][64 keys] are copied global -> LDS
//    asynchronously (global_load_lds_dwordx4, no register staging) into
//    XOR-swizzled layouts that make every MFMA operand read a conflict-free 16-byte
//    ds_read_b128.  V^T arrives with its keys permuted within each 16-key group
//    ([0-3, 8-11, 4-7, 12-15]) so the 8 keys one MFMA lane-half needs are contiguous;
//  * software pipeline: K runs one tile ahead of V (two LDS slots each), and the
//    S MFMAs of tile t+1 sit in the same basic block as the exponentials and PV
//    MFMAs of tile t, so the matrix and vector pipes overlap within a wave;
//  * the running maximum only moves when a score exceeds it by more than 2^8 (exp2
//    units), so the O rescale is rare and p <= 256 stays safe in bf16;
//    log2(e)/sqrt(hd) is folded into one fma feeding the raw v_exp_f32.
#include "wan_internal.h"

namespace wan {

namespace {

constexpr int KT = 64;  // keys per tile
constexpr float RESCALE_THRESHOLD = 8.f;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

template <typename T, int HD>
struct AttnCfg {
  static constexpr int E16 = dtype_traits<T>::per16;   // elements per 16-byte chunk
  static constexpr int KCHUNKS = HD / E16;             // 16-byte chunks per K row
  static constexpr int VCHUNKS = KT / E16;             // 16-byte chunks per V^T row
  static constexpr int KR = (KCHUNKS * 16 >= 256) ? 1 : 256 / (KCHUNKS * 16);  // rows per 256 bytes
  static constexpr int VR = (VCHUNKS * 16 >= 256) ? 1 : 256 / (VCHUNKS * 16);
  static constexpr int KMASK = (KCHUNKS < 16 ? KCHUNKS : 16) - 1;
  static constexpr int VMASK = (VCHUNKS < 16 ? VCHUNKS : 16) - 1;
  static constexpr int KBYTES = KT * HD * (int)sizeof(T);  // one K tile
  static constexpr int VBYTES = HD * KT * (int)sizeof(T);  // one V^T tile
  static constexpr int KLOADS = KBYTES / 16 / 256;         // direct loads per thread per K tile
  static constexpr int VLOADS = VBYTES / 16 / 256;
  static constexpr int NCH = HD * (int)sizeof(T) / 32;      // 32-byte k-chunks along hd
  static constexpr int ND = HD / 32;                        // 32-wide d blocks of O^T
  // swizzled byte offset of logical 16-byte chunk c of row r
  __device__ static __forceinline__ int koff(int r, int c) { return (r * KCHUNKS + (c ^ ((r / KR) & KMASK))) * 16; }
  __device__ static __forceinline__ int voff(int r, int c) { return (r * VCHUNKS + (c ^ ((r / VR) & VMASK))) * 16; }
};

// Per-thread pieces of the asynchronous tile copies, fixed for the whole key loop: the tile row and
// the 16-byte chunk this lane copies for each of its wave-instructions, and the LDS destination.
template <typename T, int HD>
struct CopyPlan {
  using C = AttnCfg<T, HD>;
  int krow[C::KLOADS], kcol[C::KLOADS];  // K: key row in the tile, element column
  int voff[C::VLOADS];                   // V^T: element offset of (d row, column) from the tile start
  __device__ __forceinline__ CopyPlan(int Lpad) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int i = 0; i < C::KLOADS; ++i) {
      const int p = (i * 4 + wave) * 64 + lane;  // 16-byte position in the tile
      const int r = p / C::KCHUNKS;
      krow[i] = r;
      kcol[i] = ((p % C::KCHUNKS) ^ ((r / C::KR) & C::KMASK)) * C::E16;  // logical chunk stored there
    }
#pragma unroll
    for (int i = 0; i < C::VLOADS; ++i) {
      const int p = (i * 4 + wave) * 64 + lane;
      const int r = p / C::VCHUNKS;  // d row
      voff[i] = r * Lpad + ((p % C::VCHUNKS) ^ ((r / C::VR) & C::VMASK)) * C::E16;
    }
  }
};

// Issue the asynchronous copies of one K tile (keys j0..j0+63, clamped to L-1: rows past L are
// masked out of the softmax) into kslot.  Wave-instruction (i, wave) fills 1 KB of LDS.
template <typename T, int HD>
__device__ __forceinline__ void load_k_tile(const CopyPlan<T, HD>& cp, const T* __restrict__ kbase, int64_t k_ss,
                                            int L, int j0, char* kslot) {
  using C = AttnCfg<T, HD>;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < C::KLOADS; ++i) {
    const int j = min(j0 + cp.krow[i], L - 1);
    const T* src = kbase + (int64_t)j * k_ss + cp.kcol[i];
    __builtin_amdgcn_global_load_lds((glb_void*)src, (lds_void*)(kslot + (i * 4 + wave) * 1024), 16, 0, 0);
  }
}

template <typename T, int HD>
__device__ __forceinline__ void load_v_tile(const CopyPlan<T, HD>& cp, const T* __restrict__ vtb, int j0,
                                            char* vslot) {
  using C = AttnCfg<T, HD>;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < C::VLOADS; ++i) {
    const T* src = vtb + j0 + cp.voff[i];
    __builtin_amdgcn_global_load_lds((glb_void*)src, (lds_void*)(vslot + (i * 4 + wave) * 1024), 16, 0, 0);
  }
}

// S^T (two 32-key blocks) of the wave's 32 queries against the K tile in kslot.
template <typename T, int HD>
__device__ __forceinline__ void scores(const u32x4 (&qf)[AttnCfg<T, HD>::NCH], const char* kslot, f32x16 (&s)[2]) {
  using C = AttnCfg<T, HD>;
  const int lane = threadIdx.x & 63, lrow = lane & 31, lhalf = lane >> 5;
  s[0] = zero16();
  s[1] = zero16();
#pragma unroll
  for (int c = 0; c < C::NCH; ++c)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(kslot + C::koff(kb * 32 + lrow, 2 * c + lhalf));
      mfma_chunk(a, qf[c], s[kb], T());
    }
}

struct SoftState {
  float m, l;
};

template <typename T, int HD>
struct Slots {
  char *k0, *k1, *v0, *v1;  // four distinct __shared__ arrays (distinct objects for alias analysis)
};

// One pipelined tile step t with static slot parity P = t % 2: issue V(t+1) -> v[1-P] and
// K(t+2) -> k[P]; softmax of S(t); S(t+1) from k[1-P]; O^T += V^T P^T from v[P].
template <typename T, int HD, int P>
__device__ __forceinline__ void tile_step(const u32x4 (&qf)[AttnCfg<T, HD>::NCH], const KVStream& kv,
                                          const CopyPlan<T, HD>& cp, const T* __restrict__ kbase,
                                          const T* __restrict__ vtb, int t, int nt, float c_log2,
                                          const Slots<T, HD>& sl, f32x16 (&s)[2], f32x16 (&sn)[2],
                                          f32x16 (&o)[AttnCfg<T, HD>::ND], SoftState& st) {
  using C = AttnCfg<T, HD>;
  const int lane = threadIdx.x & 63, lrow = lane & 31, lhalf = lane >> 5;
  char* k_this = P ? sl.k1 : sl.k0;
  char* k_next = P ? sl.k0 : sl.k1;
  char* v_this = P ? sl.v1 : sl.v0;
  char* v_next = P ? sl.v0 : sl.v1;
  const int j0 = t * KT;
  if (t + 1 < nt) load_v_tile<T, HD>(cp, vtb, j0 + KT, v_next);
  if (t + 2 < nt) load_k_tile<T, HD>(cp, kbase, kv.k_ss, kv.L, j0 + 2 * KT, k_this);

  if (j0 + KT > kv.L) {  // mask keys beyond L (only the last tile can hold any)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + kb * 32 + (r >> 2) * 8 + lhalf * 4 + (r & 3);
        if (key >= kv.L) s[kb][r] = -__builtin_inff();
      }
  }
  float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
  for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const float mnew = mx * c_log2;
  const bool need = mnew > st.m + RESCALE_THRESHOLD;
  if (__ballot(need) != 0ull) {
    const float mm = need ? mnew : st.m;
    const float alpha = __builtin_amdgcn_exp2f(st.m - mm);  // 0 on the first tile (m = -inf)
    st.m = mm;
    st.l *= alpha;
#pragma unroll
    for (int d = 0; d < C::ND; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
  }
  const float negm = -st.m;
  float lsum = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // raw v_exp_f32: the argument is <= RESCALE_THRESHOLD or -inf, so no range fix-up is needed
      const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c_log2, negm));
      s[kb][r] = p;
      lsum += p;
    }
  st.l += lsum;

  // S of the next tile, independent of the exponentials and PV products around it so the compiler
  // interleaves them (on the last step it reads a stale slot -- no copy is in flight -- and is unused).
  scores<T, HD>(qf, k_next, sn);

  // O^T += V^T P^T
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {  // 16-key chunks; this lane half's 8 keys are 16-byte chunk 2c + lhalf
      const int kb = c >> 1, r0 = (c & 1) * 8;
      bf16x8 pk;
#pragma unroll
      for (int i = 0; i < 8; ++i) pk[i] = (bf16)s[kb][r0 + i];
      const u32x4 pb = __builtin_bit_cast(u32x4, pk);
#pragma unroll
      for (int d = 0; d < C::ND; ++d) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(v_this + C::voff(d * 32 + lrow, 2 * c + lhalf));
        mfma_chunk(a, pb, o[d], T());
      }
    }
  } else {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x4 pb{__float_as_uint(s[kb][4 * g]), __float_as_uint(s[kb][4 * g + 1]),
                       __float_as_uint(s[kb][4 * g + 2]), __float_as_uint(s[kb][4 * g + 3])};
#pragma unroll
        for (int d = 0; d < C::ND; ++d) {
          // keys kb*32 + g*8 + lhalf*4 .. +3 = 16-byte chunk kb*8 + g*2 + lhalf of the fp32 V^T row
          const u32x4 a = *reinterpret_cast<const u32x4*>(v_this + C::voff(d * 32 + lrow, kb * 8 + g * 2 + lhalf));
          mfma_chunk(a, pb, o[d], T());
        }
      }
  }
  __builtin_amdgcn_s_waitcnt(0);  // this step's asynchronous tile copies have landed
  __syncthreads();
}

// One key/value stream for the wave's 32 queries; accumulates O^T (unnormalised) and (m, l).
template <typename T, int HD>
__device__ __forceinline__ void attend_stream(const u32x4 (&qf)[AttnCfg<T, HD>::NCH], const KVStream& kv, int b,
                                              int h, int H, float c_log2, const Slots<T, HD>& sl,
                                              f32x16 (&o)[AttnCfg<T, HD>::ND], SoftState& st) {
  const T* kbase = reinterpret_cast<const T*>(kv.k) + (int64_t)b * kv.k_bs + (int64_t)h * HD;
  const T* vtb = reinterpret_cast<const T*>(kv.vt) + ((int64_t)b * H + h) * HD * (int64_t)kv.Lpad;
  const int nt = (kv.L + KT - 1) / KT;

  const CopyPlan<T, HD> cp(kv.Lpad);
  __syncthreads();  // earlier users of the LDS slots are done
  load_k_tile<T, HD>(cp, kbase, kv.k_ss, kv.L, 0, sl.k0);
  load_v_tile<T, HD>(cp, vtb, 0, sl.v0);
  load_k_tile<T, HD>(cp, kbase, kv.k_ss, kv.L, KT, sl.k1);  // clamped rows when nt == 1 (unused)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  f32x16 sa[2], sb[2];
  scores<T, HD>(qf, sl.k0, sa);
  __syncthreads();  // every wave has read K(0) before step 0 refills its slot with K(2)
  for (int t = 0; t < nt; t += 2) {
    tile_step<T, HD, 0>(qf, kv, cp, kbase, vtb, t, nt, c_log2, sl, sa, sb, o, st);
    if (t + 1 < nt) tile_step<T, HD, 1>(qf, kv, cp, kbase, vtb, t + 1, nt, c_log2, sl, sb, sa, o, st);
  }
}

template <typename T, int HD, int NS, int KIND>
__global__ __launch_bounds__(256, 2) void attention_kernel(const T* __restrict__ q, int64_t q_bs, int64_t q_ss,
                                                            KVStream s0, KVStream s1, int S, int H, float c_log2,
                                                            T* __restrict__ out, int64_t o_bs, int64_t o_ss) {
  using C = AttnCfg<T, HD>;
  __shared__ u32x4 k0_raw[C::KBYTES / 16], k1_raw[C::KBYTES / 16], v0_raw[C::VBYTES / 16], v1_raw[C::VBYTES / 16];
  const Slots<T, HD> sl{reinterpret_cast<char*>(k0_raw), reinterpret_cast<char*>(k1_raw),
                        reinterpret_cast<char*>(v0_raw), reinterpret_cast<char*>(v1_raw)};
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int qrow = blockIdx.x * 128 + wave * 32 + lrow;

  // Q^T as the B operand: lane holds query qrow, 16 bytes per 32-byte chunk of hd.
  u32x4 qf[C::NCH];
  const T* qp = q + (int64_t)b * q_bs + (int64_t)min(qrow, S - 1) * q_ss + (int64_t)h * HD + lhalf * C::E16;
#pragma unroll
  for (int c = 0; c < C::NCH; ++c) qf[c] = *reinterpret_cast<const u32x4*>(qp + c * 2 * C::E16);

  f32x16 o[C::ND], acc[C::ND];
  SoftState st;
#pragma unroll
  for (int si = 0; si < NS; ++si) {
#pragma unroll
    for (int d = 0; d < C::ND; ++d) o[d] = zero16();
    st.m = -__builtin_inff();
    st.l = 0.f;
    attend_stream<T, HD>(qf, si == 0 ? s0 : s1, b, h, H, c_log2, sl, o, st);
    const float inv = 1.f / (st.l + __shfl_xor(st.l, 32, 64));
#pragma unroll
    for (int d = 0; d < C::ND; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[d][r] = (si == 0 ? 0.f : acc[d][r]) + o[d][r] * inv;
  }

  if (qrow < S) {
    T* op = out + (int64_t)b * o_bs + (int64_t)qrow * o_ss + (int64_t)h * HD;
#pragma unroll
    for (int d = 0; d < C::ND; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = d * 32 + g * 8 + lhalf * 4;
        if constexpr (sizeof(T) == 2) {
          bf16x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = (bf16)acc[d][4 * g + i];
          *reinterpret_cast<bf16x4*>(op + dd) = v;
        } else {
          *reinterpret_cast<float4*>(op + dd) =
              make_float4(acc[d][4 * g], acc[d][4 * g + 1], acc[d][4 * g + 2], acc[d][4 * g + 3]);
        }
      }
  }
}

// KIND only separates the self-attention (0) and cross-attention (1) kernel symbols in profiles.
template <typename T, int HD, int KIND>
hipError_t launch_hd(const T* q, int64_t q_bs, int64_t q_ss, KVStream s0, KVStream s1, int nstreams, int B, int S,
                     int H, float c_log2, T* o, int64_t o_bs, int64_t o_ss, hipStream_t s) {
  dim3 grid((unsigned)ceil_div(S, 128), (unsigned)H, (unsigned)B);
  if (nstreams == 2)
    hipLaunchKernelGGL((attention_kernel<T, HD, 2, KIND>), grid, dim3(256), 0, s, q, q_bs, q_ss, s0, s1, S, H, c_log2,
                       o, o_bs, o_ss);
  else
    hipLaunchKernelGGL((attention_kernel<T, HD, 1, KIND>), grid, dim3(256), 0, s, q, q_bs, q_ss, s0, s1, S, H, c_log2,
                       o, o_bs, o_ss);
  return hipGetLastError();
}

}  // namespace

template <typename T>
hipError_t launch_attention(const T* q, int64_t q_bs, int64_t q_ss, KVStream s0, KVStream s1, int nstreams, int B,
                            int S, int H, int hd, float scale, T* o, int64_t o_bs, int64_t o_ss, int kind,
                            hipStream_t s) {
  if (S <= 0 || B <= 0 || H <= 0) return hipSuccess;
  if (nstreams < 1 || nstreams > 2) return hipErrorInvalidValue;
  if (s0.L <= 0 || s0.Lpad % KT != 0 || s0.Lpad < s0.L) return hipErrorInvalidValue;
  if (nstreams == 2 && (s1.L <= 0 || s1.Lpad % KT != 0 || s1.Lpad < s1.L)) return hipErrorInvalidValue;
  const float c_log2 = scale * 1.4426950408889634f;
  if (hd == 128) {
    if (kind) return launch_hd<T, 128, 1>(q, q_bs, q_ss, s0, s1, nstreams, B, S, H, c_log2, o, o_bs, o_ss, s);
    return launch_hd<T, 128, 0>(q, q_bs, q_ss, s0, s1, nstreams, B, S, H, c_log2, o, o_bs, o_ss, s);
  }
  if (hd == 64) {
    if (kind) return launch_hd<T, 64, 1>(q, q_bs, q_ss, s0, s1, nstreams, B, S, H, c_log2, o, o_bs, o_ss, s);
    return launch_hd<T, 64, 0>(q, q_bs, q_ss, s0, s1, nstreams, B, S, H, c_log2, o, o_bs, o_ss, s);
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_attention<float>(const float*, int64_t, int64_t, KVStream, KVStream, int, int, int, int,
                                            int, float, float*, int64_t, int64_t, int, hipStream_t);
template hipError_t launch_attention<bf16>(const bf16*, int64_t, int64_t, KVStream, KVStream, int, int, int, int,
                                           int, float, bf16*, int64_t, int64_t, int, hipStream_t);

}  // namespace wan
