// Flash-style attention on 32x32 MFMA for the DiT's full 3D self-attention and
// its cross-attention.
//
// What it computes: o = softmax(q k^T / sqrt(hd)) v per (batch row, head), over
// all keys, no mask ("图解 Wan2.1 I2V" §5.3; "Wan 技术深度解析" §2.5: global,
// non-causal attention).  One launch attends one key/value stream; with its
// accumulate flag it adds its result to what o holds, which is how the caller
// sums two separately normalised attentions ("图解 Wan2.1 I2V" §5.4: image and
// text branches share q, each has its own softmax, outputs are added).
//
// How (gfx950):
//  * each wave owns 32 queries, held in registers as the B operand of
//    S^T = K Q^T.  MFMA lane l then holds query (l % 32) and 16 keys per 32-key
//    block, so the row max / sum are in-lane plus one exchange with lane l ^ 32,
//    and the same registers (as bf16) are the B operand of O^T = V^T P^T: P never
//    leaves registers;
//  * K tiles [64 keys][hd] and V^T tiles [hd][64 keys] are copied global -> LDS
//    asynchronously (global_load_lds_dwordx4, no register staging) into
//    XOR-swizzled layouts that make every MFMA operand read a conflict-free 16-byte
//    ds_read_b128.  V^T arrives with its keys permuted within each 16-key group
//    ([0-3, 8-11, 4-7, 12-15]) so the 8 keys one MFMA lane-half needs are contiguous;
//  * bf16 self-attention runs the ping-pong kernel: 8 waves (two per SIMD) share
//    each K / V^T tile, and two groups of 4 waves run half a tile apart so that one
//    wave of a SIMD does softmax + S(t+1) while the other does its PV products;
//    cross-attention and fp32 run a 4-wave kernel with one barrier per tile;
//  * operand reads are software-pipelined in small scheduling regions
//    (sched_barrier) so every LDS read has work to land behind;
//  * the running maximum only moves when a score exceeds it by more than 2^8 (exp2
//    units), so the O rescale is rare and p <= 256 stays safe in bf16;
//    log2(e)/sqrt(hd) is folded into one fma feeding the raw v_exp_f32;
//  * the ping-pong kernel does not even take a tile's row maxima unless the tile's
//    weights, computed against the running maximum as it stands, sum past 2^13 in
//    some lane (or are not finite, as on the first tile); only then does the
//    maximum move (by the rule above) and the tile get recomputed, so p <= 2^13;
//  * workgroups are ordered XCD-aware: each XCD's L2 serves a contiguous run of
//    query tiles of the same heads.
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
  static constexpr int NCH = HD * (int)sizeof(T) / 32;      // 32-byte k-chunks along hd
  static constexpr int ND = HD / 32;                        // 32-wide d blocks of O^T
  // swizzled byte offset of logical 16-byte chunk c of row r
  __device__ static __forceinline__ int koff(int r, int c) { return (r * KCHUNKS + (c ^ ((r / KR) & KMASK))) * 16; }
  __device__ static __forceinline__ int voff(int r, int c) { return (r * VCHUNKS + (c ^ ((r / VR) & VMASK))) * 16; }
};

// Per-thread pieces of the asynchronous tile copies (NW waves share each tile: waves w with the same
// w % NW take the same share), fixed for the whole key loop.  A copy's global address is a wave-uniform base (advanced per tile) plus this lane's
// 32-bit byte offset; the LDS destination of wave-instruction i is (i * NW + wave) KB into the slot.
template <typename T, int HD, int NW>
struct CopyPlan {
  using C = AttnCfg<T, HD>;
  static constexpr int KL = C::KBYTES / 1024 / NW;  // copies per wave per K tile
  static constexpr int VL = C::VBYTES / 1024 / NW;  // copies per wave per V^T tile
  static_assert(KL * NW * 1024 == C::KBYTES && VL * NW * 1024 == C::VBYTES, "tile / wave split");
  uint32_t kofs[KL];  // K: byte offset of (tile row, logical chunk) from the tile's first row
  uint32_t vofs[VL];  // V^T: byte offset of (d row, logical chunk) from the tile start
  int wave;           // wave index, uniform
  __device__ __forceinline__ CopyPlan(int64_t k_ss, int Lpad) {
    const int lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) % NW);
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int p = (i * NW + wave) * 64 + lane;  // 16-byte position in the tile
      const int r = p / C::KCHUNKS;
      const int col = ((p % C::KCHUNKS) ^ ((r / C::KR) & C::KMASK)) * C::E16;  // logical chunk stored there
      kofs[i] = (uint32_t)(((int64_t)r * k_ss + col) * (int64_t)sizeof(T));
    }
#pragma unroll
    for (int i = 0; i < VL; ++i) {
      const int p = (i * NW + wave) * 64 + lane;
      const int r = p / C::VCHUNKS;  // d row
      vofs[i] = (uint32_t)(((int64_t)r * Lpad + ((p % C::VCHUNKS) ^ ((r / C::VR) & C::VMASK)) * C::E16) *
                           (int64_t)sizeof(T));
    }
  }
};

// A wave-uniform pointer held in scalar registers (the per-tile base of the copies).
__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

// Issue the asynchronous copies of one K tile (keys j0..j0+63) into kslot.  In the last, partial
// tile the rows past L are clamped to L - 1 (their scores are masked out of the softmax).
template <typename T, int HD, int NW>
__device__ __forceinline__ void load_k_tile(const CopyPlan<T, HD, NW>& cp, const T* __restrict__ kbase,
                                            int64_t k_ss, int L, int j0, char* kslot) {
  using C = AttnCfg<T, HD>;
  using CP = CopyPlan<T, HD, NW>;
  if (j0 + KT <= L) {
    const char* base = uniform_ptr(kbase + (int64_t)j0 * k_ss);
#pragma unroll
    for (int i = 0; i < CP::KL; ++i)
      __builtin_amdgcn_global_load_lds((glb_void*)(base + cp.kofs[i]), (lds_void*)(kslot + (i * NW + cp.wave) * 1024),
                                       16, 0, 0);
  } else {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < CP::KL; ++i) {
      const int p = (i * NW + cp.wave) * 64 + lane;
      const int r = p / C::KCHUNKS;
      const int col = ((p % C::KCHUNKS) ^ ((r / C::KR) & C::KMASK)) * C::E16;
      const T* src = kbase + (int64_t)min(j0 + r, L - 1) * k_ss + col;
      __builtin_amdgcn_global_load_lds((glb_void*)src, (lds_void*)(kslot + (i * NW + cp.wave) * 1024), 16, 0, 0);
    }
  }
}

// Issue the copies of one V^T tile (columns j0..j0+63 of the [hd][Lpad] rows; j0 < Lpad).
template <typename T, int HD, int NW>
__device__ __forceinline__ void load_v_tile(const CopyPlan<T, HD, NW>& cp, const T* __restrict__ vtb, int j0,
                                            char* vslot) {
  const char* base = uniform_ptr(vtb + j0);
#pragma unroll
  for (int i = 0; i < CopyPlan<T, HD, NW>::VL; ++i)
    __builtin_amdgcn_global_load_lds((glb_void*)(base + cp.vofs[i]), (lds_void*)(vslot + (i * NW + cp.wave) * 1024),
                                     16, 0, 0);
}

// Per-lane byte offsets of the MFMA operand reads (loop invariant).  K fragment (kb, c) of this lane
// is at k[c] + kb * KB32 in a K slot; V^T fragment (d, chunk index i) at v[i] + d * VD32 in a V slot.
// The swizzle key of a row only depends on the lane's row within its 32-row block, so one offset per
// chunk serves every block.
template <typename T, int HD>
struct FragAddr {
  using C = AttnCfg<T, HD>;
  static constexpr int NV = sizeof(T) == 2 ? 4 : 8;  // V^T chunks this lane reads per tile
  static constexpr int KB32 = 32 * C::KCHUNKS * 16, VD32 = 32 * C::VCHUNKS * 16;
  uint32_t k[C::NCH], v[NV];
  __device__ __forceinline__ FragAddr() {
    const int lane = threadIdx.x & 63, lrow = lane & 31, lhalf = lane >> 5;
#pragma unroll
    for (int c = 0; c < C::NCH; ++c) k[c] = (uint32_t)C::koff(lrow, 2 * c + lhalf);
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = (uint32_t)C::voff(lrow, 2 * i + lhalf);
  }
};

// S^T (two 32-key blocks) of the wave's 32 queries against the K tile in kslot.
template <typename T, int HD>
__device__ __forceinline__ void scores(const u32x4 (&qf)[AttnCfg<T, HD>::NCH], const FragAddr<T, HD>& fa,
                                       const char* kslot, f32x16 (&s)[2]) {
  using C = AttnCfg<T, HD>;
  s[0] = zero16();
  s[1] = zero16();
#pragma unroll
  for (int c = 0; c < C::NCH; ++c)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(kslot + fa.k[c] + kb * FragAddr<T, HD>::KB32);
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

// Online-softmax bookkeeping of one tile's scores s (keys j0.. of a stream with L keys): masks keys
// >= L and moves the running maximum lazily (rescaling O and l when it does).
template <typename T, int HD>
__device__ __forceinline__ void softmax_prep(f32x16 (&s)[2], int j0, int L, float c_log2,
                                             f32x16 (&o)[AttnCfg<T, HD>::ND], SoftState& st) {
  using C = AttnCfg<T, HD>;
  const int lhalf = (threadIdx.x & 63) >> 5;
  if (j0 + KT > L) {  // mask keys beyond L (only the last tile can hold any)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + kb * 32 + (r >> 2) * 8 + lhalf * 4 + (r & 3);
        if (key >= L) s[kb][r] = -__builtin_inff();
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
}

// bf16 softmax half of a tile: the exponentials of S(t) (in s, after softmax_prep) packed into the
// PV operands pf, interleaved with S(t+1) = K(t+1) Q^T from kslot into sn.  Software-pipelined in
// small scheduling regions (the compiler moves nothing across a sched_barrier): region c issues the
// LDS reads of K chunk c + 1, then 32 / NCH exponentials and the two MFMAs of chunk c.  On a
// stream's last tile kslot holds a stale tile with no copy in flight; the S(t+1) so computed is
// never used.
template <typename T, int HD>
__device__ __forceinline__ void softmax_and_next_scores(const u32x4 (&qf)[AttnCfg<T, HD>::NCH],
                                                        const FragAddr<T, HD>& fa, const char* kslot,
                                                        f32x16 (&s)[2], f32x16 (&sn)[2], float c_log2,
                                                        SoftState& st, u32x4 (&pf)[4]) {
  using C = AttnCfg<T, HD>;
  constexpr int EPC = 32 / C::NCH;  // exponentials per S chunk
  const float negm = -st.m;
  float lsum = 0.f;
  sn[0] = zero16();
  sn[1] = zero16();
  u32x4 kf[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
    kf[0][kb] = *reinterpret_cast<const u32x4*>(kslot + fa.k[0] + kb * FragAddr<T, HD>::KB32);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < C::NCH; ++c) {
    if (c + 1 < C::NCH) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        kf[(c + 1) & 1][kb] = *reinterpret_cast<const u32x4*>(kslot + fa.k[c + 1] + kb * FragAddr<T, HD>::KB32);
    }
    __builtin_amdgcn_sched_barrier(0);  // the reads go out before this region's work
#pragma unroll
    for (int e = c * EPC; e < (c + 1) * EPC; ++e) {
      // raw v_exp_f32: the argument is <= RESCALE_THRESHOLD or -inf, so no range fix-up is needed
      const float p = __builtin_amdgcn_exp2f(fmaf(s[e >> 4][e & 15], c_log2, negm));
      s[e >> 4][e & 15] = p;
      lsum += p;
    }
    if (((c + 1) * EPC) % 8 == 0) {  // a 16-key P chunk is complete: pack this lane half's 8 keys
      const int pc = (c + 1) * EPC / 8 - 1, kb = pc >> 1, r0 = (pc & 1) * 8;
      bf16x8 pk;
#pragma unroll
      for (int i = 0; i < 8; ++i) pk[i] = (bf16)s[kb][r0 + i];
      pf[pc] = __builtin_bit_cast(u32x4, pk);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) mfma_chunk(kf[c & 1][kb], qf[c], sn[kb], T());
    __builtin_amdgcn_sched_barrier(0);
  }
  st.l += lsum;
}

// Masks the keys >= L of a stream's last tile (j0 + KT > L) to -inf.
__device__ __forceinline__ void mask_tail(f32x16 (&s)[2], int j0, int L) {
  const int lhalf = (threadIdx.x & 63) >> 5;
  if (j0 + KT > L) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + kb * 32 + (r >> 2) * 8 + lhalf * 4 + (r & 3);
        if (key >= L) s[kb][r] = -__builtin_inff();
      }
  }
}

// Largest per-lane sum of a tile's 32 weights accepted without looking at the row maximum: when the
// running maximum is current (every weight <= 2^RESCALE_THRESHOLD) the sum is at most 32 * 2^8.
constexpr float LAZY_SUM_LIMIT = 8192.f;

// The ping-pong kernel's softmax half of a tile (bf16): the weights p = 2^(s c - m) of S(t) against
// the running maximum m as it stands, packed into the PV operands pf and summed, interleaved with
// S(t+1) = K(t+1) Q^T from kslot into sn.  s keeps the raw scores.  Only if some lane's sum exceeds LAZY_SUM_LIMIT (or is not
// finite: the first tile, where m = -inf) does the wave take the row maxima: m then moves, as in
// softmax_prep, wherever the tile's maximum exceeds it by more than RESCALE_THRESHOLD, O and l are
// rescaled, and the weights are recomputed.  So every weight stays <= LAZY_SUM_LIMIT.
template <typename T, int HD>
__device__ __forceinline__ void softmax_lazy_and_next_scores(const u32x4 (&qf)[AttnCfg<T, HD>::NCH],
                                                             const FragAddr<T, HD>& fa, const char* kslot,
                                                             const f32x16 (&s)[2], f32x16 (&sn)[2], float c_log2,
                                                             f32x16 (&o)[AttnCfg<T, HD>::ND], SoftState& st,
                                                             u32x4 (&pf)[4]) {
  using C = AttnCfg<T, HD>;
  static_assert(sizeof(T) == 2, "bf16 weights");
  constexpr int EPC = 32 / C::NCH;  // exponentials per S chunk
  static_assert(EPC <= 8 && 8 % EPC == 0, "a P chunk spans whole S chunks");
  float negm = -st.m;
  float lsum = 0.f;
  sn[0] = zero16();
  sn[1] = zero16();
  u32x4 kf[2][2];
  bf16x8 pk;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
    kf[0][kb] = *reinterpret_cast<const u32x4*>(kslot + fa.k[0] + kb * FragAddr<T, HD>::KB32);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < C::NCH; ++c) {
    if (c + 1 < C::NCH) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        kf[(c + 1) & 1][kb] = *reinterpret_cast<const u32x4*>(kslot + fa.k[c + 1] + kb * FragAddr<T, HD>::KB32);
    }
    __builtin_amdgcn_sched_barrier(0);  // the reads go out before this region's work
#pragma unroll
    for (int e = c * EPC; e < (c + 1) * EPC; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[e >> 4][e & 15], c_log2, negm));
      pk[e & 7] = (bf16)p;
      lsum += p;
    }
    if (((c + 1) * EPC) % 8 == 0) {  // a 16-key P chunk is complete
      const int pc = (c + 1) * EPC / 8 - 1;
      pf[pc] = __builtin_bit_cast(u32x4, pk);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) mfma_chunk(kf[c & 1][kb], qf[c], sn[kb], T());
    __builtin_amdgcn_sched_barrier(0);
  }
  if (__ballot(!(lsum <= LAZY_SUM_LIMIT)) != 0ull) {
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = mx * c_log2;
    if (mnew > st.m + RESCALE_THRESHOLD) {
      const float alpha = __builtin_amdgcn_exp2f(st.m - mnew);  // 0 on the first tile (m = -inf)
      st.m = mnew;
      st.l *= alpha;
#pragma unroll
      for (int d = 0; d < C::ND; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
    }
    negm = -st.m;
    lsum = 0.f;
#pragma unroll
    for (int pc = 0; pc < 4; ++pc) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[pc >> 1][(pc & 1) * 8 + i], c_log2, negm));
        pk[i] = (bf16)p;
        lsum += p;
      }
      pf[pc] = __builtin_bit_cast(u32x4, pk);
    }
  }
  st.l += lsum;
}

// The ping-pong kernel's vector half of a tile (bf16, no LDS access): the weights p = 2^(s c - m) of
// S(t) against the running maximum m as it stands, packed into the PV operands pf and summed.  Only if
// some lane's sum exceeds LAZY_SUM_LIMIT (or is not finite: the first tile, where m = -inf) does the
// wave take the row maxima: m then moves, as in softmax_prep, wherever the tile's maximum exceeds it
// by more than RESCALE_THRESHOLD, O and l are rescaled and the weights recomputed.  So every weight
// stays <= LAZY_SUM_LIMIT.
template <typename T, int HD>
__device__ __forceinline__ void softmax_lazy(const f32x16 (&s)[2], float c_log2, f32x16 (&o)[AttnCfg<T, HD>::ND],
                                             SoftState& st, u32x4 (&pf)[4]) {
  using C = AttnCfg<T, HD>;
  static_assert(sizeof(T) == 2, "bf16 weights");
  float negm = -st.m;
  float lsum = 0.f;
#pragma unroll
  for (int pc = 0; pc < 4; ++pc) {
    bf16x8 pk;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // raw v_exp_f32: accepted arguments are <= 13; larger or non-finite ones are redone below
      const float p = __builtin_amdgcn_exp2f(fmaf(s[pc >> 1][(pc & 1) * 8 + i], c_log2, negm));
      pk[i] = (bf16)p;
      lsum += p;
    }
    pf[pc] = __builtin_bit_cast(u32x4, pk);
  }
  if (__ballot(!(lsum <= LAZY_SUM_LIMIT)) != 0ull) {
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = mx * c_log2;
    if (mnew > st.m + RESCALE_THRESHOLD) {
      const float alpha = __builtin_amdgcn_exp2f(st.m - mnew);  // 0 on the first tile (m = -inf)
      st.m = mnew;
      st.l *= alpha;
#pragma unroll
      for (int d = 0; d < C::ND; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
    }
    negm = -st.m;
    lsum = 0.f;
#pragma unroll
    for (int pc = 0; pc < 4; ++pc) {
      bf16x8 pk;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[pc >> 1][(pc & 1) * 8 + i], c_log2, negm));
        pk[i] = (bf16)p;
        lsum += p;
      }
      pf[pc] = __builtin_bit_cast(u32x4, pk);
    }
  }
  st.l += lsum;
}

// The ping-pong kernel's matrix half of a tile (bf16): (if NEXT) S(t+1) = K(t+1) Q^T from kslot into
// sn, then O^T += V^T(t) P^T(t) from vslot.  Units of two MFMAs, each unit's LDS fragments read two
// units ahead: the S units (hd chunk, both 32-key blocks) first, so that the next vector phase, which
// starts on S(t+1), does not wait on the last MFMAs; then the PV units (16-key chunk, pair of d
// blocks), whose accumulators the vector phase does not read.
template <typename T, int HD, bool NEXT>
__device__ __forceinline__ void read_pv_or_s_unit(const FragAddr<T, HD>& fa, const char* vslot, const char* kslot,
                                                  int u, u32x4& f0, u32x4& f1) {
  using C = AttnCfg<T, HD>;
  using F = FragAddr<T, HD>;
  constexpr int DP = C::ND / 2, NS = NEXT ? C::NCH : 0;
  if (u >= NS) {
    const int w = u - NS;
    const int c = w / DP, d0 = (w % DP) * 2;
    f0 = *reinterpret_cast<const u32x4*>(vslot + fa.v[c] + d0 * F::VD32);
    f1 = *reinterpret_cast<const u32x4*>(vslot + fa.v[c] + (d0 + 1) * F::VD32);
  } else {
    f0 = *reinterpret_cast<const u32x4*>(kslot + fa.k[u]);
    f1 = *reinterpret_cast<const u32x4*>(kslot + fa.k[u] + F::KB32);
  }
}

template <typename T, int HD, bool NEXT>
__device__ __forceinline__ void pv_and_next_scores(const FragAddr<T, HD>& fa, const char* vslot, const u32x4 (&pf)[4],
                                                   f32x16 (&o)[AttnCfg<T, HD>::ND],
                                                   const u32x4 (&qf)[AttnCfg<T, HD>::NCH], const char* kslot,
                                                   f32x16 (&sn)[2]) {
  using C = AttnCfg<T, HD>;
  constexpr int DP = C::ND / 2, NPV = 4 * DP, NS = NEXT ? C::NCH : 0, NU = NS + NPV;
  u32x4 f[3][2];  // fragments of units u % 3, read two units ahead
  read_pv_or_s_unit<T, HD, NEXT>(fa, vslot, kslot, 0, f[0][0], f[0][1]);
  read_pv_or_s_unit<T, HD, NEXT>(fa, vslot, kslot, 1, f[1][0], f[1][1]);
  if (NEXT) {
    sn[0] = zero16();
    sn[1] = zero16();
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if (u + 2 < NU) read_pv_or_s_unit<T, HD, NEXT>(fa, vslot, kslot, u + 2, f[(u + 2) % 3][0], f[(u + 2) % 3][1]);
    __builtin_amdgcn_sched_barrier(0);  // the reads go out before this unit's MFMAs
    const u32x4& f0 = f[u % 3][0];
    const u32x4& f1 = f[u % 3][1];
    if (u >= NS) {
      const int w = u - NS;
      const int c = w / DP, d0 = (w % DP) * 2;
      mfma_chunk(f0, pf[c], o[d0], T());
      mfma_chunk(f1, pf[c], o[d0 + 1], T());
    } else {
      mfma_chunk(f0, qf[u], sn[0], T());
      mfma_chunk(f1, qf[u], sn[1], T());
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// bf16 O^T += V^T P^T for one tile (V^T tile in vslot): units of two MFMAs, each reading its V^T
// fragments one unit ahead.
template <typename T, int HD>
__device__ __forceinline__ void pv_products(const FragAddr<T, HD>& fa, const char* vslot, const u32x4 (&pf)[4],
                                            f32x16 (&o)[AttnCfg<T, HD>::ND]) {
  using C = AttnCfg<T, HD>;
  constexpr int DP = C::ND / 2, NU = 4 * DP;  // unit u = (16-key chunk u / DP, d-blocks 2 (u % DP) + 0, 1)
  u32x4 va[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) va[0][j] = *reinterpret_cast<const u32x4*>(vslot + fa.v[0] + j * FragAddr<T, HD>::VD32);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if (u + 1 < NU) {
      const int c1 = (u + 1) / DP, d1 = ((u + 1) % DP) * 2;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        va[(u + 1) & 1][j] = *reinterpret_cast<const u32x4*>(vslot + fa.v[c1] + (d1 + j) * FragAddr<T, HD>::VD32);
    }
    __builtin_amdgcn_sched_barrier(0);
    const int c = u / DP, d0 = (u % DP) * 2;
#pragma unroll
    for (int j = 0; j < 2; ++j) mfma_chunk(va[u & 1][j], pf[c], o[d0 + j], T());
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------------------
// Four-wave kernel (fp32, and bf16 cross-attention): one barrier per tile.
// ---------------------------------------------------------------------------

// One pipelined tile step t with static slot parity P = t % 2: issue V(t+1) -> v[1-P] and
// K(t+2) -> k[P]; softmax of S(t); S(t+1) from k[1-P]; O^T += V^T P^T from v[P].
template <typename T, int HD, int P>
__device__ __forceinline__ void tile_step(const u32x4 (&qf)[AttnCfg<T, HD>::NCH], const FragAddr<T, HD>& fa,
                                          const KVStream& kv, const CopyPlan<T, HD, 4>& cp,
                                          const T* __restrict__ kbase, const T* __restrict__ vtb, int t, int nt,
                                          float c_log2, const Slots<T, HD>& sl, f32x16 (&s)[2], f32x16 (&sn)[2],
                                          f32x16 (&o)[AttnCfg<T, HD>::ND], SoftState& st) {
  using C = AttnCfg<T, HD>;
  char* k_this = P ? sl.k1 : sl.k0;
  char* k_next = P ? sl.k0 : sl.k1;
  char* v_this = P ? sl.v1 : sl.v0;
  char* v_next = P ? sl.v0 : sl.v1;
  const int j0 = t * KT;
  if (t + 1 < nt) load_v_tile<T, HD, 4>(cp, vtb, j0 + KT, v_next);
  if (t + 2 < nt) load_k_tile<T, HD, 4>(cp, kbase, kv.k_ss, kv.L, j0 + 2 * KT, k_this);
  softmax_prep<T, HD>(s, j0, kv.L, c_log2, o, st);
  if constexpr (sizeof(T) == 2) {
    u32x4 pf[4];
    // on the last step S(t+1) reads a stale slot (no copy is in flight) and is unused
    softmax_and_next_scores<T, HD>(qf, fa, k_next, s, sn, c_log2, st, pf);
    pv_products<T, HD>(fa, v_this, pf, o);
  } else {
    const float negm = -st.m;
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c_log2, negm));
        s[kb][r] = p;
        lsum += p;
      }
    st.l += lsum;
    scores<T, HD>(qf, fa, k_next, sn);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x4 pb{__float_as_uint(s[kb][4 * g]), __float_as_uint(s[kb][4 * g + 1]),
                       __float_as_uint(s[kb][4 * g + 2]), __float_as_uint(s[kb][4 * g + 3])};
#pragma unroll
        for (int d = 0; d < C::ND; ++d) {
          // keys kb*32 + g*8 + lhalf*4 .. +3 = 16-byte chunk kb*8 + g*2 + lhalf of the fp32 V^T row
          const u32x4 a = *reinterpret_cast<const u32x4*>(v_this + fa.v[kb * 4 + g] + d * FragAddr<T, HD>::VD32);
          mfma_chunk(a, pb, o[d], T());
        }
      }
  }
  __builtin_amdgcn_s_waitcnt(0);  // this step's asynchronous tile copies have landed
  __syncthreads();
}

// One key/value stream for the wave's 32 queries; accumulates O^T (unnormalised) and (m, l).
template <typename T, int HD>
__device__ __forceinline__ void attend_stream(const u32x4 (&qf)[AttnCfg<T, HD>::NCH], const FragAddr<T, HD>& fa,
                                              const KVStream& kv, int b, int h, int H, float c_log2,
                                              const Slots<T, HD>& sl, f32x16 (&o)[AttnCfg<T, HD>::ND],
                                              SoftState& st) {
  const T* kbase = reinterpret_cast<const T*>(kv.k) + (int64_t)b * kv.k_bs + (int64_t)h * HD;
  const T* vtb = reinterpret_cast<const T*>(kv.vt) + ((int64_t)b * H + h) * HD * (int64_t)kv.Lpad;
  const int nt = (kv.L + KT - 1) / KT;

  const CopyPlan<T, HD, 4> cp(kv.k_ss, kv.Lpad);
  __syncthreads();  // earlier users of the LDS slots are done
  load_k_tile<T, HD, 4>(cp, kbase, kv.k_ss, kv.L, 0, sl.k0);
  load_v_tile<T, HD, 4>(cp, vtb, 0, sl.v0);
  load_k_tile<T, HD, 4>(cp, kbase, kv.k_ss, kv.L, KT, sl.k1);  // clamped rows when nt == 1 (unused)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  f32x16 sa[2], sb[2];
  scores<T, HD>(qf, fa, sl.k0, sa);
  __syncthreads();  // every wave has read K(0) before step 0 refills its slot with K(2)
  for (int t = 0; t < nt; t += 2) {
    tile_step<T, HD, 0>(qf, fa, kv, cp, kbase, vtb, t, nt, c_log2, sl, sa, sb, o, st);
    if (t + 1 < nt) tile_step<T, HD, 1>(qf, fa, kv, cp, kbase, vtb, t + 1, nt, c_log2, sl, sb, sa, o, st);
  }
}

// Workgroup id -> (query tile, head, batch row), XCD-aware: workgroup ids are dealt round-robin to
// the 8 XCDs; each XCD gets a contiguous run of (batch, head, query tile) so the workgroups sharing
// an L2 stream the same head's K/V.
__device__ __forceinline__ void attn_tile_coords(int& qt, int& h, int& b) {
  const int nq = gridDim.x, nh = gridDim.y;
  const int n = nq * nh * gridDim.z;
  const int lin = blockIdx.x + nq * (blockIdx.y + nh * blockIdx.z);
  const int xcd = lin & 7;
  const int t = xcd * (n >> 3) + min(xcd, n & 7) + (lin >> 3);  // bijection on [0, n)
  qt = t % nq;
  h = (t / nq) % nh;
  b = t / (nq * nh);
}

// Key split: grid batch entry b = row * n + i becomes batch row `row` attending to keys
// [i * chunk, min((i + 1) * chunk, L)) of stream s, with o and lse moved to part i.  chunk is a multiple
// of the 64-key tile, so every part but the last ends on a whole tile and the bf16 V^T key permutation
// (within 16-key groups) is undisturbed.
template <typename T>
__device__ __forceinline__ void apply_key_split(const KeySplit& ks, int& b, KVStream& s, T* __restrict__& out,
                                                float* __restrict__& lse) {
  const int i = b % ks.n;
  b /= ks.n;
  const int key0 = i * ks.chunk;
  s.k = reinterpret_cast<const T*>(s.k) + (int64_t)key0 * s.k_ss;
  s.vt = reinterpret_cast<const T*>(s.vt) + key0;
  s.L = min(ks.chunk, s.L - key0);
  out += (int64_t)i * ks.o_stride;
  if (lse != nullptr) lse += (int64_t)i * ks.lse_stride;
}

// Normalise one stream's O^T by its row sums and add it into acc (first stream: assign).
template <typename T, int HD>
__device__ __forceinline__ void finish_stream(const f32x16 (&o)[AttnCfg<T, HD>::ND], const SoftState& st,
                                              f32x16 (&acc)[AttnCfg<T, HD>::ND]) {
  const float inv = 1.f / (st.l + __shfl_xor(st.l, 32, 64));
#pragma unroll
  for (int d = 0; d < AttnCfg<T, HD>::ND; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = o[d][r] * inv;
}

// Natural log of the row's softmax normaliser: the online state keeps sum_j exp(scale s_j) as 2^m * l
// (m in log2 units, l split over the two lane halves).  Layout [B, H, S]; lanes of the low half write.
__device__ __forceinline__ void write_lse(const SoftState& st, float* __restrict__ lse, int b, int h, int H,
                                          int qrow, int S) {
  const float l = st.l + __shfl_xor(st.l, 32, 64);
  if ((threadIdx.x & 32) == 0 && qrow < S)
    lse[((int64_t)b * H + h) * S + qrow] = (st.m + log2f(l)) * 0.69314718055994531f;
}

// Write the wave's O rows (lane: query qrow, d = 32 dblk + 8 g + 4 lhalf + 0..3).  Output channel
// n = h HD + d of query row (b, qrow) sits at out + b o_bs + qrow o_ss + (n / 32) o_cs + n % 32
// (row-major: o_cs = 32; the products' K panels: o_ss = 32, o_cs = 32 * rows per panel).
// add: the rows are added to what out holds (a second key/value stream's launch adding to the first's
// result), in fp32 before the store's rounding.
template <typename T, int HD>
__device__ __forceinline__ void store_rows(const f32x16 (&acc)[AttnCfg<T, HD>::ND], T* __restrict__ out,
                                           int64_t o_bs, int64_t o_ss, int64_t o_cs, int b, int h, int qrow, int S,
                                           bool add = false) {
  const int lhalf = (threadIdx.x & 63) >> 5;
  if (qrow >= S) return;
  T* op0 = out + (int64_t)b * o_bs + (int64_t)qrow * o_ss + (int64_t)h * (HD / 32) * o_cs;
#pragma unroll
  for (int d = 0; d < AttnCfg<T, HD>::ND; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      T* op = op0 + d * o_cs + g * 8 + lhalf * 4;  // channels 32 d + 8 g + 4 lhalf .. + 3 of the head
      if constexpr (sizeof(T) == 2) {
        bf16x4 v;
        if (add) {
          const bf16x4 old = *reinterpret_cast<const bf16x4*>(op);
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = (bf16)((float)old[i] + acc[d][4 * g + i]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = (bf16)acc[d][4 * g + i];
        }
        *reinterpret_cast<bf16x4*>(op) = v;
      } else {
        float4 v = make_float4(acc[d][4 * g], acc[d][4 * g + 1], acc[d][4 * g + 2], acc[d][4 * g + 3]);
        if (add) {
          const float4 old = *reinterpret_cast<const float4*>(op);
          v = make_float4(old.x + v.x, old.y + v.y, old.z + v.z, old.w + v.w);
        }
        *reinterpret_cast<float4*>(op) = v;
      }
    }
}

// Q^T as the B operand: lane holds query qrow (clamped), 16 bytes per 32-byte chunk of hd.
// The score scale of one query (exp2 units): c_log2, times the query row's factor when qscale [B, S]
// is given (the block's RMSNorm factor r_q, folded here instead of into the stored q row).  Both
// lanes holding a query (l and l + 32) read the same value.
__device__ __forceinline__ float query_scale(float c_log2, const float* __restrict__ qscale, int b, int qrow, int S) {
  return qscale ? c_log2 * qscale[(int64_t)b * S + min(qrow, S - 1)] : c_log2;
}

template <typename T, int HD>
__device__ __forceinline__ void load_q(const T* __restrict__ q, int64_t q_bs, int64_t q_ss, int b, int h, int qrow,
                                       int S, u32x4 (&qf)[AttnCfg<T, HD>::NCH]) {
  using C = AttnCfg<T, HD>;
  const int lhalf = (threadIdx.x & 63) >> 5;
  const T* qp = q + (int64_t)b * q_bs + (int64_t)min(qrow, S - 1) * q_ss + (int64_t)h * HD + lhalf * C::E16;
#pragma unroll
  for (int c = 0; c < C::NCH; ++c) qf[c] = *reinterpret_cast<const u32x4*>(qp + c * 2 * C::E16);
}

// One workgroup = 4 waves = 128 queries of one (b, head).
template <typename T, int HD, int KIND>
__global__ __launch_bounds__(256, 2) void attention_kernel(const T* __restrict__ q, int64_t q_bs, int64_t q_ss,
                                                            KVStream kv, int S, int H, float c_log2,
                                                            const float* __restrict__ qscale, T* __restrict__ out,
                                                            int64_t o_bs, int64_t o_ss, int64_t o_cs,
                                                            float* __restrict__ lse, KeySplit ks, int accum) {
  using C = AttnCfg<T, HD>;
  __shared__ u32x4 k0_raw[C::KBYTES / 16], k1_raw[C::KBYTES / 16], v0_raw[C::VBYTES / 16], v1_raw[C::VBYTES / 16];
  const Slots<T, HD> sl{reinterpret_cast<char*>(k0_raw), reinterpret_cast<char*>(k1_raw),
                        reinterpret_cast<char*>(v0_raw), reinterpret_cast<char*>(v1_raw)};
  int qt, h, b;
  attn_tile_coords(qt, h, b);
  if (ks.n > 1) apply_key_split<T>(ks, b, kv, out, lse);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int qrow = qt * 128 + wave * 32 + (lane & 31);
  const FragAddr<T, HD> fa;
  u32x4 qf[C::NCH];
  load_q<T, HD>(q, q_bs, q_ss, b, h, qrow, S, qf);
  const float cq = query_scale(c_log2, qscale, b, qrow, S);

  f32x16 o[C::ND], acc[C::ND];
  SoftState st;
#pragma unroll
  for (int d = 0; d < C::ND; ++d) o[d] = zero16();
  st.m = -__builtin_inff();
  st.l = 0.f;
  attend_stream<T, HD>(qf, fa, kv, b, h, H, cq, sl, o, st);
  finish_stream<T, HD>(o, st, acc);
  if (lse != nullptr) write_lse(st, lse, b, h, H, qrow, S);
  store_rows<T, HD>(acc, out, o_bs, o_ss, o_cs, b, h, qrow, S, accum != 0);
}

// ---------------------------------------------------------------------------
// Ping-pong kernel (bf16): one workgroup = 8 waves = 256 queries of one (b, head), two waves per
// SIMD.  Each wave alternates A(t) = the weights of S(t) (vector units only, no LDS access) and
// B(t) = S(t+1) = K(t+1) Q^T followed by O^T += V^T(t) P^T(t) (32 MFMAs), with a workgroup barrier
// between the two (FlashAttention-3's ping-pong schedule).  Waves 4-7 (group 1) pass one extra
// barrier at the start and waves 0-3 (group 0) one at the end, so group 1 runs a half tile behind:
// between two barriers one wave of each SIMD is in A and the other in B, and the SIMD's matrix and
// vector units work at the same time.
//
// Copies (tile t lives in slot t % 2; global phase k runs between barriers b_k and b_k+1, group 0's
// A(t) and B(t) are phases 2t and 2t+1, group 1's are 2t+1 and 2t+2).  K(t) is last read by group
// 1's B(t-1) and V^T(t-1) by group 1's B(t-1), both in phase 2t; so K(t+2) and V^T(t+1) are copied
// in phase 2t+1, by group 1's waves during their vector phase A(t) (copies issued by a wave in its
// matrix phase slow its MFMA stream), and first read in phase 2t+3 (group 0's B(t+1)).  Every copy
// thus has two phases to land; a wave waits at a barrier only for the copies it issued in its
// previous phase to be allowed in flight.
// ---------------------------------------------------------------------------

template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Barrier between phases.  The copies this wave issued in the previous phase (LAST of them) stay in
// flight: a bare s_barrier (the workgroup fence of __syncthreads() would wait for them); the
// wavefront-scope fences only stop the compiler from moving LDS accesses across it.
template <int LAST>
__device__ __forceinline__ void phase_barrier(int last) {
  if (last) wait_vm<LAST>(); else wait_vm<0>();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Tile t (static slot parity P = t % 2) as seen by one wave: barrier, A(t), barrier, B(t).  s holds
// S(t) on entry and S(t+1) on exit (S(t) is dead once A(t) has packed its weights).  `last` counts
// the copies this wave issued in its previous phase.
template <typename T, int HD, int P>
__device__ __forceinline__ void pp_tile(const u32x4 (&qf)[AttnCfg<T, HD>::NCH], const FragAddr<T, HD>& fa,
                                        const KVStream& kv, const CopyPlan<T, HD, 4>& cp,
                                        const T* __restrict__ kbase, const T* __restrict__ vtb, int t, int nt,
                                        int grp, float c_log2, const Slots<T, HD>& sl, f32x16 (&s)[2],
                                        f32x16 (&o)[AttnCfg<T, HD>::ND], SoftState& st, int& last) {
  using CP = CopyPlan<T, HD, 4>;
  constexpr int PER = CP::KL + CP::VL;  // copies per group-1 wave in its copying phase
  char* k_this = P ? sl.k1 : sl.k0;  // K(t) -> K(t+2)
  char* k_next = P ? sl.k0 : sl.k1;  // K(t+1)
  char* v_this = P ? sl.v1 : sl.v0;  // V^T(t)
  char* v_next = P ? sl.v0 : sl.v1;  // V^T(t-1) -> V^T(t+1)
  const int j0 = t * KT;
  // the copies of global phase 2t + 1, all by group 1 in its A(t) (so group 0's matrix phase B(t)
  // issues none): K(t+2) and V^T(t+1)
  auto copies = [&]() {
    if (t + 2 < nt) load_k_tile<T, HD, 4>(cp, kbase, kv.k_ss, kv.L, j0 + 2 * KT, k_this);
    if (t >= 1 && t + 1 < nt) load_v_tile<T, HD, 4>(cp, vtb, j0 + KT, v_next);
    last = (t + 2 < nt || (t >= 1 && t + 1 < nt)) ? 1 : 0;
  };
  // ---- A(t): the weights of S(t) (vector units only)
  phase_barrier<PER>(last);
  last = 0;
  if (grp == 1) copies();
  mask_tail(s, j0, kv.L);
  u32x4 pf[4];
  softmax_lazy<T, HD>(s, c_log2, o, st, pf);
  // ---- B(t): S(t+1) = K(t+1) Q^T, O^T += V^T(t) P^T(t) (matrix units)
  phase_barrier<PER>(last);
  last = 0;
  // on a stream's last tile k_next holds a stale tile with no copy in flight: S(t+1) is computed and unused
  pv_and_next_scores<T, HD, true>(fa, v_this, pf, o, qf, k_next, s);
}

template <typename T, int HD>
__device__ __forceinline__ void attend_stream_pp(const u32x4 (&qf)[AttnCfg<T, HD>::NCH], const FragAddr<T, HD>& fa,
                                                 const KVStream& kv, int b, int h, int H, int grp, float c_log2,
                                                 const Slots<T, HD>& sl, f32x16 (&o)[AttnCfg<T, HD>::ND],
                                                 SoftState& st) {
  using CP = CopyPlan<T, HD, 8>;
  const T* kbase = reinterpret_cast<const T*>(kv.k) + (int64_t)b * kv.k_bs + (int64_t)h * HD;
  const T* vtb = reinterpret_cast<const T*>(kv.vt) + ((int64_t)b * H + h) * HD * (int64_t)kv.Lpad;
  const int nt = (kv.L + KT - 1) / KT;

  const CP cp(kv.k_ss, kv.Lpad);
  __syncthreads();  // earlier users of the LDS slots are done
  load_k_tile<T, HD, 8>(cp, kbase, kv.k_ss, kv.L, 0, sl.k0);
  load_k_tile<T, HD, 8>(cp, kbase, kv.k_ss, kv.L, KT, sl.k1);  // clamped rows when nt == 1 (unused)
  load_v_tile<T, HD, 8>(cp, vtb, 0, sl.v0);
  if (nt > 1) load_v_tile<T, HD, 8>(cp, vtb, KT, sl.v1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const CopyPlan<T, HD, 4> cp4(kv.k_ss, kv.Lpad);  // group 1's share of each tile in the key loop
  f32x16 sa[2];
  scores<T, HD>(qf, fa, sl.k0, sa);
  int last = 0;
  using CP4 = CopyPlan<T, HD, 4>;
  if (grp == 1) phase_barrier<CP4::KL + CP4::VL>(0);  // group 1 runs a phase late
  for (int t = 0; t < nt; t += 2) {
    pp_tile<T, HD, 0>(qf, fa, kv, cp4, kbase, vtb, t, nt, grp, c_log2, sl, sa, o, st, last);
    if (t + 1 < nt) pp_tile<T, HD, 1>(qf, fa, kv, cp4, kbase, vtb, t + 1, nt, grp, c_log2, sl, sa, o, st, last);
  }
  if (grp == 0) phase_barrier<CP4::KL + CP4::VL>(0);  // group 0 passes the barrier ending group 1's last B
}

template <typename T, int HD, int KIND>
__global__ __launch_bounds__(512, 1) void attention_pp_kernel(const T* __restrict__ q, int64_t q_bs, int64_t q_ss,
                                                               KVStream kv, int S, int H, float c_log2,
                                                               const float* __restrict__ qscale,
                                                               T* __restrict__ out, int64_t o_bs, int64_t o_ss,
                                                               int64_t o_cs, float* __restrict__ lse, KeySplit ks) {
  using C = AttnCfg<T, HD>;
  __shared__ u32x4 k0_raw[C::KBYTES / 16], k1_raw[C::KBYTES / 16], v0_raw[C::VBYTES / 16], v1_raw[C::VBYTES / 16];
  const Slots<T, HD> sl{reinterpret_cast<char*>(k0_raw), reinterpret_cast<char*>(k1_raw),
                        reinterpret_cast<char*>(v0_raw), reinterpret_cast<char*>(v1_raw)};
  int qt, h, b;
  attn_tile_coords(qt, h, b);
  if (ks.n > 1) apply_key_split<T>(ks, b, kv, out, lse);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2;
  const int qrow = qt * 256 + wave * 32 + (lane & 31);
  const FragAddr<T, HD> fa;
  u32x4 qf[C::NCH];
  load_q<T, HD>(q, q_bs, q_ss, b, h, qrow, S, qf);
  const float cq = query_scale(c_log2, qscale, b, qrow, S);

  f32x16 o[C::ND], acc[C::ND];
  SoftState st;
#pragma unroll
  for (int d = 0; d < C::ND; ++d) o[d] = zero16();
  st.m = -__builtin_inff();
  st.l = 0.f;
  attend_stream_pp<T, HD>(qf, fa, kv, b, h, H, grp, cq, sl, o, st);
  finish_stream<T, HD>(o, st, acc);
  if (lse != nullptr) write_lse(st, lse, b, h, H, qrow, S);
  store_rows<T, HD>(acc, out, o_bs, o_ss, o_cs, b, h, qrow, S);
}

// ---------------------------------------------------------------------------
// Quantised ping-pong kernel ("Wan 技术深度解析" §5.3, FlashAttention-3 FP8: Q.K inner products in
// INT8, O = P.V in FP8, FP32 accumulation across key tiles).  The two wave groups run a phase apart
// as in the bf16 ping-pong kernel, but S(t+1) is computed in the vector phase A(t) and the matrix phase
// B(t) holds only P.V; group 0 copies the K tiles and group 1 the V^T tiles (pp_tile_q8).  Per 64-key
// tile and wave:
//  * S^T = K Q^T from INT8 codes: 8 v_mfma_i32_32x32x32_i8 (exact int32 dot products; K codes in
//    LDS, the wave's Q codes in registers);
//  * scores in exp2 units are s * (c_log2 * sq[query] * sk[tile]), with sq the query's INT8 scale
//    and sk the tile's; the running max moves only when a score exceeds it by more than Q8_TAU;
//  * P' = 2^(score - m + Q8_BIAS) <= 2^(Q8_TAU + Q8_BIAS) = 256 is rounded to E4M3 (its normal range
//    then covers 2^-12 of the running max) and O^T += V^T P'^T runs as 4
//    v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales) on E4M3 V^T codes whose keys are stored in
//    the order a lane half consumes them;
//  * the row sum l is one more FP8 product per tile, of an all-ones operand with the same E4M3 P'
//    (so numerator and denominator see the same rounded weights, and every lane holds its query's
//    l); the bias cancels in O / l, and the per-channel V scales are applied once, at the end.
// ---------------------------------------------------------------------------
constexpr float Q8_TAU = 2.f;
constexpr float Q8_BIAS = 6.f;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));

struct KVq8 {
  const uint8_t* k;   // INT8 K codes [B, L, H, hd]
  int64_t k_bs, k_ss; // byte strides
  const float* sk;    // [B, H, nb] per-64-key-block K scales
  const uint8_t* vt;  // E4M3 V^T codes [B, H, hd, Lpad], keys in P.V order within each 64-key tile
  const float* sv;    // [B, H, hd] V channel scales
  int L, Lpad;
};

template <int HD>
struct FragQ8 {
  using C = AttnCfg<uint8_t, HD>;
  static constexpr int KB32 = 32 * C::KCHUNKS * 16, VD32 = 32 * C::VCHUNKS * 16;
  uint32_t k[C::NCH], v[2];
  __device__ __forceinline__ FragQ8() {
    const int lane = threadIdx.x & 63, lrow = lane & 31, lhalf = lane >> 5;
#pragma unroll
    for (int c = 0; c < C::NCH; ++c) k[c] = (uint32_t)C::koff(lrow, 2 * c + lhalf);
#pragma unroll
    for (int i = 0; i < 2; ++i) v[i] = (uint32_t)C::voff(lrow, 2 * lhalf + i);
  }
};

__device__ __forceinline__ void mfma_i8(const u32x4& a, const u32x4& b, v16i& acc) {
  acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(v4i, a), __builtin_bit_cast(v4i, b), acc, 0, 0, 0);
}

__device__ __forceinline__ v16i zero16i() {
  v16i z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0;
  return z;
}

template <int HD>
__device__ __forceinline__ void scores_q8(const u32x4 (&qf)[AttnCfg<uint8_t, HD>::NCH], const FragQ8<HD>& fa,
                                          const char* kslot, v16i (&s)[2]) {
  s[0] = zero16i();
  s[1] = zero16i();
#pragma unroll
  for (int c = 0; c < AttnCfg<uint8_t, HD>::NCH; ++c)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      mfma_i8(*reinterpret_cast<const u32x4*>(kslot + fa.k[c] + kb * FragQ8<HD>::KB32), qf[c], s[kb]);
}

// Scores of tile t as floats (exp2 units before the max shift) -> running max bookkeeping.  Masks
// keys >= L.  Returns the tile's multiplier.
// The int32 scores are converted to float in the same registers (f aliases si's storage).
template <int HD>
__device__ __forceinline__ float softmax_prep_q8(v16i (&si)[2], int j0, int L, float cq, float skt,
                                                 f32x16 (&o)[AttnCfg<uint8_t, HD>::ND], f32x16& lacc,
                                                 SoftState& st) {
  const int lhalf = (threadIdx.x & 63) >> 5;
  f32x16 (&f)[2] = reinterpret_cast<f32x16(&)[2]>(si);
  // > 0 so that masked keys (-inf) stay -inf; a zero multiplier (all-zero query or key block) makes
  // every score ~0, which is the exact result up to 1e-30 * |s|.
  const float mul = fmaxf(cq * skt, 1e-30f);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) f[kb][r] = (float)si[kb][r];
  if (j0 + KT > L) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + kb * 32 + (r >> 2) * 8 + lhalf * 4 + (r & 3);
        if (key >= L) f[kb][r] = -__builtin_inff();
      }
  }
  float mx = fmaxf(f[0][0], f[0][1]);
#pragma unroll
  for (int r = 2; r < 16; ++r) mx = fmaxf(mx, f[0][r]);
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(mx, f[1][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const float mnew = mx * mul;
  const bool need = mnew > st.m + Q8_TAU;
  if (__ballot(need) != 0ull) {
    const float mm = need ? mnew : st.m;
    const float alpha = __builtin_amdgcn_exp2f(st.m - mm);  // 0 on the first tile (m = -inf)
    st.m = mm;
#pragma unroll
    for (int r = 0; r < 16; ++r) lacc[r] *= alpha;
#pragma unroll
    for (int d = 0; d < AttnCfg<uint8_t, HD>::ND; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
  }
  return mul;
}

__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Exponentials of tile t (f, after softmax_prep_q8) packed to E4M3 in pf (byte kb*16 + r = key
// kb*32 + (r/4)*8 + lhalf*4 + r%4), interleaved with S(t+1) from kslot into sn.
template <int HD>
__device__ __forceinline__ void softmax_and_next_scores_q8(const u32x4 (&qf)[AttnCfg<uint8_t, HD>::NCH],
                                                           const FragQ8<HD>& fa, const char* kslot, f32x16 (&f)[2],
                                                           v16i (&sn)[2], float mul, const SoftState& st,
                                                           uint32_t (&pf)[8]) {
  constexpr int NCH = AttnCfg<uint8_t, HD>::NCH;
  constexpr int EPC = 32 / NCH;  // exponentials per region
  const float negm = Q8_BIAS - st.m;
  sn[0] = zero16i();
  sn[1] = zero16i();
  u32x4 kf[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) kf[0][kb] = *reinterpret_cast<const u32x4*>(kslot + fa.k[0] + kb * FragQ8<HD>::KB32);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (c + 1 < NCH) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        kf[(c + 1) & 1][kb] = *reinterpret_cast<const u32x4*>(kslot + fa.k[c + 1] + kb * FragQ8<HD>::KB32);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = c * EPC; e < (c + 1) * EPC; ++e) {
      // argument <= Q8_TAU + Q8_BIAS = 8 or -inf: raw v_exp_f32, P' <= 256 < 448 (no E4M3 overflow)
      f[e >> 4][e & 15] = __builtin_amdgcn_exp2f(fmaf(f[e >> 4][e & 15], mul, negm));
    }
#pragma unroll
    for (int w = (c * EPC) / 4; w < ((c + 1) * EPC) / 4; ++w)
      pf[w] = pack_e4m3x4(f[w >> 2][(w & 3) * 4], f[w >> 2][(w & 3) * 4 + 1], f[w >> 2][(w & 3) * 4 + 2],
                          f[w >> 2][(w & 3) * 4 + 3]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) mfma_i8(kf[c & 1][kb], qf[c], sn[kb]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// O^T += V^T P'^T for one tile: one 32x32x64 FP8 product per 32-channel block of hd.
template <int HD>
__device__ __forceinline__ void pv_products_q8(const FragQ8<HD>& fa, const char* vslot, const uint32_t (&pf)[8],
                                               f32x16 (&o)[AttnCfg<uint8_t, HD>::ND], f32x16& lacc, int j0, int L) {
  constexpr int ND = AttnCfg<uint8_t, HD>::ND;
  const v8i pb = {(int)pf[0], (int)pf[1], (int)pf[2], (int)pf[3], (int)pf[4], (int)pf[5], (int)pf[6], (int)pf[7]};
  // l: an all-ones E4M3 operand times P' (keys >= L of the last tile excluded: their P' is 0 anyway)
  constexpr int ONE4 = 0x38383838;
  const v8i ones = {ONE4, ONE4, ONE4, ONE4, ONE4, ONE4, ONE4, ONE4};
  lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pb, lacc, 0, 0, 0, 127, 0, 127);
  u32x4 va[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) va[0][i] = *reinterpret_cast<const u32x4*>(vslot + fa.v[i]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    if (d + 1 < ND) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        va[(d + 1) & 1][i] = *reinterpret_cast<const u32x4*>(vslot + fa.v[i] + (d + 1) * FragQ8<HD>::VD32);
    }
    __builtin_amdgcn_sched_barrier(0);
    const u32x4& a0 = va[d & 1][0];
    const u32x4& a1 = va[d & 1][1];
    const v8i pa = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    o[d] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pa, pb, o[d], 0, 0, 0, 127, 0, 127);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int HD, int P>
__device__ __forceinline__ void pp_tile_q8(const u32x4 (&qf)[AttnCfg<uint8_t, HD>::NCH], const FragQ8<HD>& fa,
                                           const KVq8& kv, const CopyPlan<uint8_t, HD, 4>& cp,
                                           const uint8_t* __restrict__ kbase, const uint8_t* __restrict__ vtb,
                                           const float* __restrict__ skb, int t, int nt, int grp, float cq,
                                           const Slots<uint8_t, HD>& sl, v16i (&s)[2], v16i (&sn)[2],
                                           f32x16 (&o)[AttnCfg<uint8_t, HD>::ND], f32x16& lacc, SoftState& st) {
  using CP = CopyPlan<uint8_t, HD, 4>;
  static_assert(CP::KL == CP::VL, "equal K and V^T copy counts");
  char* k_this = P ? sl.k1 : sl.k0;  // K(t) -> K(t+2)
  char* k_next = P ? sl.k0 : sl.k1;  // K(t+1)
  char* v_this = P ? sl.v1 : sl.v0;  // V^T(t)
  char* v_next = P ? sl.v0 : sl.v1;  // V^T(t-1) -> V^T(t+1)
  const int j0 = t * KT;
  // ---- A(t): S(t+1) = K(t+1) Q^T here, so K(t) is free once the other group's A(t-1) has ended.
  // Group 0 copies K(t+2) in its A(t) and group 1 copies V^T(t+1) in its A(t); each group copies every
  // other phase and waits for all its copies at this barrier, two phases after issuing them, before
  // their first reader: no assumption about the order in which copies complete.
  phase_barrier<CP::KL>(0);
  if (grp == 0) {
    if (t + 2 < nt) load_k_tile<uint8_t, HD, 4>(cp, kbase, kv.k_ss, kv.L, j0 + 2 * KT, k_this);
  } else {
    if (t >= 1 && t + 1 < nt) load_v_tile<uint8_t, HD, 4>(cp, vtb, j0 + KT, v_next);
  }
  const float mul = softmax_prep_q8<HD>(s, j0, kv.L, cq, skb[t], o, lacc, st);
  uint32_t pf[8];
  softmax_and_next_scores_q8<HD>(qf, fa, k_next, reinterpret_cast<f32x16(&)[2]>(s), sn, mul, st, pf);
  // ---- B(t): the batch just issued stays in flight across this barrier
  phase_barrier<CP::KL>(1);
  pv_products_q8<HD>(fa, v_this, pf, o, lacc, j0, kv.L);
}

template <int HD>
__global__ __launch_bounds__(512, 1) void attention_q8_kernel(const uint8_t* __restrict__ q, int64_t q_bs,
                                                              int64_t q_ss, const float* __restrict__ sq, KVq8 kv,
                                                              int S, int H, float c_log2,
                                                              const float* __restrict__ qscale, bf16* __restrict__ out,
                                                              int64_t o_bs, int64_t o_ss, int64_t o_cs,
                                                              float* __restrict__ lse) {
  using C = AttnCfg<uint8_t, HD>;
  using CP = CopyPlan<uint8_t, HD, 8>;
  __shared__ u32x4 k0_raw[C::KBYTES / 16], k1_raw[C::KBYTES / 16], v0_raw[C::VBYTES / 16], v1_raw[C::VBYTES / 16];
  const Slots<uint8_t, HD> sl{reinterpret_cast<char*>(k0_raw), reinterpret_cast<char*>(k1_raw),
                              reinterpret_cast<char*>(v0_raw), reinterpret_cast<char*>(v1_raw)};
  int qt, h, b;
  attn_tile_coords(qt, h, b);
  const int lane = threadIdx.x & 63, lhalf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2;
  const int qrow = qt * 256 + wave * 32 + (lane & 31);
  const FragQ8<HD> fa;
  u32x4 qf[C::NCH];
  load_q<uint8_t, HD>(q, q_bs, q_ss, b, h, qrow, S, qf);
  const float cq = query_scale(c_log2, qscale, b, qrow, S) * sq[((int64_t)b * H + h) * S + min(qrow, S - 1)];

  const uint8_t* kbase = kv.k + (int64_t)b * kv.k_bs + (int64_t)h * HD;
  const uint8_t* vtb = kv.vt + ((int64_t)b * H + h) * HD * (int64_t)kv.Lpad;
  const int nt = (kv.L + KT - 1) / KT;
  const float* skb = kv.sk + ((int64_t)b * H + h) * nt;

  f32x16 o[C::ND];
#pragma unroll
  for (int d = 0; d < C::ND; ++d) o[d] = zero16();
  f32x16 lacc = zero16();  // every element: the query's running sum of E4M3 P'
  SoftState st{-__builtin_inff(), 0.f};

  const CP cp(kv.k_ss, kv.Lpad);
  load_k_tile<uint8_t, HD, 8>(cp, kbase, kv.k_ss, kv.L, 0, sl.k0);
  load_k_tile<uint8_t, HD, 8>(cp, kbase, kv.k_ss, kv.L, KT, sl.k1);  // clamped rows when nt == 1 (unused)
  load_v_tile<uint8_t, HD, 8>(cp, vtb, 0, sl.v0);
  if (nt > 1) load_v_tile<uint8_t, HD, 8>(cp, vtb, KT, sl.v1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  v16i sa[2], sb[2];
  scores_q8<HD>(qf, fa, sl.k0, sa);
  const CopyPlan<uint8_t, HD, 4> cp4(kv.k_ss, kv.Lpad);  // one group's share of each tile in the key loop
  if (grp == 1) phase_barrier<CP::KL>(0);                // group 1 runs a phase late
  for (int t = 0; t < nt; t += 2) {
    pp_tile_q8<HD, 0>(qf, fa, kv, cp4, kbase, vtb, skb, t, nt, grp, cq, sl, sa, sb, o, lacc, st);
    if (t + 1 < nt) pp_tile_q8<HD, 1>(qf, fa, kv, cp4, kbase, vtb, skb, t + 1, nt, grp, cq, sl, sb, sa, o, lacc, st);
  }
  if (grp == 0) phase_barrier<CP::KL>(0);

  // O^T / l, times the V channel scale of each output channel d = 32 dblk + 8 g + 4 lhalf + i.
  const float lt = lacc[0];
  const float inv = 1.f / lt;
  if (lse != nullptr && lhalf == 0 && qrow < S)
    lse[((int64_t)b * H + h) * S + qrow] = (st.m - Q8_BIAS + log2f(lt)) * 0.69314718055994531f;
  const float* svb = kv.sv + ((int64_t)b * H + h) * HD;
  f32x16 acc[C::ND];
#pragma unroll
  for (int d = 0; d < C::ND; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 sc = *reinterpret_cast<const float4*>(svb + d * 32 + g * 8 + lhalf * 4);
      acc[d][4 * g] = o[d][4 * g] * inv * sc.x;
      acc[d][4 * g + 1] = o[d][4 * g + 1] * inv * sc.y;
      acc[d][4 * g + 2] = o[d][4 * g + 2] * inv * sc.z;
      acc[d][4 * g + 3] = o[d][4 * g + 3] * inv * sc.w;
    }
  store_rows<bf16, HD>(acc, out, o_bs, o_ss, o_cs, b, h, qrow, S);
}

template <int HD>
hipError_t launch_q8_hd(const uint8_t* q, int64_t q_bs, int64_t q_ss, const float* sq, const KVq8& kv, int B, int S,
                        int H, float c_log2, const float* qscale, bf16* o, int64_t o_bs, int64_t o_ss, int64_t o_cs,
                        float* lse, hipStream_t s) {
  dim3 grid((unsigned)ceil_div(S, 256), (unsigned)H, (unsigned)B);
  hipLaunchKernelGGL((attention_q8_kernel<HD>), grid, dim3(512), 0, s, q, q_bs, q_ss, sq, kv, S, H, c_log2, qscale, o,
                     o_bs, o_ss, o_cs, lse);
  return hipGetLastError();
}

// KIND only separates the self-attention (0) and cross-attention (1) kernel symbols in profiles.
// bf16 self-attention uses the ping-pong kernel (256 queries per workgroup); cross-attention (a few
// hundred keys, where the per-stream prologue dominates) and fp32 use the four-wave kernel.
template <typename T, int HD, int KIND>
hipError_t launch_hd(const T* q, int64_t q_bs, int64_t q_ss, KVStream kv, int B, int S, int H, float c_log2,
                     const float* qscale, T* o, int64_t o_bs, int64_t o_ss, int64_t o_cs, float* lse, const KeySplit& ks,
                     int accum, hipStream_t s) {
  if constexpr (sizeof(T) == 2 && KIND == 0) {
    dim3 grid((unsigned)ceil_div(S, 256), (unsigned)H, (unsigned)(B * ks.n));
    hipLaunchKernelGGL((attention_pp_kernel<T, HD, KIND>), grid, dim3(512), 0, s, q, q_bs, q_ss, kv, S, H, c_log2,
                       qscale, o, o_bs, o_ss, o_cs, lse, ks);
  } else {
    dim3 grid((unsigned)ceil_div(S, 128), (unsigned)H, (unsigned)(B * ks.n));
    hipLaunchKernelGGL((attention_kernel<T, HD, KIND>), grid, dim3(256), 0, s, q, q_bs, q_ss, kv, S, H, c_log2,
                       qscale, o, o_bs, o_ss, o_cs, lse, ks, accum);
  }
  return hipGetLastError();
}

}  // namespace

template <typename T>
hipError_t launch_attention(const T* q, int64_t q_bs, int64_t q_ss, KVStream kv, int B, int S, int H, int hd,
                            float scale, T* o, int64_t o_bs, int64_t o_ss, int kind, hipStream_t s, float* lse,
                            KeySplit ks, bool accumulate, const float* qscale, int64_t o_cs) {
  if (S <= 0 || B <= 0 || H <= 0) return hipSuccess;
  if (kv.L <= 0 || kv.Lpad % KT != 0 || kv.Lpad < kv.L) return hipErrorInvalidValue;
  if (ks.n < 1 || (int64_t)B * ks.n > 65535) return hipErrorInvalidValue;
  if (ks.n > 1 && (ks.chunk <= 0 || ks.chunk % KT != 0 || (int64_t)(ks.n - 1) * ks.chunk >= kv.L))
    return hipErrorInvalidValue;
  // the ping-pong kernel (bf16 self-attention) stores only; accumulation is the four-wave kernel's
  if (accumulate && ((sizeof(T) == 2 && kind == 0) || ks.n > 1)) return hipErrorInvalidValue;
  const int acc = accumulate ? 1 : 0;
  const float c_log2 = scale * 1.4426950408889634f;
  if (hd == 128) {
    if (kind)
      return launch_hd<T, 128, 1>(q, q_bs, q_ss, kv, B, S, H, c_log2, qscale, o, o_bs, o_ss, o_cs, lse, ks, acc, s);
    return launch_hd<T, 128, 0>(q, q_bs, q_ss, kv, B, S, H, c_log2, qscale, o, o_bs, o_ss, o_cs, lse, ks, acc, s);
  }
  if (hd == 64) {
    if (kind)
      return launch_hd<T, 64, 1>(q, q_bs, q_ss, kv, B, S, H, c_log2, qscale, o, o_bs, o_ss, o_cs, lse, ks, acc, s);
    return launch_hd<T, 64, 0>(q, q_bs, q_ss, kv, B, S, H, c_log2, qscale, o, o_bs, o_ss, o_cs, lse, ks, acc, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attention_q8(const uint8_t* q8, const float* sq, const uint8_t* k8, const float* sk,
                               const uint8_t* v8t, const float* sv, int B, int S, int L, int H, int hd, bf16* o,
                               ActLayout lo, float* lse, hipStream_t s, const float* qscale) {
  if (S <= 0 || B <= 0 || H <= 0) return hipSuccess;
  if (L <= 0) return hipErrorInvalidValue;
  const int64_t dim = (int64_t)H * hd;
  const KVq8 kv{k8, (int64_t)L * dim, dim, sk, v8t, sv, L, (int)round_up(L, 128)};  // E4M3 V^T row stride
  const float c_log2 = 1.4426950408889634f / sqrtf((float)hd);
  // head_dim 128 only: a 64-key tile of 64-byte rows is too small to split over the 8 waves' copies
  if (hd == 128)
    return launch_q8_hd<128>(q8, (int64_t)S * dim, dim, sq, kv, B, S, H, c_log2, qscale, o, (int64_t)S * lo.ld, lo.ld,
                             lo.bs, lse, s);
  return hipErrorInvalidValue;
}

namespace {

// Merge of attention results over disjoint key chunks of the same queries (sequence-sharded
// attention, the RingAttention level of "Wan 技术深度解析" §5.2):
// with lse = log sum_n exp(lse_n), o = sum_n exp(lse_n - lse) o_n.
// One thread per 8 channels of one (row, head); a (row, head) pair's hd/8 threads sit in one wave,
// and consecutive pairs are consecutive heads of a row, so the o reads are contiguous.
struct MergeParts {
  const void* o[MERGE_MAX_PARTS];
  const float* lse[MERGE_MAX_PARTS];
};

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const u32x4 r = *reinterpret_cast<const u32x4*>(p);
    const T* e = reinterpret_cast<const T*>(&r);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = to_f32(e[i]);
  } else {
    const float4 a = reinterpret_cast<const float4*>(p)[0], c = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = c.x, v[5] = c.y, v[6] = c.z, v[7] = c.w;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void lse_merge_kernel(MergeParts parts, int n, int64_t pairs, int S, int H,
                                                        int hd, T* __restrict__ out, float* __restrict__ lse_out) {
  const int cpp = hd >> 3;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= pairs * cpp) return;
  const int64_t pair = t / cpp;  // row * H + h, row = b * S + s
  const int c = (int)(t - pair * cpp);
  const int64_t row = pair / H;
  const int h = (int)(pair - row * H);
  const int64_t b = row / S;
  const int64_t li = (b * H + h) * S + (row - b * S);
  float w[MERGE_MAX_PARTS];
  float m = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < MERGE_MAX_PARTS; ++i)
    if (i < n) {
      w[i] = parts.lse[i][li];
      m = fmaxf(m, w[i]);
    }
  float z = 0.f;
#pragma unroll
  for (int i = 0; i < MERGE_MAX_PARTS; ++i)
    if (i < n) {
      w[i] = expf(w[i] - m);
      z += w[i];
    }
  const float inv = 1.f / z;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int64_t off = pair * hd + c * 8;
#pragma unroll
  for (int i = 0; i < MERGE_MAX_PARTS; ++i)
    if (i < n) {
      float v[8];
      load8(reinterpret_cast<const T*>(parts.o[i]) + off, v);
      const float wi = w[i] * inv;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(wi, v[e], acc[e]);
    }
  if constexpr (sizeof(T) == 2) {
    bf16x4 lo, hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) lo[e] = (bf16)acc[e], hi[e] = (bf16)acc[4 + e];
    reinterpret_cast<bf16x4*>(out + off)[0] = lo;
    reinterpret_cast<bf16x4*>(out + off)[1] = hi;
  } else {
    reinterpret_cast<float4*>(out + off)[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    reinterpret_cast<float4*>(out + off)[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
  if (lse_out != nullptr && c == 0) lse_out[li] = m + logf(z);
}

}  // namespace

template <typename T>
hipError_t launch_lse_merge(const void* const* o_parts, const float* const* lse_parts, int n, int B, int S, int H,
                            int hd, T* o, float* lse, hipStream_t s) {
  if (n < 1 || n > MERGE_MAX_PARTS || hd % 8 != 0) return hipErrorInvalidValue;
  if (B <= 0 || S <= 0 || H <= 0) return hipSuccess;
  MergeParts mp{};
  for (int i = 0; i < n; ++i) mp.o[i] = o_parts[i], mp.lse[i] = lse_parts[i];
  const int64_t pairs = (int64_t)B * S * H;
  const int64_t threads = pairs * (hd / 8);
  hipLaunchKernelGGL(lse_merge_kernel<T>, dim3((unsigned)ceil_div(threads, 256)), dim3(256), 0, s, mp, n, pairs, S, H,
                     hd, o, lse);
  return hipGetLastError();
}

template hipError_t launch_lse_merge<float>(const void* const*, const float* const*, int, int, int, int, int, float*,
                                            float*, hipStream_t);
template hipError_t launch_lse_merge<bf16>(const void* const*, const float* const*, int, int, int, int, int, bf16*,
                                           float*, hipStream_t);

template hipError_t launch_attention<float>(const float*, int64_t, int64_t, KVStream, int, int, int, int, float,
                                            float*, int64_t, int64_t, int, hipStream_t, float*, KeySplit, bool,
                                            const float*, int64_t);
template hipError_t launch_attention<bf16>(const bf16*, int64_t, int64_t, KVStream, int, int, int, int, float, bf16*,
                                           int64_t, int64_t, int, hipStream_t, float*, KeySplit, bool, const float*,
                                           int64_t);

template <typename T>
void attention_tile(int kind, int& rows, int& per_cu) {
  if (sizeof(T) == 2 && kind == 0) {
    rows = 256;  // ping-pong kernel: 8 waves, one workgroup per compute unit
    per_cu = 1;
  } else {
    rows = 128;  // four-wave kernel, __launch_bounds__(256, 2)
    per_cu = 2;
  }
}
template void attention_tile<float>(int, int&, int&);
template void attention_tile<bf16>(int, int&, int&);

}  // namespace wan
