// Fused-dequant split-K decode attention for gfx950 (CDNA4).
//
// What it computes ("W4A16 + KV cache quantization: combined accuracy",
// section on where the errors meet; "KV Cache Quantization Analysis",
// sec. 4 KIVI and sec. 5 system integration): for every sequence and query
// head, softmax(q . k_hat / sqrt(D)) over all cached tokens, times v_hat,
// where k_hat / v_hat are the dequantized codes (x_hat = s * (q - z), or
// s * E4M3 for FP8) or the fp16 sink / residual entries.  Dequantization is
// fused into the two matrix products, so only packed bytes cross HBM.
//
// Work decomposition (workgroups of eight wavefronts, one per compute unit
// by default):
//  * the quantized 32-token blocks of all heads, flattened head-major, are
//    cut into ranges, one per workgroup (see AttnParams).  The wavefronts of a
//    workgroup take the blocks of its range from a shared counter in LDS,
//    each keeping its next kDepth blocks' loads in flight, so wavefronts the
//    memory system serves faster take more blocks and the workgroup's
//    wavefronts finish together.  For every head it meets a wavefront runs
//    an online softmax for all n_rep query heads of that KV head (GQA: every
//    KV byte is read once per step) and writes one partial (max, sum,
//    unnormalised output);
//  * INT4 / INT2 take two blocks per step: at n_rep <= 4 the two blocks
//    share the matrix columns (one block per column parity), at n_rep 8 they
//    take separate products into one accumulator (column slots);
//  * the fp16 segment (sinks + residual ring) of every head is cut into
//    32-token blocks, dealt to the workgroups that cover the head and taken
//    from a second LDS counter by wavefronts that have run out of quantized
//    blocks, so they fill the wait for the workgroup's slowest wavefront;
//  * at the end a workgroup merges, per head, its wavefronts' partials
//    (the last one from LDS) and its fp16 partials.  A head that it covers
//    alone goes straight to the output; a head shared with neighbouring
//    workgroups is counted on the head's counter (sync plane of the cache):
//    the workgroup whose arrival completes the count combines the head in
//    covering order once the others have written their merged slots.
//
// Per 32-token block a wavefront runs both products on the matrix cores with
// v_mfma_f32_16x16x32_f16 (fp32 accumulate):
//  QK:  D[token][col] = codes[token][channel] x q'[channel][col]
//  PV:  D[channel][col] = codes[channel][token] x P'[token][col]
// Column col = lane % 16 is query head (col % 8) of the KV head's group;
// columns 0-7 carry the fp16 "hi" part of the fp32 operand and columns 8-15
// its "lo" remainder (hi = f16(x), lo = f16(x - hi)), so the fp32 operand is
// represented to ~22 bits and the two column halves are summed after the
// product (DPP row_ror:8).  Integer codes enter the matrix cores as exact
// f16 subnormals (the code's bits placed in the low mantissa bits, value
// code * 2^-24, times a power of two that depends on the code's position and
// is divided out of the staged scale); E4M3 codes are converted exactly by
// the hardware.  No dequantization error is added:
//  * Key fold: q . k_hat = sum_c (q_c s_c) code_c - sum_c q_c s_c z_c, with
//    q' = q * s per channel (recomputed per block: the Key scale varies per
//    32-token group) and the zero-point sum as the accumulator's initial value;
//  * Value fold: p_t v_hat_tc = (p_t s_tg) code_tc - p_t s_tg z_tg, with
//    P' = p * s per token and channel group; the zero-point sums are
//    accumulated on the VALU and subtracted at the end.
// The softmax runs in base 2 (log2(e) / sqrt(D) folded into q).
#include <atomic>
#include <type_traits>

#include "kvq_internal.h"

// 1: the "slot written" mark is a release fetch-add and the combining
// workgroup's polls are acquire loads (the language memory model's
// hand-over); 0: the hardware ordering of device-coherent stores, their
// acknowledgement, the barrier and the mark (see the end of group_main).
#ifndef KVQ_FORMAL_ORDERING
#define KVQ_FORMAL_ORDERING 0
#endif

namespace kvq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kQScale = kLog2e * 0.08838834764831845f;   // log2(e) / sqrt(128)
constexpr float kTwo24 = 16777216.0f;

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

// value of lane (lane + 8) mod 16 within the lane's row of 16 (DPP row_ror:8)
__device__ __forceinline__ float ror8(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128,
                                                               0xF, 0xF, false));
}

// Sum / max over the four 16-lane rows of the wavefront (lanes l, l^16, l^32,
// l^48).  v_permlane32_swap / v_permlane16_swap swap the upper half of their
// first operand with the lower half of the second; with both operands holding
// x the two results are {x[l], x[l^32]} (resp. {x[l], x[l^16]}).  The results
// are copied to scalars before __builtin_bit_cast: applied directly to an
// element of the returned vector, the cast reads element 0 for both.
__device__ __forceinline__ float rows_sum(float x) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned a0 = a[0], a1 = a[1];
  x = __builtin_bit_cast(float, a0) + __builtin_bit_cast(float, a1);
  u = __builtin_bit_cast(unsigned, x);
  const auto b = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned b0 = b[0], b1 = b[1];
  return __builtin_bit_cast(float, b0) + __builtin_bit_cast(float, b1);
}

__device__ __forceinline__ float rows_max(float x) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned a0 = a[0], a1 = a[1];
  x = fmaxf(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1));
  u = __builtin_bit_cast(unsigned, x);
  const auto b = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned b0 = b[0], b1 = b[1];
  return fmaxf(__builtin_bit_cast(float, b0), __builtin_bit_cast(float, b1));
}

__device__ __forceinline__ f16x2 u2h(uint32_t w) { return __builtin_bit_cast(f16x2, w); }

__device__ __forceinline__ f16x8 cat(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const f16x2 x = u2h(a), y = u2h(b), z = u2h(c), t = u2h(d);
  return f16x8{x[0], x[1], y[0], y[1], z[0], z[1], t[0], t[1]};
}

// 8 nibbles -> slots (n0, n4, 16*n1, 16*n5, n2, n6, 16*n3, 16*n7) x 2^-24
__device__ __forceinline__ f16x8 cvt_int4(uint32_t w) {
  const uint32_t w8 = w >> 8;
  return cat(w & 0x000F000Fu, w & 0x00F000F0u, w8 & 0x000F000Fu, w8 & 0x00F000F0u);
}

// 8 bytes (two words) -> slots in byte order, x 2^-24
__device__ __forceinline__ f16x8 cvt_u8(uint32_t w0, uint32_t w1) {
  const uint32_t lo = 0x0C010C00u, hi = 0x0C030C02u;   // [0, b1, 0, b0] / [0, b3, 0, b2]
  return cat(__builtin_amdgcn_perm(0u, w0, lo), __builtin_amdgcn_perm(0u, w0, hi),
             __builtin_amdgcn_perm(0u, w1, lo), __builtin_amdgcn_perm(0u, w1, hi));
}

// 16 two-bit codes c0..c15: low half -> slots (c_k, c_{8+k}) * 4^k, high half
// (codes shifted down a byte) -> (c_{4+k}, c_{12+k}) * 4^k, k = 0..3, x 2^-24
__device__ __forceinline__ f16x8 cvt_int2(uint32_t w, bool high) {
  const uint32_t x = high ? (w >> 8) : w;
  return cat(x & 0x00030003u, x & 0x000C000Cu, x & 0x00300030u, x & 0x00C000C0u);
}

// 8 OCP E5M2 bytes -> exact f16 values in byte order: an E5M2 code is the
// upper byte of the f16 with the same value
__device__ __forceinline__ f16x8 cvt_e5m2(uint32_t w0, uint32_t w1) {
  const uint32_t lo = 0x010C000Cu, hi = 0x030C020Cu;   // [b1, 0, b0, 0] / [b3, 0, b2, 0]
  return cat(__builtin_amdgcn_perm(0u, w0, lo), __builtin_amdgcn_perm(0u, w0, hi),
             __builtin_amdgcn_perm(0u, w1, lo), __builtin_amdgcn_perm(0u, w1, hi));
}

// 8 OCP E4M3 bytes -> exact f16 values in byte order (hardware conversion)
__device__ __forceinline__ f16x8 cvt_fp8(uint32_t w0, uint32_t w1) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Prefetch depths (blocks in flight besides the one being processed); build
// knobs for tuning, the defaults keep every format at or under 256 VGPRs.
#ifndef KVQ_DEPTH_INT8
#define KVQ_DEPTH_INT8 1
#endif
#ifndef KVQ_DEPTH_FP8
#define KVQ_DEPTH_FP8 2
#endif
#ifndef KVQ_DEPTH_INT4
#define KVQ_DEPTH_INT4 3
#endif
#ifndef KVQ_DEPTH_INT2
#define KVQ_DEPTH_INT2 4
#endif

// Ring sizes of the paired path (blocks, even): the pair being processed plus
// (ring - 2) blocks in flight.
#ifndef KVQ_PAIR_RING_INT4
#define KVQ_PAIR_RING_INT4 4
#endif
#ifndef KVQ_PAIR_RING_INT2
#define KVQ_PAIR_RING_INT2 6
#endif

// FMT is a kernel variant: the kvq_format, plus kMeta16 for fp16 metadata.
template <int FMT>
struct Traits {
  static constexpr int kKind = kind_of(FMT);
  static constexpr bool kMeta16 = meta16_of(FMT);
  static constexpr bool kRope = rope_of(FMT);     // Keys stored before RoPE, in pair order
  static constexpr bool kOut = outliers_of(FMT);  // one exact outlier per quantization group
  static constexpr bool kFp8 = fp8_of(FMT);
  static constexpr int kBits = kKind == KVQ_INT4 ? 4 : (kKind == KVQ_INT2 ? 2 : 8);
  static constexpr int kRowBytes = kHeadDim * kBits / 8;   // packed bytes per token
  static constexpr int kKWords = 32 * kBits / 32;          // words per lane per 16-token tile
  static constexpr int kVWords = kRowBytes / 8;            // words per V record (= per lane)
  // blocks kept in flight besides the one being processed (bytes in flight
  // per wavefront: INT8 10 KiB, FP8 16 KiB, INT4 18 KiB, INT2 16 KiB; the
  // counts keep every format at or under 256 VGPRs, two wavefronts per SIMD)
  static constexpr int kDepthBase = kFp8 ? KVQ_DEPTH_FP8 : (kBits == 8 ? KVQ_DEPTH_INT8 : (kBits == 4 ? KVQ_DEPTH_INT4 : KVQ_DEPTH_INT2));
  // the rotation's temporaries leave room for at most two blocks in flight,
  // the outlier corrections' for two (INT4) or three (INT2)
  static constexpr int kDepthCap = kRope ? 2 : (kOut ? (kBits == 2 ? 3 : 2) : kDepthBase);
  static constexpr int kDepth = kDepthBase < kDepthCap ? kDepthBase : kDepthCap;
  // paired processing (INT4 / INT2 at n_rep <= 4, see process_pair): two blocks per step, the
  // ring holds the pair being processed and the next pairs' loads
  static constexpr bool kPairable = !kFp8 && !kRope && kBits < 8;   // (the slot path: also !kOut)
  static constexpr int kPairRing = kOut ? 4 : (kBits == 2 ? KVQ_PAIR_RING_INT2 : KVQ_PAIR_RING_INT4);
  static constexpr float kCodeScale = kFp8 ? 1.0f : kTwo24;   // undoes the subnormal placement
};

// Matrix-core operand number a (K: k-block kb of the lane's 32 channels;
// V: 16-channel tile m) from the lane's packed words.
template <int FMT>
__device__ __forceinline__ f16x8 operand(const uint32_t* w, int a) {
  if constexpr (kind_of(FMT) == KVQ_INT4) return cvt_int4(w[a]);
  else if constexpr (kind_of(FMT) == KVQ_INT2) return cvt_int2(w[a >> 1], (a & 1) != 0);
  else if constexpr (kind_of(FMT) == KVQ_FP8_E4M3) return cvt_fp8(w[2 * a], w[2 * a + 1]);
  else if constexpr (kind_of(FMT) == KVQ_FP8_E5M2) return cvt_e5m2(w[2 * a], w[2 * a + 1]);
  else return cvt_u8(w[2 * a], w[2 * a + 1]);
}

// Channel (0..31 within the lane's quarter) carried by k-slot j of k-block kb.
template <int FMT>
__device__ constexpr int k_chan(int kb, int j) {
  if constexpr (kind_of(FMT) == KVQ_INT4) return 8 * kb + (j >> 1) + 4 * (j & 1);
  else if constexpr (kind_of(FMT) == KVQ_INT2) return 16 * (kb >> 1) + 4 * (kb & 1) + (j >> 1) + 8 * (j & 1);
  else return 8 * kb + j;
}

// Within-quarter position ("slot") of channel w (0..31) in the Key operand
// order: slot 8 kb + j carries channel k_chan(kb, j).
template <int FMT>
__device__ constexpr int k_slot(int w) {
  for (int kb = 0; kb < 4; ++kb)
    for (int j = 0; j < 8; ++j)
      if (k_chan<FMT>(kb, j) == w) return 8 * kb + j;
  return 0;
}

// Power-of-two factor the conversion leaves on code i (channel for K, token
// for V); it is divided out of the staged scale.
template <int FMT>
__device__ constexpr float slot_div(int i) {
  if constexpr (kind_of(FMT) == KVQ_INT4) return (i & 1) ? 16.0f : 1.0f;
  else if constexpr (kind_of(FMT) == KVQ_INT2) return (float)(1 << (2 * (i & 3)));
  else return 1.0f;
}

template <int FMT>
struct Raw {
  uint32_t k[2][Traits<FMT>::kKWords];   // two 16-token tiles
  uint32_t v[Traits<FMT>::kVWords];
  float4 km, vm;                         // this lane's part of each metadata block: 16 bytes
                                         // of fp32 pairs, or 8 bytes of fp16 pairs in .x / .y
  uint2 ko, vo;                          // outliers: this lane's two K and two V entries
};

// Code lines are read once per call: nontemporal loads keep them from
// displacing the metadata, query and partials in the caches.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
template <bool kStream>
__device__ __forceinline__ uint4 load_stream(const uint4* ptr) {
  if constexpr (kStream) {
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr));
    return uint4{t.x, t.y, t.z, t.w};
  } else {
    return *ptr;
  }
}

// Loads one block, record rec of the code and meta planes.  rec is
// wave-uniform, so the block base is a scalar and the per-lane parts are
// 32-bit offsets.
// Every code load of a wavefront reads whole 128-byte lines: 8-bit K is
// stored as 16-byte units (tile, half, lane) and V records are split into
// 16-byte groups stored group-major, so lane l of a load reads unit l.
template <int FMT, bool kStream = true>
__device__ __forceinline__ void load_block(Raw<FMT>& r, const AttnParams& p, int64_t rec, int lane) {
  using T = Traits<FMT>;
  const int64_t id = rec;
  const uint8_t* kb = p.k_codes + id * (int64_t)(kBlock * T::kRowBytes);
  const uint8_t* vb = p.v_codes + id * (int64_t)(kBlock * T::kRowBytes);
  const uint4* k16 = reinterpret_cast<const uint4*>(kb);
  const uint32_t qd = (uint32_t)lane >> 4;
#pragma unroll
  for (int tile = 0; tile < 2; ++tile) {
    if constexpr (T::kKWords == 8) {
      const uint4 a = load_stream<kStream>(k16 + (2 * tile) * 64 + lane);
      const uint4 b = load_stream<kStream>(k16 + (2 * tile + 1) * 64 + lane);
      r.k[tile][0] = a.x; r.k[tile][1] = a.y; r.k[tile][2] = a.z; r.k[tile][3] = a.w;
      r.k[tile][4] = b.x; r.k[tile][5] = b.y; r.k[tile][6] = b.z; r.k[tile][7] = b.w;
    } else {
      const uint8_t* src = kb + ((16u * tile + ((uint32_t)lane & 15u)) * T::kRowBytes + qd * (T::kKWords * 4));
      if constexpr (T::kKWords == 4) {
        const uint4 a = load_stream<kStream>(reinterpret_cast<const uint4*>(src));
        r.k[tile][0] = a.x; r.k[tile][1] = a.y; r.k[tile][2] = a.z; r.k[tile][3] = a.w;
      } else {
        const uint2 a = *reinterpret_cast<const uint2*>(src);
        r.k[tile][0] = a.x; r.k[tile][1] = a.y;
      }
    }
  }
  const uint4* v16 = reinterpret_cast<const uint4*>(vb);
#pragma unroll
  for (int i = 0; i < T::kVWords / 4; ++i) {
    const uint4 a = load_stream<kStream>(v16 + i * 64 + lane);
    r.v[4 * i] = a.x; r.v[4 * i + 1] = a.y; r.v[4 * i + 2] = a.z; r.v[4 * i + 3] = a.w;
  }
  if constexpr (T::kMeta16) {
    const uint2 a = reinterpret_cast<const uint2*>(p.k_meta + id * 128)[lane];
    const uint2 b = reinterpret_cast<const uint2*>(p.v_meta + id * 128)[lane];
    r.km = float4{__builtin_bit_cast(float, a.x), __builtin_bit_cast(float, a.y), 0.f, 0.f};
    r.vm = float4{__builtin_bit_cast(float, b.x), __builtin_bit_cast(float, b.y), 0.f, 0.f};
  } else if constexpr (!T::kFp8) {
    r.km = reinterpret_cast<const float4*>(p.k_meta + id * 256)[lane];
    r.vm = reinterpret_cast<const float4*>(p.v_meta + id * 256)[lane];
  }
  if constexpr (T::kOut) {
    r.ko = reinterpret_cast<const uint2*>(p.k_out + id * kHeadDim)[lane];
    r.vo = reinterpret_cast<const uint2*>(p.v_out + id * kHeadDim)[lane];
  }
}

// The running max may grow by up to 2^kSlack before the accumulators are
// rescaled, so p = 2^(logit - m) <= 2^kSlack.  The P' operands p * s stay
// finite in f16 as long as s <= 255; a block holding a larger Value scale is
// processed with an exact running max instead (p <= 1, p * s <= s).
constexpr float kSlack = 8.0f;
constexpr float kLazyScaleMax = 255.0f;

// LDS staging area of one wavefront for one block (floats):
//   [0,128) K scale / slot divisor   [128,256) K s*z (pre-RoPE Keys: fp32;
//   otherwise f16 hi / lo pairs, 16-bit [256 + slot] and [384 + slot])
//   [256,384) V scale / divisor [g][t]   [384,512) V s*z [g][t]
// and with outliers (see stage_meta)
//   [512,640) K outlier corrections (slot order)   [640,768) V outlier corrections [g][t]
//   [768,832) K outlier tokens (16-bit, slot order)   [832,896) V outlier channels (16-bit)
// The paired and slot paths stage their second block from kStage on, or with
// outliers from 896 on.
constexpr int kStage = 512;
constexpr int kOutKd = 512, kOutVd = 640, kOutKx = 768, kOutVx = 832;
// Outlier corrections go through the matrix cores as (one-hot) x (q or p times
// the correction): the one-hot operand holds 2^kOhShift * 2^-24 (an f16
// subnormal, like the codes) and the staged corrections carry 2^-kOhShift,
// which keeps p * correction inside the f16 range.  Staged indices carry the
// same shift, so index ^ (token << kOhShift) is either 0 or >= 2^kOhShift.
constexpr int kOhShift = 8;
constexpr float kOhScale = 1.0f / 256.0f;

// Slot (see k_slot) of within-quarter channel w, by formula.
template <int FMT>
__device__ __forceinline__ int k_slot_of(int w) {
  if constexpr (kind_of(FMT) == KVQ_INT4) {
    const int r = w & 7;
    return (w & ~7) + (r < 4 ? 2 * r : 2 * (r - 4) + 1);
  } else if constexpr (kind_of(FMT) == KVQ_INT2) {
    const int rem = w & 15, rem2 = rem & 7;
    return 8 * (2 * (w >> 4) + (rem2 >> 2)) + 2 * (rem2 & 3) + (rem >> 3);
  } else {
    return w;
  }
}

template <int FMT>
__device__ constexpr bool k_slot_formula_ok() {
  for (int w = 0; w < 32; ++w) {
    int r = w & 7, rem = w & 15, rem2 = rem & 7;
    int f = kind_of(FMT) == KVQ_INT4 ? (w & ~7) + (r < 4 ? 2 * r : 2 * (r - 4) + 1)
          : kind_of(FMT) == KVQ_INT2 ? 8 * (2 * (w >> 4) + (rem2 >> 2)) + 2 * (rem2 & 3) + (rem >> 3) : w;
    if (f != k_slot<FMT>(w)) return false;
  }
  return true;
}
static_assert(k_slot_formula_ok<KVQ_INT8>() && k_slot_formula_ok<KVQ_INT4>() && k_slot_formula_ok<KVQ_INT2>(),
              "Key slot formula");

// Scales of the lane's two metadata pairs (V: its two token / group
// entries): fp32 (s, z) pairs or fp16 (s, m) pairs.
template <int FMT>
__device__ __forceinline__ float2 pair_scales(const float4& m) {
  if constexpr (Traits<FMT>::kMeta16) {
    const f16x2 a = u2h(__builtin_bit_cast(uint32_t, m.x)), b = u2h(__builtin_bit_cast(uint32_t, m.y));
    return float2{(float)a[0], (float)b[0]};
  } else {
    return float2{m.x, m.z};
  }
}

// Lane L holds the metadata pairs 2L and 2L+1 of each block.  The Key scale
// (with log2(e) / sqrt(D) and the slot divisor folded in) and s * z (with
// log2(e) / sqrt(D)) go to LDS in Key slot order per quarter.  fp16 pairs
// hold (s, m) with x_hat = s * q + m, so their s * z is -m.
// Pre-RoPE Keys are dequantized before the rotation instead: their staged
// Key values are s * 2^24 / slot divisor and the offset -s * z (= m for
// fp16 pairs), so that k_hat = operand value * [0] + [128].
// Outliers: a Key outlier x at (token t, channel c) adds q_c (x - x_hat(0))
// to the logit of t, x_hat(0) being what code 0 decodes to; a Value outlier
// at (t, c) adds p_t (x - x_hat(0)) to output channel c.  The corrections
// x - x_hat(0) (Keys: in logit units) times 2^-kOhShift go to [512 + slot]
// and [640 + g * 32 + t]; the Key outlier tokens to 16-bit [slot], the Value
// outlier channels to 16-bit [g * 32 + 2 (t % 16) + t / 16] (the Value
// operand pairs tokens t and t + 16), all shifted up by kOhShift.  Returns
// the largest |Value correction| of the lane's entries (0 without outliers).
template <int FMT>
__device__ __forceinline__ float stage_meta(const Raw<FMT>& r, float* st, int lane) {
  const int c = 2 * lane;                 // K stored position; V index g * 32 + t
  const int t = c & 31;
  constexpr bool kRopeK = Traits<FMT>::kRope;
  constexpr float kKs = kRopeK ? kTwo24 : kQScale;     // factor on the staged Key scale
  float sq0, sq1, kz0, kz1;
  float2 vs, vz;
  if constexpr (Traits<FMT>::kMeta16) {
    const f16x2 ka = u2h(__builtin_bit_cast(uint32_t, r.km.x)), kb = u2h(__builtin_bit_cast(uint32_t, r.km.y));
    const f16x2 va = u2h(__builtin_bit_cast(uint32_t, r.vm.x)), vb = u2h(__builtin_bit_cast(uint32_t, r.vm.y));
    sq0 = (float)ka[0] * kKs;
    sq1 = (float)kb[0] * kKs;
    kz0 = kRopeK ? (float)ka[1] : -(float)ka[1] * kQScale;
    kz1 = kRopeK ? (float)kb[1] : -(float)kb[1] * kQScale;
    vs = float2{(float)va[0] * (1.0f / slot_div<FMT>(t)), (float)vb[0] * (1.0f / slot_div<FMT>(t + 1))};
    vz = float2{-(float)va[1], -(float)vb[1]};
  } else {
    sq0 = r.km.x * kKs;
    sq1 = r.km.z * kKs;
    kz0 = kRopeK ? -(r.km.x * r.km.y) : sq0 * r.km.y;
    kz1 = kRopeK ? -(r.km.z * r.km.w) : sq1 * r.km.w;
    vs = float2{r.vm.x * (1.0f / slot_div<FMT>(t)), r.vm.z * (1.0f / slot_div<FMT>(t + 1))};
    vz = float2{r.vm.x * r.vm.y, r.vm.z * r.vm.w};
  }
  const float ks0 = sq0 * (1.0f / slot_div<FMT>(c)), ks1 = sq1 * (1.0f / slot_div<FMT>(c + 1));
  const int q0 = (c & ~31) + k_slot_of<FMT>(c & 31), q1 = (c & ~31) + k_slot_of<FMT>((c + 1) & 31);
  // Keys with a zero-point term: the term as an f16 hi / lo pair (hi at
  // 16-bit [256 + slot], lo at [384 + slot]), so that the bias is formed
  // with packed-f16 dot products against the query pairs
  uint16_t* zst = reinterpret_cast<uint16_t*>(st);
  auto zsplit = [](float x, uint16_t& h, uint16_t& l) {
    const _Float16 xh = (_Float16)x;
    h = __builtin_bit_cast(uint16_t, xh);
    l = __builtin_bit_cast(uint16_t, (_Float16)(x - (float)xh));
  };
  if constexpr (kind_of(FMT) == KVQ_INT8) {
    *reinterpret_cast<float2*>(st + q0) = float2{ks0, ks1};
    if constexpr (kRopeK) {
      *reinterpret_cast<float2*>(st + 128 + q0) = float2{kz0, kz1};
    } else {
      uint16_t h0, l0, h1, l1;
      zsplit(kz0, h0, l0);
      zsplit(kz1, h1, l1);
      *reinterpret_cast<uint32_t*>(zst + 256 + q0) = (uint32_t)h0 | ((uint32_t)h1 << 16);
      *reinterpret_cast<uint32_t*>(zst + 384 + q0) = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
  } else {
    st[q0] = ks0;
    st[q1] = ks1;
    if constexpr (kRopeK) {
      st[128 + q0] = kz0;
      st[128 + q1] = kz1;
    } else {
      zsplit(kz0, zst[256 + q0], zst[384 + q0]);
      zsplit(kz1, zst[256 + q1], zst[384 + q1]);
    }
  }
  *reinterpret_cast<float2*>(st + 256 + c) = vs;
  *reinterpret_cast<float2*>(st + 384 + c) = vz;
  if constexpr (Traits<FMT>::kOut) {
    auto value = [](uint32_t e) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(e >> 16)); };
    uint16_t* kx = reinterpret_cast<uint16_t*>(st + kOutKx);
    uint16_t* vx = reinterpret_cast<uint16_t*>(st + kOutVx);
    st[kOutKd + q0] = __builtin_fmaf(value(r.ko.x), kQScale, kz0) * kOhScale;
    st[kOutKd + q1] = __builtin_fmaf(value(r.ko.y), kQScale, kz1) * kOhScale;
    kx[q0] = (uint16_t)((r.ko.x & 31u) << kOhShift);
    kx[q1] = (uint16_t)((r.ko.y & 31u) << kOhShift);
    const float d0 = value(r.vo.x) + vz.x, d1 = value(r.vo.y) + vz.y;
    *reinterpret_cast<float2*>(st + kOutVd + c) = float2{d0 * kOhScale, d1 * kOhScale};
    const int pv = (c & ~31) + 2 * (t & 15) + (t >> 4);    // token t + 1 lands at pv + 2
    vx[pv] = (uint16_t)((r.vo.x & 31u) << kOhShift);
    vx[pv + 2] = (uint16_t)((r.vo.y & 31u) << kOhShift);
    return fmaxf(fabsf(d0), fabsf(d1));
  }
  return 0.f;
}

// One-hot operand word: for two slots, 2^kOhShift (as f16 bits) where the
// staged index equals the row's own (both shifted by kOhShift), else 0.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t one_hot(uint32_t idx, uint32_t own) {
  const u16x2 x = __builtin_bit_cast(u16x2, idx ^ own);
  const u16x2 top = {1u << kOhShift, 1u << kOhShift};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(top, x));
}

struct WaveState {
  float m;          // running max (base-2 logits) of this lane's column
  float l;          // this lane's partial softmax denominator
  f32x4 o[8];       // PV accumulator: rows 16m + 4qd + i, column col
  float z[4];       // Value zero-point sums of channel groups zg, zg + 1 (slot path: groups 0-3)
};

struct LaneInfo {
  int lane, qd, head, nrep;
  bool is_lo;       // column carries the lo remainder
  bool writer;      // hi column of a real query head: writes the results
  uint32_t hmask;   // 0xFFFFFFFF in lo columns, 0 in hi columns
  int zg;           // first Value channel group whose zero-point sum this lane keeps
  int par;          // paired path: which block of the pair this column serves (0 or 1)
  uint32_t amask;   // paired path: 0xFFFFFFFF in columns of the pair's first block, else 0
};

__device__ __forceinline__ LaneInfo lane_info(int nrep) {
  LaneInfo li;
  li.lane = threadIdx.x & 63;
  li.nrep = nrep;
  const int col = li.lane & 15;
  li.qd = li.lane >> 4;
  li.head = col & 7;
  li.is_lo = col >= 8;
  li.writer = !li.is_lo && li.head < nrep;
  li.hmask = li.is_lo ? 0xFFFFFFFFu : 0u;
  li.zg = li.is_lo ? 2 : 0;
  li.par = 0;
  li.amask = 0xFFFFFFFFu;
  return li;
}

// Slot path (n_rep 8): column col = 8 slot + head, query head col % 8 of
// the pair's block slot; hi and lo operand parts go through separate
// matrix-core products into one accumulator, so no column carries a lo part.
__device__ __forceinline__ LaneInfo lane_info_slot(int nrep) {
  LaneInfo li = lane_info(nrep);
  const int col = li.lane & 15;
  li.head = col & 7;
  li.par = col >> 3;
  li.is_lo = false;
  li.hmask = 0u;
  li.zg = 0;
  li.amask = li.par ? 0u : 0xFFFFFFFFu;
  li.writer = li.par == 0 && li.head < nrep;
  return li;
}

// Paired path (n_rep <= 4): column col = 8 lo + 4 par + head, i.e. query head
// col % 4 of the pair's block par, hi part in columns 0-7, lo in 8-15 (so
// the hi / lo partner is still lane + 8).  Both parities hold the same head;
// their softmax states are merged when the head's segment ends.
__device__ __forceinline__ LaneInfo lane_info_pair(int nrep) {
  LaneInfo li = lane_info(nrep);
  const int col = li.lane & 15;
  li.head = col & 3;
  li.par = (col >> 2) & 1;
  li.amask = li.par ? 0u : 0xFFFFFFFFu;
  li.writer = !li.is_lo && li.par == 0 && li.head < nrep;
  return li;
}

__device__ __forceinline__ void reset(WaveState& ws) {
  ws.m = neg_inf();
  ws.l = 0.f;
#pragma unroll
  for (int m = 0; m < 8; ++m) ws.o[m] = f32x4{0, 0, 0, 0};
  ws.z[0] = ws.z[1] = ws.z[2] = ws.z[3] = 0.f;
}

// hi / lo operand pairs.  A column's operand is hi = f16(x) in hi columns and
// lo = f16(x - f16(x)) in lo columns; with xz = x in lo columns and 0 in hi
// columns both are r = f16(x - f16(xz)).  v_fma_mix rounds the fp32 fma
// a * b - c once to f16; its operands may be fp32 or a half of a packed f16
// register (op_sel / op_sel_hi), so one instruction forms each half.
//
// One asm statement forms all four words of an operand (16 instructions, in
// four independent waves of four).  The compiler pads between dependent asm
// statements and does not count asm as a vector write when it spaces a
// vector write from a matrix-core read of the same register (two wait
// states), so the statement ends with s_nop 1: every word is then at least
// two wait states old when the operand is read.

// x = q * s for eight channels: q from packed f16 (both halves of qh[j], and
// of qz[j] = qh[j] in lo columns, 0 in hi columns), s[2j], s[2j + 1] fp32.
__device__ __forceinline__ f16x8 split_q4(const uint32_t* qz, const uint32_t* qh, float4 sa, float4 sb) {
  uint32_t r0, r1, r2, r3, h0, h1, h2, h3;
  asm("v_fma_mixlo_f16 %4, %8, %16, 0 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixlo_f16 %5, %9, %18, 0 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixlo_f16 %6, %10, %20, 0 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixlo_f16 %7, %11, %22, 0 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %4, %8, %17, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %5, %9, %19, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %6, %10, %21, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %7, %11, %23, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixlo_f16 %0, %12, %16, -%4 op_sel_hi:[1,0,1]\n\t"
      "v_fma_mixlo_f16 %1, %13, %18, -%5 op_sel_hi:[1,0,1]\n\t"
      "v_fma_mixlo_f16 %2, %14, %20, -%6 op_sel_hi:[1,0,1]\n\t"
      "v_fma_mixlo_f16 %3, %15, %22, -%7 op_sel_hi:[1,0,1]\n\t"
      "v_fma_mixhi_f16 %0, %12, %17, -%4 op_sel:[1,0,1] op_sel_hi:[1,0,1]\n\t"
      "v_fma_mixhi_f16 %1, %13, %19, -%5 op_sel:[1,0,1] op_sel_hi:[1,0,1]\n\t"
      "v_fma_mixhi_f16 %2, %14, %21, -%6 op_sel:[1,0,1] op_sel_hi:[1,0,1]\n\t"
      "v_fma_mixhi_f16 %3, %15, %23, -%7 op_sel:[1,0,1] op_sel_hi:[1,0,1]\n\t"
      "s_nop 1"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(h0), "=&v"(h1), "=&v"(h2), "=&v"(h3)
      : "v"(qz[0]), "v"(qz[1]), "v"(qz[2]), "v"(qz[3]), "v"(qh[0]), "v"(qh[1]), "v"(qh[2]), "v"(qh[3]),
        "v"(sa.x), "v"(sa.y), "v"(sa.z), "v"(sa.w), "v"(sb.x), "v"(sb.y), "v"(sb.z), "v"(sb.w));
  return cat(r0, r1, r2, r3);
}

// x = a * b for eight values, all fp32: word j holds (a0[j] b0[j], a1[j] b1[j]);
// az = a in lo columns, 0 in hi columns.
__device__ __forceinline__ f16x8 split_p4(const float* a0, const float* az0, const float* b0, const float* a1,
                                          const float* az1, const float* b1) {
  uint32_t r0, r1, r2, r3, h0, h1, h2, h3;
  asm("v_fma_mixlo_f16 %4, %12, %16, 0\n\t"
      "v_fma_mixlo_f16 %5, %13, %17, 0\n\t"
      "v_fma_mixlo_f16 %6, %14, %18, 0\n\t"
      "v_fma_mixlo_f16 %7, %15, %19, 0\n\t"
      "v_fma_mixhi_f16 %4, %24, %28, 0\n\t"
      "v_fma_mixhi_f16 %5, %25, %29, 0\n\t"
      "v_fma_mixhi_f16 %6, %26, %30, 0\n\t"
      "v_fma_mixhi_f16 %7, %27, %31, 0\n\t"
      "v_fma_mixlo_f16 %0, %8, %16, -%4 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixlo_f16 %1, %9, %17, -%5 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixlo_f16 %2, %10, %18, -%6 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixlo_f16 %3, %11, %19, -%7 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %0, %20, %28, -%4 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %1, %21, %29, -%5 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %2, %22, %30, -%6 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %3, %23, %31, -%7 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "s_nop 1"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(h0), "=&v"(h1), "=&v"(h2), "=&v"(h3)
      : "v"(a0[0]), "v"(a0[1]), "v"(a0[2]), "v"(a0[3]), "v"(az0[0]), "v"(az0[1]), "v"(az0[2]), "v"(az0[3]),
        "v"(b0[0]), "v"(b0[1]), "v"(b0[2]), "v"(b0[3]), "v"(a1[0]), "v"(a1[1]), "v"(a1[2]), "v"(a1[3]),
        "v"(az1[0]), "v"(az1[1]), "v"(az1[2]), "v"(az1[3]), "v"(b1[0]), "v"(b1[1]), "v"(b1[2]), "v"(b1[3]));
  return cat(r0, r1, r2, r3);
}

// hi and lo parts of x = q * s for eight channels in every lane (slot path):
// split_q4 with qz = qh gives hi = f16(x) as its first words and lo =
// f16(x - hi) as the result.
struct HiLo {
  f16x8 hi, lo;
};
__device__ __forceinline__ HiLo split_q4_both(const uint32_t* qh, float4 sa, float4 sb) {
  uint32_t r0, r1, r2, r3, h0, h1, h2, h3;
  asm("v_fma_mixlo_f16 %4, %8, %12, 0 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixlo_f16 %5, %9, %14, 0 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixlo_f16 %6, %10, %16, 0 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixlo_f16 %7, %11, %18, 0 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %4, %8, %13, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %5, %9, %15, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %6, %10, %17, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %7, %11, %19, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixlo_f16 %0, %8, %12, -%4 op_sel_hi:[1,0,1]\n\t"
      "v_fma_mixlo_f16 %1, %9, %14, -%5 op_sel_hi:[1,0,1]\n\t"
      "v_fma_mixlo_f16 %2, %10, %16, -%6 op_sel_hi:[1,0,1]\n\t"
      "v_fma_mixlo_f16 %3, %11, %18, -%7 op_sel_hi:[1,0,1]\n\t"
      "v_fma_mixhi_f16 %0, %8, %13, -%4 op_sel:[1,0,1] op_sel_hi:[1,0,1]\n\t"
      "v_fma_mixhi_f16 %1, %9, %15, -%5 op_sel:[1,0,1] op_sel_hi:[1,0,1]\n\t"
      "v_fma_mixhi_f16 %2, %10, %17, -%6 op_sel:[1,0,1] op_sel_hi:[1,0,1]\n\t"
      "v_fma_mixhi_f16 %3, %11, %19, -%7 op_sel:[1,0,1] op_sel_hi:[1,0,1]\n\t"
      "s_nop 1"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(h0), "=&v"(h1), "=&v"(h2), "=&v"(h3)
      : "v"(qh[0]), "v"(qh[1]), "v"(qh[2]), "v"(qh[3]),
        "v"(sa.x), "v"(sa.y), "v"(sa.z), "v"(sa.w), "v"(sb.x), "v"(sb.y), "v"(sb.z), "v"(sb.w));
  return HiLo{cat(h0, h1, h2, h3), cat(r0, r1, r2, r3)};
}

// The same for x = a * b with fp32 a, b (eight values: word j holds
// (a0[j] b0[j], a1[j] b1[j])).
__device__ __forceinline__ HiLo split_p4_both(const float* a0, const float* b0, const float* a1, const float* b1) {
  uint32_t r0, r1, r2, r3, h0, h1, h2, h3;
  asm("v_fma_mixlo_f16 %4, %8, %12, 0\n\t"
      "v_fma_mixlo_f16 %5, %9, %13, 0\n\t"
      "v_fma_mixlo_f16 %6, %10, %14, 0\n\t"
      "v_fma_mixlo_f16 %7, %11, %15, 0\n\t"
      "v_fma_mixhi_f16 %4, %16, %20, 0\n\t"
      "v_fma_mixhi_f16 %5, %17, %21, 0\n\t"
      "v_fma_mixhi_f16 %6, %18, %22, 0\n\t"
      "v_fma_mixhi_f16 %7, %19, %23, 0\n\t"
      "v_fma_mixlo_f16 %0, %8, %12, -%4 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixlo_f16 %1, %9, %13, -%5 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixlo_f16 %2, %10, %14, -%6 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixlo_f16 %3, %11, %15, -%7 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %0, %16, %20, -%4 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %1, %17, %21, -%5 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %2, %18, %22, -%6 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %3, %19, %23, -%7 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "s_nop 1"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(h0), "=&v"(h1), "=&v"(h2), "=&v"(h3)
      : "v"(a0[0]), "v"(a0[1]), "v"(a0[2]), "v"(a0[3]), "v"(b0[0]), "v"(b0[1]), "v"(b0[2]), "v"(b0[3]),
        "v"(a1[0]), "v"(a1[1]), "v"(a1[2]), "v"(a1[3]), "v"(b1[0]), "v"(b1[1]), "v"(b1[2]), "v"(b1[3]));
  return HiLo{cat(h0, h1, h2, h3), cat(r0, r1, r2, r3)};
}

// hi / lo pair of a fully fp32 operand (both parts in every lane):
// hi = f16(x), lo = f16(x - hi) (x - hi is exact in fp32), for two values;
// returns {hi, lo} words.  Written as ordinary code, not inline assembly:
// these registers go straight into a matrix-core instruction, and the
// compiler only keeps the required distance between a vector write and a
// matrix-core read of the same registers for instructions it can see.
__device__ __forceinline__ uint2 split_a(float x0, float x1) {
  const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
  const _Float16 l0 = (_Float16)(x0 - (float)h0), l1 = (_Float16)(x1 - (float)h1);
  return uint2{__builtin_bit_cast(uint32_t, f16x2{h0, h1}), __builtin_bit_cast(uint32_t, f16x2{l0, l1})};
}

// ---- rotary position embedding of pre-RoPE Keys (rotate-half pairs
// (i, i + 64), angle t * theta_i, theta_i = base^(-i/64)).
// theta_i in fp64.
__device__ __forceinline__ double rope_freq(float base, int i) {
  return exp2(-(double)i * (1.0 / 64.0) * log2((double)base));
}

// (cos, sin) of pos * freq: the angle is formed and reduced modulo 2 pi in
// fp64, so large positions keep full accuracy, then evaluated in fp32.
__device__ __forceinline__ float2 rope_cs(double pos, double freq) {
  constexpr double kTwoPi = 6.283185307179586;
  double a = pos * freq;
  a = a - kTwoPi * floor(a * (1.0 / kTwoPi));
  float sn, cs;
  sincosf((float)a, &sn, &cs);
  return float2{cs, sn};
}

// In-block offsets (cos, sin)(k * theta_i), k < 32, i < 64, shared by the
// workgroup in LDS: entry 64 k + i.
constexpr int kRopeTableBytes = 32 * 64 * 8;

// Query of this lane's column head (its quarter's 32 channels) from a KV
// head's n_rep query rows ([n_rep][128] fp16): packed f16 pairs in Key
// operand slot order (h[p] = slots 2p, 2p+1), and the same zeroed in hi
// columns (z).  Both are zero in columns of heads past n_rep.  The scale
// log2(e) / sqrt(D) is applied with the Key scales.  The raw load and the
// conversion are separate so the load can be issued early.
struct QRaw {
  uint4 w[4];
};

struct QOp {
  uint32_t h[16], z[16];
};

// The lane's 32 query channels: its quarter 32qd .. 32qd + 31, or for
// pre-RoPE Keys (PAIRS) the channels 16qd .. 16qd + 15 and 64 + 16qd ..
// 64 + 16qd + 15 (stored positions 32qd .. 32qd + 31 in pair order).
template <bool PAIRS = false>
__device__ __forceinline__ QRaw load_query_raw(const uint16_t* rows, int nrep, const LaneInfo& li) {
  const bool valid = li.head < nrep;
  const uint16_t* row = rows + (valid ? li.head : 0) * kHeadDim;
  QRaw r;
  if constexpr (PAIRS) {
    const uint4* a = reinterpret_cast<const uint4*>(row + 16 * li.qd);
    const uint4* b = reinterpret_cast<const uint4*>(row + kHeadDim / 2 + 16 * li.qd);
    r.w[0] = a[0]; r.w[1] = a[1]; r.w[2] = b[0]; r.w[3] = b[1];
  } else {
    const uint4* qsrc = reinterpret_cast<const uint4*>(row + 32 * li.qd);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.w[i] = qsrc[i];
  }
  return r;
}

template <int FMT>
__device__ __forceinline__ void query_operand(const QRaw& r, int nrep, const LaneInfo& li, QOp& q) {
  const uint32_t keep = li.head < nrep ? 0xFFFFFFFFu : 0u;
  const uint32_t w[16] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w, r.w[1].x, r.w[1].y, r.w[1].z, r.w[1].w,
                          r.w[2].x, r.w[2].y, r.w[2].z, r.w[2].w, r.w[3].x, r.w[3].y, r.w[3].z, r.w[3].w};
  // element of the loaded 32 holding stored position c: pair order keeps
  // channel i (position 2i) in the first 16 elements and i + 64 in the last
  auto elem = [](int c) { return Traits<FMT>::kRope ? ((c & 1) ? 16 + (c >> 1) : (c >> 1)) : c; };
#pragma unroll
  for (int pr = 0; pr < 16; ++pr) {
    const int c0 = elem(k_chan<FMT>(pr >> 2, 2 * (pr & 3))), c1 = elem(k_chan<FMT>(pr >> 2, 2 * (pr & 3) + 1));
    const uint32_t lo = (w[c0 >> 1] >> (16 * (c0 & 1))) & 0xFFFFu;
    const uint32_t hi = (w[c1 >> 1] >> (16 * (c1 & 1))) & 0xFFFFu;
    q.h[pr] = (lo | (hi << 16)) & keep;
    q.z[pr] = q.h[pr] & li.hmask;
  }
}

// The same from the query rows of KV head bh in global memory.
template <int FMT>
__device__ __forceinline__ void load_query(const AttnParams& p, int64_t bh, const LaneInfo& li, QOp& q) {
  query_operand<FMT>(load_query_raw<Traits<FMT>::kRope>(p.q + bh * p.nrep * kHeadDim, p.nrep, li), p.nrep, li, q);
}

// Static q operands (hi / lo) for Keys without a per-block scale (FP8 with
// its per-tensor scale, fp16 segment with scale 1); scale includes
// log2(e) / sqrt(D).
__device__ __forceinline__ void static_q(const QOp& q, float scale, f16x8* bk) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const float4 sc{scale, scale, scale, scale};
    bk[kb] = split_q4(q.z + 4 * kb, q.h + 4 * kb, sc, sc);
  }
}

// Online softmax over one block's 32 tokens (this lane: 8 of them, logits
// lg[tile][i] for tokens 16*tile + 4qd + i); returns p = 2^(lg - m).
__device__ __forceinline__ void softmax_block(float lg[2][4], WaveState& ws, float pr[2][4], float slack) {
  float mx = neg_inf();
#pragma unroll
  for (int tile = 0; tile < 2; ++tile)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, lg[tile][i]);
  mx = rows_max(mx);
  if (__any(mx > ws.m + slack)) {                // always true on the first block (m = -inf)
    const float m_new = fmaxf(ws.m, mx);
    const float alpha = __builtin_amdgcn_exp2f(ws.m - m_new);
#pragma unroll
    for (int m = 0; m < 8; ++m) ws.o[m] *= alpha;
#pragma unroll
    for (int g = 0; g < 4; ++g) ws.z[g] *= alpha;
    ws.l *= alpha;
    ws.m = m_new;
  }
#pragma unroll
  for (int tile = 0; tile < 2; ++tile)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[tile][i] = __builtin_amdgcn_exp2f(lg[tile][i] - ws.m);
      ws.l += pr[tile][i];
    }
}

// softmax_block for a wavefront whose inactive lanes (active = false) take no
// tokens: their state is left as it is and their p are 0.  Active lanes see at
// least one finite logit, so their new running max is finite.
__device__ __forceinline__ void softmax_block_some(float lg[2][4], WaveState& ws, float pr[2][4], float slack,
                                                   bool active) {
  float mx = neg_inf();
#pragma unroll
  for (int tile = 0; tile < 2; ++tile)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, lg[tile][i]);
  mx = rows_max(mx);
  if (!active) mx = neg_inf();
  if (__any(mx > ws.m + slack)) {
    const float m_new = fmaxf(ws.m, mx);
    const float alpha = active ? __builtin_amdgcn_exp2f(ws.m - m_new) : 1.0f;
#pragma unroll
    for (int m = 0; m < 8; ++m) ws.o[m] *= alpha;
#pragma unroll
    for (int g = 0; g < 4; ++g) ws.z[g] *= alpha;
    ws.l *= alpha;
    ws.m = active ? m_new : ws.m;
  }
#pragma unroll
  for (int tile = 0; tile < 2; ++tile)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[tile][i] = active ? __builtin_amdgcn_exp2f(lg[tile][i] - ws.m) : 0.f;
      ws.l += pr[tile][i];
    }
}

// P operand without a per-token scale (FP8: the per-tensor scale is applied
// at the end; fp16 segment: none).
__device__ __forceinline__ f16x8 p_operand(const float pr[2][4], const LaneInfo& li) {
  float z[2][4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    z[0][v] = li.is_lo ? pr[0][v] : 0.f;
    z[1][v] = li.is_lo ? pr[1][v] : 0.f;
  }
  const float one[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  return split_p4(pr[0], z[0], one, pr[1], z[1], one);
}

// Pre-RoPE Keys: this lane's RoPE frequency (theta_lane, for the block base
// angles) and the workgroup's in-block offset table.
struct RopeCtx {
  double freq;
  const float2* table;
};

// Key slot holding the other member of slot j's RoPE pair (stored positions
// 2i, 2i + 1), and whether slot j holds the first member.
template <int FMT>
__device__ constexpr int pair_slot(int j) {
  return (kind_of(FMT) == KVQ_INT4 || kind_of(FMT) == KVQ_INT2) ? (j ^ 2) : (j ^ 1);
}
template <int FMT>
__device__ constexpr bool pair_first(int j) {
  return (kind_of(FMT) == KVQ_INT4 || kind_of(FMT) == KVQ_INT2) ? ((j & 2) == 0) : ((j & 1) == 0);
}

// t0: position of the block's first token (pre-RoPE Keys only).
template <int FMT>
__device__ __forceinline__ void process_block(const Raw<FMT>& r, float* st, WaveState& ws, const QOp& q,
                                              const f16x8* bk_static, const LaneInfo& li, const RopeCtx& rc,
                                              double t0) {
  using T = Traits<FMT>;
  const int qd = li.qd;

  // ---- QK: Key codes (rows = tokens) x q' (columns)
  f32x4 acc[2];
  float vbig = 0.f;          // outliers: largest |Value correction| of the lane's entries
  float kbias = 0.f;         // zero-point term of the logits (INT Keys)
  if constexpr (T::kRope) {
    // Keys are dequantized, rotated at their positions t0 + token and split
    // into hi / lo f16 operands; the query operand is static (q, hi / lo
    // columns).  Rotation angle of (token k, frequency i) = base_i * offset_ki
    // as complex numbers: base = (t0 theta_i), staged by lane i; offset from
    // the workgroup table.
    if constexpr (!T::kFp8) stage_meta<FMT>(r, st, li.lane);
    *reinterpret_cast<float2*>(st + kStage + 2 * li.lane) = rope_cs(t0, rc.freq);
    acc[0] = f32x4{0, 0, 0, 0};
    acc[1] = acc[0];
    const int tok = li.lane & 15;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float sc[8], of[8];
      if constexpr (!T::kFp8) {
        const float4 sa = *reinterpret_cast<const float4*>(st + 32 * qd + 8 * kb);
        const float4 sb = *reinterpret_cast<const float4*>(st + 32 * qd + 8 * kb + 4);
        const float4 oa = *reinterpret_cast<const float4*>(st + 128 + 32 * qd + 8 * kb);
        const float4 ob = *reinterpret_cast<const float4*>(st + 128 + 32 * qd + 8 * kb + 4);
        sc[0] = sa.x; sc[1] = sa.y; sc[2] = sa.z; sc[3] = sa.w; sc[4] = sb.x; sc[5] = sb.y; sc[6] = sb.z; sc[7] = sb.w;
        of[0] = oa.x; of[1] = oa.y; of[2] = oa.z; of[3] = oa.w; of[4] = ob.x; of[5] = ob.y; of[6] = ob.z; of[7] = ob.w;
      }
      float2 base[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (pair_first<FMT>(j))
          base[j] = *reinterpret_cast<const float2*>(st + kStage + 2 * (16 * qd + (k_chan<FMT>(kb, j) >> 1)));
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        const f16x8 a = operand<FMT>(r.k[tile], kb);
        float x[8], y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = T::kFp8 ? (float)a[j] : __builtin_fmaf((float)a[j], sc[j], of[j]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (!pair_first<FMT>(j)) continue;
          const int js = pair_slot<FMT>(j);
          const float2 o = rc.table[64 * (16 * tile + tok) + 16 * qd + (k_chan<FMT>(kb, j) >> 1)];
          const float c = base[j].x * o.x - base[j].y * o.y;
          const float sn = base[j].y * o.x + base[j].x * o.y;
          y[j] = x[j] * c - x[js] * sn;
          y[js] = x[js] * c + x[j] * sn;
        }
        const uint2 h0 = split_a(y[0], y[1]), h1 = split_a(y[2], y[3]), h2 = split_a(y[4], y[5]),
                    h3 = split_a(y[6], y[7]);
        acc[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cat(h0.x, h1.x, h2.x, h3.x), bk_static[kb], acc[tile], 0, 0, 0);
        acc[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cat(h0.y, h1.y, h2.y, h3.y), bk_static[kb], acc[tile], 0, 0, 0);
      }
      // keep one k-block's temporaries live at a time (the unrolled loop
      // otherwise runs out of registers)
      __builtin_amdgcn_sched_barrier(0);
    }
  } else if constexpr (T::kFp8) {
    acc[0] = f32x4{0, 0, 0, 0};
    acc[1] = acc[0];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int tile = 0; tile < 2; ++tile)
        acc[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(operand<FMT>(r.k[tile], kb), bk_static[kb],
                                                           acc[tile], 0, 0, 0);
  } else {
    vbig = stage_meta<FMT>(r, st, li.lane);
    // zero-point term sum_c q_c s_c z_c over this lane's 32 channels (in
    // slot order; query pair k against the term's hi and lo pairs, four
    // independent sums), then over the four quarters; it is subtracted from
    // the logits, so the matrix-core products do not wait for it
    float bz[4] = {0.f, 0.f, 0.f, 0.f};
    const uint4* zh = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(st) + 256 + 32 * qd);
    const uint4* zl = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(st) + 384 + 32 * qd);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 h = zh[i], l = zl[i];
      const uint32_t hw[4] = {h.x, h.y, h.z, h.w}, lw[4] = {l.x, l.y, l.z, l.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        bz[i & 1] = __builtin_amdgcn_fdot2(u2h(q.h[4 * i + k]), u2h(hw[k]), bz[i & 1], false);
        bz[2 + (i & 1)] = __builtin_amdgcn_fdot2(u2h(q.h[4 * i + k]), u2h(lw[k]), bz[2 + (i & 1)], false);
      }
    }
    kbias = rows_sum((bz[0] + bz[1]) + (bz[2] + bz[3]));
    acc[0] = f32x4{0, 0, 0, 0};
    acc[1] = acc[0];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const float4 sa = *reinterpret_cast<const float4*>(st + 32 * qd + 8 * kb);
      const float4 sb = *reinterpret_cast<const float4*>(st + 32 * qd + 8 * kb + 4);
      const f16x8 bq = split_q4(q.z + 4 * kb, q.h + 4 * kb, sa, sb);
#pragma unroll
      for (int tile = 0; tile < 2; ++tile)
        acc[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(operand<FMT>(r.k[tile], kb), bq, acc[tile], 0,
                                                           0, 0);
      if constexpr (T::kOut) {
        // Key outliers: one-hot (token row, channel slot) x q times the
        // staged correction, into the same accumulators
        const float4 da = *reinterpret_cast<const float4*>(st + kOutKd + 32 * qd + 8 * kb);
        const float4 db = *reinterpret_cast<const float4*>(st + kOutKd + 32 * qd + 8 * kb + 4);
        const f16x8 bd = split_q4(q.z + 4 * kb, q.h + 4 * kb, da, db);
        const uint4 ix = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(st + kOutKx) + 32 * qd + 8 * kb);
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
          const uint32_t own = (uint32_t)(16 * tile + (li.lane & 15)) * (0x10001u << kOhShift);
          const f16x8 oh = cat(one_hot(ix.x, own), one_hot(ix.y, own), one_hot(ix.z, own), one_hot(ix.w, own));
          acc[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(oh, bd, acc[tile], 0, 0, 0);
        }
      }
    }
  }

  float lg[2][4], pr[2][4];
#pragma unroll
  for (int tile = 0; tile < 2; ++tile)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      lg[tile][i] = __builtin_fmaf(acc[tile][i] + ror8(acc[tile][i]), T::kRope ? 1.0f : T::kCodeScale, -kbias);
  float slack = kSlack;
  if constexpr (!T::kFp8) {
    const float2 sv = pair_scales<FMT>(r.vm);
    // (outliers: p times the staged correction, at most p * |correction| / 2^8)
    if (__any(sv.x > kLazyScaleMax || sv.y > kLazyScaleMax || vbig > kLazyScaleMax * 256.0f)) slack = 0.f;
  }
  softmax_block(lg, ws, pr, slack);

  // ---- PV: Value codes (rows = channels) x P' (columns)
  if constexpr (T::kFp8) {
    const f16x8 bp = p_operand(pr, li);
#pragma unroll
    for (int m = 0; m < 8; ++m)
      ws.o[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(operand<FMT>(r.v, m), bp, ws.o[m], 0, 0, 0);
  } else {
    // Value zero-point sums: this lane keeps groups zg and zg + 1
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      const float* zs = st + 384 + 32 * (li.zg + gg);
      const float4 z0 = *reinterpret_cast<const float4*>(zs + 4 * qd);
      const float4 z1 = *reinterpret_cast<const float4*>(zs + 16 + 4 * qd);
      float za = ws.z[gg];
      za = __builtin_fmaf(pr[0][0], z0.x, za); za = __builtin_fmaf(pr[0][1], z0.y, za);
      za = __builtin_fmaf(pr[0][2], z0.z, za); za = __builtin_fmaf(pr[0][3], z0.w, za);
      za = __builtin_fmaf(pr[1][0], z1.x, za); za = __builtin_fmaf(pr[1][1], z1.y, za);
      za = __builtin_fmaf(pr[1][2], z1.z, za); za = __builtin_fmaf(pr[1][3], z1.w, za);
      ws.z[gg] = za;
    }
    float pb[2][4];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile)
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[tile][i] = li.is_lo ? pr[tile][i] : 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // scales of tokens 4qd..4qd+3 (tile 0) and 16+4qd..16+4qd+3 (tile 1)
      const float4 s0 = *reinterpret_cast<const float4*>(st + 256 + 32 * g + 4 * qd);
      const float4 s1 = *reinterpret_cast<const float4*>(st + 256 + 32 * g + 16 + 4 * qd);
      const float sv0[4] = {s0.x, s0.y, s0.z, s0.w};
      const float sv1[4] = {s1.x, s1.y, s1.z, s1.w};
      const f16x8 bp = split_p4(pr[0], pb[0], sv0, pr[1], pb[1], sv1);
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const int m = 2 * g + mm;
        ws.o[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(operand<FMT>(r.v, m), bp, ws.o[m], 0, 0, 0);
      }
      if constexpr (T::kOut) {
        // Value outliers of group g: one-hot (channel row, token slot) x p
        // times the staged correction
        const float4 d0 = *reinterpret_cast<const float4*>(st + kOutVd + 32 * g + 4 * qd);
        const float4 d1 = *reinterpret_cast<const float4*>(st + kOutVd + 32 * g + 16 + 4 * qd);
        const float dv0[4] = {d0.x, d0.y, d0.z, d0.w}, dv1[4] = {d1.x, d1.y, d1.z, d1.w};
        const f16x8 bd = split_p4(pr[0], pb[0], dv0, pr[1], pb[1], dv1);
        const uint4 ix = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(st + kOutVx) + 32 * g + 8 * qd);
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const uint32_t own = (uint32_t)(16 * mm + (li.lane & 15)) * (0x10001u << kOhShift);
          const f16x8 oh = cat(one_hot(ix.x, own), one_hot(ix.y, own), one_hot(ix.z, own), one_hot(ix.w, own));
          ws.o[2 * g + mm] = __builtin_amdgcn_mfma_f32_16x16x32_f16(oh, bd, ws.o[2 * g + mm], 0, 0, 0);
        }
      }
    }
  }
}

// Two blocks of one KV head at once (INT4 / INT2, n_rep <= 4; see
// lane_info_pair): the matrix-core columns that n_rep <= 4 leaves free carry
// the second block.  Both blocks are staged; each lane forms q' and P' from
// its own block's scales (so every split instruction serves two blocks), the
// QK products of both blocks share the q' operands and each lane keeps the
// logits of its block, one softmax pass runs for both, and each PV product
// takes the P' columns of its own block (the other columns masked to zero).
// b_on = false: only block ra counts (the second-block lanes are inactive).
template <int FMT>
__device__ __forceinline__ void process_pair(const Raw<FMT>& ra, const Raw<FMT>& rb, bool b_on, float* st,
                                             WaveState& ws, const QOp& q, const LaneInfo& li) {
  using T = Traits<FMT>;
  const int qd = li.qd;
  // block b's staging follows block a's (with outliers, after its corrections)
  constexpr int kB = T::kOut ? kOutVx + 64 : kStage;
  const float vba = stage_meta<FMT>(ra, st, li.lane);     // (outliers: largest |Value correction|)
  const float vbb = stage_meta<FMT>(rb, st + kB, li.lane);
  const float* sp = st + (li.par ? kB : 0);              // this lane's block

  // zero-point term of this lane's block (see process_block)
  float bz[4] = {0.f, 0.f, 0.f, 0.f};
  const uint4* zh = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(sp) + 256 + 32 * qd);
  const uint4* zl = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(sp) + 384 + 32 * qd);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 h = zh[i], l = zl[i];
    const uint32_t hw[4] = {h.x, h.y, h.z, h.w}, lw[4] = {l.x, l.y, l.z, l.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      bz[i & 1] = __builtin_amdgcn_fdot2(u2h(q.h[4 * i + k]), u2h(hw[k]), bz[i & 1], false);
      bz[2 + (i & 1)] = __builtin_amdgcn_fdot2(u2h(q.h[4 * i + k]), u2h(lw[k]), bz[2 + (i & 1)], false);
    }
  }
  const float kbias = rows_sum((bz[0] + bz[1]) + (bz[2] + bz[3]));

  f32x4 acc_a[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
  f32x4 acc_b[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const float4 sa = *reinterpret_cast<const float4*>(sp + 32 * qd + 8 * kb);
    const float4 sb = *reinterpret_cast<const float4*>(sp + 32 * qd + 8 * kb + 4);
    const f16x8 bq = split_q4(q.z + 4 * kb, q.h + 4 * kb, sa, sb);
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      acc_a[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(operand<FMT>(ra.k[tile], kb), bq, acc_a[tile], 0, 0, 0);
      acc_b[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(operand<FMT>(rb.k[tile], kb), bq, acc_b[tile], 0, 0, 0);
    }
    if constexpr (T::kOut) {
      // Key outliers (see process_block): q times this lane's block's staged
      // corrections, against each block's one-hot (token row, channel slot)
      const float4 da = *reinterpret_cast<const float4*>(sp + kOutKd + 32 * qd + 8 * kb);
      const float4 db = *reinterpret_cast<const float4*>(sp + kOutKd + 32 * qd + 8 * kb + 4);
      const f16x8 bd = split_q4(q.z + 4 * kb, q.h + 4 * kb, da, db);
      const uint4 ia = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(st + kOutKx) + 32 * qd + 8 * kb);
      const uint4 ib =
          *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(st + kB + kOutKx) + 32 * qd + 8 * kb);
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        const uint32_t own = (uint32_t)(16 * tile + (li.lane & 15)) * (0x10001u << kOhShift);
        const f16x8 oha = cat(one_hot(ia.x, own), one_hot(ia.y, own), one_hot(ia.z, own), one_hot(ia.w, own));
        const f16x8 ohb = cat(one_hot(ib.x, own), one_hot(ib.y, own), one_hot(ib.z, own), one_hot(ib.w, own));
        acc_a[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(oha, bd, acc_a[tile], 0, 0, 0);
        acc_b[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ohb, bd, acc_b[tile], 0, 0, 0);
      }
    }
    // (with outliers, one k-block's temporaries live at a time)
    if constexpr (T::kOut) __builtin_amdgcn_sched_barrier(0);
  }
  float lg[2][4], pr[2][4];
#pragma unroll
  for (int tile = 0; tile < 2; ++tile)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = li.par ? acc_b[tile][i] : acc_a[tile][i];
      lg[tile][i] = __builtin_fmaf(x + ror8(x), T::kCodeScale, -kbias);
    }
  const float2 sva = pair_scales<FMT>(ra.vm), svb = pair_scales<FMT>(rb.vm);
  // (outliers: p times a staged correction, at most p * |correction| / 2^8)
  const bool big = sva.x > kLazyScaleMax || sva.y > kLazyScaleMax || vba > kLazyScaleMax * 256.0f ||
                   (b_on && (svb.x > kLazyScaleMax || svb.y > kLazyScaleMax || vbb > kLazyScaleMax * 256.0f));
  const float slack = __any(big) ? 0.f : kSlack;
  if (b_on) softmax_block(lg, ws, pr, slack);
  else softmax_block_some(lg, ws, pr, slack, li.par == 0);

  // Value zero-point sums (this lane's block), groups zg and zg + 1
#pragma unroll
  for (int gg = 0; gg < 2; ++gg) {
    const float* zs = sp + 384 + 32 * (li.zg + gg);
    const float4 z0 = *reinterpret_cast<const float4*>(zs + 4 * qd);
    const float4 z1 = *reinterpret_cast<const float4*>(zs + 16 + 4 * qd);
    float za = ws.z[gg];
    za = __builtin_fmaf(pr[0][0], z0.x, za); za = __builtin_fmaf(pr[0][1], z0.y, za);
    za = __builtin_fmaf(pr[0][2], z0.z, za); za = __builtin_fmaf(pr[0][3], z0.w, za);
    za = __builtin_fmaf(pr[1][0], z1.x, za); za = __builtin_fmaf(pr[1][1], z1.y, za);
    za = __builtin_fmaf(pr[1][2], z1.z, za); za = __builtin_fmaf(pr[1][3], z1.w, za);
    ws.z[gg] = za;
  }
  float pb[2][4];
#pragma unroll
  for (int tile = 0; tile < 2; ++tile)
#pragma unroll
    for (int i = 0; i < 4; ++i) pb[tile][i] = li.is_lo ? pr[tile][i] : 0.f;
  const uint32_t am = li.amask, bm = ~li.amask;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const float4 s0 = *reinterpret_cast<const float4*>(sp + 256 + 32 * g + 4 * qd);
    const float4 s1 = *reinterpret_cast<const float4*>(sp + 256 + 32 * g + 16 + 4 * qd);
    const float sv0[4] = {s0.x, s0.y, s0.z, s0.w};
    const float sv1[4] = {s1.x, s1.y, s1.z, s1.w};
    const f16x8 bp = split_p4(pr[0], pb[0], sv0, pr[1], pb[1], sv1);
    const uint4 w = __builtin_bit_cast(uint4, bp);
    const f16x8 bpa = cat(w.x & am, w.y & am, w.z & am, w.w & am);
    const f16x8 bpb = cat(w.x & bm, w.y & bm, w.z & bm, w.w & bm);
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const int m = 2 * g + mm;
      ws.o[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(operand<FMT>(ra.v, m), bpa, ws.o[m], 0, 0, 0);
      if (b_on) ws.o[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(operand<FMT>(rb.v, m), bpb, ws.o[m], 0, 0, 0);
    }
    if constexpr (T::kOut) {
      // Value outliers of group g (see process_block): p times this lane's
      // block's staged corrections, masked to each block's columns, against
      // that block's one-hot (channel row, token slot)
      const float4 d0 = *reinterpret_cast<const float4*>(sp + kOutVd + 32 * g + 4 * qd);
      const float4 d1 = *reinterpret_cast<const float4*>(sp + kOutVd + 32 * g + 16 + 4 * qd);
      const float dv0[4] = {d0.x, d0.y, d0.z, d0.w}, dv1[4] = {d1.x, d1.y, d1.z, d1.w};
      const uint4 wd = __builtin_bit_cast(uint4, split_p4(pr[0], pb[0], dv0, pr[1], pb[1], dv1));
      const f16x8 bda = cat(wd.x & am, wd.y & am, wd.z & am, wd.w & am);
      const f16x8 bdb = cat(wd.x & bm, wd.y & bm, wd.z & bm, wd.w & bm);
      const uint4 ia = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(st + kOutVx) + 32 * g + 8 * qd);
      const uint4 ib =
          *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(st + kB + kOutVx) + 32 * g + 8 * qd);
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const uint32_t own = (uint32_t)(16 * mm + (li.lane & 15)) * (0x10001u << kOhShift);
        const f16x8 oha = cat(one_hot(ia.x, own), one_hot(ia.y, own), one_hot(ia.z, own), one_hot(ia.w, own));
        ws.o[2 * g + mm] = __builtin_amdgcn_mfma_f32_16x16x32_f16(oha, bda, ws.o[2 * g + mm], 0, 0, 0);
        if (b_on) {
          const f16x8 ohb = cat(one_hot(ib.x, own), one_hot(ib.y, own), one_hot(ib.z, own), one_hot(ib.w, own));
          ws.o[2 * g + mm] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ohb, bdb, ws.o[2 * g + mm], 0, 0, 0);
        }
      }
    }
    if constexpr (T::kOut) __builtin_amdgcn_sched_barrier(0);
  }
}

// Two blocks of one KV head at once at n_rep 8 (INT4 / INT2; see
// lane_info_slot): column col = 8 slot + head holds the pair's block slot,
// and the hi and lo parts of q' and P' are separate operands, each with its
// own matrix-core product into the same accumulator.  Every lane forms both
// parts of its own block's q' and P' (two split instructions give two
// operand halves), so each split instruction, each zero-point term and the
// softmax serve one (head, block) column, none a lo column.  The PV products
// take the P' columns of their block (the other slot's columns masked to
// zero).  b_on = false: only block ra counts.
template <int FMT>
__device__ __forceinline__ void process_slots(const Raw<FMT>& ra, const Raw<FMT>& rb, bool b_on, float* st,
                                              WaveState& ws, const QOp& q, const LaneInfo& li) {
  using T = Traits<FMT>;
  const int qd = li.qd;
  stage_meta<FMT>(ra, st, li.lane);
  stage_meta<FMT>(rb, st + kStage, li.lane);
  const float* sp = st + (li.par ? kStage : 0);          // this lane's block

  float bz[4] = {0.f, 0.f, 0.f, 0.f};
  const uint4* zh = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(sp) + 256 + 32 * qd);
  const uint4* zl = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(sp) + 384 + 32 * qd);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 h = zh[i], l = zl[i];
    const uint32_t hw[4] = {h.x, h.y, h.z, h.w}, lw[4] = {l.x, l.y, l.z, l.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      bz[i & 1] = __builtin_amdgcn_fdot2(u2h(q.h[4 * i + k]), u2h(hw[k]), bz[i & 1], false);
      bz[2 + (i & 1)] = __builtin_amdgcn_fdot2(u2h(q.h[4 * i + k]), u2h(lw[k]), bz[2 + (i & 1)], false);
    }
  }
  const float kbias = rows_sum((bz[0] + bz[1]) + (bz[2] + bz[3]));

  f32x4 acc_a[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
  f32x4 acc_b[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const float4 sa = *reinterpret_cast<const float4*>(sp + 32 * qd + 8 * kb);
    const float4 sb = *reinterpret_cast<const float4*>(sp + 32 * qd + 8 * kb + 4);
    const HiLo bq = split_q4_both(q.h + 4 * kb, sa, sb);
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      const f16x8 ka = operand<FMT>(ra.k[tile], kb), kbo = operand<FMT>(rb.k[tile], kb);
      acc_a[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, bq.hi, acc_a[tile], 0, 0, 0);
      acc_b[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kbo, bq.hi, acc_b[tile], 0, 0, 0);
      acc_a[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, bq.lo, acc_a[tile], 0, 0, 0);
      acc_b[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kbo, bq.lo, acc_b[tile], 0, 0, 0);
    }
  }
  float lg[2][4], pr[2][4];
#pragma unroll
  for (int tile = 0; tile < 2; ++tile)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      lg[tile][i] = __builtin_fmaf(li.par ? acc_b[tile][i] : acc_a[tile][i], T::kCodeScale, -kbias);
  const float2 sva = pair_scales<FMT>(ra.vm), svb = pair_scales<FMT>(rb.vm);
  const bool big = sva.x > kLazyScaleMax || sva.y > kLazyScaleMax || (b_on && (svb.x > kLazyScaleMax || svb.y > kLazyScaleMax));
  const float slack = __any(big) ? 0.f : kSlack;
  if (b_on) softmax_block(lg, ws, pr, slack);
  else softmax_block_some(lg, ws, pr, slack, li.par == 0);

  // Value zero-point sums of all four groups (this lane's block)
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const float* zs = sp + 384 + 32 * g;
    const float4 z0 = *reinterpret_cast<const float4*>(zs + 4 * qd);
    const float4 z1 = *reinterpret_cast<const float4*>(zs + 16 + 4 * qd);
    float za = ws.z[g];
    za = __builtin_fmaf(pr[0][0], z0.x, za); za = __builtin_fmaf(pr[0][1], z0.y, za);
    za = __builtin_fmaf(pr[0][2], z0.z, za); za = __builtin_fmaf(pr[0][3], z0.w, za);
    za = __builtin_fmaf(pr[1][0], z1.x, za); za = __builtin_fmaf(pr[1][1], z1.y, za);
    za = __builtin_fmaf(pr[1][2], z1.z, za); za = __builtin_fmaf(pr[1][3], z1.w, za);
    ws.z[g] = za;
  }
  const uint32_t am = li.amask, bm = ~li.amask;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const float4 s0 = *reinterpret_cast<const float4*>(sp + 256 + 32 * g + 4 * qd);
    const float4 s1 = *reinterpret_cast<const float4*>(sp + 256 + 32 * g + 16 + 4 * qd);
    const float sv0[4] = {s0.x, s0.y, s0.z, s0.w};
    const float sv1[4] = {s1.x, s1.y, s1.z, s1.w};
    const HiLo bp = split_p4_both(pr[0], sv0, pr[1], sv1);
    const uint4 wh = __builtin_bit_cast(uint4, bp.hi), wl = __builtin_bit_cast(uint4, bp.lo);
    const f16x8 ha = cat(wh.x & am, wh.y & am, wh.z & am, wh.w & am);
    const f16x8 la = cat(wl.x & am, wl.y & am, wl.z & am, wl.w & am);
    const f16x8 hb = cat(wh.x & bm, wh.y & bm, wh.z & bm, wh.w & bm);
    const f16x8 lb = cat(wl.x & bm, wl.y & bm, wl.z & bm, wl.w & bm);
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const int m = 2 * g + mm;
      const f16x8 va = operand<FMT>(ra.v, m), vb = operand<FMT>(rb.v, m);
      ws.o[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, ha, ws.o[m], 0, 0, 0);
      ws.o[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vb, hb, ws.o[m], 0, 0, 0);
      ws.o[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, la, ws.o[m], 0, 0, 0);
      ws.o[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vb, lb, ws.o[m], 0, 0, 0);
    }
  }
}

// Slot path: fold the other slot's state (lane + 8 in the row: same quarter,
// same head, other block slot) into this lane's, so both slots' lanes hold
// the head's state over both.  An empty state (m = -inf) weighs 0.
__device__ __forceinline__ void merge_slots(WaveState& ws) {
  const float mo = ror8(ws.m);
  const float mn = fmaxf(ws.m, mo);
  const float a = ws.m == neg_inf() ? 0.f : __builtin_amdgcn_exp2f(ws.m - mn);
  const float b = mo == neg_inf() ? 0.f : __builtin_amdgcn_exp2f(mo - mn);
  ws.l = __builtin_fmaf(a, ws.l, b * ror8(ws.l));
#pragma unroll
  for (int g = 0; g < 4; ++g) ws.z[g] = __builtin_fmaf(a, ws.z[g], b * ror8(ws.z[g]));
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) ws.o[m][i] = __builtin_fmaf(a, ws.o[m][i], b * ror8(ws.o[m][i]));
  ws.m = mn;
}

// Slot path counterpart of finish_segment (after merge_slots): the lane's
// column already holds whole values, so only the four quarters are summed.
__device__ __forceinline__ void finish_slot_segment(const WaveState& ws, const LaneInfo& li, float* slot,
                                                    float oscale) {
  const float l = rows_sum(ws.l);
  float zs[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) zs[g] = rows_sum(ws.z[g]);
  float* dst = slot + li.head * kPartStride;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    float4 o;
    o.x = ws.o[m][0] * oscale - zs[m >> 1];
    o.y = ws.o[m][1] * oscale - zs[m >> 1];
    o.z = ws.o[m][2] * oscale - zs[m >> 1];
    o.w = ws.o[m][3] * oscale - zs[m >> 1];
    if (li.writer) *reinterpret_cast<float4*>(dst + 4 + 16 * m + 4 * li.qd) = o;
  }
  if (li.writer && li.qd == 0) {
    dst[0] = ws.m;
    dst[1] = l;
  }
}

// Paired path: fold the second-block columns' softmax state (lane ^ 4: same
// quarter, same hi / lo half, other parity) into the first's, so that every
// lane holds its head's state over both.  An empty state (m = -inf) weighs 0.
__device__ __forceinline__ void merge_parity(WaveState& ws) {
  const float mo = __shfl_xor(ws.m, 4);
  const float mn = fmaxf(ws.m, mo);
  const float a = ws.m == neg_inf() ? 0.f : __builtin_amdgcn_exp2f(ws.m - mn);
  const float b = mo == neg_inf() ? 0.f : __builtin_amdgcn_exp2f(mo - mn);
  ws.l = __builtin_fmaf(a, ws.l, b * __shfl_xor(ws.l, 4));
  ws.z[0] = __builtin_fmaf(a, ws.z[0], b * __shfl_xor(ws.z[0], 4));
  ws.z[1] = __builtin_fmaf(a, ws.z[1], b * __shfl_xor(ws.z[1], 4));
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) ws.o[m][i] = __builtin_fmaf(a, ws.o[m][i], b * __shfl_xor(ws.o[m][i], 4));
  ws.m = mn;
}

// A workgroup's merged slots are read by another workgroup (on another
// compute unit, possibly another XCD): they are written and read with
// device-coherent accesses (relaxed atomics at agent scope), which go past
// the non-coherent caches without the L2-wide write-back and invalidate that
// device-scope fences cost.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sums over quarters and hi + lo columns, then writes one partial slot:
// m, l, o[128] per query head (o unnormalised).  The slot is read only by
// this workgroup, after a barrier.
__device__ __forceinline__ void finish_segment(const WaveState& ws, const LaneInfo& li, float* slot, float oscale,
                                               bool has_z) {
  const float l = rows_sum(ws.l);
  float zs[4] = {0.f, 0.f, 0.f, 0.f};
  if (has_z) {
    const float z0 = rows_sum(ws.z[0]), z1 = rows_sum(ws.z[1]);
    // hi columns hold groups 0, 1; their lo partners (lane + 8) groups 2, 3
    zs[0] = z0; zs[1] = z1; zs[2] = ror8(z0); zs[3] = ror8(z1);
  }
  float* dst = slot + li.head * kPartStride;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    float4 o;
    o.x = (ws.o[m][0] + ror8(ws.o[m][0])) * oscale - zs[m >> 1];
    o.y = (ws.o[m][1] + ror8(ws.o[m][1])) * oscale - zs[m >> 1];
    o.z = (ws.o[m][2] + ror8(ws.o[m][2])) * oscale - zs[m >> 1];
    o.w = (ws.o[m][3] + ror8(ws.o[m][3])) * oscale - zs[m >> 1];
    if (li.writer) *reinterpret_cast<float4*>(dst + 4 + 16 * m + 4 * li.qd) = o;
  }
  if (li.writer && li.qd == 0) {
    dst[0] = ws.m;
    dst[1] = l;
  }
}

// Wavefront-local LDS hand-over: the LDS unit serves one wavefront's
// instructions in order, so once this wavefront's writes have completed its
// lanes read each other's data; the clobber keeps the compiler from moving
// LDS accesses across the point.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// One 32-token block fb of the fp16 segment (sink tokens, then the residual
// ring) of head bh, into its own partial slot.  Keys feed the matrix cores
// straight from their rows; Values are transposed through the wavefront's
// LDS area into the (channel, 8 tokens) operand order.
constexpr int kSegVStride = 136;     // halves per staged Value row (16-byte aligned)

// Row of segment token k: a sink, a ring slot, or (fused append, fresh != null)
// for the newest token the input row, which fp16_block also copies to its
// ring slot.
__device__ __forceinline__ const uint16_t* seg_row(const AttnParams& p, const uint16_t* sink,
                                                   const uint16_t* ring, const uint16_t* fresh, int64_t bh, int k) {
  if (fresh && k == p.n_sink + p.n_res - 1) return fresh + bh * kHeadDim;
  if (k < p.n_sink) return sink + (bh * p.sink_cap + k) * kHeadDim;
  const int slot = (p.ring_first + (k - p.n_sink)) % p.ring_slots;
  return ring + (bh * p.ring_slots + slot) * kHeadDim;
}

// ROPE: the segment holds pre-RoPE Keys; each is rotated at its position
// (sinks: their index; residual token u of the body: S + u) with angles
// evaluated directly (fp64 reduction), the lane's channels taken in pair
// order like the quantized blocks.
template <bool ROPE>
__device__ void fp16_block(const AttnParams& p, int64_t bh, int fb, uint16_t* vt, float* slot) {
  const LaneInfo li = lane_info(p.nrep);
  const int lane = li.lane;
  const int nt = p.n_sink + p.n_res;
  // fused append: the block holding the newest token (a residual token) copies
  // its Key and Value rows from the input to its ring slot, 16 bytes per lane;
  // no other block of this call reads that slot
  if (p.new_k && fb == (nt - 1) / kBlock && lane < 32) {
    const int kv = lane >> 4, chunk = lane & 15;
    const uint16_t* ring = kv ? p.v_ring : p.k_ring;
    const uint16_t* dst = seg_row(p, nullptr, ring, nullptr, bh, nt - 1) + 8 * chunk;
    *reinterpret_cast<uint4*>(const_cast<uint16_t*>(dst)) =
        *reinterpret_cast<const uint4*>((kv ? p.new_v : p.new_k) + bh * kHeadDim + 8 * chunk);
  }
  QOp q;
  f16x8 bk[4];
  load_query<ROPE ? (KVQ_INT8 | kRope) : KVQ_INT8>(p, bh, li, q);   // scale 1
  static_q(q, kQScale, bk);
  WaveState ws;
  reset(ws);
  // Key rows of this lane's two tokens (one per 16-token tile): its quarter's
  // 32 channels, or in pair order channels 16qd .. +15 and 64 + 16qd .. +15
  uint4 kr[2][4];
  int kpos[2];
#pragma unroll
  for (int tile = 0; tile < 2; ++tile) {
    int k = 32 * fb + 16 * tile + (lane & 15);
    k = k < nt ? k : nt - 1;                           // masked below; any valid row keeps values finite
    kpos[tile] = k < p.n_sink ? k : p.sink_cap + kBlock * p.nblk + (k - p.n_sink);
    const uint16_t* row = seg_row(p, p.k_sink, p.k_ring, p.new_k, bh, k);
    if constexpr (ROPE) {
      const uint4* a = reinterpret_cast<const uint4*>(row + 16 * li.qd);
      const uint4* b = reinterpret_cast<const uint4*>(row + kHeadDim / 2 + 16 * li.qd);
      kr[tile][0] = a[0]; kr[tile][1] = a[1]; kr[tile][2] = b[0]; kr[tile][3] = b[1];
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(row + 32 * li.qd);
#pragma unroll
      for (int i = 0; i < 4; ++i) kr[tile][i] = src[i];
    }
  }
  // Value row of token lane % 32, channel half lane / 32, into LDS
  {
    int k = 32 * fb + (lane & 31);
    k = k < nt ? k : nt - 1;
    const uint4* src = reinterpret_cast<const uint4*>(seg_row(p, p.v_sink, p.v_ring, p.new_v, bh, k) + 64 * (lane >> 5));
    uint4* dst = reinterpret_cast<uint4*>(vt + (lane & 31) * kSegVStride + 64 * (lane >> 5));
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = src[i];
  }
  f32x4 acc[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    if constexpr (ROPE) {
      // slot j of k-block kb holds stored position 8kb + j: channel pair
      // m = 4kb + j / 2, member j % 2
      double fr[4];
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) fr[mm] = rope_freq(p.rope_theta, 16 * li.qd + 4 * kb + mm);
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        float y[8];
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
          const int m = 4 * kb + mm;
          const uint4 wa = kr[tile][m >> 3], wb = kr[tile][2 + (m >> 3)];
          const uint32_t ua[4] = {wa.x, wa.y, wa.z, wa.w}, ub[4] = {wb.x, wb.y, wb.z, wb.w};
          const float x0 = (float)u2h(ua[(m & 7) >> 1])[m & 1];
          const float x1 = (float)u2h(ub[(m & 7) >> 1])[m & 1];
          const float2 cs = rope_cs((double)kpos[tile], fr[mm]);
          y[2 * mm] = x0 * cs.x - x1 * cs.y;
          y[2 * mm + 1] = x1 * cs.x + x0 * cs.y;
        }
        const uint2 h0 = split_a(y[0], y[1]), h1 = split_a(y[2], y[3]), h2 = split_a(y[4], y[5]),
                    h3 = split_a(y[6], y[7]);
        acc[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cat(h0.x, h1.x, h2.x, h3.x), bk[kb], acc[tile], 0, 0, 0);
        acc[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cat(h0.y, h1.y, h2.y, h3.y), bk[kb], acc[tile], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        const uint4 w = kr[tile][kb];
        acc[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cat(w.x, w.y, w.z, w.w), bk[kb], acc[tile], 0, 0, 0);
      }
    }
  }
  float lg[2][4], pr[2][4];
#pragma unroll
  for (int tile = 0; tile < 2; ++tile)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = 32 * fb + 16 * tile + 4 * li.qd + i;
      const float x = acc[tile][i] + ror8(acc[tile][i]);
      lg[tile][i] = k < nt ? x : neg_inf();
    }
  softmax_block(lg, ws, pr, kSlack);
  const f16x8 bp = p_operand(pr, li);
  wave_lds_sync();                                      // staged Value rows visible to every lane
  const int r = lane & 15;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    // channel 16m + r of tokens T0, T4, T1, T5, T2, T6, T3, T7 (T = 4qd + 0..3, 16 + 4qd + 0..3)
    f16x8 a;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      a[2 * v] = __builtin_bit_cast(_Float16, vt[(4 * li.qd + v) * kSegVStride + 16 * m + r]);
      a[2 * v + 1] = __builtin_bit_cast(_Float16, vt[(16 + 4 * li.qd + v) * kSegVStride + 16 * m + r]);
    }
    ws.o[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bp, ws.o[m], 0, 0, 0);
  }
  wave_lds_sync();                                      // reads done before the area is reused
  finish_segment(ws, li, slot, 1.0f, false);
}

constexpr int kGroupThreads = 64 * kGroupWaves;
// per-wavefront LDS area: the block staging of process_block, or the Value
// rows of an fp16 block (never both at once)
constexpr int kStageBytes = (kStage * 4 > kBlock * kSegVStride * 2) ? kStage * 4 : kBlock * kSegVStride * 2;
// then the wavefront's last segment partial (n_rep <= 8 query heads)
constexpr int kWaveLds = kStageBytes + 8 * kPartStride * 4;
// workgroup LDS: the wavefronts' areas, the block counter, the record ids of
// a paged range (then, for pre-RoPE Keys, the in-block offset table)
constexpr int kLdsHeader = 32 + 4 * kGroupWaves;    // counters, each wavefront's final head, covering info
constexpr int kLdsBytes = kGroupWaves * kWaveLds + kLdsHeader + 4 * kMaxPagedRange;
// The first kFp16Lds fp16 partials of a workgroup's first head are kept in
// LDS after kLdsBytes (the merge reads them as LDS instead of from the
// workspace), the RoPE table after them.
constexpr int kFp16Lds = 4;
constexpr int kFp16LdsBytes = kFp16Lds * 8 * kPartStride * 4;
static_assert(kStageBytes >= (kStage + 128) * 4, "stage area holds the RoPE base angles after the block metadata");
static_assert(kStageBytes >= 2 * kStage * 4, "the stage area holds two blocks (paired and slot paths)");
static_assert(kStageBytes >= (kOutVx + 64) * 4, "stage area holds the outlier corrections after the block metadata");
static_assert(kStageBytes >= 2 * (kOutVx + 64) * 4, "stage area holds two blocks with outliers (paired path)");

// One workgroup: range [jb, jb + len) of the flattened quantized blocks,
// touching heads h0..h1.
struct GroupRange {
  int64_t jb;
  int len, h0, h1;
};

// The flattened blocks are cut into stretches of range_len blocks, each
// stretch into range_parts consecutive ranges: part p of a stretch starts at
// floor(p L / k) + (p odd ? d : 0) (L = range_len, k = range_parts, d =
// group_skew), so odd-numbered workgroups take d fewer blocks than their
// even neighbours.  Following heads: L = nblk, k ranges per head; equal
// ranges of R blocks across head boundaries: L = 2 R, k = 2.  The host keeps
// k L < 2^31, so every quotient below is a 32-bit multiply-shift.
// range_start(g) is the first block of workgroup g's range and range_of(x)
// the workgroup whose range holds flattened block x.
__device__ __forceinline__ uint32_t div_len(const AttnParams& p, uint32_t x) {     // x / L, x < 2^31
  return (uint32_t)(((uint64_t)x * p.len_magic) >> p.len_shift);
}
__device__ __forceinline__ uint32_t div_parts(const AttnParams& p, uint32_t x) {   // x / k, x < 2^31
  return (uint32_t)(((uint64_t)x * p.parts_magic) >> p.parts_shift);
}
__device__ __forceinline__ int64_t part_start(const AttnParams& p, uint32_t part) {
  return (int64_t)div_parts(p, part * (uint32_t)p.range_len) + ((part & 1) ? p.group_skew : 0);
}
__device__ __forceinline__ int64_t range_start(const AttnParams& p, int64_t g) {
  const uint32_t s = div_parts(p, (uint32_t)g);
  return (int64_t)s * p.range_len + part_start(p, (uint32_t)g - s * (uint32_t)p.range_parts);
}
__device__ __forceinline__ int64_t range_of(const AttnParams& p, int64_t x) {
  const uint32_t s = div_len(p, (uint32_t)x), r = (uint32_t)x - s * (uint32_t)p.range_len;
  uint32_t part = div_len(p, (r + 1) * (uint32_t)p.range_parts - 1);   // last part starting at or before r,
  if (part_start(p, part) > r) --part;                                 // skew aside (an odd part starts d later)
  return (int64_t)s * p.range_parts + part;
}

__device__ __forceinline__ GroupRange group_range(const AttnParams& p, int g) {
  GroupRange r;
  const int64_t total = (int64_t)p.bh_count * p.nblk;
  r.jb = range_start(p, g);
  const int64_t e = range_start(p, g + 1);
  r.len = r.jb < total ? (int)((e < total ? e : total) - r.jb) : 0;
  r.h0 = r.len ? (int)((uint32_t)r.jb / (uint32_t)p.nblk) : 0;             // jb < 2^31
  r.h1 = r.len ? (int)((uint32_t)(r.jb + r.len - 1) / (uint32_t)p.nblk) : -1;
  return r;
}

// Workgroups whose range touches head h: g_lo .. g_lo + count - 1.
__device__ __forceinline__ int64_t covering_lo(const AttnParams& p, int64_t h) {
  return range_of(p, h * p.nblk);
}
__device__ __forceinline__ int64_t covering_count(const AttnParams& p, int64_t h) {
  return range_of(p, (h + 1) * p.nblk - 1) - covering_lo(p, h) + 1;
}

__device__ __forceinline__ int64_t slot_floats(const AttnParams& p) { return (int64_t)p.nrep * kPartStride; }

// Head of flattened block j (j < 2^31): j / nblk by multiply and shift.
__device__ __forceinline__ uint32_t head_of(const AttnParams& p, uint32_t j) {
  return (uint32_t)(((uint64_t)j * p.nblk_magic) >> p.nblk_shift);
}

// Online-softmax combine of N partials (m, l, o) into (M, L, O), in order:
// M = max, then every non-empty partial weighted by 2^(m - M) (an empty
// partial, m = -inf, weighs 0 and its o is not read).
template <int N>
__device__ __forceinline__ void fold(float& M, float& L, float& O, const float* m, const float* l, const float* o) {
  float Mn = M;
#pragma unroll
  for (int j = 0; j < N; ++j) Mn = fmaxf(Mn, m[j]);
  if (Mn != neg_inf()) {                         // rescale what was summed before
    const float a = M == neg_inf() ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
    L *= a;
    O *= a;
  }
  M = Mn;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    if (m[j] != neg_inf()) {
      const float wt = __builtin_amdgcn_exp2f(m[j] - M);
      L = __builtin_fmaf(wt, l[j], L);
      O = __builtin_fmaf(wt, o[j], O);
    }
  }
}

// fold for four channels that share their partials' (m, l).
template <int N>
__device__ __forceinline__ void fold4(float& M, float& L, float4& O, const float* m, const float* l,
                                      const float4* o) {
  float Mn = M;
#pragma unroll
  for (int j = 0; j < N; ++j) Mn = fmaxf(Mn, m[j]);
  if (Mn != neg_inf()) {
    const float a = M == neg_inf() ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
    L *= a;
    O.x *= a; O.y *= a; O.z *= a; O.w *= a;
  }
  M = Mn;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    if (m[j] != neg_inf()) {
      const float wt = __builtin_amdgcn_exp2f(m[j] - M);
      L = __builtin_fmaf(wt, l[j], L);
      O.x = __builtin_fmaf(wt, o[j].x, O.x);
      O.y = __builtin_fmaf(wt, o[j].y, O.y);
      O.z = __builtin_fmaf(wt, o[j].z, O.z);
      O.w = __builtin_fmaf(wt, o[j].w, O.w);
    }
  }
}

// Four consecutive floats of a merged slot, device-coherent (two 64-bit
// relaxed atomics at agent scope).
__device__ __forceinline__ void st_dev4(float* p, float4 v) {
  uint64_t* q = reinterpret_cast<uint64_t*>(p);
  __hip_atomic_store(q, ((uint64_t)__builtin_bit_cast(uint32_t, v.y) << 32) | __builtin_bit_cast(uint32_t, v.x),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, ((uint64_t)__builtin_bit_cast(uint32_t, v.w) << 32) | __builtin_bit_cast(uint32_t, v.z),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float4 ld_dev4(const float* p) {
  uint64_t* q = reinterpret_cast<uint64_t*>(const_cast<float*>(p));
  const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return float4{__builtin_bit_cast(float, (uint32_t)a), __builtin_bit_cast(float, (uint32_t)(a >> 32)),
                __builtin_bit_cast(float, (uint32_t)b), __builtin_bit_cast(float, (uint32_t)(b >> 32))};
}

constexpr int kReduceItems = 4;           // items per thread and pass of reduce_fp16_head
constexpr int kReduceBatch = 4;           // slots per item whose loads are issued together

// out[b][h] of all n_rep query heads of (sequence, KV head) h, from the
// head's fp16-block slots (written by this workgroup before a barrier):
//   sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,  M = max_s m_s
// (the exact regrouping of one softmax over all tokens), over the slots in
// order.  Items are (query head, four channels), kReduceItems per thread and
// pass; the loads of kReduceBatch slots of all of a thread's items are issued
// before any is used (one memory round trip per batch).
__device__ void reduce_fp16_head(const AttnParams& p, int64_t h) {
  const int total = p.nrep * (kHeadDim / 4);
  const int ns = p.fp16_blocks;
  const float* sb = p.part_fp16 + h * p.fp16_blocks * slot_floats(p);
  for (int base = 0; base < total; base += kReduceItems * kGroupThreads) {
    float M[kReduceItems], L[kReduceItems];
    float4 O[kReduceItems];
#pragma unroll
    for (int k = 0; k < kReduceItems; ++k) {
      M[k] = neg_inf();
      L[k] = 0.f;
      O[k] = float4{0.f, 0.f, 0.f, 0.f};
    }
    for (int s0 = 0; s0 < ns; s0 += kReduceBatch) {
      float m[kReduceItems][kReduceBatch], l[kReduceItems][kReduceBatch];
      float4 o[kReduceItems][kReduceBatch];
#pragma unroll
      for (int k = 0; k < kReduceItems; ++k) {
        const int r = base + (int)threadIdx.x + k * kGroupThreads;
#pragma unroll
        for (int j = 0; j < kReduceBatch; ++j) {
          if (r < total && s0 + j < ns) {
            const float* sp = sb + (s0 + j) * slot_floats(p) + (r >> 5) * kPartStride;
            m[k][j] = sp[0];
            l[k][j] = sp[1];
            o[k][j] = *reinterpret_cast<const float4*>(sp + 4 + 4 * (r & 31));
          } else {
            m[k][j] = neg_inf();
            l[k][j] = 0.f;
            o[k][j] = float4{0.f, 0.f, 0.f, 0.f};
          }
        }
      }
#pragma unroll
      for (int k = 0; k < kReduceItems; ++k) fold4<kReduceBatch>(M[k], L[k], O[k], m[k], l[k], o[k]);
    }
#pragma unroll
    for (int k = 0; k < kReduceItems; ++k) {
      const int r = base + (int)threadIdx.x + k * kGroupThreads;
      if (r < total) {
        const f16x2 lo = {(_Float16)(O[k].x / L[k]), (_Float16)(O[k].y / L[k])};
        const f16x2 hi = {(_Float16)(O[k].z / L[k]), (_Float16)(O[k].w / L[k])};
        *reinterpret_cast<uint2*>(p.out + (h * p.nrep + (r >> 5)) * kHeadDim + 4 * (r & 31)) =
            uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
      }
    }
  }
}

// Bound on the polls of a head's counter while the other covering
// workgroups finish writing their slots.  They have all arrived, so they are
// running and write without waiting on anything; the bound only guarantees
// that every wavefront exits.
constexpr int kSpinLimit = 1 << 22;

// The combine of the shared heads h0 (last0) and / or h1 (last1) that this
// workgroup's arrival completed: once every other covering workgroup's
// "written" mark is in the counter, the counter is set back to 0 and each
// output row is
//   sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,  M = max_s m_s
// over the covering workgroups' merged partials in covering order (the
// exact regrouping of one softmax over all tokens), this workgroup's own
// from LDS, the others' by device-coherent loads issued after the marks
// were seen, kCombineBatch slots per round trip.
constexpr int kCombineBatch = 8;
// floats of the combine's batch results in LDS (the stage areas of wavefronts 2 on)
constexpr int kRedFloats = (kGroupWaves - 2) * kWaveLds / 4;

__device__ void combine_shared(const AttnParams& p, int g, int h0, int h1, bool last0, bool last1, int lo0, int lo1,
                               int nc0, int nc1, const float* own0, const float* own1, float* red) {
  if (threadIdx.x == 0) {
    for (int s = 0; s < 2; ++s) {
      const bool on = s == 0 ? last0 : last1;
      if (!on) continue;
      const int h = s == 0 ? h0 : h1, nc = s == 0 ? nc0 : nc1;
      for (int it = 0; it < kSpinLimit; ++it) {
        const int c = __hip_atomic_load(p.sync + h, KVQ_FORMAL_ORDERING ? __ATOMIC_ACQUIRE : __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
        if ((c >> 16) >= nc - 1) break;
        __builtin_amdgcn_s_sleep(2);
      }
      __hip_atomic_store(p.sync + h, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  const int per = p.nrep * (kHeadDim / 4);
  const int n0 = last0 ? per : 0;
  const int total = n0 + (last1 ? per : 0);
  // Items are (head, query head, four channels).  An item's slots are cut
  // into batches of kCombineBatch; each batch is folded on its own, and the
  // batch results are folded in batch order, so the result does not depend
  // on how the work is spread.  With threads to spare, G groups of `total`
  // threads fold every G-th batch each into LDS (red: 8 floats per batch and
  // item) and one thread per item folds them; otherwise one thread per item
  // does both in turn.
  const int nmax = (last0 && nc0 > (last1 ? nc1 : 0)) ? nc0 : (last1 ? nc1 : nc0);
  const int nbat = (nmax + kCombineBatch - 1) / kCombineBatch;
  int G = kGroupThreads / total;
  G = G < nbat ? G : nbat;
  if ((int64_t)nbat * total * 8 > kRedFloats) G = 1;
  G = G > 1 ? G : 1;
  auto item = [&](int idx, int& h, int& nc, int& hq, int& c4, bool& first) {
    first = idx < n0;
    h = first ? h0 : h1;
    nc = first ? nc0 : nc1;
    const int r = first ? idx : idx - n0;
    hq = r >> 5;
    c4 = r & 31;
  };
  // the fold of slots s0 .. s0 + kCombineBatch - 1 (those below nc) of an item
  auto batch = [&](int idx, int s0, float& M, float& L, float4& O) {
    int h, nc, hq, c4;
    bool first;
    item(idx, h, nc, hq, c4, first);
    const float* own = (first ? own0 : own1) + hq * kPartStride;
    const int64_t glo = first ? lo0 : lo1;
    const int me = g - (int)glo;                 // this workgroup's place among the covering ones
    const float* base = p.part_group + (glo + h) * slot_floats(p) + hq * kPartStride;
    float m[kCombineBatch], l[kCombineBatch];
    float4 o[kCombineBatch];
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) {
      const int s = s0 + j;
      if (s >= nc) {
        m[j] = neg_inf();
        l[j] = 0.f;
        o[j] = float4{0.f, 0.f, 0.f, 0.f};
      } else if (s == me) {
        m[j] = own[0];
        l[j] = own[1];
        o[j] = *reinterpret_cast<const float4*>(own + 4 + 4 * c4);
      } else {
        const float* sp = base + s * slot_floats(p);
        m[j] = ld_dev(sp);
        l[j] = ld_dev(sp + 1);
        o[j] = ld_dev4(sp + 4 + 4 * c4);
      }
    }
    M = neg_inf();
    L = 0.f;
    O = float4{0.f, 0.f, 0.f, 0.f};
    fold4<kCombineBatch>(M, L, O, m, l, o);
  };
  auto write_out = [&](int idx, float L, float4 O) {
    int h, nc, hq, c4;
    bool first;
    item(idx, h, nc, hq, c4, first);
    const f16x2 lo = {(_Float16)(O.x / L), (_Float16)(O.y / L)};
    const f16x2 hi = {(_Float16)(O.z / L), (_Float16)(O.w / L)};
    *reinterpret_cast<uint2*>(p.out + ((int64_t)h * p.nrep + hq) * kHeadDim + 4 * c4) =
        uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
  };
  auto nbat_of = [&](int idx) {
    const int nc = idx < n0 ? nc0 : nc1;
    return (nc + kCombineBatch - 1) / kCombineBatch;
  };
  {
    const int gi = G > 1 ? (int)threadIdx.x / total : 0;
    const int idx = (int)threadIdx.x - gi * total;
    float M = neg_inf(), L = 0.f;
    float4 O = {0.f, 0.f, 0.f, 0.f};
    if (gi < G && idx < total) {
      const int nb = nbat_of(idx);
      for (int b = gi; b < nb; b += G) {
        float bm, bl;
        float4 bo;
        batch(idx, b * kCombineBatch, bm, bl, bo);
        if (G > 1) {
          float* r = red + 8 * (b * total + idx);
          r[0] = bm;
          r[1] = bl;
          *reinterpret_cast<float4*>(r + 4) = bo;
        } else {
          fold4<1>(M, L, O, &bm, &bl, &bo);
        }
      }
    }
    if (G > 1) {                                // uniform over the workgroup
      __syncthreads();
      if ((int)threadIdx.x < total) {
        const int nb = nbat_of(threadIdx.x);
        for (int b = 0; b < nb; ++b) {
          const float* r = red + 8 * (b * total + (int)threadIdx.x);
          const float bm = r[0], bl = r[1];
          const float4 bo = *reinterpret_cast<const float4*>(r + 4);
          fold4<1>(M, L, O, &bm, &bl, &bo);
        }
      }
    }
    if ((int)threadIdx.x < total) write_out(threadIdx.x, L, O);
  }
}

// The workgroup's wavefronts stream the blocks of its range: each keeps
// kDepth blocks in flight beyond the one it processes and takes its next
// block from a counter in LDS, so a wavefront that the memory system serves
// faster processes more blocks and all finish together (in deterministic
// mode wavefront w takes blocks w, w + 8, w + 16, ... instead).  Every
// wavefront keeps one online softmax per head it meets and writes one partial
// per head of the range (the last one into its LDS area).  Then the
// wavefronts take the workgroup's fp16 blocks from a second LDS counter, and
// the workgroup merges, per head, its wavefronts' and fp16 partials.
// MODE: kSingle (process_block), kPairs (process_pair; INT4 / INT2 at
// n_rep <= 4) or kSlots (process_slots; INT4 / INT2 at n_rep 8); the last
// two take blocks two at a time, with a ring of kPairRing blocks.
constexpr int kSingle = 0, kPairs = 1, kSlots = 2;
template <int FMT, int MODE>
__device__ void group_main(const AttnParams& p, char* lds) {
  using T = Traits<FMT>;
  constexpr bool PAIR = MODE != kSingle;
  constexpr int D = PAIR ? T::kPairRing : T::kDepth + 1;
  static_assert(!PAIR || (T::kPairable && D % 2 == 0 && D >= 4), "paired ring");
  const int g = blockIdx.x;
  const int v = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wavefront index, uniform
  const LaneInfo li = MODE == kPairs ? lane_info_pair(p.nrep) : (MODE == kSlots ? lane_info_slot(p.nrep)
                                                                                 : lane_info(p.nrep));
  const GroupRange gr = group_range(p, g);
  if (!gr.len) return;                        // (never: every workgroup has a range)
  const uint32_t nblk = (uint32_t)p.nblk;
  float* stage = reinterpret_cast<float*>(lds + v * kWaveLds);
  int* ctr = reinterpret_cast<int*>(lds + kGroupWaves * kWaveLds);
  int* fin_head = reinterpret_cast<int*>(lds + kGroupWaves * kWaveLds + 16);
  int* recs = reinterpret_cast<int*>(lds + kGroupWaves * kWaveLds + kLdsHeader);
  // the workgroups covering the range's first and last heads: cov[0] / cov[2]
  // the first of them, cov[1] / cov[3] how many (a head strictly between is
  // this workgroup's alone); kept in LDS, read at the end of the call
  int* cov = reinterpret_cast<int*>(lds + kGroupWaves * kWaveLds + 16 + 4 * kGroupWaves);
  auto cover = [&](int h, int& lo, int& nc) {
    lo = h == gr.h0 ? cov[0] : (h == gr.h1 ? cov[2] : g);
    nc = h == gr.h0 ? cov[1] : (h == gr.h1 ? cov[3] : 1);
  };

  // paged caches: the record ids of the range's blocks, read from the block
  // table once (a page id outside the pool reads record 0 instead)
  if (p.table) {
    for (int i = threadIdx.x; i < gr.len; i += kGroupThreads) {
      const int64_t j = gr.jb + i;
      const int64_t bhj = head_of(p, (uint32_t)j);
      const int64_t r = block_record(p.table, p.table_stride, p.page_blocks, p.num_pages, p.hkv, p.nb_cap,
                                     bhj / p.hkv, bhj % p.hkv, j - bhj * nblk);
      recs[i] = r < 0 ? 0 : (int)r;
    }
  }
  // pre-RoPE Keys: the in-block offsets (cos, sin)(k theta_i), k < 32, i < 64
  float2* rtab = reinterpret_cast<float2*>(lds + kLdsBytes + kFp16LdsBytes);
  if constexpr (T::kRope) {
    for (int e = threadIdx.x; e < 32 * 64; e += kGroupThreads)
      rtab[e] = rope_cs((double)(e >> 6), rope_freq(p.rope_theta, e & 63));
  }
  RopeCtx rc{};
  if constexpr (T::kRope) rc = RopeCtx{rope_freq(p.rope_theta, li.lane), rtab};
  // the block counter starts at zero; the barrier comes before any block
  // load is issued, so no wavefront waits on another's loads
  if (threadIdx.x == 0) {
    ctr[0] = ctr[1] = 0;                         // quantized units, fp16 blocks
    cov[0] = (int)covering_lo(p, gr.h0);
    cov[1] = (int)covering_count(p, gr.h0);
    cov[2] = gr.h1 == gr.h0 ? cov[0] : g;        // a later head starts inside this range
    cov[3] = gr.h1 == gr.h0 ? cov[1] : (int)(range_of(p, (int64_t)(gr.h1 + 1) * p.nblk - 1) - g + 1);
  }
  __syncthreads();

  // query rows of the range's first head, loaded before the blocks
  const QRaw q0 = load_query_raw<T::kRope>(p.q + (int64_t)gr.h0 * p.nrep * kHeadDim, p.nrep, li);

  // block ring: D - 1 blocks prefetched ahead of the one being processed;
  // rid = block index within the range (-1 past its end), rbh = its head.
  // Loads past the end read block 0 of head 0 with ordinary loads: every
  // wavefront's surplus loads hit the same lines, which stay in the cache.
  const uint64_t rot = ((uint32_t)g * 0x9E3779B9u) >> 12;     // a 20-bit fraction
  const uint32_t jb = (uint32_t)gr.jb, je = (uint32_t)(gr.jb + gr.len);
  Raw<FMT> buf[D];
  int rid[D], rbh[D], rblk[D];
  int kst = 0;
  // Heads of the range shared with neighbouring workgroups count this
  // workgroup's arrival on their counters (sync plane).  The arrival is made
  // by the one wavefront whose claim is the first past the range (claims are
  // numbered, so exactly one gets index len), while the workgroup still has
  // its last blocks in flight: the arrival order then follows the order in
  // which the workgroups run out of blocks, and the atomics' round trips are
  // hidden behind those blocks.  The returned counts go to LDS once the
  // wavefront's loop is over.
  int arr0 = 0, arr1 = 0;
  bool arrived = false;
  uint32_t tsink = 0;
  auto arrive = [&]() {
    arrived = true;
    if (li.lane == 0) {
      if (cov[1] > 1) arr0 = __hip_atomic_fetch_add(p.sync + gr.h0, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (gr.h1 != gr.h0 && cov[3] > 1)
        arr1 = __hip_atomic_fetch_add(p.sync + gr.h1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // Single-block path: touch one word of every 128-byte line of the
    // workgroup's first fp16 blocks (Key and Value rows), so that they are
    // in the caches when the wavefronts take them up after their last
    // quantized blocks (measured: INT8 and FP8 calls -0.2 to -0.5 us; the
    // paired paths have no registers to spare for it).
    if constexpr (MODE == kSingle) {
      const int nt = p.n_sink + p.n_res;
      int done = 0;
      for (int hh = gr.h0; hh <= gr.h1 && done < 4; ++hh) {
        const int lo_h = hh == gr.h0 ? cov[0] : (hh == gr.h1 ? cov[2] : g);
        const int nc_h = hh == gr.h0 ? cov[1] : (hh == gr.h1 ? cov[3] : 1);
        for (int fb = g - lo_h; fb < p.fp16_blocks && done < 4; fb += nc_h, ++done) {
          int k = 32 * fb + (li.lane & 31);
          k = k < nt ? k : nt - 1;
          const int half = li.lane >> 5;
          const uint16_t* kr = seg_row(p, p.k_sink, p.k_ring, p.new_k, hh, k) + 64 * half;
          const uint16_t* vr = seg_row(p, p.v_sink, p.v_ring, p.new_v, hh, k) + 64 * half;
          tsink ^= *reinterpret_cast<const uint32_t*>(kr) ^ *reinterpret_cast<const uint32_t*>(vr);
        }
      }
    }
  };
  auto fetch = [&](Raw<FMT>& r, int& id, int& bhout, int& blkout) {
    int idx;
    if (p.deterministic) {
      idx = v + kGroupWaves * kst;
      ++kst;
    } else {
      idx = 0;
      if (li.lane == 0) idx = atomicAdd(ctr, 1);
      idx = __builtin_amdgcn_readfirstlane(idx);
    }
    if (idx < gr.len) {
      id = idx;
      uint32_t j = jb + (uint32_t)idx;
      const uint32_t bh = head_of(p, j);
      // visit the blocks of each head's part of the range (n blocks from ps)
      // starting at a per-workgroup fraction of it, so that the workgroups'
      // streams sit at unrelated addresses rather than in step:
      // j -> ps + (j - ps + floor(rot n / 2^20)) mod n
      const uint32_t ps = bh * nblk > jb ? bh * nblk : jb;
      const uint32_t pe = (bh + 1) * nblk < je ? (bh + 1) * nblk : je;
      const uint32_t n = pe - ps;
      uint32_t x = j - ps + (uint32_t)((rot * n) >> 20);   // < 2n
      x = x >= n ? x - n : x;
      j = ps + x;
      bhout = (int)bh;
      blkout = (int)(j - bh * nblk);
      const int64_t rec = p.table ? (int64_t)__builtin_amdgcn_readfirstlane(recs[j - (uint32_t)gr.jb])
                                  : (int64_t)bh * p.nb_cap + (j - bh * nblk);
      load_block<FMT>(r, p, rec, li.lane);
    } else {
      id = -1;
      bhout = 0;
      blkout = 0;
      if (idx == gr.len) arrive();
      load_block<FMT, false>(r, p, 0, li.lane);
    }
  };
  // Paired path: the range's blocks are handed out as units of two
  // consecutive blocks of one head (a head part of odd length ends with a
  // single block).  Units of the first head part come first, then ceil(nblk
  // / 2) units per whole head, then those of the last part; like single
  // blocks, each part's units are visited from a per-workgroup rotation.
  const uint32_t e0 = (uint32_t)gr.h0 * nblk + nblk < je ? (uint32_t)gr.h0 * nblk + nblk : je;
  const uint32_t u0 = (e0 - jb + 1) / 2;
  const uint32_t hn = (nblk + 1) / 2;
  const uint32_t units = gr.h1 > gr.h0 ? u0 + (uint32_t)(gr.h1 - gr.h0 - 1) * hn + (je - (uint32_t)gr.h1 * nblk + 1) / 2
                                       : u0;
  bool two[D / 2 > 0 ? D / 2 : 1];
  auto fetch_pair = [&](Raw<FMT>& ra, Raw<FMT>& rb, int& id, int& bhout, bool& has2) {
    int idx;
    if (p.deterministic) {
      idx = v + kGroupWaves * kst;
      ++kst;
    } else {
      idx = 0;
      if (li.lane == 0) idx = atomicAdd(ctr, 1);
      idx = __builtin_amdgcn_readfirstlane(idx);
    }
    if ((uint32_t)idx < units) {
      id = idx;
      uint32_t bh, ps, pe, r;
      if ((uint32_t)idx < u0) {
        bh = (uint32_t)gr.h0;
        ps = jb;
        pe = e0;
        r = (uint32_t)idx;
      } else {
        const uint32_t t = (uint32_t)idx - u0;
        const uint32_t k = (uint32_t)(((uint64_t)t * p.half_magic) >> p.half_shift);   // t / hn
        bh = (uint32_t)gr.h0 + 1 + k;
        r = t - k * hn;
        ps = bh * nblk;
        pe = ps + nblk < je ? ps + nblk : je;
      }
      const uint32_t nu = (pe - ps + 1) / 2;
      uint32_t x = r + (uint32_t)((rot * nu) >> 20);        // < 2 nu
      x = x >= nu ? x - nu : x;
      const uint32_t ja = ps + 2 * x;
      has2 = ja + 1 < pe;
      bhout = (int)bh;
      auto rec = [&](uint32_t j) {
        return p.table ? (int64_t)__builtin_amdgcn_readfirstlane(recs[j - jb])
                       : (int64_t)bh * p.nb_cap + (j - bh * nblk);
      };
      load_block<FMT>(ra, p, rec(ja), li.lane);
      if (has2) load_block<FMT>(rb, p, rec(ja + 1), li.lane);
      else load_block<FMT, false>(rb, p, 0, li.lane);
    } else {
      id = -1;
      bhout = 0;
      has2 = false;
      if (idx == (int)units) arrive();
      load_block<FMT, false>(ra, p, 0, li.lane);
      load_block<FMT, false>(rb, p, 0, li.lane);
    }
  };
  if constexpr (PAIR) {
#pragma unroll
    for (int d = 0; d < D - 2; d += 2) fetch_pair(buf[d], buf[d + 1], rid[d], rbh[d], two[d / 2]);
  } else {
#pragma unroll
    for (int d = 0; d < D - 1; ++d) fetch(buf[d], rid[d], rbh[d], rblk[d]);
  }

  // The fp16 blocks (sinks + residual ring) of the range's heads, each into
  // its own partial slot: fp16 block fb of head h belongs to covering
  // workgroup g_lo(h) + fb mod count(h); fp16_of maps the workgroup's k-th to
  // (h, fb).  They are processed at the end (see below).
  auto fp16_of = [&](int k, int& h, int& fb) -> bool {
    for (int hh = gr.h0; hh <= gr.h1; ++hh) {
      int lo_h, nc_h;
      cover(hh, lo_h, nc_h);
      const int64_t nc = nc_h, fb0 = g - lo_h;
      const int cnt = fb0 < p.fp16_blocks ? (int)((p.fp16_blocks - fb0 + nc - 1) / nc) : 0;
      if (k < cnt) {
        h = hh;
        fb = (int)(fb0 + k * nc);
        return true;
      }
      k -= cnt;
    }
    return false;
  };

  auto wave_slot = [&](int h, int w) { return p.part_wave + ((int64_t)kGroupWaves * (g + h) + w) * slot_floats(p); };
  if (li.writer && li.qd == 0) {
    for (int h = gr.h0; h <= gr.h1; ++h) {
      float* dst = wave_slot(h, v) + li.head * kPartStride;
      dst[0] = neg_inf();
      dst[1] = 0.f;
    }
  }

  {
    const float oscale = T::kFp8 ? p.v_scale : T::kCodeScale;
    QOp qop;
    f16x8 bk_static[4];
    query_operand<FMT>(q0, p.nrep, li, qop);  // qop holds the query of head qhead
    int qhead = gr.h0;
    WaveState ws;
    reset(ws);
    int cur = -1;
    if constexpr (PAIR) {
      // the segment of head h starts: close the previous one (both parities merged)
      auto begin_head = [&](int h) {
        if (h == cur) return;
        if (cur >= 0) {
          if constexpr (MODE == kSlots) {
            merge_slots(ws);
            finish_slot_segment(ws, li, wave_slot(cur, v), oscale);
          } else {
            merge_parity(ws);
            finish_segment(ws, li, wave_slot(cur, v), oscale, true);
          }
          reset(ws);
        }
        cur = h;
        if (cur != qhead) {
          load_query<FMT>(p, cur, li, qop);
          qhead = cur;
        }
      };
      // one step per ring position d (a compile-time constant, so the ring
      // stays in registers); false once no unit is left
      auto step = [&](auto dc) -> bool {
        constexpr int d = decltype(dc)::value;
        constexpr int f = (d + D - 2) % D;
        fetch_pair(buf[f], buf[f + 1], rid[f], rbh[f], two[f / 2]);
        if (rid[d] < 0) return false;        // units are taken in order: none left
        begin_head(rbh[d]);
        if constexpr (MODE == kSlots) process_slots<FMT>(buf[d], buf[d + 1], two[d / 2], stage, ws, qop, li);
        else process_pair<FMT>(buf[d], buf[d + 1], two[d / 2], stage, ws, qop, li);
        return true;
      };
      static_assert(D <= 8, "paired ring of at most 8 blocks");
      for (;;) {
        if (!step(std::integral_constant<int, 0>{})) break;
        if (!step(std::integral_constant<int, 2>{})) break;
        if constexpr (D > 4)
          if (!step(std::integral_constant<int, (D > 4 ? 4 : 0)>{})) break;
        if constexpr (D > 6)
          if (!step(std::integral_constant<int, (D > 6 ? 6 : 0)>{})) break;
      }
    } else {
      for (;;) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
          fetch(buf[(d + D - 1) % D], rid[(d + D - 1) % D], rbh[(d + D - 1) % D], rblk[(d + D - 1) % D]);
          if (rid[d] < 0) goto done;           // blocks are taken in order: none left
          if (rbh[d] != cur) {
            if (cur >= 0) {
              finish_segment(ws, li, wave_slot(cur, v), oscale, !T::kFp8);
              reset(ws);
            }
            cur = rbh[d];
            if (cur != qhead) {
              load_query<FMT>(p, cur, li, qop);
              qhead = cur;
            }
            if constexpr (T::kFp8 || T::kRope) static_q(qop, T::kFp8 ? p.k_scale * kQScale : kQScale, bk_static);
          }
          process_block<FMT>(buf[d], stage, ws, qop, bk_static, li, rc,
                             (double)p.sink_cap + (double)kBlock * rblk[d]);
        }
      }
    }
  done:
    // the wavefront's last segment goes to its own LDS partial area, the
    // earlier ones went to global memory
    float* part = reinterpret_cast<float*>(lds + v * kWaveLds + kStageBytes);
    if (cur >= 0) {
      if constexpr (MODE == kSlots) {
        merge_slots(ws);
        finish_slot_segment(ws, li, part, oscale);
      } else {
        if constexpr (MODE == kPairs) merge_parity(ws);
        finish_segment(ws, li, part, oscale, !T::kFp8);
      }
    }
    if (li.lane == 0) fin_head[v] = cur;
    asm volatile("" ::"v"(tsink));             // keeps the touch loads (their values are not used)
    if (arrived && li.lane == 0) {             // the arrival's returned counts
      ctr[2] = arr0;
      ctr[3] = arr1;
    }
  }

  // The fp16 blocks are taken from a second LDS counter by the wavefronts as
  // they run out of quantized blocks, so this work fills the wait for the
  // workgroup's slowest one (measured faster than doing them at the start,
  // under the first block loads, for every workload).
  {
    for (;;) {
      int idx = 0;
      if (li.lane == 0) idx = atomicAdd(ctr + 1, 1);
      idx = __builtin_amdgcn_readfirstlane(idx);
      int h, fb;
      if (!fp16_of(idx, h, fb)) break;
      // (the first kFp16Lds of the first head's: idx is then their place among that head's)
      float* dst = h == gr.h0 && idx < kFp16Lds
                       ? reinterpret_cast<float*>(lds + kLdsBytes) + idx * slot_floats(p)
                       : p.part_fp16 + ((int64_t)h * p.fp16_blocks + fb) * slot_floats(p);
      fp16_block<T::kRope>(p, h, fb, reinterpret_cast<uint16_t*>(stage), dst);
    }
  }
  __syncthreads();                            // every wavefront's partials written

  // ---- end of the call.  Heads in the middle of the range are covered by
  // this workgroup alone; the first and the last head may be shared with
  // neighbouring workgroups.  A shared head's counter (sync plane) has taken
  // each covering workgroup's arrival in its low 16 bits (see arrive); the
  // workgroup whose arrival completed the count combines the head, every
  // other one writes its merged slot and then adds its "written" mark (bit
  // 16).
  const int lo0 = cov[0], nc0 = cov[1], lo1 = cov[2], nc1 = cov[3];
  const bool sh0 = nc0 > 1, sh1 = gr.h1 != gr.h0 && nc1 > 1;
  int prev0 = 0, prev1 = 0;
  if (threadIdx.x == 0) {
    prev0 = ctr[2];
    prev1 = ctr[3];
  }
  bool last0 = false, last1 = false;
  // own merged partials of a shared head this workgroup combines, in the
  // (free) stage areas of wavefronts 0 and 1
  auto own_slot = [&](int s) { return reinterpret_cast<float*>(lds + s * kWaveLds); };

  // Merge the wavefronts' partials of each head, then the fp16 blocks of
  // the head that this workgroup handled (fb = g - g_lo(h) + k count(h)).
  // Items are (head, query head, four channels) of all the range's heads,
  // one per thread and pass; a pass issues its loads (the wavefront slots,
  // the first kFoldFp16 fp16 slots) before it uses any.  The result goes to
  // the output (a head of this workgroup alone), to LDS (a shared head this
  // workgroup combines) or to the workgroup's slot (device-coherent stores).
  {
    constexpr int kFoldFp16 = 4;
    const int nf = p.fp16_blocks;
    const int per = p.nrep * (kHeadDim / 4);
    const int total = (gr.h1 - gr.h0 + 1) * per;
    for (int base = 0; base < total; base += kGroupThreads) {
      const int idx = base + (int)threadIdx.x;
      const int h = gr.h0 + (idx < total ? idx / per : 0), r = idx % per, hh = r >> 5, c4 = r & 31;
      float M = neg_inf(), L = 0.f;
      float4 O = {0.f, 0.f, 0.f, 0.f};
      if (idx < total) {
        int lo_h, nc_h;
        cover(h, lo_h, nc_h);
        const int64_t nc = nc_h, fb0 = g - lo_h;
        float m[kGroupWaves], l[kGroupWaves], fm[kFoldFp16], fl[kFoldFp16];
        float4 o[kGroupWaves], fo[kFoldFp16];
#pragma unroll
        for (int w = 0; w < kGroupWaves; ++w) {
          // the wavefront's last segment is in its LDS area (read as LDS, not
          // through a generic pointer); an earlier one in its workspace slot
          const float* lp = reinterpret_cast<const float*>(lds + w * kWaveLds + kStageBytes) + hh * kPartStride;
          const float2 ml = *reinterpret_cast<const float2*>(lp);
          m[w] = ml.x;
          l[w] = ml.y;
          o[w] = *reinterpret_cast<const float4*>(lp + 4 + 4 * c4);
          if (fin_head[w] != h) {                 // (nontemporal: a load of another kind than
            const float* sp = wave_slot(h, w) + hh * kPartStride;   // the LDS one, never merged with it)
            const f32x2 a = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(sp));
            const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sp + 4 + 4 * c4));
            m[w] = a.x;
            l[w] = a.y;
            o[w] = float4{t.x, t.y, t.z, t.w};
          }
        }
        // the first kFp16Lds of the first head's are in LDS (read as LDS)
        const bool in_lds = h == gr.h0;
        static_assert(kFoldFp16 == kFp16Lds, "one pass reads the LDS fp16 partials");
        auto load_fp16 = [&](int64_t first) {
#pragma unroll
          for (int j = 0; j < kFoldFp16; ++j) {
            const int64_t fb = first + j * nc;
            if (fb < nf && in_lds && first == fb0) {
              const float* lp = reinterpret_cast<const float*>(lds + kLdsBytes) + j * slot_floats(p) + hh * kPartStride;
              const float2 ml = *reinterpret_cast<const float2*>(lp);
              fm[j] = ml.x;
              fl[j] = ml.y;
              fo[j] = *reinterpret_cast<const float4*>(lp + 4 + 4 * c4);
            } else if (fb < nf) {
              const float* sp = p.part_fp16 + ((int64_t)h * nf + fb) * slot_floats(p) + hh * kPartStride;
              fm[j] = sp[0];
              fl[j] = sp[1];
              fo[j] = *reinterpret_cast<const float4*>(sp + 4 + 4 * c4);
            } else {
              fm[j] = neg_inf();
              fl[j] = 0.f;
              fo[j] = float4{0.f, 0.f, 0.f, 0.f};
            }
          }
        };
        load_fp16(fb0);
        fold4<kGroupWaves>(M, L, O, m, l, o);
        fold4<kFoldFp16>(M, L, O, fm, fl, fo);
        for (int64_t first = fb0 + kFoldFp16 * nc; first < nf; first += kFoldFp16 * nc) {
          load_fp16(first);                       // more than kFoldFp16 fp16 blocks here
          fold4<kFoldFp16>(M, L, O, fm, fl, fo);
        }
      }
      if (base == 0) {                            // which shared heads this workgroup combines
        int* lf = ctr + 2;                        // the arrival's counts are in prev0 / prev1 now
        if (threadIdx.x == 0) {
          lf[0] = sh0 && (prev0 & 0xFFFF) == nc0 - 1;
          lf[1] = sh1 && (prev1 & 0xFFFF) == nc1 - 1;
        }
        __syncthreads();
        last0 = lf[0] != 0;
        last1 = lf[1] != 0;
      }
      if (idx < total) {
        const bool shared = (h == gr.h0 && sh0) || (h == gr.h1 && sh1);
        if (!shared) {                            // this workgroup's head alone: the output row
          const f16x2 lo = {(_Float16)(O.x / L), (_Float16)(O.y / L)};
          const f16x2 hi = {(_Float16)(O.z / L), (_Float16)(O.w / L)};
          *reinterpret_cast<uint2*>(p.out + ((int64_t)h * p.nrep + hh) * kHeadDim + 4 * c4) =
              uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        } else {
          const bool mine = h == gr.h0 ? last0 : last1;
          if (mine) {                             // (LDS and workspace addresses kept apart, so
            float* dst = own_slot(h == gr.h0 ? 0 : 1) + hh * kPartStride;   // that neither goes generic)
            if (c4 == 0) {
              dst[0] = M;
              dst[1] = L;
            }
            *reinterpret_cast<float4*>(dst + 4 + 4 * c4) = O;
          } else {
            float* dst = p.part_group + ((int64_t)g + h) * slot_floats(p) + hh * kPartStride;
            if (c4 == 0) {
              st_dev(dst, M);
              st_dev(dst + 1, L);
            }
            st_dev4(dst + 4 + 4 * c4, O);
          }
        }
      }
    }
  }
  // Shared heads combined elsewhere: the merged slot is written (each store
  // acknowledged), then the "written" mark.  The stores are device-coherent
  // (write-through past the compute unit's caches) and acknowledged before
  // the mark is added, so a combining workgroup that has seen the mark and
  // then loads the slot device-coherently reads these values.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    constexpr int kMarkOrder = KVQ_FORMAL_ORDERING ? __ATOMIC_RELEASE : __ATOMIC_RELAXED;
    if (sh0 && !last0) __hip_atomic_fetch_add(p.sync + gr.h0, 1 << 16, kMarkOrder, __HIP_MEMORY_SCOPE_AGENT);
    if (sh1 && !last1) __hip_atomic_fetch_add(p.sync + gr.h1, 1 << 16, kMarkOrder, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (last0 || last1)                          // (partials of the slot groups in wavefronts 2.. 's areas)
    combine_shared(p, g, gr.h0, gr.h1, last0, last1, lo0, lo1, nc0, nc1, own_slot(0), own_slot(1),
                   reinterpret_cast<float*>(lds + 2 * kWaveLds));
}


// No quantized blocks yet: workgroup g takes the fp16 blocks of head g and
// combines them.
template <bool ROPE>
__device__ void fp16_group(const AttnParams& p, char* lds) {
  const int g = blockIdx.x;
  const int v = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wavefront index, uniform
  for (int fb = v; fb < p.fp16_blocks; fb += kGroupWaves)
    fp16_block<ROPE>(p, g, fb, reinterpret_cast<uint16_t*>(lds + v * kWaveLds),
               p.part_fp16 + ((int64_t)g * p.fp16_blocks + fb) * slot_floats(p));
  __syncthreads();                            // the head's partials, all written by this workgroup
  reduce_fp16_head(p, g);
}

template <int FMT, int MODE = kSingle>
__global__ __launch_bounds__(kGroupThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16)))
  char lds[kLdsBytes + kFp16LdsBytes + (Traits<FMT>::kRope ? kRopeTableBytes : 0)];
  if (p.nblk == 0) fp16_group<Traits<FMT>::kRope>(p, lds);
  else group_main<FMT, MODE>(p, lds);
}

}  // namespace

// Workspace of kv_decode_attention_noalloc (partials of the split-K combine,
// which any contents may start from).  In host code `scratch` names a host
// stand-in, not device memory: only the address from hipGetSymbolAddress is
// ever handed to a kernel.
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch[kMaxScratchDevices];
}  // namespace

hipError_t attention_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void* a = g_scratch[dev].load(std::memory_order_acquire);
  if (!a) {                                     // first call on this device: it is current
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    g_scratch[dev].store(a, std::memory_order_release);   // racing first calls store the same address
  }
  *ptr = a;
  return hipSuccess;
}

hipError_t launch_attention(int variant, const AttnParams& p, hipStream_t s) {
  const dim3 grid((unsigned)p.groups), block(kGroupThreads);
  // INT4 / INT2: two blocks per step, process_pair at n_rep <= 4, process_slots at n_rep 8
#define KVQ_LAUNCH2(V, M) hipLaunchKernelGGL((attn_kernel<V, M>), grid, block, 0, s, p); return hipGetLastError()
  if (p.nrep <= 4) {
    switch (variant) {
      case KVQ_INT4: KVQ_LAUNCH2(KVQ_INT4, kPairs);
      case KVQ_INT2: KVQ_LAUNCH2(KVQ_INT2, kPairs);
      case KVQ_INT4 | kMeta16: KVQ_LAUNCH2(KVQ_INT4 | kMeta16, kPairs);
      case KVQ_INT2 | kMeta16: KVQ_LAUNCH2(KVQ_INT2 | kMeta16, kPairs);
      case KVQ_INT4 | kOutliers: KVQ_LAUNCH2(KVQ_INT4 | kOutliers, kPairs);
      case KVQ_INT2 | kOutliers: KVQ_LAUNCH2(KVQ_INT2 | kOutliers, kPairs);
      case KVQ_INT4 | kMeta16 | kOutliers: KVQ_LAUNCH2(KVQ_INT4 | kMeta16 | kOutliers, kPairs);
      case KVQ_INT2 | kMeta16 | kOutliers: KVQ_LAUNCH2(KVQ_INT2 | kMeta16 | kOutliers, kPairs);
      default: break;
    }
  } else {
    switch (variant) {
      case KVQ_INT4: KVQ_LAUNCH2(KVQ_INT4, kSlots);
      case KVQ_INT2: KVQ_LAUNCH2(KVQ_INT2, kSlots);
      case KVQ_INT4 | kMeta16: KVQ_LAUNCH2(KVQ_INT4 | kMeta16, kSlots);
      case KVQ_INT2 | kMeta16: KVQ_LAUNCH2(KVQ_INT2 | kMeta16, kSlots);
      default: break;
    }
  }
#undef KVQ_LAUNCH2
  switch (variant) {
    case KVQ_INT8: hipLaunchKernelGGL(attn_kernel<KVQ_INT8>, grid, block, 0, s, p); break;
    case KVQ_INT4: hipLaunchKernelGGL(attn_kernel<KVQ_INT4>, grid, block, 0, s, p); break;
    case KVQ_INT2: hipLaunchKernelGGL(attn_kernel<KVQ_INT2>, grid, block, 0, s, p); break;
    case KVQ_FP8_E4M3: hipLaunchKernelGGL(attn_kernel<KVQ_FP8_E4M3>, grid, block, 0, s, p); break;
    case KVQ_FP8_E5M2: hipLaunchKernelGGL(attn_kernel<KVQ_FP8_E5M2>, grid, block, 0, s, p); break;
    case KVQ_INT8 | kMeta16: hipLaunchKernelGGL(attn_kernel<KVQ_INT8 | kMeta16>, grid, block, 0, s, p); break;
    case KVQ_INT4 | kMeta16: hipLaunchKernelGGL(attn_kernel<KVQ_INT4 | kMeta16>, grid, block, 0, s, p); break;
    case KVQ_INT2 | kMeta16: hipLaunchKernelGGL(attn_kernel<KVQ_INT2 | kMeta16>, grid, block, 0, s, p); break;
    case KVQ_INT8 | kRope: hipLaunchKernelGGL(attn_kernel<KVQ_INT8 | kRope>, grid, block, 0, s, p); break;
    case KVQ_INT4 | kRope: hipLaunchKernelGGL(attn_kernel<KVQ_INT4 | kRope>, grid, block, 0, s, p); break;
    case KVQ_INT2 | kRope: hipLaunchKernelGGL(attn_kernel<KVQ_INT2 | kRope>, grid, block, 0, s, p); break;
    case KVQ_FP8_E4M3 | kRope: hipLaunchKernelGGL(attn_kernel<KVQ_FP8_E4M3 | kRope>, grid, block, 0, s, p); break;
    case KVQ_FP8_E5M2 | kRope: hipLaunchKernelGGL(attn_kernel<KVQ_FP8_E5M2 | kRope>, grid, block, 0, s, p); break;
    case KVQ_INT8 | kOutliers: hipLaunchKernelGGL(attn_kernel<KVQ_INT8 | kOutliers>, grid, block, 0, s, p); break;
    case KVQ_INT4 | kOutliers: hipLaunchKernelGGL(attn_kernel<KVQ_INT4 | kOutliers>, grid, block, 0, s, p); break;
    case KVQ_INT2 | kOutliers: hipLaunchKernelGGL(attn_kernel<KVQ_INT2 | kOutliers>, grid, block, 0, s, p); break;
    case KVQ_INT8 | kMeta16 | kOutliers:
      hipLaunchKernelGGL(attn_kernel<KVQ_INT8 | kMeta16 | kOutliers>, grid, block, 0, s, p); break;
    case KVQ_INT4 | kMeta16 | kOutliers:
      hipLaunchKernelGGL(attn_kernel<KVQ_INT4 | kMeta16 | kOutliers>, grid, block, 0, s, p); break;
    case KVQ_INT2 | kMeta16 | kOutliers:
      hipLaunchKernelGGL(attn_kernel<KVQ_INT2 | kMeta16 | kOutliers>, grid, block, 0, s, p); break;
    case KVQ_INT8 | kMeta16 | kRope:
      hipLaunchKernelGGL(attn_kernel<KVQ_INT8 | kMeta16 | kRope>, grid, block, 0, s, p); break;
    case KVQ_INT4 | kMeta16 | kRope:
      hipLaunchKernelGGL(attn_kernel<KVQ_INT4 | kMeta16 | kRope>, grid, block, 0, s, p); break;
    case KVQ_INT2 | kMeta16 | kRope:
      hipLaunchKernelGGL(attn_kernel<KVQ_INT2 | kMeta16 | kRope>, grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
