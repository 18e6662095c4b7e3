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
// Work decomposition (grid = [1 + body splits, Hkv, B], 256 threads):
//  * blockIdx.x == 0 handles the fp16 segment (sinks + residual ring) of one
//    (sequence, KV head) with plain fp32 VALU code;
//  * every other workgroup owns a range of 4 * blocks_per_wave quantized
//    32-token blocks of one (sequence, KV head); each of its four wavefronts
//    streams blocks_per_wave consecutive blocks and keeps an online softmax
//    for all n_rep query heads of the KV head (GQA: every KV byte is read
//    once per step);
//  * each workgroup writes one partial (max, sum, unnormalised output) per
//    query head; reduce_kernel combines the partials in a fixed order.
//
// Per 32-token block a wavefront runs both products on the matrix cores with
// v_mfma_f32_16x16x32_f16 (fp32 accumulate):
//  QK:  D[token][col] = codes[token][channel] x q'[channel][col]
//  PV:  D[channel][col] = codes[channel][token] x P'[token][col]
// Column col = lane % 16 is query head (col % 8) of the KV head's group;
// columns 0-7 carry the fp16 "hi" part of the fp32 operand and columns 8-15
// its "lo" remainder (hi = f16(x), lo = f16(x - hi)), so the fp32 operand is
// represented to ~22 bits and the two column halves are summed after the
// product (DPP row_ror:8).  Codes enter as exact small integers in f16 (or
// exact E4M3 values), so no dequantization error is added:
//  * Key fold: q . k_hat = sum_c (q_c s_c) code_c - sum_c q_c s_c z_c, with
//    q' = q * s per channel (recomputed per block: the Key scale varies per
//    32-token group) and the zero-point sum as the accumulator's initial value;
//  * Value fold: p_t v_hat_tc = (p_t s_tg) code_tc - p_t s_tg z_tg, with
//    P' = p * s per token and channel group; the zero-point sums are
//    accumulated on the VALU and subtracted at the end.
// The softmax runs in base 2 (log2(e) / sqrt(D) folded into q).
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

// value of lane (lane + 8) mod 16 within the lane's row of 16 (DPP row_ror:8)
__device__ __forceinline__ float ror8(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128,
                                                               0xF, 0xF, false));
}

__device__ __forceinline__ float xor_shfl(float x, int m) { return __shfl_xor(x, m, 64); }

__device__ __forceinline__ f16x2 u2h(uint32_t w) { return __builtin_bit_cast(f16x2, w); }

// (0x6400 | c) is the f16 value 1024 + c for c < 1024; subtracting 1024 is exact.
__device__ __forceinline__ f16x2 magic_sub(uint32_t w) {
  const f16x2 k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  return u2h(w | 0x64006400u) - k1024;
}

__device__ __forceinline__ f16x8 cat(f16x2 a, f16x2 b, f16x2 c, f16x2 d) {
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 8 nibbles -> slots (n0, n4, 16*n1, 16*n5, n2, n6, 16*n3, 16*n7)
__device__ __forceinline__ f16x8 cvt_int4(uint32_t w) {
  const uint32_t w8 = w >> 8;
  return cat(magic_sub(w & 0x000F000Fu), magic_sub(w & 0x00F000F0u), magic_sub(w8 & 0x000F000Fu),
             magic_sub(w8 & 0x00F000F0u));
}

// 8 bytes (two words) -> slots in byte order
__device__ __forceinline__ f16x8 cvt_u8(uint32_t w0, uint32_t w1) {
  const uint32_t lo = 0x04010400u, hi = 0x04030402u;   // [0x64, b1, 0x64, b0] / [.., b3, .., b2]
  return cat(u2h(__builtin_amdgcn_perm(0x64646464u, w0, lo)) - f16x2{1024, 1024},
             u2h(__builtin_amdgcn_perm(0x64646464u, w0, hi)) - f16x2{1024, 1024},
             u2h(__builtin_amdgcn_perm(0x64646464u, w1, lo)) - f16x2{1024, 1024},
             u2h(__builtin_amdgcn_perm(0x64646464u, w1, hi)) - f16x2{1024, 1024});
}

// 16 two-bit codes c0..c15: low half -> slots (c_k, c_{8+k}) * 4^k, high half
// (codes shifted down a byte) -> (c_{4+k}, c_{12+k}) * 4^k, k = 0..3
__device__ __forceinline__ f16x8 cvt_int2(uint32_t w, bool high) {
  const uint32_t x = high ? (w >> 8) : w;
  return cat(magic_sub(x & 0x00030003u), magic_sub(x & 0x000C000Cu), magic_sub(x & 0x00300030u),
             magic_sub(x & 0x00C000C0u));
}

// 8 OCP E4M3 bytes -> exact f16 values in byte order (hardware conversion)
__device__ __forceinline__ f16x8 cvt_fp8(uint32_t w0, uint32_t w1) {
  return cat(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false),
             __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true),
             __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false),
             __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true));
}

template <int FMT>
struct Traits {
  static constexpr bool kFp8 = FMT == KVQ_FP8_E4M3;
  static constexpr int kBits = FMT == KVQ_INT4 ? 4 : (FMT == KVQ_INT2 ? 2 : 8);
  static constexpr int kRowBytes = kHeadDim * kBits / 8;   // packed bytes per token
  static constexpr int kKWords = 32 * kBits / 32;          // words per lane per 16-token tile
  static constexpr int kVWords = kRowBytes / 8;            // words per V record (= per lane)
};

// Matrix-core operand number a (K: k-block kb of the lane's 32 channels;
// V: 16-channel tile m) from the lane's packed words.
template <int FMT>
__device__ __forceinline__ f16x8 operand(const uint32_t* w, int a) {
  if constexpr (FMT == KVQ_INT4) return cvt_int4(w[a]);
  else if constexpr (FMT == KVQ_INT2) return cvt_int2(w[a >> 1], (a & 1) != 0);
  else if constexpr (FMT == KVQ_FP8_E4M3) return cvt_fp8(w[2 * a], w[2 * a + 1]);
  else return cvt_u8(w[2 * a], w[2 * a + 1]);
}

// Channel (0..31 within the lane's quarter) carried by k-slot j of k-block kb.
template <int FMT>
__device__ constexpr int k_chan(int kb, int j) {
  if constexpr (FMT == KVQ_INT4) return 8 * kb + (j >> 1) + 4 * (j & 1);
  else if constexpr (FMT == KVQ_INT2) return 16 * (kb >> 1) + 4 * (kb & 1) + (j >> 1) + 8 * (j & 1);
  else return 8 * kb + j;
}

// Power-of-two factor the conversion leaves on code i (channel for K, token
// for V); it is divided out of the staged scale.
template <int FMT>
__device__ constexpr float slot_div(int i) {
  if constexpr (FMT == KVQ_INT4) return (i & 1) ? 16.0f : 1.0f;
  else if constexpr (FMT == KVQ_INT2) return (float)(1 << (2 * (i & 3)));
  else return 1.0f;
}

template <int FMT>
struct Raw {
  uint32_t k[2][Traits<FMT>::kKWords];   // two 16-token tiles
  uint32_t v[Traits<FMT>::kVWords];
  float4 km, vm;                         // this lane's 16 bytes of each meta block
};

template <int FMT>
__device__ __forceinline__ void load_block(Raw<FMT>& r, const AttnParams& p, int64_t bh, int64_t blk,
                                           int lane) {
  using T = Traits<FMT>;
  const int64_t blkoff = (bh * p.nb_cap + blk) * (int64_t)(kBlock * T::kRowBytes);
  const int qd = lane >> 4;
#pragma unroll
  for (int tile = 0; tile < 2; ++tile) {
    const uint8_t* src = p.k_codes + blkoff + (int64_t)(16 * tile + (lane & 15)) * T::kRowBytes +
                         qd * (T::kKWords * 4);
    if constexpr (T::kKWords == 8) {
      const uint4 a = reinterpret_cast<const uint4*>(src)[0];
      const uint4 b = reinterpret_cast<const uint4*>(src)[1];
      r.k[tile][0] = a.x; r.k[tile][1] = a.y; r.k[tile][2] = a.z; r.k[tile][3] = a.w;
      r.k[tile][4] = b.x; r.k[tile][5] = b.y; r.k[tile][6] = b.z; r.k[tile][7] = b.w;
    } else if constexpr (T::kKWords == 4) {
      const uint4 a = *reinterpret_cast<const uint4*>(src);
      r.k[tile][0] = a.x; r.k[tile][1] = a.y; r.k[tile][2] = a.z; r.k[tile][3] = a.w;
    } else {
      const uint2 a = *reinterpret_cast<const uint2*>(src);
      r.k[tile][0] = a.x; r.k[tile][1] = a.y;
    }
  }
  const uint4* vsrc = reinterpret_cast<const uint4*>(p.v_codes + blkoff + (int64_t)lane * (T::kVWords * 4));
#pragma unroll
  for (int i = 0; i < T::kVWords / 4; ++i) {
    const uint4 a = vsrc[i];
    r.v[4 * i] = a.x; r.v[4 * i + 1] = a.y; r.v[4 * i + 2] = a.z; r.v[4 * i + 3] = a.w;
  }
  if constexpr (!T::kFp8) {
    const int64_t moff = (bh * p.nb_cap + blk) * 256 + lane * 4;
    r.km = *reinterpret_cast<const float4*>(p.k_meta + moff);
    r.vm = *reinterpret_cast<const float4*>(p.v_meta + moff);
  }
}

// LDS staging area of one wavefront for one block (floats):
//   [0,128) K scale / slot divisor   [128,256) K s*z
//   [256,384) V scale / divisor [g][t]   [384,512) V s*z [g][t]
constexpr int kStage = 512;

template <int FMT>
__device__ __forceinline__ void stage_meta(const Raw<FMT>& r, float* st, int lane) {
  // lane L < 32 holds s[4L..4L+3], lane L + 32 the matching z
  const float kz0 = __shfl_down(r.km.x, 32, 64), kz1 = __shfl_down(r.km.y, 32, 64);
  const float kz2 = __shfl_down(r.km.z, 32, 64), kz3 = __shfl_down(r.km.w, 32, 64);
  const float vz0 = __shfl_down(r.vm.x, 32, 64), vz1 = __shfl_down(r.vm.y, 32, 64);
  const float vz2 = __shfl_down(r.vm.z, 32, 64), vz3 = __shfl_down(r.vm.w, 32, 64);
  if (lane < 32) {
    const int c = 4 * lane;                      // K channel
    float4 ks = {r.km.x / slot_div<FMT>(c), r.km.y / slot_div<FMT>(c + 1),
                 r.km.z / slot_div<FMT>(c + 2), r.km.w / slot_div<FMT>(c + 3)};
    float4 kz = {r.km.x * kz0, r.km.y * kz1, r.km.z * kz2, r.km.w * kz3};
    *reinterpret_cast<float4*>(st + c) = ks;
    *reinterpret_cast<float4*>(st + 128 + c) = kz;
    const int t = c & 31;                        // V: group lane / 8, tokens t..t+3
    float4 vs = {r.vm.x / slot_div<FMT>(t), r.vm.y / slot_div<FMT>(t + 1),
                 r.vm.z / slot_div<FMT>(t + 2), r.vm.w / slot_div<FMT>(t + 3)};
    float4 vz = {r.vm.x * vz0, r.vm.y * vz1, r.vm.z * vz2, r.vm.w * vz3};
    *reinterpret_cast<float4*>(st + 256 + c) = vs;
    *reinterpret_cast<float4*>(st + 384 + c) = vz;
  }
}

struct WaveState {
  float m;          // running max (base-2 logits) of this lane's column
  float l;          // this lane's partial softmax denominator
  f32x4 o[8];       // PV accumulator: rows 16m + 4qd + i, column col
  float zacc[4];    // Value zero-point sums per channel group
};

template <int FMT>
__device__ __forceinline__ void process_block(const Raw<FMT>& r, float* st, WaveState& ws,
                                              const float* qf, const float* qfb, const f16x8* bk_static,
                                              bool is_lo, int lane) {
  using T = Traits<FMT>;
  const int qd = lane >> 4;

  // ---- QK: Key codes (rows = tokens) x q' (columns)
  f32x4 acc[2];
  if constexpr (T::kFp8) {
    acc[0] = f32x4{0, 0, 0, 0};
    acc[1] = acc[0];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int tile = 0; tile < 2; ++tile)
        acc[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(operand<FMT>(r.k[tile], kb), bk_static[kb],
                                                           acc[tile], 0, 0, 0);
    }
  } else {
    stage_meta<FMT>(r, st, lane);
    float sk[32], szk[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 a = *reinterpret_cast<const float4*>(st + 32 * qd + 4 * i);
      const float4 b = *reinterpret_cast<const float4*>(st + 128 + 32 * qd + 4 * i);
      sk[4 * i] = a.x; sk[4 * i + 1] = a.y; sk[4 * i + 2] = a.z; sk[4 * i + 3] = a.w;
      szk[4 * i] = b.x; szk[4 * i + 1] = b.y; szk[4 * i + 2] = b.z; szk[4 * i + 3] = b.w;
    }
    // zero-point term sum_c q_c s_c z_c of this lane's 32 channels, then the
    // other three quarters
    float bias = 0.f;
#pragma unroll
    for (int c = 0; c < 32; ++c) bias = __builtin_fmaf(qf[c], szk[c], bias);
    bias += xor_shfl(bias, 16);
    bias += xor_shfl(bias, 32);
    const float c0 = is_lo ? 0.f : -bias;
    acc[0] = f32x4{c0, c0, c0, c0};
    acc[1] = acc[0];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f16x8 bq;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = k_chan<FMT>(kb, j);
        const _Float16 hi = (_Float16)(qfb[c] * sk[c]);          // 0 in hi columns
        bq[j] = (_Float16)__builtin_fmaf(qf[c], sk[c], -(float)hi); // hi, or the lo remainder
      }
#pragma unroll
      for (int tile = 0; tile < 2; ++tile)
        acc[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(operand<FMT>(r.k[tile], kb), bq, acc[tile], 0,
                                                           0, 0);
    }
  }

  // ---- online softmax over the block's 32 tokens (this lane: 8 of them)
  float lg[2][4];
  float mx = neg_inf();
#pragma unroll
  for (int tile = 0; tile < 2; ++tile)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lg[tile][i] = acc[tile][i] + ror8(acc[tile][i]);
      mx = fmaxf(mx, lg[tile][i]);
    }
  mx = fmaxf(mx, xor_shfl(mx, 16));
  mx = fmaxf(mx, xor_shfl(mx, 32));
  const float m_new = fmaxf(ws.m, mx);
  if (__any(m_new > ws.m)) {
    const float alpha = exp2f(ws.m - m_new);     // 0 on the first block (m = -inf)
#pragma unroll
    for (int m = 0; m < 8; ++m) ws.o[m] *= alpha;
#pragma unroll
    for (int g = 0; g < 4; ++g) ws.zacc[g] *= alpha;
    ws.l *= alpha;
    ws.m = m_new;
  }
  float pr[2][4];
#pragma unroll
  for (int tile = 0; tile < 2; ++tile)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[tile][i] = exp2f(lg[tile][i] - ws.m);
      ws.l += pr[tile][i];
    }

  // ---- PV: Value codes (rows = channels) x P' (columns)
  if constexpr (T::kFp8) {
    f16x8 bp;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        const float x = pr[tile][v];
        const _Float16 hi = (_Float16)(is_lo ? x : 0.f);
        bp[2 * v + tile] = (_Float16)(x - (float)hi);
      }
    }
#pragma unroll
    for (int m = 0; m < 8; ++m)
      ws.o[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(operand<FMT>(r.v, m), bp, ws.o[m], 0, 0, 0);
  } else {
    float pb[2][4];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile)
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[tile][i] = is_lo ? pr[tile][i] : 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // scales of tokens 4qd..4qd+3 (tile 0) and 16+4qd..16+4qd+3 (tile 1)
      const float4 s0 = *reinterpret_cast<const float4*>(st + 256 + 32 * g + 4 * qd);
      const float4 s1 = *reinterpret_cast<const float4*>(st + 256 + 32 * g + 16 + 4 * qd);
      const float4 z0 = *reinterpret_cast<const float4*>(st + 384 + 32 * g + 4 * qd);
      const float4 z1 = *reinterpret_cast<const float4*>(st + 384 + 32 * g + 16 + 4 * qd);
      const float sv[2][4] = {{s0.x, s0.y, s0.z, s0.w}, {s1.x, s1.y, s1.z, s1.w}};
      const float zv[2][4] = {{z0.x, z0.y, z0.z, z0.w}, {z1.x, z1.y, z1.z, z1.w}};
      f16x8 bp;
      float za = ws.zacc[g];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
          const _Float16 hi = (_Float16)(pb[tile][v] * sv[tile][v]);
          bp[2 * v + tile] = (_Float16)__builtin_fmaf(pr[tile][v], sv[tile][v], -(float)hi);
          za = __builtin_fmaf(pr[tile][v], zv[tile][v], za);
        }
      }
      ws.zacc[g] = za;
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const int m = 2 * g + mm;
        ws.o[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(operand<FMT>(r.v, m), bp, ws.o[m], 0, 0, 0);
      }
    }
  }
}

// ---------------------------------------------------------------- LDS map
constexpr int kCombineFloats = kWavesPerSplit * 8 * 130;                 // m, l, o[128] per head
constexpr int kBodyLdsFloats = kWavesPerSplit * 2 * kStage > kCombineFloats ? kWavesPerSplit * 2 * kStage
                                                                            : kCombineFloats;
constexpr int kSegChunk = 32;
constexpr int kSegKStride = 130;                                         // halves per K row (bank spread)
constexpr int kSegBytes = 8 * 128 * 4 + kSegChunk * kSegKStride * 2 + kSegChunk * 128 * 2 + 8 * kSegChunk * 4;
constexpr int kLdsBytes = kBodyLdsFloats * 4 > kSegBytes ? kBodyLdsFloats * 4 : kSegBytes;

template <int FMT>
__device__ void body_split(const AttnParams& p, int b, int g, int split, char* lds) {
  using T = Traits<FMT>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;
  const int qd = lane >> 4;
  const int head = col & 7;
  const bool is_lo = col >= 8;
  const bool valid_head = head < p.nrep;
  const int64_t bh = (int64_t)b * p.hkv + g;
  float* ldsf = reinterpret_cast<float*>(lds);
  float* stage = ldsf + wave * 2 * kStage;

  // query in base-2 logit units, this lane's head and 32 channels
  const float qscale = kLog2e * 0.08838834764831845f;   // log2(e) / sqrt(128)
  float qf[32], qfb[32];
  {
    const uint16_t* qsrc = p.q + (((int64_t)b * p.hkv + g) * p.nrep + (valid_head ? head : 0)) * kHeadDim + 32 * qd;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 w = reinterpret_cast<const uint4*>(qsrc)[i];
      const uint32_t ws_[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = valid_head ? (float)u2h(ws_[j])[0] * qscale : 0.f;
        const float c = valid_head ? (float)u2h(ws_[j])[1] * qscale : 0.f;
        qf[8 * i + 2 * j] = a;
        qf[8 * i + 2 * j + 1] = c;
      }
    }
  }
  f16x8 bk_static[4];
  if constexpr (T::kFp8) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = qf[k_chan<FMT>(kb, j)] * p.k_scale;
        const _Float16 hi = (_Float16)(is_lo ? x : 0.f);
        bk_static[kb][j] = (_Float16)(x - (float)hi);
      }
  } else {
#pragma unroll
    for (int c = 0; c < 32; ++c) qfb[c] = is_lo ? qf[c] : 0.f;
  }

  WaveState ws;
  ws.m = neg_inf();
  ws.l = 0.f;
#pragma unroll
  for (int m = 0; m < 8; ++m) ws.o[m] = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int gg = 0; gg < 4; ++gg) ws.zacc[gg] = 0.f;

  const int64_t first = ((int64_t)split * kWavesPerSplit + wave) * p.blocks_per_wave;
  int64_t nb = (int64_t)p.nblk - first;
  if (nb > p.blocks_per_wave) nb = p.blocks_per_wave;
  if (nb > 0) {
    Raw<FMT> ra, rb;
    load_block<FMT>(ra, p, bh, first, lane);
    for (int64_t i = 0; i < nb; i += 2) {
      if (i + 1 < nb) load_block<FMT>(rb, p, bh, first + i + 1, lane);
      process_block<FMT>(ra, stage, ws, qf, qfb, bk_static, is_lo, lane);
      if (i + 1 >= nb) break;
      if (i + 2 < nb) load_block<FMT>(ra, p, bh, first + i + 2, lane);
      process_block<FMT>(rb, stage + kStage, ws, qf, qfb, bk_static, is_lo, lane);
    }
  }

  // ---- finish this wavefront: sum over quarters, hi + lo columns
  float l = ws.l;
  l += xor_shfl(l, 16);
  l += xor_shfl(l, 32);
  float z[4];
#pragma unroll
  for (int gg = 0; gg < 4; ++gg) {
    z[gg] = ws.zacc[gg];
    z[gg] += xor_shfl(z[gg], 16);
    z[gg] += xor_shfl(z[gg], 32);
  }
  const float vscale = T::kFp8 ? p.v_scale : 1.0f;
  __syncthreads();                                   // staging area is reused below
  float* cm = ldsf + wave * 8 * 130;                 // [head][m, l, o[128]]
#pragma unroll
  for (int m = 0; m < 8; ++m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float o = (ws.o[m][i] + ror8(ws.o[m][i]) - z[m >> 1]) * vscale;
      if (!is_lo && valid_head) cm[head * 130 + 2 + 16 * m + 4 * qd + i] = o;
    }
  }
  if (!is_lo && valid_head && qd == 0) {
    cm[head * 130] = ws.m;
    cm[head * 130 + 1] = l;
  }
  __syncthreads();

  // ---- combine the four wavefronts and write this split's partials
  for (int e = tid; e < p.nrep * kHeadDim; e += 256) {
    const int h = e >> 7, c = e & 127;
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < kWavesPerSplit; ++w) M = fmaxf(M, ldsf[w * 8 * 130 + h * 130]);
    float L = 0.f, O = 0.f;
    if (M != neg_inf()) {
#pragma unroll
      for (int w = 0; w < kWavesPerSplit; ++w) {
        const float mw = ldsf[w * 8 * 130 + h * 130];
        if (mw != neg_inf()) {
          const float f = exp2f(mw - M);
          L = __builtin_fmaf(f, ldsf[w * 8 * 130 + h * 130 + 1], L);
          O = __builtin_fmaf(f, ldsf[w * 8 * 130 + h * 130 + 2 + c], O);
        }
      }
    }
    float* dst = p.part + ((bh * p.nsplit + split + 1) * p.nrep + h) * kPartStride;
    dst[4 + c] = O;
    if (c == 0) {
      dst[0] = M;
      dst[1] = L;
    }
  }
}

// fp16 segment: sink tokens and the residual ring, plain fp32 arithmetic.
__device__ void fp16_segment(const AttnParams& p, int b, int g, char* lds) {
  const int tid = threadIdx.x;
  const int hh = tid >> 5;            // query head of the group
  const int c4 = tid & 31;            // channels 4*c4 .. 4*c4+3
  float* qs = reinterpret_cast<float*>(lds);                                  // [8][128]
  uint16_t* kc = reinterpret_cast<uint16_t*>(lds + 8 * 128 * 4);              // [32][130]
  uint16_t* vc = kc + kSegChunk * kSegKStride;                                // [32][128]
  float* lgs = reinterpret_cast<float*>(vc + kSegChunk * 128);                // [8][32]
  const int64_t bh = (int64_t)b * p.hkv + g;
  const float qscale = kLog2e * 0.08838834764831845f;
  if (hh < p.nrep) {
    const uint16_t* qsrc = p.q + (bh * p.nrep + hh) * kHeadDim + 4 * c4;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      qs[hh * 128 + 4 * c4 + j] = (float)__builtin_bit_cast(_Float16, qsrc[j]) * qscale;
  }
  float m = neg_inf(), l = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
  const int nt = p.n_sink + p.n_res;
  for (int base = 0; base < nt; base += kSegChunk) {
    __syncthreads();
    for (int e = tid; e < kSegChunk * 16; e += 256) {
      const int t = e >> 4, c8 = (e & 15) * 8;
      const int k = base + t;
      uint4 kk = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (k < nt) {
        const uint16_t* kp;
        const uint16_t* vp;
        if (k < p.n_sink) {
          const int64_t s_off = (bh * (int64_t)p.sink_cap + k) * kHeadDim + c8;
          kp = p.k_sink + s_off;
          vp = p.v_sink + s_off;
        } else {
          const int slot = (p.ring_first + (k - p.n_sink)) % p.ring_slots;
          const int64_t r_off = (bh * p.ring_slots + slot) * kHeadDim + c8;
          kp = p.k_ring + r_off;
          vp = p.v_ring + r_off;
        }
        kk = *reinterpret_cast<const uint4*>(kp);
        vv = *reinterpret_cast<const uint4*>(vp);
      }
      uint32_t* kd = reinterpret_cast<uint32_t*>(kc + t * kSegKStride + c8);
      kd[0] = kk.x; kd[1] = kk.y; kd[2] = kk.z; kd[3] = kk.w;
      *reinterpret_cast<uint4*>(vc + t * 128 + c8) = vv;
    }
    __syncthreads();
    {
      const int t = tid & 31;                 // token of the chunk
      if (hh < p.nrep) {
        float acc = 0.f;
        if (base + t < nt) {
          for (int c = 0; c < kHeadDim; ++c)
            acc = __builtin_fmaf(qs[hh * 128 + c], (float)__builtin_bit_cast(_Float16, kc[t * kSegKStride + c]),
                                 acc);
        }
        lgs[hh * kSegChunk + t] = (base + t < nt) ? acc : neg_inf();
      }
    }
    __syncthreads();
    if (hh < p.nrep) {
      float cmax = neg_inf();
      for (int t = 0; t < kSegChunk; ++t) cmax = fmaxf(cmax, lgs[hh * kSegChunk + t]);
      const float m_new = fmaxf(m, cmax);
      const float alpha = exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] *= alpha;
      m = m_new;
      for (int t = 0; t < kSegChunk; ++t) {
        const float pt = exp2f(lgs[hh * kSegChunk + t] - m);
        l += pt;
        const uint2 vw = *reinterpret_cast<const uint2*>(vc + t * 128 + 4 * c4);
        o[0] = __builtin_fmaf(pt, (float)u2h(vw.x)[0], o[0]);
        o[1] = __builtin_fmaf(pt, (float)u2h(vw.x)[1], o[1]);
        o[2] = __builtin_fmaf(pt, (float)u2h(vw.y)[0], o[2]);
        o[3] = __builtin_fmaf(pt, (float)u2h(vw.y)[1], o[3]);
      }
    }
  }
  if (hh < p.nrep) {
    float* dst = p.part + ((bh * p.nsplit + 0) * p.nrep + hh) * kPartStride;
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[4 + 4 * c4 + j] = o[j];
    if (c4 == 0) {
      dst[0] = m;
      dst[1] = l;
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void attn_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int g = blockIdx.y, b = blockIdx.z;
  if (blockIdx.x == 0) {
    fp16_segment(p, b, g, lds);
  } else {
    body_split<FMT>(p, b, g, blockIdx.x - 1, lds);
  }
}

// out[b][h] = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, M = max_s m_s
__global__ __launch_bounds__(128) void reduce_kernel(ReduceParams p) {
  const int hq = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
  const int g = hq / p.nrep, hh = hq % p.nrep;
  const int64_t stride = (int64_t)p.nrep * kPartStride;
  const float* base = p.part + (((int64_t)b * p.hkv + g) * p.nsplit * p.nrep + hh) * kPartStride;
  float M = neg_inf();
  for (int s = 0; s < p.nsplit; ++s) M = fmaxf(M, base[s * stride]);
  float L = 0.f, O = 0.f;
  for (int s = 0; s < p.nsplit; ++s) {
    const float ms = base[s * stride];
    if (ms != neg_inf()) {
      const float f = exp2f(ms - M);
      L = __builtin_fmaf(f, base[s * stride + 1], L);
      O = __builtin_fmaf(f, base[s * stride + 4 + c], O);
    }
  }
  const _Float16 r = (_Float16)(O / L);
  p.out[((int64_t)b * p.hkv * p.nrep + hq) * kHeadDim + c] = __builtin_bit_cast(uint16_t, r);
}

}  // namespace

hipError_t launch_attention(int fmt, const AttnParams& p, int batch, hipStream_t s) {
  const dim3 grid(p.nsplit, p.hkv, batch), block(256);
  switch (fmt) {
    case KVQ_INT8: hipLaunchKernelGGL(attn_kernel<KVQ_INT8>, grid, block, 0, s, p); break;
    case KVQ_INT4: hipLaunchKernelGGL(attn_kernel<KVQ_INT4>, grid, block, 0, s, p); break;
    case KVQ_INT2: hipLaunchKernelGGL(attn_kernel<KVQ_INT2>, grid, block, 0, s, p); break;
    case KVQ_FP8_E4M3: hipLaunchKernelGGL(attn_kernel<KVQ_FP8_E4M3>, grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceParams& p, int batch, hipStream_t s) {
  hipLaunchKernelGGL(reduce_kernel, dim3(p.hkv * p.nrep, batch), dim3(128), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvq
