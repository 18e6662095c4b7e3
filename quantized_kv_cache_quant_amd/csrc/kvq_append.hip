// Quantize-on-append kernels for gfx950.
//
// "KV Cache Quantization Analysis", sec. 5 (system integration): the new
// token's K and V are quantized right after they are computed and stored in
// the cache.  Sec. 3 / sec. 4 (KIVI): Keys per channel, Values per token,
// the most recent tokens kept in full precision.  Sec. 2: affine
// quantization q = round(x / s + z), x_hat = s * (q - z).  Sec. 4 (FP8 /
// INT8): OCP E4M3 or E5M2 with an fp32 scale.  With fp16 metadata a group
// stores an fp16 scale (rounded up) and its minimum m as an fp16 offset:
// q = round((x - m) / s), x_hat = s * q + m.
//
// Two kernels, enqueued in this order on one stream:
//  flush_kernel  one workgroup per (32-token block leaving the residual
//                window, KV head, sequence): gathers the block's fp16 K / V
//                from the ring or the new input, computes the per-channel K
//                and per-token V scale / zero-point, encodes and writes the
//                packed codes in the documented plane layouts.
//  copy_kernel   copies new sink tokens and new residual tokens into their
//                fp16 planes (ring slot u mod (R + 32)).  It runs after the
//                flush because it may overwrite ring slots the flush read.
//                On a cache's first append it also zeroes the attention
//                arrival counters.
// A flush that reads no ring slot (no body token was in the ring before the
// append, as on a cache's first append) does the copy itself, in extra
// workgroups of its launch, and copy_kernel is not launched.
//
// Bit-exactness: every quantization step is one correctly rounded IEEE fp32
// operation in the order of the formula, exactly like the CPU oracle: the
// division x / s by the exact reciprocal-and-remainder sequence of div_rn
// (FP8: div_rn_any while the per-tensor scale lies in [2^-60, 2^60], true
// division outside), no contraction (this file is built with
// -ffp-contract=off and correctly rounded fp32 division), rint
// round-half-even.
#include "kvq_internal.h"

#pragma clang fp contract(off)

namespace kvq {
namespace {

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// The correctly rounded quotient x / s from y = RN(1 / s) (one correctly
// rounded division per group): q = RN(x y) lies within one ulp of x / s,
// r = RN(x - q s) is one fused multiply-add, and RN(q + r y), another, is
// RN(x / s) (Markstein's theorem on division by a correctly rounded
// reciprocal; it holds without overflow or underflow, which is the case
// here: x is an fp16 value or the difference of two, and s a group scale of
// fp16 data, so |x / s| stays below 2^49 and above 2^-41 or is 0).
__device__ __forceinline__ float div_rn(float x, float s, float y) {
  const float q = x * y;
  const float r = __builtin_fmaf(-q, s, x);
  return __builtin_fmaf(r, y, q);
}

// Integer code of x in a group with scale s (reciprocal y = RN(1 / s)) and
// zero-point z (fp32 pairs: rint(x / s + z)) or, with fp16 metadata
// (OFFSET), offset z = m: rint((x - m) / s).  Each step is one correctly
// rounded fp32 operation, clamped to the code range.
template <int BITS, bool OFFSET>
__device__ __forceinline__ uint32_t encode_int(float x, float s, float z, float y) {
  constexpr float kQmax = (float)((1 << BITS) - 1);
  float v;
  if constexpr (OFFSET) {
    v = x - z;
    v = div_rn(v, s, y);
  } else {
    v = div_rn(x, s, y);
    v = v + z;
  }
  v = __builtin_rintf(v);
  v = fminf(fmaxf(v, 0.0f), kQmax);
  return (uint32_t)v;
}

// div_rn for every fp16 dividend, signed zeros and infinities included (an
// FP8 code keeps the sign of zero): a zero remainder means q * s = x exactly,
// so q (with its sign) is the quotient; a NaN remainder comes from x = +-inf,
// where q = x * y is already +-inf
__device__ __forceinline__ float div_rn_any(float x, float s, float y) {
  const float q = x * y;
  const float r = __builtin_fmaf(-q, s, x);
  return fabsf(r) > 0.0f ? __builtin_fmaf(r, y, q) : q;
}

// Smallest fp16 >= x, for finite 0 <= x <= 65504 (bit pattern; -0 gives -0).
__device__ __forceinline__ uint32_t f16_round_up(float x) {
  const _Float16 h = (_Float16)x;                  // round to nearest even
  uint32_t b = __builtin_bit_cast(uint16_t, h);
  if ((float)h < x) b += 1;                        // the next fp16 up (x > 0)
  return b;
}

// Two fp32 values -> two OCP FP8 bytes (low 16 bits of the result) after the
// explicit clamp to the format's largest finite value; the hardware
// conversion rounds to nearest even.  E4M3: +-448; E5M2: +-57344.
template <bool E5M2>
__device__ __forceinline__ uint32_t encode_fp8_pair(float a, float b, float s, float y, bool fast) {
  constexpr float kMax = E5M2 ? 57344.0f : 448.0f;
  float va = fminf(fmaxf(fast ? div_rn_any(a, s, y) : a / s, -kMax), kMax);
  float vb = fminf(fmaxf(fast ? div_rn_any(b, s, y) : b / s, -kMax), kMax);
  if constexpr (E5M2) return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(va, vb, 0, false) & 0xFFFFu;
  else return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(va, vb, 0, false) & 0xFFFFu;
}

// Token index (0..31 inside a block) of slot j (0..7) of V record quarter qd.
__device__ __forceinline__ int record_token(int qd, int j) {
  return (j < 4) ? (4 * qd + j) : (16 + 4 * qd + (j - 4));
}

// 16-byte chunk `chunk` of copied token k (sinks first, then residual
// tokens) of K (kv = 0) or V (kv = 1) of (sequence b, KV head h): from the
// input to the sink plane or to the token's ring slot u mod (R + 32).
__device__ __forceinline__ void copy_chunk(const CopyParams& p, int b, int h, int64_t k, int kv, int chunk) {
  const int64_t t = k < p.n_sink_copy ? p.n_old + k : p.ring_first_t + (k - p.n_sink_copy);   // absolute
  const int64_t i = t - p.n_old;                   // input token
  uint16_t* dst;
  if (t < p.sink) {
    uint16_t* plane = kv ? p.v_sink : p.k_sink;
    dst = plane + (((int64_t)b * p.hkv + h) * p.sink + t) * kHeadDim + chunk * 8;
  } else {
    const int64_t u = t - p.sink;                  // u >= n_q_new: a residual token
    uint16_t* plane = kv ? p.v_ring : p.k_ring;
    dst = plane + (((int64_t)b * p.hkv + h) * p.ring_slots + (u % p.ring_slots)) * kHeadDim + chunk * 8;
  }
  const uint16_t* src = (kv ? p.v_in : p.k_in) + (((int64_t)b * p.T + i) * p.hkv + h) * kHeadDim + chunk * 8;
  *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}

template <int VAR>
__global__ __launch_bounds__(256) void flush_kernel(FlushParams p) {
  constexpr int kKind = kind_of(VAR);
  constexpr bool kFp8 = fp8_of(VAR);
  constexpr bool kE5M2 = kKind == KVQ_FP8_E5M2;
  constexpr bool kM16 = meta16_of(VAR);
  constexpr bool kRopeK = rope_of(VAR);     // K rows in RoPE pair order
  constexpr bool kOut = outliers_of(VAR);   // one exact outlier per group
  constexpr int kBits = kKind == KVQ_INT4 ? 4 : (kKind == KVQ_INT2 ? 2 : 8);
  constexpr int kRowBytes = kHeadDim * kBits / 8;   // packed bytes per token
  constexpr float kQmax = (float)((1 << kBits) - 1);

  // the block's K and V as their fp16 bits (exact; widened to fp32 where
  // read): rows of kRowH halves, 16-byte aligned for the gather's stores
  constexpr int kRowH = kHeadDim + 8;
  __shared__ __attribute__((aligned(16))) uint16_t ksh[kBlock][kRowH];
  __shared__ __attribute__((aligned(16))) uint16_t vsh[kBlock][kRowH];
  auto ks_at = [&](int t, int c) { return half_bits_to_float(ksh[t][c]); };
  auto vs_at = [&](int t, int c) { return half_bits_to_float(vsh[t][c]); };
  __shared__ float sk[kHeadDim], zk[kHeadDim], rk[kHeadDim];            // rk = RN(1 / sk)
  __shared__ float sv[kBlock][kVGroups], zv[kBlock][kVGroups], rv[kBlock][kVGroups];
  __shared__ int ko[kHeadDim];               // outliers: token of each channel's outlier
  __shared__ int vo[kBlock][kVGroups];       // outliers: channel (in group) of each token's outlier

  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  if ((int)blockIdx.x >= p.flush_x) {               // fused copy: chunks of (b, h) in this workgroup's 256
    const int64_t xc = (int64_t)blockIdx.x - p.flush_x;
    if (xc == 0 && h == 0 && p.cp.sync_zero)
      for (int e = tid; e < p.hkv; e += 256) p.cp.sync_zero[(int64_t)b * p.hkv + e] = 0;
    const int64_t e = xc * 256 + tid;
    if (e < p.cp.n_copy * 32) copy_chunk(p.cp, b, h, e >> 5, (int)((e >> 4) & 1), (int)(e & 15));
    return;                                         // uniform over the workgroup, before any barrier
  }
  const int64_t blk = (int64_t)p.first_block + blockIdx.x;
  const int64_t bh = (int64_t)b * p.hkv + h;
  // record of this block in the code / meta planes (paged: through the block
  // table); a page id outside the pool leaves the block unwritten
  const int64_t rec = block_record(p.table, p.table_stride, p.page_blocks, p.num_pages, p.hkv, p.nb_cap, b, h, blk);
  if (rec < 0) return;                                // uniform over the workgroup, before any barrier
  // FP8: x / s by div_rn from y = RN(1 / s) when s lies in [2^-60, 2^60] (no
  // overflow or underflow for fp16 x), else by true division
  const float ky = 1.0f / p.k_scale, vy = 1.0f / p.v_scale;
  const bool kfast = p.k_scale >= 0x1p-60f && p.k_scale <= 0x1p60f;
  const bool vfast = p.v_scale >= 0x1p-60f && p.v_scale <= 0x1p60f;

  // 1) gather the block's 32 tokens: 512 16-byte chunks per tensor, two of K
  //    and two of V per thread, all four loads issued before the LDS stores
  //    (a workgroup per block: the hardware's dispatch keeps eight resident
  //    per compute unit; a persistent loop prefetching the next block into
  //    registers measured slower).
  //    Ring slot of body index u: (u0 + t) mod (R + 32) with u0 the block's
  //    first index reduced once (t < 32 <= R + 32: one subtraction).
  {
    int64_t ring0 = 0;
    if (blk * kBlock < p.n_body_old) ring0 = (blk * kBlock) % p.ring_slots;
    uint4 kc[2], vc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid + 256 * i;
      const int t = e >> 4;
      const int c8 = (e & 15) * 8;
      const int64_t u = blk * kBlock + t;             // body index
      const uint16_t* ksrc;
      const uint16_t* vsrc;
      if (u < p.n_body_old) {                         // still in the residual ring
        int64_t slot = ring0 + t;
        if (slot >= p.ring_slots) slot -= p.ring_slots;
        const int64_t off = (bh * p.ring_slots + slot) * kHeadDim + c8;
        ksrc = p.k_ring + off;
        vsrc = p.v_ring + off;
      } else {                                        // arrives with this append
        const int64_t i_in = u + p.sink - p.n_old;
        const int64_t off = (((int64_t)b * p.T + i_in) * p.hkv + h) * kHeadDim + c8;
        ksrc = p.k_in + off;
        vsrc = p.v_in + off;
      }
      kc[i] = *reinterpret_cast<const uint4*>(ksrc);
      vc[i] = *reinterpret_cast<const uint4*>(vsrc);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid + 256 * i;
      const int t = e >> 4;
      const int c8 = (e & 15) * 8;
      *reinterpret_cast<uint4*>(&ksh[t][c8]) = kc[i];
      *reinterpret_cast<uint4*>(&vsh[t][c8]) = vc[i];
    }
  }
  __syncthreads();

  // 2) scale / zero-point: K per channel over the 32 tokens, V per token
  //    over each group of 32 channels
  if constexpr (!kFp8) {
    if (tid < kHeadDim) {
      const int c = tid;
      float mn, mx;
      if constexpr (kOut) {
        // the outlier: largest magnitude, lowest token index on ties; the
        // range comes from the other 31 values
        int oi = 0;
        float oa = fabsf(ks_at(0, c));
        for (int t = 1; t < kBlock; ++t)
          if (fabsf(ks_at(t, c)) > oa) { oa = fabsf(ks_at(t, c)); oi = t; }
        const int first = oi == 0 ? 1 : 0;
        mn = ks_at(first, c);
        mx = mn;
        for (int t = 0; t < kBlock; ++t) {
          if (t == oi) continue;
          mn = fminf(mn, ks_at(t, c));
          mx = fmaxf(mx, ks_at(t, c));
        }
        ko[c] = oi;
        const uint32_t xb = __builtin_bit_cast(uint16_t, (_Float16)ks_at(oi, c));   // exact: an fp16 input
        p.k_out[rec * kHeadDim + (kRopeK ? rope_stored_pos(c) : c)] = (uint32_t)oi | (xb << 16);
      } else {
        mn = ks_at(0, c);
        mx = ks_at(0, c);
        for (int t = 1; t < kBlock; ++t) {
          mn = fminf(mn, ks_at(t, c));
          mx = fmaxf(mx, ks_at(t, c));
        }
      }
      mn = mn + 0.0f;                                 // a zero minimum is +0
      if constexpr (kM16) {                           // fp16 (s rounded up, m = min)
        uint32_t sb = f16_round_up((mx - mn) / kQmax);
        if ((sb & 0x7FFFu) == 0) sb = 0x3C00u;        // constant group (range +-0): s = 1
        const uint32_t mb = __builtin_bit_cast(uint16_t, (_Float16)mn);   // exact
        sk[c] = half_bits_to_float(sb);
        zk[c] = mn;
        rk[c] = 1.0f / sk[c];
        const int sp = kRopeK ? rope_stored_pos(c) : c;   // stored position of channel c
        reinterpret_cast<uint32_t*>(p.k_meta)[rec * kHeadDim + sp] = sb | (mb << 16);
      } else {
        float s = (mx - mn) / kQmax;
        if (s == 0.0f) s = 1.0f;
        const float z = (-mn) / s;
        sk[c] = s;
        zk[c] = z;
        rk[c] = 1.0f / s;
        float* km = p.k_meta + rec * (2 * kHeadDim);   // [stored position][s, z]
        const int sp = kRopeK ? rope_stored_pos(c) : c;
        *reinterpret_cast<float2*>(km + 2 * sp) = make_float2(s, z);
      }
    } else {
      const int e = tid - kHeadDim;
      const int t = e >> 2, g = e & 3;
      float mn, mx;
      if constexpr (kOut) {
        int oi = 0;
        float oa = fabsf(vs_at(t, kVGroup * g));
        for (int c = 1; c < kVGroup; ++c)
          if (fabsf(vs_at(t, kVGroup * g + c)) > oa) { oa = fabsf(vs_at(t, kVGroup * g + c)); oi = c; }
        const int first = oi == 0 ? 1 : 0;
        mn = vs_at(t, kVGroup * g + first);
        mx = mn;
        for (int c = 0; c < kVGroup; ++c) {
          if (c == oi) continue;
          mn = fminf(mn, vs_at(t, kVGroup * g + c));
          mx = fmaxf(mx, vs_at(t, kVGroup * g + c));
        }
        vo[t][g] = oi;
        const uint32_t xb = __builtin_bit_cast(uint16_t, (_Float16)vs_at(t, kVGroup * g + oi));
        p.v_out[rec * (kVGroups * kBlock) + g * kBlock + t] = (uint32_t)oi | (xb << 16);
      } else {
        mn = vs_at(t, kVGroup * g);
        mx = mn;
        for (int c = 1; c < kVGroup; ++c) {
          mn = fminf(mn, vs_at(t, kVGroup * g + c));
          mx = fmaxf(mx, vs_at(t, kVGroup * g + c));
        }
      }
      mn = mn + 0.0f;
      if constexpr (kM16) {
        uint32_t sb = f16_round_up((mx - mn) / kQmax);
        if ((sb & 0x7FFFu) == 0) sb = 0x3C00u;
        const uint32_t mb = __builtin_bit_cast(uint16_t, (_Float16)mn);
        sv[t][g] = half_bits_to_float(sb);
        zv[t][g] = mn;
        rv[t][g] = 1.0f / sv[t][g];
        reinterpret_cast<uint32_t*>(p.v_meta)[rec * (kVGroups * kBlock) + g * kBlock + t] =
            sb | (mb << 16);
      } else {
        float s = (mx - mn) / kQmax;
        if (s == 0.0f) s = 1.0f;
        const float z = (-mn) / s;
        sv[t][g] = s;
        zv[t][g] = z;
        rv[t][g] = 1.0f / s;
        float* vm = p.v_meta + rec * (2 * kVGroups * kBlock);  // [group][token][s, z]
        *reinterpret_cast<float2*>(vm + 2 * (g * kBlock + t)) = make_float2(s, z);
      }
    }
    __syncthreads();
  }

  // 3) K codes, stored position p at bit (p * bits) of its token's codes (LSB
  //    first); position p holds channel p, or in RoPE pair order channel
  //    (p >> 1) + 64 (p & 1).
  //    INT4 / INT2: token-major rows.  8-bit codes: 16-byte units ordered
  //    (tile, half, lane); unit (tile, half, 16 qd + r) holds channels
  //    32 qd + 16 half .. + 15 of token 16 tile + r.
  {
    constexpr int kWordsPerRow = kRowBytes / 4;
    uint32_t* dst = reinterpret_cast<uint32_t*>(p.k_codes + rec * kBlock * kRowBytes);
    for (int w = tid; w < kBlock * kWordsPerRow; w += 256) {
      int t, wi;
      if constexpr (kBits == 8) {
        const int u = w >> 2;                       // 16-byte unit
        const int lane = u & 63, half = (u >> 6) & 1, tile = u >> 7;
        t = 16 * tile + (lane & 15);
        wi = 8 * (lane >> 4) + 4 * half + (w & 3);
      } else {
        t = w / kWordsPerRow;
        wi = w % kWordsPerRow;
      }
      uint32_t word = 0;
      // channel held by stored position sp of the row
      auto chan = [](int sp) { return kRopeK ? rope_channel(sp) : sp; };
      if constexpr (kFp8) {
        const int c = wi * 4;
        word = encode_fp8_pair<kE5M2>(ks_at(t, chan(c)), ks_at(t, chan(c + 1)), p.k_scale, ky, kfast) |
               (encode_fp8_pair<kE5M2>(ks_at(t, chan(c + 2)), ks_at(t, chan(c + 3)), p.k_scale, ky, kfast) << 16);
      } else {
        constexpr int kPer = 32 / kBits;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const int c = chan(wi * kPer + j);
          uint32_t code = encode_int<kBits, kM16>(ks_at(t, c), sk[c], zk[c], rk[c]);
          if constexpr (kOut) code = ko[c] == t ? 0u : code;            // the outlier's code is 0
          word |= code << (j * kBits);
        }
      }
      dst[w] = word;
    }
  }

  // 4) V codes: 64 records per block in the attention kernel's operand
  //    order, stored as 16-byte groups: group i of record l at 16 (64 i + l)
  {
    constexpr int kRecWords = kHeadDim * kBits / 16 / 4;   // words per record
    uint32_t* dst = reinterpret_cast<uint32_t*>(p.v_codes + rec * kBlock * kRowBytes);
    for (int w = tid; w < 64 * kRecWords; w += 256) {
      const int lane = (w >> 2) & 63;
      const int wi = 4 * (w >> 8) + (w & 3);
      const int qd = lane >> 4, r = lane & 15;
      uint32_t word = 0;
      // code of (token t, channel ch) in group g; an outlier's code is 0
      auto oz = [&](uint32_t code, int t, int ch, int g) {
        return (kOut && vo[t][g] == (ch & (kVGroup - 1))) ? 0u : code;
      };
      if constexpr (kBits == 4) {                 // word m: nibble j = T[j], channel 16m + r
        const int ch = 16 * wi + r;
        const int g = ch / kVGroup;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int t = record_token(qd, j);
          word |= oz(encode_int<4, kM16>(vs_at(t, ch), sv[t][g], zv[t][g], rv[t][g]), t, ch, g) << (4 * j);
        }
      } else if constexpr (kBits == 8) {          // bytes 8m..8m+7 = T0 T4 T1 T5 T2 T6 T3 T7
        const int ch = 16 * (wi >> 1) + r;
        const int g = ch / kVGroup;
        // slot k of the 8 bytes holds record token (k >> 1) + 4 * (k & 1)
        const int base = 4 * (wi & 1);
        auto sel = [](int k) { return (k >> 1) + 4 * (k & 1); };
        if constexpr (kFp8) {
          const float x0 = vs_at(record_token(qd, sel(base + 0)), ch);
          const float x1 = vs_at(record_token(qd, sel(base + 1)), ch);
          const float x2 = vs_at(record_token(qd, sel(base + 2)), ch);
          const float x3 = vs_at(record_token(qd, sel(base + 3)), ch);
          word = encode_fp8_pair<kE5M2>(x0, x1, p.v_scale, vy, vfast) | (encode_fp8_pair<kE5M2>(x2, x3, p.v_scale, vy, vfast) << 16);
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int t = record_token(qd, sel(base + k));
            word |= oz(encode_int<8, kM16>(vs_at(t, ch), sv[t][g], zv[t][g], rv[t][g]), t, ch, g) << (8 * k);
          }
        }
      } else {                                    // INT2 word p: A = 32p + r, B = 32p + 16 + r
        const int cha = 32 * wi + r, chb = cha + 16;
        const int ga = cha / kVGroup, gb = chb / kVGroup;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t0 = record_token(qd, j), t1 = record_token(qd, 4 + j);
          word |= oz(encode_int<2, kM16>(vs_at(t0, cha), sv[t0][ga], zv[t0][ga], rv[t0][ga]), t0, cha, ga) << (2 * j);
          word |= oz(encode_int<2, kM16>(vs_at(t0, chb), sv[t0][gb], zv[t0][gb], rv[t0][gb]), t0, chb, gb) << (8 + 2 * j);
          word |= oz(encode_int<2, kM16>(vs_at(t1, cha), sv[t1][ga], zv[t1][ga], rv[t1][ga]), t1, cha, ga) << (16 + 2 * j);
          word |= oz(encode_int<2, kM16>(vs_at(t1, chb), sv[t1][gb], zv[t1][gb], rv[t1][gb]), t1, chb, gb) << (24 + 2 * j);
        }
      }
      dst[w] = word;
    }
  }
}

// One thread per 16-byte chunk of one token row of K or V, over the tokens
// that are copied (sinks, then residual tokens; a long prefill quantizes the
// others straight from the input and launches no thread for them).
__global__ __launch_bounds__(256) void copy_kernel(CopyParams p) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  if (p.sync_zero && e < p.hkv) p.sync_zero[(int64_t)b * p.hkv + e] = 0;
  const int64_t total = p.n_copy * p.hkv * 2 * 16;
  if (e >= total) return;
  const int chunk = (int)(e & 15);
  int64_t rest = e >> 4;
  const int kv = (int)(rest & 1);
  rest >>= 1;
  const int h = (int)(rest % p.hkv);
  copy_chunk(p, b, h, rest / p.hkv, kv, chunk);
}

}  // namespace

hipError_t launch_flush(int variant, const FlushParams& p, int batch, hipStream_t s) {
  if (p.flush_x <= 0 || p.copy_x < 0 || (int64_t)p.flush_x + p.copy_x > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(p.flush_x + p.copy_x), p.hkv, batch), block(256);
  switch (variant) {
    case KVQ_INT8: hipLaunchKernelGGL(flush_kernel<KVQ_INT8>, grid, block, 0, s, p); break;
    case KVQ_INT4: hipLaunchKernelGGL(flush_kernel<KVQ_INT4>, grid, block, 0, s, p); break;
    case KVQ_INT2: hipLaunchKernelGGL(flush_kernel<KVQ_INT2>, grid, block, 0, s, p); break;
    case KVQ_FP8_E4M3: hipLaunchKernelGGL(flush_kernel<KVQ_FP8_E4M3>, grid, block, 0, s, p); break;
    case KVQ_FP8_E5M2: hipLaunchKernelGGL(flush_kernel<KVQ_FP8_E5M2>, grid, block, 0, s, p); break;
    case KVQ_INT8 | kMeta16: hipLaunchKernelGGL(flush_kernel<KVQ_INT8 | kMeta16>, grid, block, 0, s, p); break;
    case KVQ_INT4 | kMeta16: hipLaunchKernelGGL(flush_kernel<KVQ_INT4 | kMeta16>, grid, block, 0, s, p); break;
    case KVQ_INT2 | kMeta16: hipLaunchKernelGGL(flush_kernel<KVQ_INT2 | kMeta16>, grid, block, 0, s, p); break;
    case KVQ_INT8 | kRope: hipLaunchKernelGGL(flush_kernel<KVQ_INT8 | kRope>, grid, block, 0, s, p); break;
    case KVQ_INT4 | kRope: hipLaunchKernelGGL(flush_kernel<KVQ_INT4 | kRope>, grid, block, 0, s, p); break;
    case KVQ_INT2 | kRope: hipLaunchKernelGGL(flush_kernel<KVQ_INT2 | kRope>, grid, block, 0, s, p); break;
    case KVQ_FP8_E4M3 | kRope: hipLaunchKernelGGL(flush_kernel<KVQ_FP8_E4M3 | kRope>, grid, block, 0, s, p); break;
    case KVQ_FP8_E5M2 | kRope: hipLaunchKernelGGL(flush_kernel<KVQ_FP8_E5M2 | kRope>, grid, block, 0, s, p); break;
    case KVQ_INT8 | kOutliers: hipLaunchKernelGGL(flush_kernel<KVQ_INT8 | kOutliers>, grid, block, 0, s, p); break;
    case KVQ_INT4 | kOutliers: hipLaunchKernelGGL(flush_kernel<KVQ_INT4 | kOutliers>, grid, block, 0, s, p); break;
    case KVQ_INT2 | kOutliers: hipLaunchKernelGGL(flush_kernel<KVQ_INT2 | kOutliers>, grid, block, 0, s, p); break;
    case KVQ_INT8 | kMeta16 | kOutliers:
      hipLaunchKernelGGL(flush_kernel<KVQ_INT8 | kMeta16 | kOutliers>, grid, block, 0, s, p); break;
    case KVQ_INT4 | kMeta16 | kOutliers:
      hipLaunchKernelGGL(flush_kernel<KVQ_INT4 | kMeta16 | kOutliers>, grid, block, 0, s, p); break;
    case KVQ_INT2 | kMeta16 | kOutliers:
      hipLaunchKernelGGL(flush_kernel<KVQ_INT2 | kMeta16 | kOutliers>, grid, block, 0, s, p); break;
    case KVQ_INT8 | kMeta16 | kRope:
      hipLaunchKernelGGL(flush_kernel<KVQ_INT8 | kMeta16 | kRope>, grid, block, 0, s, p); break;
    case KVQ_INT4 | kMeta16 | kRope:
      hipLaunchKernelGGL(flush_kernel<KVQ_INT4 | kMeta16 | kRope>, grid, block, 0, s, p); break;
    case KVQ_INT2 | kMeta16 | kRope:
      hipLaunchKernelGGL(flush_kernel<KVQ_INT2 | kMeta16 | kRope>, grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_copy(const CopyParams& p, int batch, hipStream_t s) {
  const int64_t total = p.n_copy * p.hkv * 2 * 16;
  int64_t blocks = (total + 255) / 256;
  if (p.sync_zero) blocks = blocks > (p.hkv + 255) / 256 ? blocks : (p.hkv + 255) / 256;   // zeroing threads
  if (blocks == 0) return hipSuccess;              // nothing to copy
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks, batch), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvq
