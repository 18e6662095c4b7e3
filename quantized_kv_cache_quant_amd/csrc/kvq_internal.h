// Internal interface between the host library (kvq_host.cpp) and the HIP
// kernels (kvq_append.hip, kvq_attn.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

constexpr int kBlock = 32;        // tokens per quantized block (= Key group)
constexpr int kHeadDim = 128;     // the only head_dim of this version
constexpr int kVGroup = 32;       // channels per Value group
constexpr int kVGroups = kHeadDim / kVGroup;
constexpr int kPartStride = 132;  // floats per partial: m, l, 2 pad, o[128]
constexpr int kMaxBlocksPerWave = 1024;
constexpr int kFp16BlocksPerWave = 2;

inline int format_bits(int fmt) { return fmt == KVQ_INT4 ? 4 : (fmt == KVQ_INT2 ? 2 : 8); }

// ---------------------------------------------------------------- append
struct FlushParams {
  const uint16_t* k_in;   // fp16 [B][T][Hkv][D]
  const uint16_t* v_in;
  const uint16_t* k_ring; // fp16 [B][Hkv][RS][D]
  const uint16_t* v_ring;
  uint8_t* k_codes;       // [B][Hkv][NB*32][D*b/8]
  uint8_t* v_codes;       // [B][Hkv][NB][32*D*b/8]
  float* k_meta;          // [B][Hkv][NB][D][2]       (s, z) per channel
  float* v_meta;          // [B][Hkv][NB][D/32][32][2] (s, z) per group and token
  int64_t n_old;          // tokens per sequence before this append
  int32_t T;              // tokens appended
  int32_t hkv;
  int32_t sink;           // S
  int32_t ring_slots;     // R + 32
  int32_t nb_cap;         // NB
  int32_t first_block;    // n_q_old / 32
  int64_t n_body_old;     // max(0, n_old - S)
  float k_scale, v_scale; // FP8
};

struct CopyParams {
  const uint16_t* k_in;
  const uint16_t* v_in;
  uint16_t* k_ring;
  uint16_t* v_ring;
  uint16_t* k_sink;
  uint16_t* v_sink;
  int64_t n_old;
  int64_t n_q_new;        // quantized body tokens after the append
  int32_t T, hkv, sink, ring_slots;
};

hipError_t launch_flush(int fmt, const FlushParams& p, int n_blocks, int batch, hipStream_t s);
hipError_t launch_copy(const CopyParams& p, int batch, hipStream_t s);

// ------------------------------------------------------------- attention
// Partial results: kPartStride floats per query head, n_rep heads per slot.
//   fp16 region  slot bh * fp16_waves_per_head + f   (f-th fp16 wavefront of head bh)
//   body region  slot fp16_slots + w + bh            (body wavefront w's share of head bh)
// A body wavefront w streams the flattened quantized blocks [w*L, (w+1)*L) of
// all heads (head-major), so head bh is covered by the wavefronts
// floor(bh*nblk/L) .. floor(((bh+1)*nblk - 1)/L) and w + bh never collides.
struct AttnParams {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const float* k_meta;
  const float* v_meta;
  const uint16_t* k_ring;
  const uint16_t* v_ring;
  const uint16_t* k_sink;
  const uint16_t* v_sink;
  const uint16_t* q;      // fp16 [B][Hq][D]
  float* part;            // partial slots (see above)
  int32_t hkv;
  int32_t nrep;           // NR = Hq / Hkv (1, 2, 4 or 8)
  int32_t nb_cap;         // NB (block stride of the code / meta planes)
  int32_t nblk;           // quantized blocks currently held per head (n_q / 32)
  int32_t ring_slots;
  int32_t sink_cap;       // S of the layout (row stride of the sink planes)
  int32_t n_sink;         // sink tokens held
  int32_t n_res;          // residual tokens held
  int32_t ring_first;     // ring slot of the oldest residual token (n_q mod RS)
  int32_t bh_count;       // B * Hkv
  int32_t body_per_wave;  // L: quantized blocks per body wavefront
  int32_t body_waves;     // ceil(bh_count * nblk / L)
  int32_t fp16_blocks;    // ceil((n_sink + n_res) / 32) per head
  int32_t fp16_per_wave;  // fp16 blocks per fp16 wavefront
  int32_t fp16_waves_per_head;
  float k_scale, v_scale; // FP8
};

struct ReduceParams {
  const float* part;
  uint16_t* out;          // fp16 [B][Hq][D]
  int32_t hkv, nrep, nblk, body_per_wave, fp16_waves_per_head, bh_count;
};

hipError_t launch_attention(int fmt, const AttnParams& p, int64_t waves, hipStream_t s);
hipError_t launch_reduce(const ReduceParams& p, int batch, hipStream_t s);
// Attention workgroups (one wavefront each) a compute unit holds at once.
int attention_waves_per_cu(int fmt);

}  // namespace kvq
