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
#ifndef KVQ_GROUP_WAVES
#define KVQ_GROUP_WAVES 8
#endif
#ifndef KVQ_GROUPS_PER_CU
#define KVQ_GROUPS_PER_CU 1
#endif
constexpr int kGroupWaves = KVQ_GROUP_WAVES;        // wavefronts per attention workgroup (power of 2)
constexpr int kGroupsPerCu = KVQ_GROUPS_PER_CU;     // workgroup ranges per compute unit (library split)
constexpr int kMaxBlocksPerGroup = 1 << 20;
constexpr int kMaxPagedRange = 4096;     // paged caches: blocks per workgroup range (ids staged in LDS)

// Kernel variant: the kvq_format, plus kMeta16 when an INT format stores
// fp16 (scale, offset) pairs and kRope when the Keys are stored before RoPE.
constexpr int kMeta16 = 8;
constexpr int kRope = 16;
constexpr int kOutliers = 32;
__host__ __device__ constexpr int kind_of(int variant) { return variant & 7; }
__host__ __device__ constexpr bool meta16_of(int variant) { return (variant & kMeta16) != 0; }
__host__ __device__ constexpr bool rope_of(int variant) { return (variant & kRope) != 0; }
__host__ __device__ constexpr bool outliers_of(int variant) { return (variant & kOutliers) != 0; }
__host__ __device__ constexpr bool fp8_of(int variant) {
  return kind_of(variant) == KVQ_FP8_E4M3 || kind_of(variant) == KVQ_FP8_E5M2;
}
inline int variant_of(const kvq_layout& L) {
  return L.format | (L.meta_fp16 ? kMeta16 : 0) | (L.rope_theta > 0.f ? kRope : 0) | (L.outliers ? kOutliers : 0);
}

// Stored position of channel c in a pre-RoPE Key row (pairs side by side)
// and the channel at stored position p.
__host__ __device__ constexpr int rope_stored_pos(int c) { return 2 * (c % (kHeadDim / 2)) + c / (kHeadDim / 2); }
__host__ __device__ constexpr int rope_channel(int p) { return (p >> 1) + (kHeadDim / 2) * (p & 1); }
inline int format_bits(int fmt) { return fmt == KVQ_INT4 ? 4 : (fmt == KVQ_INT2 ? 2 : 8); }

// ---------------------------------------------------------------- append
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
  int32_t* sync_zero;     // non-null on a cache's first append: [B][Hkv] counters set to 0
  int64_t n_sink_copy;    // appended tokens copied: n_sink_copy sinks from token n_old, then
  int64_t n_copy;         // n_copy - n_sink_copy residual tokens from token ring_first_t
  int64_t ring_first_t;   // (the tokens in between are quantized straight from the input)
};

struct FlushParams {
  const uint16_t* k_in;   // fp16 [B][T][Hkv][D]
  const uint16_t* v_in;
  const uint16_t* k_ring; // fp16 [B][Hkv][RS][D]
  const uint16_t* v_ring;
  uint8_t* k_codes;       // [B][Hkv][NB][32*D*b/8]
  uint8_t* v_codes;       // [B][Hkv][NB][32*D*b/8]
  float* k_meta;          // [B][Hkv][NB][D][2]       (s, z) per channel (fp16 (s, m) pairs: meta16)
  float* v_meta;          // [B][Hkv][NB][D/32][32][2] (s, z) per group and token
  uint32_t* k_out;        // outliers: [B][Hkv][NB][D] entries (index | fp16 << 16)
  uint32_t* v_out;        // outliers: [B][Hkv][NB][D/32][32] entries
  int64_t n_old;          // tokens per sequence before this append
  int32_t T;              // tokens appended
  int32_t hkv;
  int32_t sink;           // S
  int32_t ring_slots;     // R + 32
  int32_t nb_cap;         // NB
  int32_t first_block;    // n_q_old / 32
  int64_t n_body_old;     // max(0, n_old - S)
  float k_scale, v_scale; // FP8
  const int32_t* table;   // paged: block table [B][table_stride], else null
  int32_t table_stride;
  int32_t page_blocks;    // P
  int32_t num_pages;
  // Fused copy (a flush that reads no ring slot, such as a cache's first
  // append): workgroups x >= flush_x of each (KV head, sequence) copy that
  // pair's tokens of cp, 256 16-byte chunks per workgroup; copy_x of them.
  int32_t flush_x;        // blocks flushed per (sequence, KV head): the flush's workgroups in x
  int32_t copy_x;         // 0: no fused copy (copy_kernel runs after the flush)
  CopyParams cp;
};

// Record index of logical block blk of (sequence b, head h) in the code and
// meta planes: contiguous (b * Hkv + h) * NB + blk, or paged
// (page * Hkv + h) * P + blk % P with page = table[b][blk / P]; -1 when the
// page id lies outside the pool.
__host__ __device__ inline int64_t block_record(const int32_t* table, int32_t stride, int32_t page_blocks,
                                                int32_t num_pages, int32_t hkv, int32_t nb_cap, int64_t b,
                                                int64_t h, int64_t blk) {
  if (!table) return (b * hkv + h) * nb_cap + blk;
  const int32_t page = table[b * stride + blk / page_blocks];
  if (page < 0 || page >= num_pages) return -1;
  return ((int64_t)page * hkv + h) * page_blocks + blk % page_blocks;
}


hipError_t launch_flush(int variant, const FlushParams& p, int batch, hipStream_t s);
hipError_t launch_copy(const CopyParams& p, int batch, hipStream_t s);

// ------------------------------------------------------------- attention
// Work: the quantized blocks of all heads, flattened head-major (block j is
// block j mod nblk of head j / nblk), are cut into ranges, one per workgroup
// of kGroupWaves wavefronts (whole heads cut into equal parts of at most
// kGroupWaves blocks when those fit one workgroup per compute unit, else into
// equal parts when the workgroups divide among the heads evenly, else equal
// ranges across head boundaries); the wavefronts of a
// workgroup take the blocks of its range in turn.  The fp16 segment of every
// head (sinks, then residual ring) is cut into 32-token blocks, dealt round
// robin to the workgroups whose range touches the head.
// Partial results (kPartStride floats per query head, n_rep heads per slot):
//   part_fp16   slot bh * fp16_blocks + fb       fp16 block fb of head bh
//   part_wave   slot kGroupWaves * (g + bh) + w   wavefront w of workgroup g, head bh
//   part_group  slot g + bh                      workgroup g, head bh (its wavefronts merged)
// Workgroup g's range [start(g), start(g + 1)) (start: range_start in
// kvq_attn.hip, increasing in g) touches heads floor(start(g) / nblk) ..
// floor((start(g + 1) - 1) / nblk), so g + bh never collides between
// workgroups.  Each workgroup folds its
// wavefront partials and the fp16 slots it produced per head.  A head the
// workgroup covers alone is written to the output.  A head shared with other
// workgroups is counted on its sync counter: arrivals in the low 16 bits,
// "slot written" marks in bit 16 and up.  The workgroup whose arrival
// completes the count combines the head (its own merged partial from LDS,
// the others' part_group slots once all their marks are in) and sets the
// counter back to 0; every other covering workgroup writes its part_group
// slot and then adds its mark.
// With no quantized block (nblk == 0) workgroup g takes the fp16 blocks of head g.
struct AttnParams {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const float* k_meta;
  const float* v_meta;
  const uint32_t* k_out;  // outliers (see FlushParams)
  const uint32_t* v_out;
  const uint16_t* k_ring;
  const uint16_t* v_ring;
  const uint16_t* k_sink;
  const uint16_t* v_sink;
  const uint16_t* q;      // fp16 [B][Hq][D]
  uint16_t* out;          // fp16 [B][Hq][D]
  int32_t* sync;          // [B][Hkv] counters of shared heads (0 between calls)
  const uint16_t* new_k;  // fused append: fp16 [B][1][Hkv][D] of the newest token, else null;
  const uint16_t* new_v;  // it is read from here and copied to its ring slot
  float* part_fp16;
  float* part_wave;
  float* part_group;
  int32_t hkv;
  int32_t nrep;           // NR = Hq / Hkv (1, 2, 4 or 8)
  int32_t nb_cap;         // NB (block stride of the code / meta planes)
  int32_t nblk;           // quantized blocks currently held per head (n_q / 32)
  uint32_t nblk_magic;    // j / nblk == (j * nblk_magic) >> nblk_shift for 0 <= j < 2^31
  int32_t nblk_shift;
  uint32_t half_magic;    // the same for the divisor ceil(nblk / 2)
  int32_t half_shift;
  int32_t ring_slots;
  int32_t sink_cap;       // S of the layout (row stride of the sink planes)
  int32_t n_sink;         // sink tokens held
  int32_t n_res;          // residual tokens held
  int32_t ring_first;     // ring slot of the oldest residual token (n_q mod RS)
  int32_t bh_count;       // B * Hkv
  int32_t range_len;      // L: blocks per stretch (nblk: ranges follow heads; 2 R: equal ranges of R)
  int32_t range_parts;    // k: workgroup ranges per stretch (k L < 2^31)
  int32_t group_skew;     // d: odd parts start d blocks later (0 <= d < floor(L / k))
  uint32_t len_magic;     // x / L == (x * len_magic) >> len_shift for 0 <= x < 2^31
  int32_t len_shift;
  uint32_t parts_magic;   // the same for the divisor k
  int32_t parts_shift;
  int32_t groups;         // workgroups in the grid
  int32_t fp16_blocks;    // ceil((n_sink + n_res) / 32) per head
  int32_t deterministic;  // 1: wavefront w takes blocks w, w + 8, ... of its range
  float k_scale, v_scale; // FP8
  float rope_theta;       // pre-RoPE Keys: the RoPE base
  const int32_t* table;   // paged: block table [B][table_stride] (record ids via block_record)
  int32_t table_stride;
  int32_t page_blocks;
  int32_t num_pages;
};

hipError_t launch_attention(int variant, const AttnParams& p, hipStream_t s);

// Library-owned workspace of kv_decode_attention_noalloc: a file-scope device
// array of kScratchBytes in kvq_attn.hip, one copy per GPU for the life of
// the process.  attention_scratch returns the current device's copy (its
// address is looked up once per device, with that device current).
constexpr uint64_t kScratchBytes = 32ull << 20;
hipError_t attention_scratch(void** ptr);

// ------------------------------------------------------------- read probe
constexpr int kProbeThreads = 512;        // threads per workgroup, as the attention kernel
hipError_t launch_read_probe(const void* buf, uint64_t units, uint32_t* sink, int groups, hipStream_t s);
// units workgroups; read16 / write16: 16-byte words read / written per unit
hipError_t launch_rw_probe(const void* src, void* dst, uint64_t units, int read16, int write16, hipStream_t s);

}  // namespace kvq
