// Host side of the C ABI in include/kvq.h: layout validation, byte sizing,
// plane placement, token routing and launch configuration.  Nothing here
// touches device memory; kernels are enqueued on the caller's stream.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>

#include "kvq_internal.h"

using namespace kvq;

namespace {

constexpr uint64_t kPlaneAlign = 256;

uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Window {
  int64_t n_sink, n_q, r;
};

// Routing after n tokens: S sinks, n_q quantized body tokens (a multiple of
// 32, leaving at least R body tokens in fp16), r residual tokens.
Window window(const kvq_layout& L, int64_t n) {
  Window w;
  w.n_sink = n < L.sink_tokens ? n : L.sink_tokens;
  int64_t body = n - w.n_sink;
  int64_t over = body - L.residual_tokens;
  w.n_q = over > 0 ? (over / kBlock) * kBlock : 0;
  w.r = body - w.n_q;
  return w;
}

int32_t nb_cap(const kvq_layout& L) {
  int64_t over = (int64_t)L.max_tokens - L.sink_tokens - L.residual_tokens;
  return over > 0 ? (int32_t)(over / kBlock) : 0;
}

// Plane sizes in bytes for a validated layout.
void plane_sizes(const kvq_layout& L, uint64_t sz[KVQ_NUM_PLANES]) {
  const uint64_t bh = (uint64_t)L.batch * L.num_kv_heads;
  // block records of the quantized planes: [B][Hkv][NB], or the page pool
  const uint64_t recs = L.page_blocks > 0 ? (uint64_t)L.num_pages * L.num_kv_heads * L.page_blocks
                                          : bh * (uint64_t)nb_cap(L);
  const uint64_t bits = (uint64_t)format_bits(L.format);
  const uint64_t d = (uint64_t)L.head_dim;
  const bool fp8 = fp8_of(L.format);
  const uint64_t eb = L.meta_fp16 ? 2 : 4;           // bytes per scale / zero-point
  sz[KVQ_PLANE_K_CODES] = recs * kBlock * d * bits / 8;
  sz[KVQ_PLANE_V_CODES] = sz[KVQ_PLANE_K_CODES];
  sz[KVQ_PLANE_K_META] = fp8 ? 0 : recs * 2 * d * eb;
  sz[KVQ_PLANE_V_META] = fp8 ? 0 : recs * 2 * (d / L.v_group_channels) * kBlock * eb;
  sz[KVQ_PLANE_K_RING] = bh * (uint64_t)(L.residual_tokens + kBlock) * d * 2;
  sz[KVQ_PLANE_V_RING] = sz[KVQ_PLANE_K_RING];
  sz[KVQ_PLANE_K_SINK] = bh * (uint64_t)L.sink_tokens * d * 2;
  sz[KVQ_PLANE_V_SINK] = sz[KVQ_PLANE_K_SINK];
  sz[KVQ_PLANE_K_OUT] = L.outliers ? recs * d * 4 : 0;                       // one entry per channel
  sz[KVQ_PLANE_V_OUT] = L.outliers ? recs * (d / L.v_group_channels) * kBlock * 4 : 0;
  sz[KVQ_PLANE_SYNC] = bh * 4;                                               // int32 per (sequence, KV head)
}

// Compute units of the current device (256 when no device answers), cached
// per device id; concurrent first calls store the same value.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

int64_t device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  int cached = dev < kMaxDevices ? g_cus[dev].load(std::memory_order_relaxed) : 0;
  if (cached > 0) return cached;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < kMaxDevices) g_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

struct AttnPlan {
  int64_t range_len, range_parts, group_skew;   // see AttnParams
  int64_t max_range, min_range;                 // longest and shortest workgroup range
  int64_t groups, fp16_blocks, slots;
};

// The library's own split gives the workgroups on odd-numbered XCDs (odd
// workgroup index: workgroup g runs on XCD g mod 8) kOddSkewPermille / 1000
// of a range fewer blocks than their even neighbours: on MI355X the odd XCDs
// stream measurably slower, so equal ranges finish unequally.
#ifndef KVQ_ODD_SKEW_PERMILLE
#define KVQ_ODD_SKEW_PERMILLE 40
#endif
constexpr int64_t kOddSkewPermille = KVQ_ODD_SKEW_PERMILLE;

// Split the work: the quantized blocks of all heads into one range per
// workgroup; the fp16 segment of each head into 32-token blocks handled by
// the workgroups whose range touches the head (one workgroup per head when
// no block is quantized yet).  Partial slots: one per fp16 block, plus, for
// the quantized blocks, kGroupWaves + 1 per (workgroup, head) index g + bh.
// Ranges: stretches of range_len blocks, each cut into range_parts parts
// (part p from floor(p L / k) + (p odd ? d : 0), see range_start in
// kvq_attn.hip):
//  * bpg > 0: ranges of exactly bpg blocks (L = bpg, k = 1);
//  * bpg = 0 (the library's split, one range per compute unit): when the
//    compute units divide among the heads evenly (k = CUs / heads ranges per
//    head are as long as an even cut of all blocks over the CUs, to within
//    1/32), every head is cut into k parts (L = nblk), so no range straddles
//    two heads and each head is shared by exactly k workgroups; otherwise
//    all blocks are cut into equal ranges of R blocks across head boundaries
//    (L = 2 R, k = 2).
// Paged caches stage a range's record ids in LDS, so their ranges hold at
// most kMaxPagedRange blocks.
AttnPlan plan(const kvq_layout& L, int64_t nblk, int64_t n_fp16_tokens, int32_t bpg) {
  AttnPlan a{};
  const int64_t bh = (int64_t)L.batch * L.num_kv_heads;
  a.fp16_blocks = (n_fp16_tokens + kBlock - 1) / kBlock;
  const int64_t total = bh * nblk;
  a.range_len = 1;
  a.range_parts = 1;
  a.group_skew = 0;
  if (total == 0) {
    a.groups = bh;
    a.slots = bh * a.fp16_blocks;
    return a;
  }
  const int64_t cap = L.page_blocks > 0 ? kMaxPagedRange : (int64_t(1) << 29);
  if (bpg > 0) {                                    // exact ranges of bpg blocks
    a.range_len = bpg;
    a.range_parts = 1;
  } else {
    const int64_t target = device_cus() * kGroupsPerCu;
    const int64_t even = std::min((total + target - 1) / target, cap);
    const int64_t k = bh <= target ? target / bh : 0;
    const int64_t per = k > 0 ? (nblk + k - 1) / k : 0;
    // a small call: every head in parts of at most one block per wavefront,
    // as long as they fit one workgroup per compute unit (a workgroup's merge
    // and a shared head's combine cost the same whatever its share, so fewer,
    // fuller workgroups finish sooner than one block each)
    const int64_t ks = (nblk + kGroupWaves - 1) / kGroupWaves;
    if (bh * ks <= target && kGroupWaves <= cap && ks * nblk < (int64_t(1) << 31)) {
      a.range_len = nblk;                           // ks parts of every head
      a.range_parts = ks;
    } else if (k > 0 && nblk >= k && per <= even + even / 32 && per <= cap && k * nblk < (int64_t(1) << 31)) {
      a.range_len = nblk;                           // k parts of every head
      a.range_parts = k;
    } else {
      a.range_len = 2 * even;                       // equal ranges of `even` blocks
      a.range_parts = 2;
    }
    const int64_t lo = a.range_len / a.range_parts, hi = (a.range_len + a.range_parts - 1) / a.range_parts;
    a.group_skew = std::min(lo * kOddSkewPermille / 1000, lo - 1);
    a.group_skew = std::max<int64_t>(0, std::min(a.group_skew, cap - hi));
  }
  const int64_t lo = a.range_len / a.range_parts, hi = (a.range_len + a.range_parts - 1) / a.range_parts;
  a.max_range = hi + a.group_skew;
  a.min_range = lo - a.group_skew;
  // workgroups: every part that starts before the end
  auto start = [&](int64_t g) {
    const int64_t s = g / a.range_parts, part = g - s * a.range_parts;
    return s * a.range_len + part * a.range_len / a.range_parts + ((part & 1) ? a.group_skew : 0);
  };
  a.groups = (total + a.range_len - 1) / a.range_len * a.range_parts;
  while (a.groups > 1 && start(a.groups - 1) >= total) --a.groups;
  a.slots = bh * a.fp16_blocks + (kGroupWaves + 1) * (a.groups + bh);
  return a;
}

// Multiply-shift division by d for dividends below 2^31: with 2^l >= d,
// m = ceil(2^(31+l) / d) < 2^32 and m d - 2^(31+l) < d, so
// floor(j m / 2^(31+l)) = floor(j / d) whenever j < 2^31.
void div_magic(uint64_t d, uint32_t& magic, int32_t& shift) {
  if (d == 0) d = 1;
  int l = 0;
  while ((1ull << l) < d) ++l;
  shift = 31 + l;
  magic = (uint32_t)(((1ull << (31 + l)) + d - 1) / d);
}

uint64_t slot_bytes(const kvq_layout& L) {
  return (uint64_t)(L.num_q_heads / L.num_kv_heads) * kPartStride * sizeof(float);
}

}  // namespace

// Validation and kernel parameters of an attention call over the first
// n_tokens tokens of the cache (every check before anything is enqueued).
static int32_t prepare_attention(const kvq_cache* c, int64_t n_tokens, const void* q, void* out, void* ws,
                                 uint64_t ws_bytes, int32_t bpg, int32_t deterministic, AttnParams& p) {
  if (!c || !c->base || !q || !out) return KVQ_ERR_NULL;
  const kvq_layout& L = c->layout;
  int32_t st = kvq_layout_validate(&L);
  if (st != KVQ_OK) return st;
  if (bpg < 0 || bpg > kMaxBlocksPerGroup || (deterministic != 0 && deterministic != 1)) return KVQ_ERR_LAYOUT;
  if (L.page_blocks > 0 && bpg > kMaxPagedRange) return KVQ_ERR_LAYOUT;
  if (L.page_blocks > 0 && !c->block_table) return KVQ_ERR_NULL;
  if (!aligned(q, 16) || !aligned(out, 16)) return KVQ_ERR_ALIGN;
  if (n_tokens == 0) return KVQ_ERR_EMPTY;
  const Window w = window(L, n_tokens);
  const int64_t nblk = w.n_q / kBlock;
  const int64_t bh = (int64_t)L.batch * L.num_kv_heads;
  // workspace is checked before anything touches the device
  if (!ws) return KVQ_ERR_WORKSPACE;
  const AttnPlan a = plan(L, nblk, w.n_sink + w.r, bpg);
  const uint64_t sb = slot_bytes(L);
  if ((uint64_t)a.slots * sb > ws_bytes) return KVQ_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return KVQ_ERR_ALIGN;
  if (bh * nblk > 0x7fffffffLL || a.groups > 0x7fffffffLL) return KVQ_ERR_UNSUPPORTED;
  // a head's arrival counter holds up to 65535 arrivals and 32767 "written"
  // marks: at most 32767 workgroups may cover one head
  if (nblk > 0 && (nblk + a.min_range - 1) / a.min_range + 1 > 32767) return KVQ_ERR_UNSUPPORTED;
  // the kernels' range arithmetic is 32-bit: range_len * range_parts < 2^31
  if (nblk > 0 && a.range_len * a.range_parts >= (int64_t(1) << 31)) return KVQ_ERR_UNSUPPORTED;

  char* base = static_cast<char*>(c->base);
  auto plane = [&](int i) { return base + c->plane_off[i]; };
  p = AttnParams{};
  p.k_codes = reinterpret_cast<const uint8_t*>(plane(KVQ_PLANE_K_CODES));
  p.v_codes = reinterpret_cast<const uint8_t*>(plane(KVQ_PLANE_V_CODES));
  p.k_meta = reinterpret_cast<const float*>(plane(KVQ_PLANE_K_META));
  p.v_meta = reinterpret_cast<const float*>(plane(KVQ_PLANE_V_META));
  p.k_out = reinterpret_cast<const uint32_t*>(plane(KVQ_PLANE_K_OUT));
  p.v_out = reinterpret_cast<const uint32_t*>(plane(KVQ_PLANE_V_OUT));
  p.k_ring = reinterpret_cast<const uint16_t*>(plane(KVQ_PLANE_K_RING));
  p.v_ring = reinterpret_cast<const uint16_t*>(plane(KVQ_PLANE_V_RING));
  p.k_sink = reinterpret_cast<const uint16_t*>(plane(KVQ_PLANE_K_SINK));
  p.v_sink = reinterpret_cast<const uint16_t*>(plane(KVQ_PLANE_V_SINK));
  p.sync = reinterpret_cast<int32_t*>(plane(KVQ_PLANE_SYNC));
  p.q = static_cast<const uint16_t*>(q);
  p.out = static_cast<uint16_t*>(out);
  p.part_fp16 = static_cast<float*>(ws);
  p.part_wave = p.part_fp16 + bh * a.fp16_blocks * (sb / sizeof(float));
  p.part_group = p.part_wave + (nblk > 0 ? kGroupWaves * (a.groups + bh) : 0) * (int64_t)(sb / sizeof(float));
  p.hkv = L.num_kv_heads;
  p.nrep = L.num_q_heads / L.num_kv_heads;
  p.nb_cap = c->n_blocks_cap;
  p.nblk = (int32_t)nblk;
  div_magic((uint64_t)nblk, p.nblk_magic, p.nblk_shift);
  div_magic(((uint64_t)nblk + 1) / 2, p.half_magic, p.half_shift);   // the block pairs of a whole head
  p.ring_slots = c->ring_slots;
  p.sink_cap = L.sink_tokens;
  p.n_sink = (int32_t)w.n_sink;
  p.n_res = (int32_t)w.r;
  p.ring_first = (int32_t)(w.n_q % c->ring_slots);
  p.bh_count = (int32_t)bh;
  p.range_len = (int32_t)a.range_len;
  p.range_parts = (int32_t)a.range_parts;
  p.group_skew = (int32_t)a.group_skew;
  div_magic((uint64_t)a.range_len, p.len_magic, p.len_shift);
  div_magic((uint64_t)a.range_parts, p.parts_magic, p.parts_shift);
  p.groups = (int32_t)a.groups;
  p.fp16_blocks = (int32_t)a.fp16_blocks;
  p.deterministic = deterministic;
  p.k_scale = L.k_scale;
  p.v_scale = L.v_scale;
  p.table = c->block_table;
  p.table_stride = c->table_stride;
  p.page_blocks = L.page_blocks;
  p.num_pages = L.num_pages;
  p.rope_theta = L.rope_theta;
  return KVQ_OK;
}

extern "C" {

const char* kvq_status_string(int32_t s) {
  switch (s) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_ERR_NULL: return "KVQ_ERR_NULL: a required pointer is NULL";
    case KVQ_ERR_LAYOUT: return "KVQ_ERR_LAYOUT: inconsistent sizes";
    case KVQ_ERR_UNSUPPORTED: return "KVQ_ERR_UNSUPPORTED: valid but not implemented";
    case KVQ_ERR_CAPACITY: return "KVQ_ERR_CAPACITY: capacity exceeded or buffer too small";
    case KVQ_ERR_ALIGN: return "KVQ_ERR_ALIGN: misaligned buffer";
    case KVQ_ERR_WORKSPACE: return "KVQ_ERR_WORKSPACE: workspace missing or too small";
    case KVQ_ERR_HIP: return "KVQ_ERR_HIP: kernel launch failed";
    case KVQ_ERR_EMPTY: return "KVQ_ERR_EMPTY: attention over an empty cache";
    default: return "unknown kvq status";
  }
}

int32_t kvq_layout_validate(const kvq_layout* L) {
  if (!L) return KVQ_ERR_NULL;
  if (L->batch < 1 || L->num_kv_heads < 1 || L->num_q_heads < 1 || L->head_dim < 1 ||
      L->max_tokens < 1 || L->residual_tokens < 0 || L->sink_tokens < 0 ||
      L->k_group_tokens < 1 || L->v_group_channels < 1)
    return KVQ_ERR_LAYOUT;
  if (L->num_q_heads % L->num_kv_heads) return KVQ_ERR_LAYOUT;
  if (L->head_dim % L->v_group_channels) return KVQ_ERR_LAYOUT;
  if (L->format < KVQ_INT8 || L->format > KVQ_FP8_E5M2) return KVQ_ERR_LAYOUT;
  if (L->meta_fp16 != 0 && L->meta_fp16 != 1) return KVQ_ERR_LAYOUT;
  if (fp8_of(L->format)) {
    if (!std::isfinite(L->k_scale) || !std::isfinite(L->v_scale) || !(L->k_scale > 0.f) ||
        !(L->v_scale > 0.f) || L->meta_fp16)
      return KVQ_ERR_LAYOUT;
  }
  if (L->sink_tokens > L->max_tokens) return KVQ_ERR_LAYOUT;
  if (L->page_blocks < 0 || (L->page_blocks > 0 && L->num_pages < 1)) return KVQ_ERR_LAYOUT;
  if (!std::isfinite(L->rope_theta) || L->rope_theta < 0.f) return KVQ_ERR_LAYOUT;
  if (L->outliers != 0 && L->outliers != 1) return KVQ_ERR_LAYOUT;
  if (L->outliers && fp8_of(L->format)) return KVQ_ERR_LAYOUT;           // FP8 has no groups
  // block records are 32-bit in the attention kernel
  if (L->page_blocks > 0 && (int64_t)L->num_pages * L->num_kv_heads * L->page_blocks > 0x7fffffffLL)
    return KVQ_ERR_UNSUPPORTED;
  if (L->head_dim != kHeadDim || L->k_group_tokens != kBlock || L->v_group_channels != kVGroup)
    return KVQ_ERR_UNSUPPORTED;
  const int nrep = L->num_q_heads / L->num_kv_heads;
  if (nrep != 1 && nrep != 2 && nrep != 4 && nrep != 8) return KVQ_ERR_UNSUPPORTED;
  if (L->outliers && L->rope_theta > 0.f) return KVQ_ERR_UNSUPPORTED;
  // grid.y = Hkv and grid.z = B must fit the launch limits
  if (L->num_kv_heads > 65535 || L->batch > 65535) return KVQ_ERR_UNSUPPORTED;
  if ((int64_t)L->residual_tokens + kBlock > (int64_t)1 << 30) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

int32_t kvq_cache_bytes(const kvq_layout* L, uint64_t* bytes) {
  if (!L || !bytes) return KVQ_ERR_NULL;
  int32_t st = kvq_layout_validate(L);
  if (st != KVQ_OK) return st;
  uint64_t sz[KVQ_NUM_PLANES];
  plane_sizes(*L, sz);
  uint64_t total = 0;
  for (int i = 0; i < KVQ_NUM_PLANES; ++i) total = align_up(total, kPlaneAlign) + sz[i];
  *bytes = align_up(total, kPlaneAlign);
  return KVQ_OK;
}

int32_t kvq_cache_init(kvq_cache* c, const kvq_layout* L, void* base, uint64_t bytes) {
  if (!c || !L || !base) return KVQ_ERR_NULL;
  uint64_t need = 0;
  int32_t st = kvq_cache_bytes(L, &need);
  if (st != KVQ_OK) return st;
  if (!aligned(base, kPlaneAlign)) return KVQ_ERR_ALIGN;
  if (bytes < need) return KVQ_ERR_CAPACITY;
  std::memset(c, 0, sizeof(*c));
  c->layout = *L;
  c->base = base;
  c->bytes = bytes;
  c->n_tokens = 0;
  c->n_blocks_cap = nb_cap(*L);
  c->ring_slots = L->residual_tokens + kBlock;
  uint64_t sz[KVQ_NUM_PLANES];
  plane_sizes(*L, sz);
  uint64_t off = 0;
  for (int i = 0; i < KVQ_NUM_PLANES; ++i) {
    off = align_up(off, kPlaneAlign);
    c->plane_off[i] = off;
    c->plane_bytes[i] = sz[i];
    off += sz[i];
  }
  return KVQ_OK;
}

int32_t kvq_cache_plane(const kvq_cache* c, int32_t plane, uint64_t* offset, uint64_t* bytes) {
  if (!c || !offset || !bytes) return KVQ_ERR_NULL;
  if (plane < 0 || plane >= KVQ_NUM_PLANES) return KVQ_ERR_LAYOUT;
  *offset = c->plane_off[plane];
  *bytes = c->plane_bytes[plane];
  return KVQ_OK;
}

int32_t kvq_cache_window(const kvq_cache* c, int64_t* n_sink, int64_t* n_q, int64_t* n_res) {
  if (!c || !n_sink || !n_q || !n_res) return KVQ_ERR_NULL;
  Window w = window(c->layout, c->n_tokens);
  *n_sink = w.n_sink;
  *n_q = w.n_q;
  *n_res = w.r;
  return KVQ_OK;
}

int32_t kvq_cache_set_block_table(kvq_cache* c, const void* table, int32_t stride) {
  if (!c) return KVQ_ERR_NULL;
  const kvq_layout& L = c->layout;
  if (L.page_blocks <= 0) return KVQ_ERR_LAYOUT;
  if (!table) {
    c->block_table = nullptr;
    c->table_stride = 0;
    return KVQ_OK;
  }
  const int64_t pages = ((int64_t)c->n_blocks_cap + L.page_blocks - 1) / L.page_blocks;
  if (stride < pages || stride < 1) return KVQ_ERR_LAYOUT;
  if (!aligned(table, 4)) return KVQ_ERR_ALIGN;
  c->block_table = static_cast<const int32_t*>(table);
  c->table_stride = stride;
  return KVQ_OK;
}

int32_t kv_quant_append(kvq_cache* c, const void* K, const void* V, int32_t T, void* stream) {
  if (!c || !c->base) return KVQ_ERR_NULL;
  const kvq_layout& L = c->layout;
  int32_t st = kvq_layout_validate(&L);
  if (st != KVQ_OK) return st;
  if (L.page_blocks > 0 && !c->block_table) return KVQ_ERR_NULL;
  if (T < 0) return KVQ_ERR_LAYOUT;
  if (T == 0) return KVQ_OK;
  if (!K || !V) return KVQ_ERR_NULL;
  if (!aligned(K, 16) || !aligned(V, 16)) return KVQ_ERR_ALIGN;
  if (c->n_tokens + (int64_t)T > (int64_t)L.max_tokens) return KVQ_ERR_CAPACITY;
  const int64_t n_old = c->n_tokens;
  const int64_t n_new = n_old + T;
  const Window w0 = window(L, n_old);
  const Window w1 = window(L, n_new);
  if (w1.n_q / kBlock > c->n_blocks_cap) return KVQ_ERR_CAPACITY;  // cannot happen for valid caches
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(c->base);
  auto plane = [&](int i) { return base + c->plane_off[i]; };

  // copy of new sink tokens and new residual tokens to their fp16 planes
  bool fused = false;
  CopyParams cp{};
  cp.k_in = static_cast<const uint16_t*>(K);
  cp.v_in = static_cast<const uint16_t*>(V);
  cp.k_ring = reinterpret_cast<uint16_t*>(plane(KVQ_PLANE_K_RING));
  cp.v_ring = reinterpret_cast<uint16_t*>(plane(KVQ_PLANE_V_RING));
  cp.k_sink = reinterpret_cast<uint16_t*>(plane(KVQ_PLANE_K_SINK));
  cp.v_sink = reinterpret_cast<uint16_t*>(plane(KVQ_PLANE_V_SINK));
  cp.n_old = n_old;
  cp.n_q_new = w1.n_q;
  cp.T = T;
  cp.hkv = L.num_kv_heads;
  cp.sink = L.sink_tokens;
  cp.ring_slots = c->ring_slots;
  // copied tokens: new sinks [n_old, min(n_new, S)), then new residual tokens
  // [max(n_old, S + n_q_new), n_new)
  cp.n_sink_copy = std::max<int64_t>(0, std::min<int64_t>(n_new, L.sink_tokens) - n_old);
  cp.ring_first_t = std::max<int64_t>(n_old, (int64_t)L.sink_tokens + w1.n_q);
  cp.n_copy = cp.n_sink_copy + std::max<int64_t>(0, n_new - cp.ring_first_t);
  // the first append of a cache also sets the attention arrival counters to 0
  cp.sync_zero = n_old == 0 ? reinterpret_cast<int32_t*>(plane(KVQ_PLANE_SYNC)) : nullptr;

  // 1) quantize the blocks that leave the residual window (reads ring slots
  //    of old tokens, so it runs before the copy below overwrites any slot)
  const int64_t n_flush = (w1.n_q - w0.n_q) / kBlock;
  if (n_flush > 0) {
    FlushParams p{};
    p.k_in = static_cast<const uint16_t*>(K);
    p.v_in = static_cast<const uint16_t*>(V);
    p.k_ring = reinterpret_cast<const uint16_t*>(plane(KVQ_PLANE_K_RING));
    p.v_ring = reinterpret_cast<const uint16_t*>(plane(KVQ_PLANE_V_RING));
    p.k_codes = reinterpret_cast<uint8_t*>(plane(KVQ_PLANE_K_CODES));
    p.v_codes = reinterpret_cast<uint8_t*>(plane(KVQ_PLANE_V_CODES));
    p.k_meta = reinterpret_cast<float*>(plane(KVQ_PLANE_K_META));
    p.v_meta = reinterpret_cast<float*>(plane(KVQ_PLANE_V_META));
    p.k_out = reinterpret_cast<uint32_t*>(plane(KVQ_PLANE_K_OUT));
    p.v_out = reinterpret_cast<uint32_t*>(plane(KVQ_PLANE_V_OUT));
    p.n_old = n_old;
    p.T = T;
    p.hkv = L.num_kv_heads;
    p.sink = L.sink_tokens;
    p.ring_slots = c->ring_slots;
    p.nb_cap = c->n_blocks_cap;
    p.first_block = (int32_t)(w0.n_q / kBlock);
    p.n_body_old = n_old - w0.n_sink;
    p.k_scale = L.k_scale;
    p.v_scale = L.v_scale;
    p.table = c->block_table;
    p.table_stride = c->table_stride;
    p.page_blocks = L.page_blocks;
    p.num_pages = L.num_pages;
    if (n_flush > 0x7fffffff) return KVQ_ERR_UNSUPPORTED;
    p.flush_x = (int32_t)n_flush;
    // a flush that reads no ring slot (nothing of the body was in the ring
    // before this append) takes the copy as extra workgroups of its launch:
    // the two touch disjoint planes, so they may run together
    if (p.n_body_old == 0) {
      const int64_t cx = std::max<int64_t>((cp.n_copy * 32 + 255) / 256, cp.sync_zero ? 1 : 0);
      if (n_flush + cx <= 0x7fffffff) {
        p.copy_x = (int32_t)cx;
        p.cp = cp;
        fused = true;
      }
    }
    if (launch_flush(variant_of(L), p, L.batch, s) != hipSuccess) return KVQ_ERR_HIP;
  }
  // 2) the copy, after the flush: it may overwrite ring slots the flush read
  if (!fused && launch_copy(cp, L.batch, s) != hipSuccess) return KVQ_ERR_HIP;
  c->n_tokens = n_new;
  return KVQ_OK;
}

int32_t kvq_workspace_bytes(const kvq_cache* c, int32_t bpg, uint64_t* bytes) {
  if (!c || !bytes) return KVQ_ERR_NULL;
  if (bpg < 0 || bpg > kMaxBlocksPerGroup) return KVQ_ERR_LAYOUT;
  const kvq_layout& L = c->layout;
  const uint64_t bh = (uint64_t)L.batch * L.num_kv_heads;
  // worst case over every cache length: all NB blocks quantized and the
  // largest fp16 segment (S sinks + R + 31 residual tokens); the library's
  // own split uses at most one workgroup per compute unit
  const uint64_t total = bh * (uint64_t)c->n_blocks_cap;
  const uint64_t nf = bh * (((uint64_t)L.sink_tokens + L.residual_tokens + kBlock - 1 + kBlock - 1) / kBlock);
  uint64_t groups = 0;
  if (total > 0) groups = bpg > 0 ? (total + bpg - 1) / bpg : std::min<uint64_t>(total, (uint64_t)(device_cus() * kGroupsPerCu));
  if (total > 0 && L.page_blocks > 0)        // paged ranges hold at most kMaxPagedRange blocks
    groups = std::max<uint64_t>(groups, (total + kMaxPagedRange - 1) / kMaxPagedRange);
  *bytes = (nf + (total > 0 ? (kGroupWaves + 1) * (groups + bh) : 0)) * slot_bytes(L);
  return KVQ_OK;
}

int32_t kv_decode_attention_split(const kvq_cache* c, const void* q, void* out, void* ws,
                                  uint64_t ws_bytes, int32_t bpg, int32_t deterministic, void* stream) {
  AttnParams p;
  const int32_t st = prepare_attention(c, c ? c->n_tokens : 0, q, out, ws, ws_bytes, bpg, deterministic, p);
  if (st != KVQ_OK) return st;
  const kvq_layout& L = c->layout;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (launch_attention(variant_of(L), p, s) != hipSuccess) return KVQ_ERR_HIP;
  return KVQ_OK;
}

int32_t kv_decode_attention(const kvq_cache* c, const void* q, void* out, void* ws,
                            uint64_t ws_bytes, void* stream) {
  return kv_decode_attention_split(c, q, out, ws, ws_bytes, 0, 0, stream);
}

int32_t kv_decode_attention_noalloc(const kvq_cache* c, const void* q, void* out, void* stream) {
  // every check first, the workspace size against the library's scratch
  // included, with a host stand-in address (alignment and arithmetic only;
  // those parameters are discarded): nothing touches the device on an error
  alignas(256) static const char stand_in[256] = {};
  AttnParams p;
  void* probe = const_cast<char*>(stand_in);
  int32_t st = prepare_attention(c, c ? c->n_tokens : 0, q, out, probe, kScratchBytes, 0, 0, p);
  if (st != KVQ_OK) return st;
  void* ws = nullptr;
  if (attention_scratch(&ws) != hipSuccess) return KVQ_ERR_HIP;
  st = prepare_attention(c, c->n_tokens, q, out, ws, kScratchBytes, 0, 0, p);
  if (st != KVQ_OK) return st;
  if (launch_attention(variant_of(c->layout), p, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return KVQ_ERR_HIP;
  return KVQ_OK;
}

int32_t kv_append_decode_attention(kvq_cache* c, const void* K, const void* V, const void* q, void* out,
                                   void* ws, uint64_t ws_bytes, void* stream) {
  if (!c || !c->base || !K || !V) return KVQ_ERR_NULL;
  const kvq_layout& L = c->layout;
  int32_t st = kvq_layout_validate(&L);
  if (st != KVQ_OK) return st;
  if (L.page_blocks > 0 && !c->block_table) return KVQ_ERR_NULL;
  if (!aligned(K, 16) || !aligned(V, 16)) return KVQ_ERR_ALIGN;
  const int64_t n_old = c->n_tokens;
  if (n_old + 1 > (int64_t)L.max_tokens) return KVQ_ERR_CAPACITY;
  AttnParams p;                                   // attention over the n_old + 1 tokens
  st = prepare_attention(c, n_old + 1, q, out, ws, ws_bytes, 0, 0, p);
  if (st != KVQ_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const Window w0 = window(L, n_old), w1 = window(L, n_old + 1);
  // one launch when the token only enters the residual ring: not the cache's
  // first append (which also zeroes the counters), not a sink, and no block
  // leaves the window; the attention kernel reads the token from K, V and
  // copies it to its ring slot
  if (n_old > 0 && n_old >= L.sink_tokens && w1.n_q == w0.n_q) {
    p.new_k = static_cast<const uint16_t*>(K);
    p.new_v = static_cast<const uint16_t*>(V);
    if (launch_attention(variant_of(L), p, s) != hipSuccess) return KVQ_ERR_HIP;
    c->n_tokens = n_old + 1;
    return KVQ_OK;
  }
  st = kv_quant_append(c, K, V, 1, stream);       // every validation already passed above
  if (st != KVQ_OK) return st;
  if (launch_attention(variant_of(L), p, s) != hipSuccess) return KVQ_ERR_HIP;
  return KVQ_OK;
}

int32_t kvq_read_probe(const void* buf, uint64_t bytes, void* sink, uint64_t sink_bytes, int32_t groups,
                       void* stream) {
  if (!buf || !sink) return KVQ_ERR_NULL;
  if (bytes % 16 != 0 || groups < 0) return KVQ_ERR_LAYOUT;
  if (!aligned(buf, 16) || !aligned(sink, 16)) return KVQ_ERR_ALIGN;
  const int64_t g = groups > 0 ? groups : device_cus();
  if (g > 0x7fffffffLL) return KVQ_ERR_UNSUPPORTED;
  if ((uint64_t)g * kProbeThreads * 4 > sink_bytes) return KVQ_ERR_WORKSPACE;
  if (bytes == 0) return KVQ_OK;
  if (launch_read_probe(buf, bytes / 16, static_cast<uint32_t*>(sink), (int)g,
                        reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return KVQ_ERR_HIP;
  return KVQ_OK;
}

int32_t kvq_rw_probe(const void* src, uint64_t src_bytes, void* dst, uint64_t dst_bytes, uint32_t read_bytes,
                     uint32_t write_bytes, void* stream) {
  if (!src || !dst) return KVQ_ERR_NULL;
  if (read_bytes == 0 || read_bytes % 4096 != 0 || read_bytes > 32768 || write_bytes % 16 != 0 ||
      write_bytes > 65536 || src_bytes % read_bytes != 0)
    return KVQ_ERR_LAYOUT;
  if (!aligned(src, 16) || !aligned(dst, 16)) return KVQ_ERR_ALIGN;
  const uint64_t units = src_bytes / read_bytes;
  if (units > 0x7fffffffULL) return KVQ_ERR_UNSUPPORTED;
  if (units * write_bytes > dst_bytes) return KVQ_ERR_WORKSPACE;
  if (units == 0) return KVQ_OK;
  if (launch_rw_probe(src, dst, units, (int)(read_bytes / 16), (int)(write_bytes / 16),
                      reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return KVQ_ERR_HIP;
  return KVQ_OK;
}

}  // extern "C"
