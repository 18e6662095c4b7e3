/*
 * kvq.h -- quantized KV cache for MI355X (gfx950): C ABI.
 *
 * Two hot calls, as the method describes its integration ("KV Cache
 * Quantization Analysis", sec. 5, system integration): quantize the new
 * token's K and V right after they are produced and store them
 * (kv_quant_append), and dequantize inside attention (kv_decode_attention).
 * Everything else here is sizing, validation and set-up.
 *
 * Conventions (every entry point):
 *  - Return value: KVQ_OK (0) or a negative kvq_status.  No exceptions, no
 *    aborts, no device allocation, no host<->device synchronisation.
 *  - Memory: the caller owns every buffer.  Device pointers are plain HIP
 *    device addresses; "stream" is a hipStream_t passed as void* (NULL =
 *    the default stream).  All device work is enqueued on that stream.
 *  - Validation happens on the host before anything is enqueued.  A call
 *    that returns a validation error (NULL, LAYOUT, UNSUPPORTED, CAPACITY,
 *    ALIGN, WORKSPACE, EMPTY) has changed nothing.  KVQ_ERR_HIP means a
 *    kernel launch failed; the cache contents are then undefined.
 *  - A cache must not be used from two streams at once, and two attention
 *    calls on one cache must not overlap (they share the cache's sync
 *    plane); the host struct is not thread-safe.
 *  - Inputs must be finite (no NaN / Inf); this is not checked.
 *
 * Cache layout (one cache per layer; all sequences of the batch hold the
 * same number of tokens n).  Readings of the pages, fixed here:
 *  - the first S tokens are attention sinks kept in fp16 ("W4A16 + KV cache
 *    quantization: combined accuracy", layer-sensitivity section);
 *  - the other tokens ("body", index u = t - S) are quantized 32 at a time,
 *    keeping at least R recent body tokens in fp16 ("KV Cache Quantization
 *    Analysis", sec. 3, full-precision recent window): after n tokens,
 *    n_q = 32 * floor(max(0, n - S - R) / 32) body tokens are quantized and
 *    r = n - S - n_q stay in an fp16 ring of R + 32 slots (token u in slot
 *    u mod (R + 32));
 *  - INT formats: Keys per channel over each block of 32 tokens, Values per
 *    token over groups of 32 channels (same page, sec. 3 and sec. 4, KIVI);
 *    q = clamp(rint(x / s + z), 0, 2^b - 1), s = (max - min) / (2^b - 1)
 *    (s = 1 for a constant group), z = -min / s, each a single fp32 IEEE
 *    operation (same page, sec. 2, affine quantization);
 *  - FP8: OCP E4M3 (max 448) of clamp(x / s, -448, 448), or OCP E5M2 (max
 *    57344) of clamp(x / s, -57344, 57344), rounded to nearest even, with
 *    one fp32 scale for K and one for V per layer (same page, sec. 4, FP8 /
 *    INT8, which names both formats);
 *  - fp16 metadata (meta_fp16 = 1, INT formats): one fp16 scale and one fp16
 *    offset per group, 16 bits each as in the block formats of the 27B KL
 *    study's KV-cache size table.  s = (max - min) / (2^b - 1) in fp32,
 *    rounded up to the next fp16 (1 for a constant group); the offset is
 *    m = min (exact in fp16); q = clamp(rint((x - m) / s), 0, 2^b - 1) in
 *    fp32 steps; x_hat = s * q + m (the same affine map, with s * z = -m).
 *
 * Planes inside the caller's device buffer (offsets from kvq_cache_plane;
 * NB = max(0, max_tokens - S - R) / 32 blocks, D = head_dim, b = bits):
 *   K codes  [B][Hkv][NB][32*D*b/8].  The codes of one token are D*b/8
 *            bytes, channel c at bit (c*b mod 8) of byte floor(c*b/8)
 *            (FP8: one E4M3 byte per channel).  INT4, INT2: the 32 tokens'
 *            rows one after another.  INT8, FP8: 16-byte units, unit
 *            (2*tile + half)*64 + 16*qd + r = bytes 32*qd + 16*half .. +15
 *            of token 16*tile + r.
 *   V codes  [B][Hkv][NB][32*D*b/8] per 32-token block: 64 records of
 *            D*b/16 bytes, cut into 16-byte groups; group i of record l
 *            starts at byte 16*(64*i + l) of the block.
 *            Record l = 16*qd + r holds channels 16*m + r
 *            (m = 0 .. D/16-1) of the tokens T = (4qd .. 4qd+3,
 *            16+4qd .. 16+4qd+3):
 *              INT4       word m, nibble j = code(T[j], 16m + r)
 *              INT8, FP8  bytes 8m..8m+7 = T[0],T[4],T[1],T[5],T[2],T[6],T[3],T[7]
 *              INT2       word p: byte 0 / 1 = channel 32p + r / 32p + 16 + r
 *                         of T[0..3], byte 2 / 3 = the same channels of T[4..7]
 *            (the order in which the attention kernel's matrix-core operands
 *            are loaded).
 *   K meta   [B][Hkv][NB][D][2] fp32: (s, z) of each channel (INT only)
 *   V meta   [B][Hkv][NB][D/32][32][2] fp32: (s, z) of each channel group
 *            and token (INT only)
 *            With meta_fp16 both meta planes have the same shapes and hold
 *            fp16 (s, m) pairs (half the bytes).
 *   K ring, V ring  [B][Hkv][R+32][D] fp16
 *   K sink, V sink  [B][Hkv][S][D] fp16
 *   sync     [B][Hkv] int32 counters of the attention call.  For a head
 *            whose blocks are split over several workgroups, each of them
 *            adds 1 on arrival (low 16 bits) and, unless its arrival
 *            completed the count, 1 << 16 once its partial is written; the
 *            one that completed the count waits for the others' marks,
 *            combines the head's partials and sets the counter back to 0.
 *            At most 32767 workgroups may share a head (checked by the
 *            host: larger splits return KVQ_ERR_UNSUPPORTED).
 *            Set to 0 by the cache's first kv_quant_append and 0 again
 *            after every attention call; no other call touches it.
 * Each plane starts on a 256-byte boundary.
 *
 * FP8 E5M2 codes use the INT8 / FP8 byte layouts above.
 *
 * Dense-and-sparse outliers (outliers = 1, INT formats; "KV Cache
 * Quantization Analysis", sec. 2 outliers and sec. 4 KVQuant per-vector
 * dense-and-sparse): in every quantization group (a Key channel's 32 tokens
 * of a block, a Value token's 32-channel group) the value of largest
 * magnitude (lowest index on ties) is kept exactly as fp16 with its index,
 * the group's scale and zero-point (or offset) come from the other 31
 * values, and the outlier's own code is 0.  Entries are 32-bit: index in the
 * group in the low 16 bits, fp16 value in the high 16 bits.
 *   K out    [B][Hkv][NB][D] entries (token index in the block per channel;
 *            stored-position order like K meta)
 *   V out    [B][Hkv][NB][D/32][32] entries (channel index in the group per
 *            group and token, the V meta order)
 * Not combined with pre-RoPE Keys (KVQ_ERR_UNSUPPORTED).
 *
 * Pre-RoPE Keys (rope_theta > 0; "KV Cache Quantization Analysis", sec. 3
 * RoPE problem and sec. 4 KVQuant: quantize Keys per channel before the
 * rotary encoding, rotate after dequantization).  kv_quant_append then takes
 * Keys *before* RoPE, and attention rotates every cached Key (sinks,
 * quantized body, residual) at its position t (0-based index in the
 * sequence) with the rotate-half pairs (i, i + D/2): angle t * theta_i,
 * theta_i = rope_theta^(-2i/D).  The query passed to attention is already
 * rotated at its own position.  Each K row of the code and meta planes is
 * stored in pair order: stored position 2i holds channel i, 2i + 1 holds
 * channel i + D/2 (the byte layout above applies to stored positions).
 *
 * Paged cache (page_blocks = P >= 1): the four quantized planes (K / V
 * codes, K / V meta) are pools of num_pages pages instead of [B][Hkv][NB]
 * arrays.  A page holds P consecutive 32-token blocks of one sequence for
 * all Hkv heads: block-sized records ordered [page][Hkv][P], each record in
 * the block layout above.  Logical block j (0 .. NB-1) of sequence b, head
 * h, is record (page * Hkv + h) * P + j % P with page = table[b * stride +
 * j / P] ("KV Cache Quantization Analysis", sec. 5: paged blocks are
 * orthogonal to quantization, and low-bit blocks hold more tokens per page;
 * "Quantization and the KV cache: two ways to run a model lighter", section
 * on how the KV-cache side works: the cache is split into small blocks, a
 * table per request lists its blocks, and requests with the same prompt may
 * share blocks).  The table
 * is an int32 device array set by kvq_cache_set_block_table, owned and
 * filled by the caller before the calls that touch those blocks.  Pages of
 * different sequences may be shared only where their quantized blocks are
 * identical (the same tokens).  A page id outside [0, num_pages) is a
 * caller error: the kernels never touch memory outside the pool for it (the
 * block is not written, and attention reads page 0 in its place, so that
 * sequence's output is undefined).  The fp16 ring and sink planes stay per
 * sequence.
 *
 * Limits of this version (KVQ_ERR_UNSUPPORTED otherwise): head_dim == 128,
 * k_group_tokens == 32, v_group_channels == 32, num_q_heads / num_kv_heads
 * in {1, 2, 4, 8}.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_NULL = -1,         /* a required pointer is NULL */
  KVQ_ERR_LAYOUT = -2,       /* inconsistent sizes (e.g. Hq % Hkv != 0, T < 0) */
  KVQ_ERR_UNSUPPORTED = -3,  /* valid but not implemented (see limits above) */
  KVQ_ERR_CAPACITY = -4,     /* append past max_tokens, or buffer too small */
  KVQ_ERR_ALIGN = -5,        /* buffer not aligned (base: 256 B, tensors: 16 B) */
  KVQ_ERR_WORKSPACE = -6,    /* workspace NULL or smaller than required */
  KVQ_ERR_HIP = -7,          /* a kernel launch failed */
  KVQ_ERR_EMPTY = -8         /* attention over an empty cache */
} kvq_status;

typedef enum { KVQ_INT8 = 0, KVQ_INT4 = 1, KVQ_INT2 = 2, KVQ_FP8_E4M3 = 3, KVQ_FP8_E5M2 = 4 } kvq_format;

/* One layer's cache geometry.  Per-layer formats (e.g. INT8 on the first and
 * last layers, INT4 in between) use one layout and one cache per layer. */
typedef struct {
  int32_t batch;             /* B >= 1 */
  int32_t num_kv_heads;      /* Hkv >= 1 */
  int32_t num_q_heads;       /* Hq, a multiple of Hkv (GQA: q head h reads KV head h / (Hq/Hkv)) */
  int32_t head_dim;          /* D (128) */
  int32_t max_tokens;        /* capacity in tokens per sequence */
  int32_t format;            /* kvq_format */
  int32_t k_group_tokens;    /* tokens per Key scale group (32) */
  int32_t v_group_channels;  /* channels per Value scale group (32) */
  int32_t residual_tokens;   /* R >= 0: recent body tokens always kept in fp16 */
  int32_t sink_tokens;       /* S >= 0: first tokens always kept in fp16 */
  float k_scale;             /* FP8 only: Key scale, finite and > 0 */
  float v_scale;             /* FP8 only: Value scale, finite and > 0 */
  int32_t meta_fp16;         /* INT only: 0 = fp32 (s, z) pairs, 1 = fp16 (s, m) pairs; 0 for FP8 */
  int32_t page_blocks;       /* 0: contiguous planes; P >= 1: paged, P 32-token blocks per page */
  int32_t num_pages;         /* paged only: pages in the pool (>= 1) */
  float rope_theta;          /* 0: Keys stored as given; > 0 (finite): pre-RoPE Keys, RoPE base */
  int32_t outliers;          /* INT only: 1 = one exact fp16 outlier per quantization group */
} kvq_layout;

enum {
  KVQ_PLANE_K_CODES = 0, KVQ_PLANE_V_CODES, KVQ_PLANE_K_META, KVQ_PLANE_V_META,
  KVQ_PLANE_K_RING, KVQ_PLANE_V_RING, KVQ_PLANE_K_SINK, KVQ_PLANE_V_SINK,
  KVQ_PLANE_K_OUT, KVQ_PLANE_V_OUT, KVQ_PLANE_SYNC,
  KVQ_NUM_PLANES
};

/* Host-side handle of one cache.  Plain data owned by the caller; filled by
 * kvq_cache_init; n_tokens is advanced by kv_quant_append only after its
 * kernels were enqueued successfully.  Copying the struct together with the
 * device buffer's bytes saves and restores the cache. */
typedef struct {
  kvq_layout layout;
  void* base;                          /* device buffer */
  uint64_t bytes;                      /* its size */
  int64_t n_tokens;                    /* tokens per sequence currently cached */
  int32_t n_blocks_cap;                /* NB */
  int32_t ring_slots;                  /* R + 32 */
  uint64_t plane_off[KVQ_NUM_PLANES];  /* byte offsets from base */
  uint64_t plane_bytes[KVQ_NUM_PLANES];
  const int32_t* block_table;          /* paged only: device int32 [B][table_stride] */
  int32_t table_stride;                /* pages per sequence row of block_table */
} kvq_cache;

/* Static string naming a status code. */
const char* kvq_status_string(int32_t status);

/* Check a layout.  Returns KVQ_OK, KVQ_ERR_NULL, KVQ_ERR_LAYOUT or
 * KVQ_ERR_UNSUPPORTED. */
int32_t kvq_layout_validate(const kvq_layout* layout);

/* Device bytes needed for one cache with this layout (*bytes, host memory). */
int32_t kvq_cache_bytes(const kvq_layout* layout, uint64_t* bytes);

/* Bind a caller-allocated device buffer (256-B aligned, >= kvq_cache_bytes)
 * to *cache and set it empty (n_tokens = 0).  Enqueues nothing: plane
 * contents are undefined until written by kv_quant_append. */
int32_t kvq_cache_init(kvq_cache* cache, const kvq_layout* layout, void* dev_base, uint64_t bytes);

/* Byte offset and size of one plane (KVQ_PLANE_*) inside the buffer. */
int32_t kvq_cache_plane(const kvq_cache* cache, int32_t plane, uint64_t* offset, uint64_t* bytes);

/* Current routing: sinks held, quantized body tokens, fp16 residual tokens. */
int32_t kvq_cache_window(const kvq_cache* cache, int64_t* n_sink, int64_t* n_q, int64_t* n_residual);

/* Paged layouts: bind the block table, an int32 device array [B][stride]
 * (4-B aligned) whose row b lists the physical pages of sequence b's
 * logical pages 0 .. ceil(NB / P) - 1 (stride >= that count).  The library
 * keeps the pointer and reads the table on the device at every append and
 * attention call; the caller may change its contents between calls.  NULL
 * unbinds it.  Errors: KVQ_ERR_LAYOUT for a contiguous layout or a stride
 * below ceil(NB / P), KVQ_ERR_ALIGN.  kv_quant_append and the attention
 * calls return KVQ_ERR_NULL on a paged cache without a table. */
int32_t kvq_cache_set_block_table(kvq_cache* cache, const void* table, int32_t stride);

/* Quantize-on-append ("KV Cache Quantization Analysis", sec. 5: quantize
 * the new K, V right after they are computed, then store).
 * K, V: device fp16 [B][T][Hkv][D], contiguous, 16-B aligned, read only.
 * Appends T >= 0 tokens to every sequence: sinks and residual tokens are
 * copied to their fp16 planes; every block of 32 body tokens that leaves the
 * residual window is quantized (from the ring or directly from K, V) and its
 * codes and scale/zero planes written.  Errors: KVQ_ERR_CAPACITY if
 * n_tokens + T > max_tokens (nothing enqueued). */
int32_t kv_quant_append(kvq_cache* cache, const void* K, const void* V, int32_t T, void* stream);

/* Workspace bytes kv_decode_attention_split needs on the current device for
 * any n_tokens up to max_tokens with the given blocks_per_group (0 = the
 * library's choice): partials of (4 + 128) floats per query head, one per
 * fp16 block of 32 tokens and, for the quantized blocks, nine per (workgroup
 * + head) index (eight wavefronts' and their merge).  A larger blocks_per_group never needs more.
 * Errors: KVQ_ERR_NULL; KVQ_ERR_LAYOUT for blocks_per_group outside
 * [0, 2^20]. */
int32_t kvq_workspace_bytes(const kvq_cache* cache, int32_t blocks_per_group, uint64_t* bytes);

/* Fused-dequant decode attention ("KV Cache Quantization Analysis", sec. 4
 * and sec. 5: dequantization fused into the attention matmuls; "W4A16 + KV
 * cache quantization: combined accuracy", softmax(Q K^T / sqrt(d)) with GQA).
 * q: device fp16 [B][Hq][D]; out: device fp16 [B][Hq][D]; both 16-B aligned.
 * For every sequence b and query head h:
 *   out[b][h] = sum_t softmax_t(q[b][h] . k_hat[b][g][t] / sqrt(D)) v_hat[b][g][t]
 * over all n_tokens cached tokens, g = h / (Hq/Hkv), with k_hat, v_hat the
 * dequantized (or fp16) cache entries.  Split-K in one kernel: workgroups
 * write partials (max, sum, unnormalised output) into ws, merged per
 * workgroup; the last workgroup to finish a (sequence, KV head) combines
 * that head's partials into out, in a fixed order.
 * ws: device scratch of >= kvq_workspace_bytes(cache, 0) bytes, 16-B
 * aligned, any contents, overwritten; calls that share a workspace must be
 * ordered on one stream.  Blocks are handed to wavefronts as the memory
 * system serves them, so repeated calls may differ in the last bits (see the
 * deterministic mode below).  Errors: KVQ_ERR_EMPTY if n_tokens == 0. */
int32_t kv_decode_attention(const kvq_cache* cache, const void* q, void* out, void* ws,
                            uint64_t ws_bytes, void* stream);

/* One decode step of one layer, the two hot calls back to back as the method
 * integrates them ("KV Cache Quantization Analysis", sec. 5, system
 * integration: quantize the new K, V right after they are produced, then
 * dequantize inside attention): kv_quant_append of one token (K, V: device
 * fp16 [B][1][Hkv][D]) followed by kv_decode_attention over the cache that
 * includes it, with the results of those two calls (the same kernel, the
 * library's own split).  When the token only enters the fp16
 * residual ring (not the cache's first append, not a sink, no block leaves
 * the window: 31 of every 32 decode steps) it is one kernel launch: the
 * attention kernel reads the token from K, V and copies it to its ring slot;
 * otherwise the two calls are enqueued in turn.  Every check of both calls
 * runs before anything is enqueued, so an error leaves the cache unchanged;
 * n_tokens advances by one on success.  Errors: those of kv_quant_append
 * (T = 1) and kv_decode_attention. */
int32_t kv_append_decode_attention(kvq_cache* cache, const void* K, const void* V, const void* q, void* out,
                                   void* ws, uint64_t ws_bytes, void* stream);

/* kv_decode_attention with an explicit split.  The quantized 32-token blocks
 * of all heads, flattened head-major, are cut into ranges of blocks_per_group
 * blocks (a range may cross from one head into the next), one per workgroup
 * of 8 wavefronts; 0 selects the library's choice, one range per compute
 * unit.  deterministic = 0: a workgroup's wavefronts take its blocks in the
 * order they become free; deterministic = 1: wavefront w takes blocks w,
 * w + 8, w + 16, ... of the range, and repeated calls give identical bits.
 * The fp16 segment (sinks + residual ring) is handled in 32-token blocks.
 * Results of every choice agree up to fp32 rounding.  Errors: KVQ_ERR_LAYOUT
 * for blocks_per_group outside [0, 2^20] or deterministic not 0 or 1;
 * KVQ_ERR_WORKSPACE if ws_bytes is below what this n_tokens and split need
 * (checked before any launch); KVQ_ERR_UNSUPPORTED beyond 2^31 - 1
 * quantized blocks. */
int32_t kv_decode_attention_split(const kvq_cache* cache, const void* q, void* out, void* ws,
                                  uint64_t ws_bytes, int32_t blocks_per_group, int32_t deterministic,
                                  void* stream);

/* kv_decode_attention without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The same kernel and the same results
 * (the library's own split); the partials go to a workspace the library owns:
 * a 32 MiB device array, one copy per GPU, held until the process ends.  The
 * call allocates and frees nothing.  All calls on one GPU share that array,
 * so two calls whose kernels may overlap on one GPU (other streams, other
 * threads) race and give undefined results; calls ordered on one stream do
 * not.  Its address is looked up on the first call on each device.
 * Errors: those of kv_decode_attention; KVQ_ERR_WORKSPACE when the call
 * needs more than the 32 MiB (kvq_workspace_bytes(cache, 0) above 32 MiB;
 * checked before any device call); KVQ_ERR_HIP if the array cannot be
 * located on the current device. */
int32_t kv_decode_attention_noalloc(const kvq_cache* cache, const void* q, void* out, void* stream);

/* Diagnostic, not part of the method: a plain streaming read of a device
 * buffer, which measures the HBM read rate this GPU delivers to a kernel of
 * the attention call's shape (the benchmark reports attention calls against
 * it as well as against the nominal peak).  groups workgroups of 512 threads
 * (0 = one per compute unit) each read one contiguous part of buf (bytes, a
 * multiple of 16) with 16-byte nontemporal loads, eight in flight per thread;
 * each thread writes the XOR of the words it read to its uint32 of sink, so
 * no load can be dropped.  buf and sink are device pointers, 16-B aligned;
 * sink_bytes >= 4 * 512 * groups.  Errors: KVQ_ERR_NULL, KVQ_ERR_LAYOUT
 * (bytes not a multiple of 16, groups < 0), KVQ_ERR_ALIGN, KVQ_ERR_WORKSPACE
 * (sink too small), KVQ_ERR_HIP. */
int32_t kvq_read_probe(const void* buf, uint64_t bytes, void* sink, uint64_t sink_bytes, int32_t groups,
                       void* stream);

/* Diagnostic, not part of the method: the traffic of a flush and nothing
 * else, which measures the ceiling of kv_quant_append's quantization kernel
 * on this GPU (the benchmark reports the prompt's quantization against it).
 * One workgroup of 256 threads per unit of read_bytes of src (src_bytes /
 * read_bytes units): it reads the unit whole (16-byte loads, all in flight
 * together; thread t the unit's 16-byte words t, t + 256, ...), folds what
 * each thread read by XOR into one 16-byte word w (four uint32 lanes), then
 * writes the unit's write_bytes of dst, thread t the words j = t, t + 256,
 * ... as w + j (uint32 lanes, wrapping).  A flush of head_dim 128 reads
 * 16384 bytes per 32-token block and writes its codes and metadata.  src and
 * dst are device pointers, 16-B aligned; read_bytes a multiple of 4096 up to
 * 32768; write_bytes a multiple of 16 up to 65536; src_bytes a multiple of
 * read_bytes; dst_bytes >= units * write_bytes.  Errors: KVQ_ERR_NULL,
 * KVQ_ERR_LAYOUT (sizes), KVQ_ERR_ALIGN, KVQ_ERR_WORKSPACE (dst too small),
 * KVQ_ERR_UNSUPPORTED (more than 2^31 - 1 units), KVQ_ERR_HIP. */
int32_t kvq_rw_probe(const void* src, uint64_t src_bytes, void* dst, uint64_t dst_bytes, uint32_t read_bytes,
                     uint32_t write_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
