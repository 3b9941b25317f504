/*
 * thdattn: causal attention with EOD (document) mask reset over THD-packed
 * sequences, for one context-parallel rank's share, on AMD MI355X (gfx950).
 *
 * The operation ("kvallgather cp thd load balance", Ascend/MindSpeed pull
 * request, sections "What this PR does / why we need it?" and "Does this PR
 * introduce any user-facing change?"):
 *   - THD-packed input: documents of lengths L_0..L_{n-1} are packed end to
 *     end, T = sum L_i tokens; every L_i must be divisible by 2*cp;
 *   - EOD-aware symmetric partitioning: each document is cut into 2*cp equal
 *     chunks of c_i = L_i/(2cp) tokens; rank r owns chunks r and 2cp-1-r; its
 *     T_local = T/cp query rows run document by document, chunk r first;
 *   - KV-all-gather context parallelism: K and V arrive already all-gathered
 *     in rank-major order (rank 0's shard, then rank 1's, ...) and are indexed
 *     directly, without a reorder copy;
 *   - causal attention with the mask reset at every EOD: the query at global
 *     position g of document i sees the keys cu_i..g of that document only;
 *   - MHA, GQA (q head h uses kv head h / (Hq/Hkv)) and expanded MLA
 *     (d_qk != d_v).
 *
 * Tensor layouts (row-major, contiguous, "TND"):
 *   q    bf16 [T_local, Hq,  d_qk]      this rank's queries
 *   k    bf16 [T,       Hkv, d_qk]      gathered, rank-major
 *   v    bf16 [T,       Hkv, d_v ]      gathered, rank-major
 *   o    bf16 [T_local, Hq,  d_v ]      output (round to nearest even)
 *   lse  fp32 [T_local, Hq]             natural-log sum of exp of the scores
 *   d_o  bf16 [T_local, Hq,  d_v ]      upstream gradient (backward)
 *   dq   fp32 [T_local, Hq,  d_qk]      backward outputs; dk/dv are this
 *   dk   fp32 [T,       Hkv, d_qk]      rank's partial sums in the gathered
 *   dv   fp32 [T,       Hkv, d_v ]      layout, exact zeros for unseen keys
 *                                       (bf16 from thd_attn_bwd_bf16kv)
 *
 * Conventions for every entry point:
 *   - return 0 (THD_OK) or a negative thd_status; nothing aborts or throws
 *     across this interface; thd_last_error() gives a message for the
 *     calling thread's last failure;
 *   - host pointers are caller-owned and only read (or written, for outputs)
 *     during the call; device pointers are caller-owned device memory;
 *   - kernels are enqueued on the given HIP stream (NULL = default stream)
 *     and the call returns before they finish; all argument checks are
 *     synchronous and host-side;
 *   - every entry point is thread-safe.
 */
#ifndef THDATTN_H
#define THDATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  THD_OK = 0,
  THD_EINVAL = -1,        /* a required pointer is NULL, a count or scale is out of range */
  THD_ENOTDIV = -2,       /* a subsequence length is not divisible by 2*cp */
  THD_ERANGE = -3,        /* cp < 1, rank outside [0, cp), T >= 2^31, bad tile size */
  THD_EALIGN = -4,        /* a device pointer is not 16-byte aligned */
  THD_EMISMATCH = -5,     /* metadata does not fit the call (tile sizes, device) */
  THD_EHIP = -6,          /* the HIP runtime reported an error */
  THD_ENOMEM = -7,        /* host or device allocation failed */
  THD_EUNSUPPORTED = -8   /* no kernel for these head dims or group size */
} thd_status;

/* Version of the tile-table contract (the per-tile bounds and work items below). */
#define THD_META_VERSION 4

/* Fields of a metadata object, for thd_meta_copy. All int32.
 *   Q_GLOBAL  [T_local]       global packed position of each local query row
 *   KV_ROW    [T]             gathered (rank-major) row of each global token
 *   CHUNK_OFF [n_docs*2cp]    gathered row of the first token of each chunk
 *   TILES     [n_tiles*8]     per query tile: q_local_start, q_global_start,
 *                             n_rows, doc, slot, kv_start, n_kv_tiles,
 *                             n_full_kv_tiles (tiles never straddle a chunk;
 *                             KV tile j covers keys kv_start + j*block_n ...,
 *                             up to the last row's position; the first
 *                             n_full_kv_tiles need no causal mask)
 *   ORDER     [n_tiles]       tile indices, most KV tiles first (ties by index)
 *   KVTILES   [n_kvtiles*8]   per key tile (backward; together they cover
 *                             every key once): doc, kv_global_start, n_keys,
 *                             q_tile_begin, q_tile_end (the query tiles that
 *                             see the tile, empty for unseen keys), 0, 0, 0
 *   ITEMS     [n_items*4]     forward work items, longest first: tile,
 *                             kv_tile_begin, kv_tile_end, part slot (-1 when
 *                             the tile is not split)
 *   SPLITS    [n_splits*4]    tiles whose key range is split: tile, first part
 *                             slot, number of parts, 0
 *   DOC_END   [n_docs]        global position one past each document's last
 *                             real token (cu_i + L_i without padding; see
 *                             thd_build_metadata_padded)
 *   PACK_ROWS [n_pack_rows*4] packed plans (thd_build_packed_metadata): per row
 *                             of the packed tiles, in tile order: local row,
 *                             first and last key slot it sees, 1 if real
 *                             (0 for a pad row)
 *   PACK_KEYS [n_pack_keys]   packed plans: gathered row of each key slot;
 *                             each packed tile's slots start at its
 *                             kv_start and fill n_kv_tiles whole KV tiles
 * With concurrency C > 0 (work items of one kv head the device runs at once)
 * and fewer than 2C tiles, the key range of tiles longer than
 * kv_split = max(ceil(sum of n_kv_tiles / C), 8) KV tiles is cut into
 * min(ceil(n_kv_tiles / kv_split), n_full_kv_tiles) near-equal parts, every
 * part starting with a KV tile its rows see whole; the forward merges the
 * parts' partial results. */
enum {
  THD_FIELD_Q_GLOBAL = 0,
  THD_FIELD_KV_ROW = 1,
  THD_FIELD_CHUNK_OFF = 2,
  THD_FIELD_TILES = 3,
  THD_FIELD_ORDER = 4,
  THD_FIELD_KVTILES = 5,
  THD_FIELD_ITEMS = 6,
  THD_FIELD_SPLITS = 7,
  THD_FIELD_DOC_END = 8,
  THD_FIELD_PACK_ROWS = 9,
  THD_FIELD_PACK_KEYS = 10
};

typedef struct thd_meta thd_meta;   /* opaque, library-owned, reference-counted */

typedef struct {
  int64_t total_tokens;     /* T */
  int64_t local_tokens;     /* T / cp */
  int64_t n_tiles;
  int64_t n_kvtiles;
  int64_t useful_pairs;     /* visible (local query, key) pairs: sum L_i (L_i + 1) / (2cp) */
  int64_t max_kv_tiles;     /* largest n_kv_tiles of any tile */
  int64_t n_items;          /* forward work items */
  int64_t n_splits;         /* tiles whose key range is split */
  int64_t n_part_slots;     /* partial-result slots (sum of parts over split tiles) */
  int64_t pad_tokens;       /* pad tokens over all documents (0 without padding) */
  int32_t concurrency, kv_split;
  int32_t n_docs, cp, rank, block_t, block_n, version;
  int32_t device;           /* device holding the uploaded copy, -1 = host only */
  int32_t cache_hit;        /* 1 if this handle came from the cache */
  int32_t is_pass;          /* 1 for a pass plan (thd_build_pass_metadata) */
  int32_t item_ints;        /* ints per ITEMS record: 4, or 8 for a pass plan */
  uint64_t shard_mask;      /* pass plans: bit s set = keys of rank s's shard */
  int64_t n_packed_tiles;   /* packed plans: tiles made of several partial tiles */
  int64_t n_pack_rows;      /* packed plans: rows of the packed tiles (PACK_ROWS) */
  int64_t n_pack_keys;      /* packed plans: key slots (PACK_KEYS) */
  int32_t is_packed;        /* 1 for a packed plan (thd_build_packed_metadata) */
  int32_t reserved;
} thd_meta_info_t;

/* Message for the calling thread's last failed call ("" if none). An
 * interface convention of this library: the pages define no error interface. */
const char* thd_last_error(void);

/* Symmetric EOD-aware partition of a packed batch for one rank.
 * Source: "feat: kvallgather cp thd load balance #3820" (Ascend/MindSpeed),
 * "What this PR does / why we need it?" (EOD-aware symmetric partitioning,
 * rank-major K/V) and "Does this PR introduce any user-facing change?" (every
 * subsequence length divisible by 2 * context-parallel size).
 *   seqlens[n_docs]: packed subsequence lengths (host, int32, each >= 1 and
 *   divisible by 2*cp). Writes T and T_local, and any of the host arrays that
 *   are non-NULL: q_global[T_local], kv_row[T], chunk_off[n_docs*2*cp]
 *   (layouts as for THD_FIELD_*). Errors: THD_EINVAL, THD_ENOTDIV, THD_ERANGE. */
int thd_plan_partition(const int32_t* seqlens, int32_t n_docs, int32_t cp, int32_t rank,
                       int64_t* total_tokens, int64_t* local_tokens,
                       int32_t* q_global, int32_t* kv_row, int32_t* chunk_off);

/* Source: "feat: kvallgather cp thd load balance #3820", "What this PR does /
 * why we need it?" (metadata cached to avoid recomputing it every call). The
 * tile tables are this library's own plan for the kernels.
 * Build (or fetch from the cache) the metadata of one rank's attention: the
 * partition maps, per-tile document/causal bounds for block_t query tokens by
 * block_n keys, the largest-first tile order, the forward work items (see
 * THD_FIELD_ITEMS; concurrency >= 0, 0 = never split a tile) and the backward
 * key tiles. device >= 0 also uploads the arrays to that device (once per
 * cache entry); device = -1 builds host arrays only. The cache key holds every
 * input (all lengths, cp, rank, block sizes, concurrency, contract version,
 * device). On success *out is a new reference: release it with
 * thd_meta_release. */
int thd_build_metadata(const int32_t* seqlens, int32_t n_docs, int32_t cp, int32_t rank,
                       int32_t block_t, int32_t block_n, int32_t concurrency, int32_t device,
                       thd_meta** out);

/* Padding-tolerant partitioning. It relaxes the divisibility rule of "feat:
 * kvallgather cp thd load balance #3820", "Does this PR introduce any
 * user-facing change?", which this library keeps for thd_build_metadata. A
 * document of R_i >= 1 real tokens is stored padded to
 * L_i = ceil(R_i / (2*cp)) * 2*cp tokens: its R_i real tokens first, then
 * L_i - R_i pad tokens (any finite values). The padded batch is partitioned,
 * gathered and laid out exactly like an unpadded one of lengths L_i
 * (thd_plan_partition with those lengths gives the maps). Pads follow every real token of their
 * document, so the causal mask already hides them from real queries: real rows
 * get exactly the attention of the unpadded documents. Pad rows get O = 0 and
 * LSE = +inf (so exp(S - LSE) = 0: the backward gives pad rows dQ = 0 whatever
 * dO holds there, and pad keys dK = dV = 0).
 * thd_pad_lengths writes L_i into padded[n_docs] (host). Errors: THD_EINVAL
 * (NULL pointer, n_docs < 1, a length < 1), THD_ERANGE (cp < 1 or a padded
 * length beyond int32). */
int thd_pad_lengths(const int32_t* real_lengths, int32_t n_docs, int32_t cp, int32_t* padded);

/* thd_build_metadata for the padded layout of real_lengths[n_docs] (host):
 * the arrays of the padded lengths L_i, plus DOC_END = cu_i + R_i. The cache
 * key holds the real lengths. */
int thd_build_metadata_padded(const int32_t* real_lengths, int32_t n_docs, int32_t cp,
                              int32_t rank, int32_t block_t, int32_t block_n,
                              int32_t concurrency, int32_t device, thd_meta** out);

/* Short-segment packing: a forward plan whose last, partial query tiles of
 * consecutive chunks are grouped into packed tiles. Reading of the per-row
 * [start, end) key bounds of the FlashMask kernels on "[Optim] FlashMask-4
 * Overlap support part 1 (NVSHMEM backend) - #166", applied to the documents
 * of "feat: kvallgather cp thd load balance #3820". Plain tiles are those of
 * thd_build_metadata; the partial tiles (fewer than block_t rows) are taken
 * in tile order and a tile joins the open group while the group holds at most
 * block_t rows and at most block_n * K key slots, K = max_kv_tiles or, when
 * the plain tiles would be split (see THD_FIELD_ITEMS), the smaller of it and
 * their kv_split: packed tiles are never split. (A tile of the same document
 * as the group's previous member adds only the keys past that member's.) Each group of two or more becomes one packed tile, listed after
 * the plain ones: TILES record [-1, first PACK_ROWS row, rows, -1, -1, first
 * PACK_KEYS slot, n_kv_tiles, 0]. Its documents' keys take consecutive slots,
 * one document after the other, and each row sees exactly its causal keys as
 * one window of slots. ORDER and ITEMS are formed over this tile list as in
 * thd_build_metadata (packed tiles are never split). The result is the same
 * attention as the plain plan's, with fewer workgroups when many documents
 * end in short tiles. Forward only: thd_attn_bwd refuses it (no KVTILES).
 *   lengths[n_docs]: as seqlens of thd_build_metadata (padded = 0), or as
 *   real_lengths of thd_build_metadata_padded (padded = 1). Other arguments,
 *   the cache and the errors as thd_build_metadata, plus THD_EINVAL for padded
 *   not 0 or 1. */
int thd_build_packed_metadata(const int32_t* lengths, int32_t n_docs, int32_t cp, int32_t rank,
                              int32_t block_t, int32_t block_n, int32_t concurrency,
                              int32_t padded, int32_t device, thd_meta** out);

/* Sizes and counters of a metadata object (see thd_meta_info_t); the
 * metadata of "feat: kvallgather cp thd load balance #3820", "What this PR
 * does / why we need it?". Errors: THD_EINVAL (NULL meta or info). */
int thd_meta_info(const thd_meta* meta, thd_meta_info_t* info);

/* Copy count int32 values of a field (THD_FIELD_*) into host memory dst;
 * count must equal the field's length (THD_EINVAL otherwise, or for an
 * unknown field or NULL dst). Exposes the cached metadata ("feat:
 * kvallgather cp thd load balance #3820", "What this PR does / why we need
 * it?") for bit-exact checks. */
int thd_meta_copy(const thd_meta* meta, int32_t field, int32_t* dst, int64_t count);

/* Drop one reference (NULL is ignored). The entry stays cached until evicted
 * (least recently used, 64 entries); device memory is freed when the last
 * reference to an evicted entry goes. */
void thd_meta_release(thd_meta* meta);

/* Metadata cache ("feat: kvallgather cp thd load balance #3820", "What this
 * PR does / why we need it?": metadata caching). Counters since the last
 * clear (any output may be NULL); thd_cache_clear drops every cached entry
 * that no caller still holds. */
int thd_cache_stats(int64_t* hits, int64_t* misses, int64_t* uploads, int64_t* entries);
int thd_cache_clear(void);

/* Head shapes of "feat: kvallgather cp thd load balance #3820", "What this
 * PR does / why we need it?" (MHA, GQA, expanded MLA).
 * Tile sizes the kernels expect for a head shape: block_t query tokens per
 * tile and block_n keys per KV tile. THD_EUNSUPPORTED if no kernel exists.
 * These sizes serve the forward and the backward alike. */
int thd_preferred_tiles(int32_t hq, int32_t hkv, int32_t d_qk, int32_t d_v,
                        int32_t* block_t, int32_t* block_n);

/* The tile choice of this library for the forward of "feat: kvallgather cp
 * thd load balance #3820" (single fused attention call, causal with EOD
 * reset). Tile sizes for the forward of one batch (seqlens[n_docs] as laid out, i.e.
 * padded lengths for the padded layout; host). The forward also has 32-key
 * tile kernels for d_qk <= 128, run three workgroups per CU instead of two.
 * They are chosen (block_n = 32) when they compute at least 7% fewer key
 * slots than 64-key tiles: a query tile visits its document's keys up to its
 * last row, rounded up to whole KV tiles, so short chunks leave most of a
 * 64-key tile masked. They are also chosen when concurrency32 > 0 (the
 * device's thd_fwd_concurrency for block_n = 32; 0 skips this rule), query
 * tiles hold at most 32 tokens (Hq/Hkv >= 4) and the batch has at least
 * 2 * concurrency32 query tiles, so that no tile's key range is split: a
 * large grid of short query tiles then gains from the third workgroup per CU.
 * Otherwise block_n = 64. block_t as thd_preferred_tiles. Metadata built with
 * block_n = 32 serves thd_attn_fwd only: thd_attn_bwd needs block_n = 64
 * (THD_EMISMATCH otherwise). Errors as thd_plan_partition, plus
 * THD_EUNSUPPORTED and THD_EINVAL (concurrency32 < 0). */
int thd_preferred_fwd_tiles(const int32_t* seqlens, int32_t n_docs, int32_t cp, int32_t rank,
                            int32_t hq, int32_t hkv, int32_t d_qk, int32_t d_v,
                            int32_t concurrency32, int32_t* block_t, int32_t* block_n);

/* Scheduling input of this library's planner (no page passage; it balances
 * the single fused forward call of "feat: kvallgather cp thd load balance
 * #3820" over the device). Forward work items of one kv head to plan for on a device: its CUs times
 * the forward workgroups per CU for this KV tile size (2 for block_n = 64, 3
 * for 32), times 7/8, over hkv (at least 1). The 7/8 leaves the split parts
 * slightly longer, which measured faster than filling every slot. Pass it as
 * thd_build_metadata's concurrency. Errors: THD_EINVAL (hkv < 1, block_n not 32 or 64, NULL
 * output, no such device), THD_EHIP. */
int thd_fwd_concurrency(int32_t device, int32_t hkv, int32_t block_n, int32_t* concurrency);

/* Bytes of device workspace thd_attn_fwd needs for the partial results of
 * split tiles (0 when no tile is split). Errors: THD_EINVAL (NULL meta or
 * bytes, bad head counts, d_v < 1). */
int thd_attn_fwd_workspace(const thd_meta* meta, int32_t hq, int32_t hkv, int32_t d_v,
                           int64_t* bytes);

/* Forward: o and lse for every local query row and q head.
 * Source: "feat: kvallgather cp thd load balance #3820", "What this PR does /
 * why we need it?" (THD attention with direct rank-major K/V indexing in a
 * single fused call; MHA, GQA, expanded MLA) and "Does this PR introduce any
 * user-facing change?" (causal attention with the mask reset at every EOD).
 * meta must come from thd_build_metadata (or thd_build_metadata_padded, or
 * thd_build_packed_metadata) with the tile sizes of thd_preferred_tiles or
 * thd_preferred_fwd_tiles and the current device.
 * softmax_scale >= 0 and finite; 0 selects 1/sqrt(d_qk). Supported (d_qk, d_v): (64,64), (128,128),
 * (192,128); Hq/Hkv <= 128. q, k, v, o, lse must be 16-byte aligned; k and v
 * must each be smaller than 4 GiB (THD_ERANGE otherwise). workspace (16-byte
 * aligned, at least thd_attn_fwd_workspace bytes; may be NULL when that is 0)
 * holds the split tiles' partial results; the forward allocates nothing.
 * o_f32 (optional, NULL to skip; fp32 [T_local, Hq, d_v], 16-byte aligned):
 * when given, the probabilities enter the P.V product as bf16 (hi, lo) pairs
 * and O is also written here in fp32, exact up to fp32 accumulation. It is
 * meant for training: thd_attn_bwd then takes D = rowsum(dO * O) from it
 * instead of recomputing D from the scores. */
int thd_attn_fwd(const thd_meta* meta, const void* q, const void* k, const void* v,
                 void* o, float* lse, float* o_f32, int32_t hq, int32_t hkv, int32_t d_qk,
                 int32_t d_v, float softmax_scale, void* workspace, int64_t workspace_bytes,
                 void* hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the forward
 * of thd_attn_fwd with the same arguments, checks and results, minus the
 * workspace. The split tiles' partial results go to a file-scope device array
 * of 64 MiB (THD_FWD_NOALLOC_SCRATCH_BYTES), one copy per device, held until
 * the process ends; its device address is looked up once per device, on the
 * first call there. The call allocates nothing: the caller passes every input
 * and output, and the metadata must already be built on this device.
 * THD_ERANGE when the partial results need more than the array holds
 * (thd_attn_fwd_workspace gives the need; build the metadata with a smaller
 * concurrency, or call thd_attn_fwd). Every call on one device shares that
 * device's array, which keeps the last call's contents (no part of it needs
 * to start at zero): calls that overlap on one device, on other streams or
 * threads, race on it and must be serialised by the caller. */
#define THD_FWD_NOALLOC_SCRATCH_BYTES (64ll << 20)
int thd_attn_fwd_noalloc(const thd_meta* meta, const void* q, const void* k, const void* v,
                         void* o, float* lse, float* o_f32, int32_t hq, int32_t hkv,
                         int32_t d_qk, int32_t d_v, float softmax_scale, void* hip_stream);

/* All-gather overlap, shard by shard. Source: "[Optim] FlashMask-4 Overlap
 * support part 1 (NVSHMEM backend) - #166" (PaddlePaddle/flash-attention),
 * feature list: the forward overlapped with the K/V all-gather. Here without
 * any in-kernel waiting: the all-gather of "feat: kvallgather cp thd load
 * balance #3820" delivers rank s's shard (its chunks s and 2cp-1-s of every
 * document, rows [s*T_local, (s+1)*T_local) of the gathered K/V) as a unit, and
 * the caller runs one forward pass per delivered shard (or set of shards), on
 * a stream that waits for the delivery (an event). Passes merge into a running
 * state; the last one writes o and lse, equal to thd_attn_fwd's up to the
 * order of summation.
 *
 * thd_build_pass_metadata: the metadata of a pass over the keys of the source
 * ranks in shard_mask (bit s = rank s; at least one bit, none at or above cp;
 * cp <= 64). Same arguments and cache as thd_build_metadata (the mask is part
 * of the key); block_n must be 64. Its TILES are thd_build_metadata's; ITEMS
 * are 8 ints per work item, [tile, first key, end key (exclusive), part slot,
 * KV tiles, KV tiles every row sees whole, 0, 0], one per maximal run of
 * consecutive chunks the tile's rows see that a listed rank holds, longest
 * first; SPLITS holds [tile, first part slot, parts, 0] for every tile.
 * Errors as thd_build_metadata, plus THD_EINVAL (bad mask), THD_ERANGE (cp > 64). */
int thd_build_pass_metadata(const int32_t* seqlens, int32_t n_docs, int32_t cp, int32_t rank,
                            int32_t block_t, int32_t block_n, uint64_t shard_mask,
                            int32_t device, thd_meta** out);

/* thd_build_pass_metadata for the padded layout of real_lengths[n_docs] (host),
 * as thd_build_metadata_padded is for thd_build_metadata: the pass plan of the
 * padded lengths, plus DOC_END = cu_i + R_i, which the last pass reads to write
 * pad rows as O = 0, LSE = +inf. Sources: as thd_build_pass_metadata, and the
 * divisibility rule of "feat: kvallgather cp thd load balance #3820" ("Does
 * this PR introduce any user-facing change?") relaxed by padding as in
 * thd_pad_lengths. Errors as thd_build_pass_metadata and thd_pad_lengths. */
int thd_build_pass_metadata_padded(const int32_t* real_lengths, int32_t n_docs, int32_t cp,
                                   int32_t rank, int32_t block_t, int32_t block_n,
                                   uint64_t shard_mask, int32_t device, thd_meta** out);

/* Bytes of running state the passes of one forward share (the caller's;
 * fp32 O [T_local, Hq, d_v] then its base-2 log-sum-exp [T_local, Hq]). A
 * pass needs no other workspace. Source: as thd_build_pass_metadata.
 * Errors: THD_EINVAL (bad heads, d_v < 1, NULL state_bytes), THD_EMISMATCH
 * (not a pass plan). */
int thd_attn_fwd_pass_state_bytes(const thd_meta* meta, int32_t hq, int32_t hkv, int32_t d_v,
                                  int64_t* state_bytes);

#define THD_PASS_FIRST 1   /* the state holds nothing yet (its contents are ignored) */
#define THD_PASS_LAST 2    /* write o and lse instead of the state */

/* One pass: attention of every local row over the keys of the pass's shards,
 * merged (log-sum-exp weights) into the state; with THD_PASS_LAST the merged
 * result is written to o (bf16) and lse (natural log) instead. Rows that saw
 * no key in any pass so far hold an empty state (lse -inf; written as O = 0,
 * LSE = -inf by a last pass). One workgroup per query tile and kv head walks
 * all of the tile's runs in the pass and merges straight into the state, so a
 * pass allocates nothing and launches one kernel. Arguments and layouts as
 * thd_attn_fwd (o and lse may be NULL unless THD_PASS_LAST); state (16-byte
 * aligned, thd_attn_fwd_pass_state_bytes long). Every key a pass reads lies in
 * its shards' rows of k and v, so the other rows may still be in flight.
 * Passes of one forward run in order on one stream (each reads the state the
 * last one wrote). Errors as thd_attn_fwd, plus THD_EMISMATCH (metadata not a
 * pass plan) and THD_EINVAL (unknown flags). */
int thd_attn_fwd_pass(const thd_meta* meta, const void* q, const void* k, const void* v,
                      void* o, float* lse, float* state, int32_t flags, int32_t hq,
                      int32_t hkv, int32_t d_qk, int32_t d_v, float softmax_scale,
                      void* hip_stream);

/* Bytes of device workspace thd_attn_bwd needs (caller allocates): D and
 * the base-2 log-sum-exp, two fp32 [T_local, Hq] arrays. Errors: THD_EINVAL. */
int thd_attn_bwd_workspace(const thd_meta* meta, int32_t hq, int64_t* bytes);

/* Backward of thd_attn_fwd. The pages give no backward formula; the
 * gradients are those of the forward's definition, and dk, dv in the gathered
 * layout are what the all-gather's backward (a reduce-scatter over the ranks;
 * "[Optim] FlashMask-4 Overlap support part 1 (NVSHMEM backend) - #166",
 * feature list: reduce-scatter in the backward) sums to their owners.
 * softmax_scale as for thd_attn_fwd (0 selects 1/sqrt(d_qk)); same head
 * dims, alignment and size limits; metadata with block_n = 64, not a pass
 * plan nor a packed plan (THD_EMISMATCH).
 * Backward: dq, and this rank's partial dk, dv (all fp32, layouts above),
 * from the forward's lse and the upstream gradient d_o. dk and dv are written
 * in full (zeros for keys no local query sees). The softmax-gradient term
 * D = rowsum(dO * O) needs O exact: it is taken from o_f32 (the forward's
 * fp32 output, see thd_attn_fwd; 16-byte aligned) when that is not NULL, and
 * otherwise recomputed as rowsum(P * dP) from the scores (one more pass over
 * the keys), since the forward's bf16 o would make D's rounding the largest
 * error in the gradients. The workspace (size from thd_attn_bwd_workspace,
 * 16-byte aligned) holds D and the log-sum-exp in base 2 for every local row
 * and q head. */
int thd_attn_bwd(const thd_meta* meta, const void* q, const void* k, const void* v,
                 const float* lse, const float* o_f32, const void* d_o,
                 float* dq, float* dk, float* dv,
                 int32_t hq, int32_t hkv, int32_t d_qk, int32_t d_v, float softmax_scale,
                 void* workspace, int64_t workspace_bytes, void* hip_stream);

/* thd_attn_bwd with this rank's partial dk and dv written in bf16: the same
 * fp32 results rounded to nearest even, in the same layouts, so that the
 * reduce-scatter which sums the ranks' partials ("[Optim] FlashMask-4 Overlap
 * support part 1 (NVSHMEM backend) - #166", feature list: reduce-scatter
 * overlapped with the backward) moves half the bytes. Each partial then
 * carries a rounding error of up to 2^-9 of its magnitude into that sum. dq
 * stays fp32 (it never leaves the rank). dk: bf16 [T, Hkv, d_qk], dv: bf16
 * [T, Hkv, d_v], 16-byte aligned; every other argument, the workspace and the
 * errors as thd_attn_bwd. */
int thd_attn_bwd_bf16kv(const thd_meta* meta, const void* q, const void* k, const void* v,
                        const float* lse, const float* o_f32, const void* d_o,
                        float* dq, void* dk, void* dv,
                        int32_t hq, int32_t hkv, int32_t d_qk, int32_t d_v, float softmax_scale,
                        void* workspace, int64_t workspace_bytes, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* THDATTN_H */
