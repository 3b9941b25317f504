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
#define THD_META_VERSION 3

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
  THD_FIELD_DOC_END = 8
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
} thd_meta_info_t;

/* Message for the calling thread's last failed call ("" if none). */
const char* thd_last_error(void);

/* Symmetric EOD-aware partition of a packed batch for one rank.
 *   seqlens[n_docs]: packed subsequence lengths (host, int32, each >= 1 and
 *   divisible by 2*cp). Writes T and T_local, and any of the host arrays that
 *   are non-NULL: q_global[T_local], kv_row[T], chunk_off[n_docs*2*cp]
 *   (layouts as for THD_FIELD_*). Errors: THD_EINVAL, THD_ENOTDIV, THD_ERANGE. */
int thd_plan_partition(const int32_t* seqlens, int32_t n_docs, int32_t cp, int32_t rank,
                       int64_t* total_tokens, int64_t* local_tokens,
                       int32_t* q_global, int32_t* kv_row, int32_t* chunk_off);

/* Build (or fetch from the cache) the metadata of one rank's attention: the
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

/* Padding-tolerant partitioning (relaxes the divisibility rule above). A
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

int thd_meta_info(const thd_meta* meta, thd_meta_info_t* info);

/* Copy count int32 values of a field (THD_FIELD_*) into host memory dst;
 * count must equal the field's length. */
int thd_meta_copy(const thd_meta* meta, int32_t field, int32_t* dst, int64_t count);

/* Drop one reference (NULL is ignored). */
void thd_meta_release(thd_meta* meta);

/* Cache counters since the last clear; thd_cache_clear drops every cached
 * entry that no caller still holds. */
int thd_cache_stats(int64_t* hits, int64_t* misses, int64_t* uploads, int64_t* entries);
int thd_cache_clear(void);

/* Tile sizes the kernels expect for a head shape: block_t query tokens per
 * tile and block_n keys per KV tile. THD_EUNSUPPORTED if no kernel exists.
 * These sizes serve the forward and the backward alike. */
int thd_preferred_tiles(int32_t hq, int32_t hkv, int32_t d_qk, int32_t d_v,
                        int32_t* block_t, int32_t* block_n);

/* Tile sizes for the forward of one batch (seqlens[n_docs] as laid out, i.e.
 * padded lengths for the padded layout; host). The forward also has 32-key
 * tile kernels for d_qk <= 128, run three workgroups per CU instead of two.
 * They are chosen (block_n = 32) when they compute at least 7% fewer key
 * slots than 64-key tiles: a query tile visits its document's keys up to its
 * last row, rounded up to whole KV tiles, so short chunks leave most of a
 * 64-key tile masked. Otherwise block_n = 64. block_t as thd_preferred_tiles.
 * Metadata built with block_n = 32 serves thd_attn_fwd only: thd_attn_bwd
 * needs block_n = 64 (THD_EMISMATCH otherwise). Errors as
 * thd_plan_partition, plus THD_EUNSUPPORTED. */
int thd_preferred_fwd_tiles(const int32_t* seqlens, int32_t n_docs, int32_t cp, int32_t rank,
                            int32_t hq, int32_t hkv, int32_t d_qk, int32_t d_v, int32_t* block_t,
                            int32_t* block_n);

/* Forward work items of one kv head to plan for on a device: its CUs times
 * the forward workgroups per CU for this KV tile size (2 for block_n = 64, 3
 * for 32), times 7/8, over hkv (at least 1). The 7/8 leaves the split parts
 * slightly longer, which measured faster than filling every slot. Pass it as
 * thd_build_metadata's concurrency. Errors: THD_EINVAL (hkv < 1, block_n not 32 or 64, NULL
 * output, no such device), THD_EHIP. */
int thd_fwd_concurrency(int32_t device, int32_t hkv, int32_t block_n, int32_t* concurrency);

/* Bytes of device workspace thd_attn_fwd needs for the partial results of
 * split tiles (0 when no tile is split). */
int thd_attn_fwd_workspace(const thd_meta* meta, int32_t hq, int32_t hkv, int32_t d_v,
                           int64_t* bytes);

/* Forward: o and lse for every local query row and q head.
 * meta must come from thd_build_metadata with the tile sizes of
 * thd_preferred_tiles or thd_preferred_fwd_tiles and the current device. softmax_scale > 0 (callers
 * usually pass 1/sqrt(d_qk)). Supported (d_qk, d_v): (64,64), (128,128),
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

/* Bytes of device workspace thd_attn_bwd needs (caller allocates). */
int thd_attn_bwd_workspace(const thd_meta* meta, int32_t hq, int64_t* bytes);

/* Backward: dq, and this rank's partial dk, dv (all fp32, layouts above),
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

#ifdef __cplusplus
}
#endif

#endif /* THDATTN_H */
