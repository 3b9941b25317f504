// Internal declarations shared by the host planner, the cache, the C ABI and
// the kernel launchers. Not part of the public interface.
#pragma once

#include <cstdint>
#include <memory>
#include <string>
#include <vector>

#include "thdattn.h"

namespace thd {

// Error carrying a thd_status code; converted to a return value at the ABI.
struct Error {
  int code;
  std::string msg;
};

[[noreturn]] void fail(int code, const std::string& msg);

// Host-side plan and tile tables for one (lengths, cp, rank, block_t, block_n).
// Field meanings are documented with THD_FIELD_* in thdattn.h.
struct Plan {
  std::vector<int32_t> seqlens;   // stored (padded) lengths
  std::vector<int32_t> real;      // real lengths (equal to seqlens without padding)
  int32_t cp = 1, rank = 0, block_t = 1, block_n = 1, concurrency = 0, kv_split = 0;
  int64_t total = 0, local = 0, useful_pairs = 0, max_kv_tiles = 0, n_part_slots = 0;
  int64_t pad_tokens = 0;
  // A pass plan (all-gather overlap) covers only the keys of the source ranks
  // in shard_mask: its items are 8 ints with absolute key ranges, and splits
  // holds one [tile, first part slot, parts, 0] record per tile. For the
  // kernel: pass_runs lists the items by part slot (so a tile's runs are
  // consecutive), pass_order the tiles with runs, most KV tiles first, then
  // the tiles without (n_run_tiles of the former).
  bool pass = false;
  uint64_t shard_mask = 0;
  std::vector<int32_t> pass_runs, pass_order;
  int64_t n_run_tiles = 0;
  // A packed plan (short-segment packing) also lists packed tiles
  // (q_local_start = -1): their rows in pack_rows [local row, first slot, last
  // slot, real] and their key slots' gathered rows in pack_keys. It has no
  // backward key tiles.
  bool packed = false;
  int64_t n_packed = 0;
  // For the dK/dV kernel: the key tiles ordered by how many local query
  // tokens see them, most first (stable), so the longest workgroups start
  // first (a scheduling choice; every key tile writes only its own rows).
  std::vector<int32_t> kv_order;
  std::vector<int32_t> q_global, kv_row, chunk_off, tiles, order, kvtiles, items, splits, doc_end;
  std::vector<int32_t> pack_rows, pack_keys;
  int item_ints() const { return pass ? 8 : 4; }
};

// Checks lengths/cp/rank; throws Error. Returns T.
int64_t validate_partition(const int32_t* seqlens, int32_t n_docs, int32_t cp, int32_t rank);

// Fills q_global / kv_row / chunk_off (any may be null) for validated input.
void plan_partition(const int32_t* seqlens, int32_t n_docs, int32_t cp, int32_t rank,
                    int32_t* q_global, int32_t* kv_row, int32_t* chunk_off);

// Builds the full plan (partition maps + tile tables). real_lengths (may be
// null: no padding) gives each document's real tokens, 1 <= R_i <= L_i.
// packed: group the partial tiles of consecutive documents into packed tiles
// before the order and the work items are formed (see pack_partial_tiles).
std::unique_ptr<Plan> build_plan(const int32_t* seqlens, int32_t n_docs, int32_t cp,
                                 int32_t rank, int32_t block_t, int32_t block_n,
                                 int32_t concurrency, const int32_t* real_lengths,
                                 bool packed = false);

// The plan of one forward pass over the keys held by the source ranks in
// shard_mask (bit s = rank s's shard): same tiles, items over maximal runs of
// such chunks (see build_pass_plan). real_lengths as for build_plan.
std::unique_ptr<Plan> build_pass_plan(const int32_t* seqlens, int32_t n_docs, int32_t cp,
                                      int32_t rank, int32_t block_t, int32_t block_n,
                                      uint64_t shard_mask, const int32_t* real_lengths);

// Device copies of the arrays the kernels read.
struct DeviceMeta {
  int device = -1;
  void* base = nullptr;          // one allocation holding every array
  const int32_t* kv_row = nullptr;
  const int32_t* tiles = nullptr;
  const int32_t* order = nullptr;
  const int32_t* kvtiles = nullptr;
  const int32_t* q_global = nullptr;
  const int32_t* items = nullptr;
  const int32_t* splits = nullptr;
  const int32_t* doc_end = nullptr;
  const int32_t* pack_rows = nullptr;
  const int32_t* pack_keys = nullptr;
  const int32_t* pass_runs = nullptr;
  const int32_t* pass_order = nullptr;
  const int32_t* kv_order = nullptr;
};

struct MetaEntry {
  std::unique_ptr<Plan> plan;
  DeviceMeta dev;
  ~MetaEntry();
};

}  // namespace thd

// The opaque handle handed out at the ABI: one reference to a cache entry.
struct thd_meta {
  std::shared_ptr<thd::MetaEntry> entry;
  bool cache_hit = false;
};

namespace thd {

// Fixed kernel geometry: 4 waves of 64 lanes, 32 query rows per wave, and
// 64-key KV tiles.
constexpr int kWaves = 4;
constexpr int kRowsPerWg = 128;
constexpr int kBlockN = 64;
// The forward also runs 32-key tiles (d_qk <= 128), three workgroups per CU:
// for batches of short documents, whose query tiles see few KV tiles.
constexpr int kBlockNShort = 32;

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* o_f32;       // optional fp32 copy of O (split P in the PV product); null to skip
  float* partial;     // workspace: per (part slot, kv head) O rows (fp32) then their lse
                      // (split tiles of a one-pass plan)
  const int32_t* tiles;
  const int32_t* items;
  const int32_t* splits;
  const int32_t* kv_row;
  const int32_t* doc_end;   // per document: one past its last real token
  int32_t n_items, n_splits, hq, hkv, group, block_t, block_n;
  int64_t total;
  float scale_log2;   // softmax_scale * log2(e)
  // Pass plans only: the running state (O [T_local, Hq, d_v] fp32 then its
  // log2-sum-exp [T_local, Hq]), the THD_PASS_FIRST / THD_PASS_LAST flags,
  // each tile's runs (pass_runs, 8 ints each, from splits' first slot) and
  // the tiles to run (pass_order; n_items of them).
  int32_t ranged, pass_flags;
  float* state;
  int64_t local;
  const int32_t* pass_runs;
  const int32_t* pass_order;
  // Packed plans only: rows [local row, first slot, last slot, real] of the
  // packed tiles, and each key slot's gathered row.
  int32_t packed;
  const int32_t* pack_rows;
  const int32_t* pack_keys;
};

#if defined(__HIPCC__)
#define THD_HOST_DEVICE __host__ __device__
#else
#define THD_HOST_DEVICE
#endif

// Floats of forward workspace per (part slot, kv head): the part's O rows
// (rows * d_v) then its per-row log2-sum-exp (rows), padded to a multiple of 4
// so every slot starts 16-byte aligned.
THD_HOST_DEVICE inline int64_t fwd_partial_floats(int32_t block_t, int32_t group, int32_t d_v) {
  return (int64_t(block_t) * group * (d_v + 1) + 3) / 4 * 4;
}

// Bytes of the file-scope device array that thd_attn_fwd_noalloc uses as the
// forward's workspace (one copy per device).
constexpr int64_t kFwdStaticScratchBytes = THD_FWD_NOALLOC_SCRATCH_BYTES;

// Device address of that array on `device`, which must be the current device;
// looked up on the first call per device. Returns a hipError_t value.
int fwd_static_scratch(int device, void** ptr);

// Kernel launchers (defined in the .hip files). Return a hipError_t value.
int launch_fwd(const FwdParams& p, int d_qk, int d_v, void* stream);
// One forward pass of a pass plan: each listed tile walks its runs and merges
// its result into the running state.
int launch_fwd_pass(const FwdParams& p, int d_qk, int d_v, void* stream);
// Workgroups of the forward kernel for this KV tile size that fit one CU.
int fwd_workgroups_per_cu(int block_n);

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const float* lse;
  const float* o_f32;   // optional exact O (fp32); D = rowsum(dO * O) from it when given
  const void* d_o;
  float* dq;
  void* dk;           // fp32, or bf16 when kv_bf16
  void* dv;
  float* delta;       // workspace: D [T_local, Hq]
  float* lse2;        // workspace: lse * log2(e) [T_local, Hq]
  const int32_t* tiles;
  const int32_t* order;      // dQ workgroup b takes query tile order[b / hkv] (largest first)
  const int32_t* kvtiles;
  const int32_t* kv_order;   // dK/dV workgroup b takes key tile kv_order[b / hkv]
  const int32_t* kv_row;
  int32_t n_tiles, n_kvtiles, hq, hkv, group, block_t;
  int32_t kv_bf16;    // dk, dv stored as bf16 (round to nearest even) instead of fp32
  int64_t total, local;
  float scale;        // softmax_scale
  float scale_log2;   // softmax_scale * log2(e)
};

// Bytes of one [T_local, Hq] fp32 array in the backward workspace, padded so
// the next array starts 256-byte aligned; the workspace holds two (D, lse2).
inline int64_t bwd_ws_array_bytes(int64_t local, int32_t hq) {
  return (local * hq * int64_t(sizeof(float)) + 255) / 256 * 256;
}

int launch_bwd(const BwdParams& p, int d_qk, int d_v, void* stream);
bool bwd_supported(int d_qk, int d_v);
bool fwd_supported(int d_qk, int d_v);
// Whether the forward has a kernel for this KV tile size and d_qk.
bool fwd_block_n_supported(int d_qk, int block_n);

}  // namespace thd
