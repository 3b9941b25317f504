// The C ABI: argument checks, the metadata cache, and kernel launches.
//
// Metadata is cached because it depends only on the packed lengths, cp, rank
// and tile sizes, which repeat from step to step ("kvallgather cp thd load
// balance", Ascend/MindSpeed, "What this PR does / why we need it?": metadata
// caching to avoid repeated calculations). The key holds every input that
// changes the arrays (the full length list, not just T or the document
// count), plus the contract version and the device of the uploaded copy.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <list>
#include <mutex>
#include <new>
#include <string>
#include <unordered_map>

#include "internal.h"

namespace thd {
namespace {

thread_local std::string g_last_error;

template <class F>
int guarded(F&& body) {
  try {
    body();
    return THD_OK;
  } catch (const Error& e) {
    g_last_error = e.msg;
    return e.code;
  } catch (const std::bad_alloc&) {
    g_last_error = "host allocation failed";
    return THD_ENOMEM;
  } catch (...) {
    g_last_error = "unexpected internal error";
    return THD_EINVAL;
  }
}

void check_hip(hipError_t err, const char* what) {
  if (err != hipSuccess)
    fail(err == hipErrorOutOfMemory ? THD_ENOMEM : THD_EHIP,
         std::string(what) + ": " + hipGetErrorString(err));
}

// Restores the caller's current device when it goes out of scope.
struct DeviceScope {
  int saved = -1;
  explicit DeviceScope(int device) {
    check_hip(hipGetDevice(&saved), "hipGetDevice");
    if (saved != device) check_hip(hipSetDevice(device), "hipSetDevice");
  }
  ~DeviceScope() {
    int now = -1;
    if (hipGetDevice(&now) == hipSuccess && now != saved && saved >= 0) (void)hipSetDevice(saved);
  }
};

void upload(MetaEntry& e, int device) {
  const Plan& p = *e.plan;
  DeviceScope scope(device);
  constexpr int kParts = 13;
  const std::vector<int32_t>* parts[kParts] = {&p.kv_row,    &p.tiles,     &p.order,
                                               &p.kvtiles,   &p.q_global,  &p.items,
                                               &p.splits,    &p.doc_end,   &p.pack_rows,
                                               &p.pack_keys, &p.pass_runs, &p.pass_order,
                                               &p.kv_order};
  size_t offs[kParts];
  size_t bytes = 0;
  for (int i = 0; i < kParts; ++i) {
    offs[i] = bytes;
    bytes += (parts[i]->size() * sizeof(int32_t) + 255) / 256 * 256;
  }
  void* base = nullptr;
  check_hip(hipMalloc(&base, bytes == 0 ? 256 : bytes), "hipMalloc(metadata)");
  std::vector<char> staging(bytes);
  for (int i = 0; i < kParts; ++i)
    if (!parts[i]->empty())
      std::memcpy(staging.data() + offs[i], parts[i]->data(), parts[i]->size() * sizeof(int32_t));
  const hipError_t err = hipMemcpy(base, staging.data(), bytes, hipMemcpyHostToDevice);
  if (err != hipSuccess) {
    (void)hipFree(base);
    check_hip(err, "hipMemcpy(metadata)");
  }
  char* b = static_cast<char*>(base);
  e.dev.device = device;
  e.dev.base = base;
  e.dev.kv_row = reinterpret_cast<const int32_t*>(b + offs[0]);
  e.dev.tiles = reinterpret_cast<const int32_t*>(b + offs[1]);
  e.dev.order = reinterpret_cast<const int32_t*>(b + offs[2]);
  e.dev.kvtiles = reinterpret_cast<const int32_t*>(b + offs[3]);
  e.dev.q_global = reinterpret_cast<const int32_t*>(b + offs[4]);
  e.dev.items = reinterpret_cast<const int32_t*>(b + offs[5]);
  e.dev.splits = reinterpret_cast<const int32_t*>(b + offs[6]);
  e.dev.doc_end = reinterpret_cast<const int32_t*>(b + offs[7]);
  e.dev.pack_rows = reinterpret_cast<const int32_t*>(b + offs[8]);
  e.dev.pack_keys = reinterpret_cast<const int32_t*>(b + offs[9]);
  e.dev.pass_runs = reinterpret_cast<const int32_t*>(b + offs[10]);
  e.dev.pass_order = reinterpret_cast<const int32_t*>(b + offs[11]);
  e.dev.kv_order = reinterpret_cast<const int32_t*>(b + offs[12]);
}

// Least-recently-used cache of metadata entries. Entries still referenced by a
// caller's handle outlive their eviction. The cache object is never destroyed,
// so no device memory is freed after the HIP runtime has shut down.
struct Cache {
  std::mutex mu;
  std::unordered_map<std::string, std::shared_ptr<MetaEntry>> map;
  std::list<std::string> lru;  // front: most recently used
  std::unordered_map<std::string, std::list<std::string>::iterator> where;
  int64_t hits = 0, misses = 0, uploads = 0;
  static constexpr size_t kCapacity = 64;
};

Cache& cache() {
  static Cache* c = new Cache;
  return *c;
}

std::string make_key(const int32_t* seqlens, const int32_t* real, int32_t n_docs, int32_t cp,
                     int32_t rank, int32_t block_t, int32_t block_n, int32_t concurrency,
                     int32_t device, bool pass, uint64_t shard_mask, bool packed) {
  const int32_t head[13] = {THD_META_VERSION, cp,     rank,    block_t,
                            block_n,          concurrency, device, n_docs,
                            real != nullptr ? 1 : 0, pass ? 1 : 0, int32_t(shard_mask & 0xffffffffu),
                            int32_t(shard_mask >> 32), packed ? 1 : 0};
  const size_t n = size_t(n_docs) * sizeof(int32_t);
  std::string key(sizeof(head) + (real != nullptr ? 2 : 1) * n, '\0');
  std::memcpy(&key[0], head, sizeof(head));
  std::memcpy(&key[sizeof(head)], seqlens, n);
  if (real != nullptr) std::memcpy(&key[sizeof(head) + n], real, n);
  return key;
}

const MetaEntry& entry_of(const thd_meta* meta) {
  if (meta == nullptr || !meta->entry || !meta->entry->plan) fail(THD_EINVAL, "meta is NULL");
  return *meta->entry;
}

void check_ptr(const void* p, const char* name, size_t align) {
  if (p == nullptr) fail(THD_EINVAL, std::string(name) + " is NULL");
  if (reinterpret_cast<uintptr_t>(p) % align != 0)
    fail(THD_EALIGN, std::string(name) + " is not " + std::to_string(align) + "-byte aligned");
}

const DeviceMeta& device_meta(const MetaEntry& e) {
  if (e.dev.base == nullptr)
    fail(THD_EMISMATCH, "metadata was built without a device copy (device = -1)");
  int cur = -1;
  check_hip(hipGetDevice(&cur), "hipGetDevice");
  if (cur != e.dev.device)
    fail(THD_EMISMATCH, "metadata lives on device " + std::to_string(e.dev.device) +
                            " but the current device is " + std::to_string(cur));
  return e.dev;
}

int preferred_block_t(int32_t group) { return kRowsPerWg / group; }

void check_heads(int32_t hq, int32_t hkv) {
  if (hq < 1 || hkv < 1) fail(THD_EINVAL, "head counts must be >= 1");
  if (hq % hkv != 0) fail(THD_EINVAL, "hq must be a multiple of hkv");
  if (hq / hkv > kRowsPerWg) fail(THD_EUNSUPPORTED, "hq / hkv must be <= 128");
}

// softmax_scale = 0 selects the default 1/sqrt(d_qk), the usual scaling of
// dot-product attention (the subject page gives no scale of its own).
float resolve_scale(float scale, int32_t d_qk) {
  if (!(std::isfinite(scale) && scale >= 0.0f))
    fail(THD_EINVAL, "softmax_scale must be finite and >= 0 (0 = 1/sqrt(d_qk))");
  return scale == 0.0f ? float(1.0 / std::sqrt(double(d_qk))) : scale;
}

void check_rows(const Plan& p, int32_t group) {
  if (int64_t(p.block_t) * group > kRowsPerWg)
    fail(THD_EMISMATCH, "metadata block_t " + std::to_string(p.block_t) + " times group " +
                            std::to_string(group) + " exceeds 128 rows");
}

void check_fwd_tiles(const Plan& p, int32_t group, int32_t d_qk) {
  if (!fwd_block_n_supported(d_qk, p.block_n))
    fail(THD_EMISMATCH, "metadata block_n " + std::to_string(p.block_n) +
                            " has no forward kernel for d_qk=" + std::to_string(d_qk) +
                            " (64, or 32 for d_qk <= 128)");
  check_rows(p, group);
}

void check_bwd_tiles(const Plan& p, int32_t group) {
  if (p.block_n != kBlockN)
    fail(THD_EMISMATCH, "metadata block_n " + std::to_string(p.block_n) + " != backward kernels' " +
                            std::to_string(kBlockN));
  check_rows(p, group);
}

// The kernels address K and V with 32-bit byte offsets.
void check_kv_bytes(int64_t total, int32_t hkv, int32_t d_qk, int32_t d_v) {
  const int64_t row = int64_t(hkv) * 2 * std::max(d_qk, d_v);
  if (total * row >= (int64_t(1) << 32)) fail(THD_ERANGE, "K or V exceeds 4 GiB");
}

// L_i = ceil(R_i / 2cp) * 2cp (see thd_pad_lengths).
void pad_lengths(const int32_t* real, int32_t n_docs, int32_t cp, int32_t* padded) {
  if (real == nullptr || padded == nullptr) fail(THD_EINVAL, "a length array is NULL");
  if (n_docs < 1) fail(THD_EINVAL, "n_docs must be >= 1");
  if (cp < 1) fail(THD_ERANGE, "cp must be >= 1");
  for (int32_t i = 0; i < n_docs; ++i) {
    if (real[i] < 1) fail(THD_EINVAL, "document " + std::to_string(i) + " has length < 1");
    const int64_t two = 2 * int64_t(cp);
    const int64_t l = (int64_t(real[i]) + two - 1) / two * two;
    if (l > INT32_MAX) fail(THD_ERANGE, "padded length beyond int32");
    padded[i] = int32_t(l);
  }
}

// Shared by thd_build_metadata (real = NULL), thd_build_metadata_padded,
// thd_build_pass_metadata (pass) and thd_build_packed_metadata (packed).
void build_metadata_impl(const int32_t* seqlens, const int32_t* real, int32_t n_docs, int32_t cp,
                         int32_t rank, int32_t block_t, int32_t block_n, int32_t concurrency,
                         int32_t device, thd_meta** out, bool pass = false,
                         uint64_t shard_mask = 0, bool packed = false) {
  if (out == nullptr) fail(THD_EINVAL, "out is NULL");
  *out = nullptr;
  validate_partition(seqlens, n_docs, cp, rank);
  if (device < -1) fail(THD_EINVAL, "device must be >= -1");
  if (concurrency < 0) fail(THD_EINVAL, "concurrency must be >= 0");
  if (device >= 0) {
    int count = 0;
    check_hip(hipGetDeviceCount(&count), "hipGetDeviceCount");
    if (device >= count) fail(THD_EINVAL, "no such device " + std::to_string(device));
  }
  const std::string key = make_key(seqlens, real, n_docs, cp, rank, block_t, block_n,
                                   concurrency, device, pass, shard_mask, packed);
  Cache& c = cache();
  std::lock_guard<std::mutex> lock(c.mu);
  auto hit = c.map.find(key);
  auto handle = std::make_unique<thd_meta>();
  if (hit != c.map.end()) {
    ++c.hits;
    c.lru.splice(c.lru.begin(), c.lru, c.where[key]);
    handle->entry = hit->second;
    handle->cache_hit = true;
  } else {
    ++c.misses;
    auto e = std::make_shared<MetaEntry>();
    e->plan = pass ? build_pass_plan(seqlens, n_docs, cp, rank, block_t, block_n, shard_mask, real)
                   : build_plan(seqlens, n_docs, cp, rank, block_t, block_n, concurrency, real,
                                packed);
    if (device >= 0) {
      upload(*e, device);
      ++c.uploads;
    }
    c.map.emplace(key, e);
    c.lru.push_front(key);
    c.where[key] = c.lru.begin();
    while (c.map.size() > Cache::kCapacity) {
      const std::string& victim = c.lru.back();
      c.map.erase(victim);
      c.where.erase(victim);
      c.lru.pop_back();
    }
    handle->entry = std::move(e);
  }
  *out = handle.release();
}

}  // namespace

MetaEntry::~MetaEntry() {
  if (dev.base != nullptr) {
    int saved = -1;
    if (hipGetDevice(&saved) == hipSuccess) {
      if (saved != dev.device) (void)hipSetDevice(dev.device);
      (void)hipFree(dev.base);
      if (saved != dev.device) (void)hipSetDevice(saved);
    }
  }
}

}  // namespace thd

using namespace thd;

extern "C" {

const char* thd_last_error(void) { return g_last_error.c_str(); }

int thd_plan_partition(const int32_t* seqlens, int32_t n_docs, int32_t cp, int32_t rank,
                       int64_t* total_tokens, int64_t* local_tokens, int32_t* q_global,
                       int32_t* kv_row, int32_t* chunk_off) {
  return guarded([&] {
    const int64_t total = validate_partition(seqlens, n_docs, cp, rank);
    if (total_tokens != nullptr) *total_tokens = total;
    if (local_tokens != nullptr) *local_tokens = total / cp;
    plan_partition(seqlens, n_docs, cp, rank, q_global, kv_row, chunk_off);
  });
}

int thd_build_metadata(const int32_t* seqlens, int32_t n_docs, int32_t cp, int32_t rank,
                       int32_t block_t, int32_t block_n, int32_t concurrency, int32_t device,
                       thd_meta** out) {
  return guarded([&] {
    build_metadata_impl(seqlens, nullptr, n_docs, cp, rank, block_t, block_n, concurrency, device,
                        out);
  });
}

int thd_pad_lengths(const int32_t* real_lengths, int32_t n_docs, int32_t cp, int32_t* padded) {
  return guarded([&] { pad_lengths(real_lengths, n_docs, cp, padded); });
}

int thd_build_metadata_padded(const int32_t* real_lengths, int32_t n_docs, int32_t cp,
                              int32_t rank, int32_t block_t, int32_t block_n,
                              int32_t concurrency, int32_t device, thd_meta** out) {
  return guarded([&] {
    if (out == nullptr) fail(THD_EINVAL, "out is NULL");
    *out = nullptr;
    if (n_docs < 1) fail(THD_EINVAL, "n_docs must be >= 1");
    std::vector<int32_t> padded(n_docs);
    pad_lengths(real_lengths, n_docs, cp, padded.data());
    build_metadata_impl(padded.data(), real_lengths, n_docs, cp, rank, block_t, block_n,
                        concurrency, device, out);
  });
}

int thd_build_packed_metadata(const int32_t* lengths, int32_t n_docs, int32_t cp, int32_t rank,
                              int32_t block_t, int32_t block_n, int32_t concurrency,
                              int32_t padded, int32_t device, thd_meta** out) {
  return guarded([&] {
    if (out == nullptr) fail(THD_EINVAL, "out is NULL");
    *out = nullptr;
    if (padded != 0 && padded != 1) fail(THD_EINVAL, "padded must be 0 or 1");
    if (padded == 0) {
      build_metadata_impl(lengths, nullptr, n_docs, cp, rank, block_t, block_n, concurrency,
                          device, out, false, 0, true);
      return;
    }
    if (n_docs < 1) fail(THD_EINVAL, "n_docs must be >= 1");
    std::vector<int32_t> stored(n_docs);
    pad_lengths(lengths, n_docs, cp, stored.data());
    build_metadata_impl(stored.data(), lengths, n_docs, cp, rank, block_t, block_n, concurrency,
                        device, out, false, 0, true);
  });
}

int thd_meta_info(const thd_meta* meta, thd_meta_info_t* info) {
  return guarded([&] {
    const MetaEntry& e = entry_of(meta);
    if (info == nullptr) fail(THD_EINVAL, "info is NULL");
    const Plan& p = *e.plan;
    info->total_tokens = p.total;
    info->local_tokens = p.local;
    info->n_tiles = int64_t(p.tiles.size() / 8);
    info->n_kvtiles = int64_t(p.kvtiles.size() / 8);
    info->useful_pairs = p.useful_pairs;
    info->max_kv_tiles = p.max_kv_tiles;
    info->n_items = int64_t(p.items.size() / p.item_ints());
    info->n_splits = int64_t(p.splits.size() / 4);
    info->n_part_slots = p.n_part_slots;
    info->pad_tokens = p.pad_tokens;
    info->concurrency = p.concurrency;
    info->kv_split = p.kv_split;
    info->n_docs = int32_t(p.seqlens.size());
    info->cp = p.cp;
    info->rank = p.rank;
    info->block_t = p.block_t;
    info->block_n = p.block_n;
    info->version = THD_META_VERSION;
    info->device = e.dev.base != nullptr ? e.dev.device : -1;
    info->cache_hit = meta->cache_hit ? 1 : 0;
    info->is_pass = p.pass ? 1 : 0;
    info->item_ints = p.item_ints();
    info->shard_mask = p.shard_mask;
    info->is_packed = p.packed ? 1 : 0;
    info->n_packed_tiles = p.n_packed;
    info->n_pack_rows = int64_t(p.pack_rows.size() / 4);
    info->n_pack_keys = int64_t(p.pack_keys.size());
  });
}

int thd_meta_copy(const thd_meta* meta, int32_t field, int32_t* dst, int64_t count) {
  return guarded([&] {
    const Plan& p = *entry_of(meta).plan;
    const std::vector<int32_t>* src = nullptr;
    switch (field) {
      case THD_FIELD_Q_GLOBAL: src = &p.q_global; break;
      case THD_FIELD_KV_ROW: src = &p.kv_row; break;
      case THD_FIELD_CHUNK_OFF: src = &p.chunk_off; break;
      case THD_FIELD_TILES: src = &p.tiles; break;
      case THD_FIELD_ORDER: src = &p.order; break;
      case THD_FIELD_KVTILES: src = &p.kvtiles; break;
      case THD_FIELD_ITEMS: src = &p.items; break;
      case THD_FIELD_SPLITS: src = &p.splits; break;
      case THD_FIELD_DOC_END: src = &p.doc_end; break;
      case THD_FIELD_PACK_ROWS: src = &p.pack_rows; break;
      case THD_FIELD_PACK_KEYS: src = &p.pack_keys; break;
      default: fail(THD_EINVAL, "unknown field " + std::to_string(field));
    }
    if (count != int64_t(src->size()))
      fail(THD_EINVAL, "count " + std::to_string(count) + " != field length " +
                           std::to_string(src->size()));
    if (count > 0 && dst == nullptr) fail(THD_EINVAL, "dst is NULL");
    if (count > 0) std::memcpy(dst, src->data(), size_t(count) * sizeof(int32_t));
  });
}

void thd_meta_release(thd_meta* meta) {
  if (meta == nullptr) return;
  std::lock_guard<std::mutex> lock(cache().mu);
  delete meta;
}

int thd_cache_stats(int64_t* hits, int64_t* misses, int64_t* uploads, int64_t* entries) {
  return guarded([&] {
    Cache& c = cache();
    std::lock_guard<std::mutex> lock(c.mu);
    if (hits) *hits = c.hits;
    if (misses) *misses = c.misses;
    if (uploads) *uploads = c.uploads;
    if (entries) *entries = int64_t(c.map.size());
  });
}

int thd_cache_clear(void) {
  return guarded([&] {
    Cache& c = cache();
    std::lock_guard<std::mutex> lock(c.mu);
    c.map.clear();
    c.where.clear();
    c.lru.clear();
    c.hits = c.misses = c.uploads = 0;
  });
}

int thd_preferred_tiles(int32_t hq, int32_t hkv, int32_t d_qk, int32_t d_v, int32_t* block_t,
                        int32_t* block_n) {
  return guarded([&] {
    check_heads(hq, hkv);
    if (!fwd_supported(d_qk, d_v))
      fail(THD_EUNSUPPORTED, "no kernel for d_qk=" + std::to_string(d_qk) +
                                 ", d_v=" + std::to_string(d_v));
    if (block_t == nullptr || block_n == nullptr) fail(THD_EINVAL, "output pointer is NULL");
    *block_t = preferred_block_t(hq / hkv);
    *block_n = kBlockN;
  });
}

int thd_preferred_fwd_tiles(const int32_t* seqlens, int32_t n_docs, int32_t cp, int32_t rank,
                            int32_t hq, int32_t hkv, int32_t d_qk, int32_t d_v,
                            int32_t concurrency32, int32_t* block_t, int32_t* block_n) {
  return guarded([&] {
    validate_partition(seqlens, n_docs, cp, rank);
    check_heads(hq, hkv);
    if (!fwd_supported(d_qk, d_v))
      fail(THD_EUNSUPPORTED, "no kernel for d_qk=" + std::to_string(d_qk) +
                                 ", d_v=" + std::to_string(d_v));
    if (block_t == nullptr || block_n == nullptr) fail(THD_EINVAL, "output pointer is NULL");
    if (concurrency32 < 0) fail(THD_EINVAL, "concurrency32 must be >= 0");
    // Key slots the forward computes (visited KV tiles times their size) with
    // 64- and with 32-key tiles: query tile t0.. of chunk k sees the document's
    // keys up to k*c + t0 + rows. Short tiles pay when they drop more than 7%
    // of the slots (keys past each tile's last row that a 64-key tile still
    // computes); below that their extra barriers and the tighter register
    // budget of the third workgroup cost more than they save.
    // Second rule, when the caller gives the 32-key concurrency
    // (thd_fwd_concurrency): query tiles of at most 32 tokens (four or more q
    // heads per kv head) in a grid large enough that 32-key tiles need no
    // split (at least two work items per slot). There the third workgroup per
    // CU pays even without saved slots: 3-5% on GQA batches of 266 to 1050
    // tiles, in both P paths, where MHA's 128-token tiles lose 10-18%.
    const int32_t bt = preferred_block_t(hq / hkv);
    int64_t slots64 = 0, slots32 = 0, n_tiles = 0;
    for (int32_t i = 0; i < n_docs; ++i) {
      const int64_t c = seqlens[i] / (2 * cp);
      for (int s = 0; s < 2; ++s) {
        const int64_t k = s == 0 ? rank : 2 * cp - 1 - rank;
        for (int64_t t0 = 0; t0 < c; t0 += bt) {
          const int64_t kv_len = k * c + t0 + std::min<int64_t>(bt, c - t0);
          slots64 += (kv_len + kBlockN - 1) / kBlockN * kBlockN;
          slots32 += (kv_len + kBlockNShort - 1) / kBlockNShort * kBlockNShort;
          ++n_tiles;
        }
      }
    }
    const bool saves_slots = 100 * slots32 <= 93 * slots64;
    const bool large_grid = concurrency32 > 0 && bt <= 32 && n_tiles >= 2 * int64_t(concurrency32);
    *block_t = bt;
    *block_n = fwd_block_n_supported(d_qk, kBlockNShort) && (saves_slots || large_grid)
                   ? kBlockNShort
                   : kBlockN;
  });
}

int thd_fwd_concurrency(int32_t device, int32_t hkv, int32_t block_n, int32_t* concurrency) {
  return guarded([&] {
    if (hkv < 1) fail(THD_EINVAL, "hkv must be >= 1");
    if (block_n != kBlockN && block_n != kBlockNShort)
      fail(THD_EINVAL, "block_n must be " + std::to_string(kBlockN) + " or " +
                           std::to_string(kBlockNShort));
    if (concurrency == nullptr) fail(THD_EINVAL, "concurrency is NULL");
    int count = 0;
    check_hip(hipGetDeviceCount(&count), "hipGetDeviceCount");
    if (device < 0 || device >= count) fail(THD_EINVAL, "no such device " + std::to_string(device));
    int cus = 0;
    check_hip(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device),
              "hipDeviceGetAttribute");
    // Seven eighths of the slots: parts then come out a little longer and
    // fewer, which saves part startups and combine traffic (MLA workload, 9
    // documents of 1024-8192 tokens, cp = 8: 8 split tiles instead of 13,
    // kernel plus combine about 1% faster, within run-to-run spread; the split
    // rule does not split at all below about five eighths there).
    *concurrency = std::max(1, cus * fwd_workgroups_per_cu(block_n) * 7 / (8 * hkv));
  });
}

int thd_attn_fwd_workspace(const thd_meta* meta, int32_t hq, int32_t hkv, int32_t d_v,
                           int64_t* bytes) {
  return guarded([&] {
    const Plan& p = *entry_of(meta).plan;
    check_heads(hq, hkv);
    if (d_v < 1) fail(THD_EINVAL, "d_v must be >= 1");
    if (bytes == nullptr) fail(THD_EINVAL, "bytes is NULL");
    *bytes = p.n_part_slots * hkv * fwd_partial_floats(p.block_t, hq / hkv, d_v) *
             int64_t(sizeof(float));
  });
}

}  // extern "C"

namespace thd {
namespace {

// Shared by thd_attn_fwd (caller workspace) and thd_attn_fwd_noalloc (the
// per-device static array; use_static = true, workspace ignored).
void attn_fwd_impl(const thd_meta* meta, const void* q, const void* k, const void* v, void* o,
                   float* lse, float* o_f32, int32_t hq, int32_t hkv, int32_t d_qk, int32_t d_v,
                   float softmax_scale, void* workspace, int64_t workspace_bytes, bool use_static,
                   void* hip_stream) {
  const MetaEntry& e = entry_of(meta);
  const Plan& p = *e.plan;
  check_heads(hq, hkv);
  if (!fwd_supported(d_qk, d_v))
    fail(THD_EUNSUPPORTED, "no forward kernel for d_qk=" + std::to_string(d_qk) +
                               ", d_v=" + std::to_string(d_v));
  softmax_scale = resolve_scale(softmax_scale, d_qk);
  const int32_t group = hq / hkv;
  check_fwd_tiles(p, group, d_qk);
  if (p.pass) fail(THD_EMISMATCH, "metadata is a pass plan: call thd_attn_fwd_pass");
  check_ptr(q, "q", 16);
  check_ptr(k, "k", 16);
  check_ptr(v, "v", 16);
  check_ptr(o, "o", 16);
  check_ptr(lse, "lse", 16);
  if (o_f32 != nullptr) check_ptr(o_f32, "o_f32", 16);
  const int64_t need = p.n_part_slots * hkv * fwd_partial_floats(p.block_t, group, d_v) *
                       int64_t(sizeof(float));
  if (use_static) {
    if (need > kFwdStaticScratchBytes)
      fail(THD_ERANGE, "the split tiles' partial results need " + std::to_string(need) +
                           " bytes; the no-allocation forward holds at most " +
                           std::to_string(kFwdStaticScratchBytes) +
                           " (build the metadata with a smaller concurrency, or call "
                           "thd_attn_fwd with a workspace)");
  } else if (need > 0) {
    check_ptr(workspace, "workspace", 16);
    if (workspace_bytes < need)
      fail(THD_EINVAL, "workspace has " + std::to_string(workspace_bytes) + " bytes, needs " +
                           std::to_string(need));
  }
  const DeviceMeta& d = device_meta(e);
  const int64_t n_items = int64_t(p.items.size() / 4);
  if (n_items * hkv >= (int64_t(1) << 31)) fail(THD_ERANGE, "grid too large");
  check_kv_bytes(p.total, hkv, d_qk, d_v);
  if (use_static) {
    void* ptr = nullptr;
    check_hip(hipError_t(fwd_static_scratch(d.device, &ptr)), "hipGetSymbolAddress(scratch)");
    workspace = ptr;
  }
  FwdParams fp{};
  fp.q = q;
  fp.k = k;
  fp.v = v;
  fp.o = o;
  fp.lse = lse;
  fp.o_f32 = o_f32;
  fp.partial = static_cast<float*>(workspace);
  fp.tiles = d.tiles;
  fp.items = d.items;
  fp.splits = d.splits;
  fp.kv_row = d.kv_row;
  fp.doc_end = d.doc_end;
  fp.packed = p.packed ? 1 : 0;
  fp.pack_rows = d.pack_rows;
  fp.pack_keys = d.pack_keys;
  fp.n_items = int32_t(n_items);
  fp.n_splits = int32_t(p.splits.size() / 4);
  fp.hq = hq;
  fp.hkv = hkv;
  fp.group = group;
  fp.block_t = p.block_t;
  fp.block_n = p.block_n;
  fp.total = p.total;
  fp.scale_log2 = softmax_scale * 1.4426950408889634f;
  check_hip(hipError_t(launch_fwd(fp, d_qk, d_v, hip_stream)), "forward launch");
}

}  // namespace
}  // namespace thd

extern "C" {

int thd_attn_fwd(const thd_meta* meta, const void* q, const void* k, const void* v, void* o,
                 float* lse, float* o_f32, int32_t hq, int32_t hkv, int32_t d_qk, int32_t d_v,
                 float softmax_scale, void* workspace, int64_t workspace_bytes,
                 void* hip_stream) {
  return guarded([&] {
    attn_fwd_impl(meta, q, k, v, o, lse, o_f32, hq, hkv, d_qk, d_v, softmax_scale, workspace,
                  workspace_bytes, false, hip_stream);
  });
}

int thd_attn_fwd_noalloc(const thd_meta* meta, const void* q, const void* k, const void* v,
                         void* o, float* lse, float* o_f32, int32_t hq, int32_t hkv,
                         int32_t d_qk, int32_t d_v, float softmax_scale, void* hip_stream) {
  return guarded([&] {
    attn_fwd_impl(meta, q, k, v, o, lse, o_f32, hq, hkv, d_qk, d_v, softmax_scale, nullptr, 0,
                  true, hip_stream);
  });
}

int thd_build_pass_metadata(const int32_t* seqlens, int32_t n_docs, int32_t cp, int32_t rank,
                            int32_t block_t, int32_t block_n, uint64_t shard_mask,
                            int32_t device, thd_meta** out) {
  return guarded([&] {
    build_metadata_impl(seqlens, nullptr, n_docs, cp, rank, block_t, block_n, 0, device, out,
                        true, shard_mask);
  });
}

int thd_build_pass_metadata_padded(const int32_t* real_lengths, int32_t n_docs, int32_t cp,
                                   int32_t rank, int32_t block_t, int32_t block_n,
                                   uint64_t shard_mask, int32_t device, thd_meta** out) {
  return guarded([&] {
    if (out == nullptr) fail(THD_EINVAL, "out is NULL");
    *out = nullptr;
    if (n_docs < 1) fail(THD_EINVAL, "n_docs must be >= 1");
    std::vector<int32_t> padded(n_docs);
    pad_lengths(real_lengths, n_docs, cp, padded.data());
    build_metadata_impl(padded.data(), real_lengths, n_docs, cp, rank, block_t, block_n, 0,
                        device, out, true, shard_mask);
  });
}

int thd_attn_fwd_pass_state_bytes(const thd_meta* meta, int32_t hq, int32_t hkv, int32_t d_v,
                                  int64_t* state_bytes) {
  return guarded([&] {
    const Plan& p = *entry_of(meta).plan;
    check_heads(hq, hkv);
    if (d_v < 1) fail(THD_EINVAL, "d_v must be >= 1");
    if (!p.pass) fail(THD_EMISMATCH, "metadata is not a pass plan");
    if (state_bytes == nullptr) fail(THD_EINVAL, "state_bytes is NULL");
    *state_bytes = p.local * hq * (int64_t(d_v) + 1) * int64_t(sizeof(float));
  });
}

int thd_attn_fwd_pass(const thd_meta* meta, const void* q, const void* k, const void* v, void* o,
                      float* lse, float* state, int32_t flags, int32_t hq, int32_t hkv,
                      int32_t d_qk, int32_t d_v, float softmax_scale, void* hip_stream) {
  return guarded([&] {
    const MetaEntry& e = entry_of(meta);
    const Plan& p = *e.plan;
    check_heads(hq, hkv);
    if (!fwd_supported(d_qk, d_v))
      fail(THD_EUNSUPPORTED, "no forward kernel for d_qk=" + std::to_string(d_qk) +
                                 ", d_v=" + std::to_string(d_v));
    softmax_scale = resolve_scale(softmax_scale, d_qk);
    if (!p.pass) fail(THD_EMISMATCH, "metadata is not a pass plan (thd_build_pass_metadata)");
    if (p.block_n != kBlockN)
      fail(THD_EMISMATCH, "pass plans take block_n = " + std::to_string(kBlockN));
    if ((flags & ~(THD_PASS_FIRST | THD_PASS_LAST)) != 0) fail(THD_EINVAL, "unknown pass flags");
    const int32_t group = hq / hkv;
    check_fwd_tiles(p, group, d_qk);
    check_ptr(q, "q", 16);
    check_ptr(k, "k", 16);
    check_ptr(v, "v", 16);
    check_ptr(state, "state", 16);
    if (flags & THD_PASS_LAST) {
      check_ptr(o, "o", 16);
      check_ptr(lse, "lse", 16);
    }
    const DeviceMeta& d = device_meta(e);
    const int64_t n_tiles = int64_t(p.tiles.size() / 8);
    if (n_tiles * hkv >= (int64_t(1) << 31)) fail(THD_ERANGE, "grid too large");
    // A first pass sets every row's state and a last one writes every row's
    // output, so they visit every tile; the others only the tiles with runs.
    const int64_t n_wg = (flags & (THD_PASS_FIRST | THD_PASS_LAST)) != 0 ? n_tiles : p.n_run_tiles;
    check_kv_bytes(p.total, hkv, d_qk, d_v);
    FwdParams fp{};
    fp.q = q;
    fp.k = k;
    fp.v = v;
    fp.o = o;
    fp.lse = lse;
    fp.o_f32 = nullptr;
    fp.partial = nullptr;
    fp.tiles = d.tiles;
    fp.items = d.items;
    fp.splits = d.splits;
    fp.kv_row = d.kv_row;
    fp.doc_end = d.doc_end;
    fp.n_items = int32_t(n_wg);
    fp.n_splits = int32_t(n_tiles);
    fp.pass_runs = d.pass_runs;
    fp.pass_order = d.pass_order;
    fp.hq = hq;
    fp.hkv = hkv;
    fp.group = group;
    fp.block_t = p.block_t;
    fp.block_n = p.block_n;
    fp.total = p.total;
    fp.scale_log2 = softmax_scale * 1.4426950408889634f;
    fp.ranged = 1;
    fp.pass_flags = flags;
    fp.state = state;
    fp.local = p.local;
    check_hip(hipError_t(launch_fwd_pass(fp, d_qk, d_v, hip_stream)), "forward pass launch");
  });
}

int thd_attn_bwd_workspace(const thd_meta* meta, int32_t hq, int64_t* bytes) {
  return guarded([&] {
    const Plan& p = *entry_of(meta).plan;
    if (hq < 1) fail(THD_EINVAL, "hq must be >= 1");
    if (bytes == nullptr) fail(THD_EINVAL, "bytes is NULL");
    *bytes = 2 * bwd_ws_array_bytes(p.local, hq);
  });
}

}  // extern "C"

namespace thd {
namespace {

// Both backward entry points: dk and dv in fp32, or in bf16 (kv_bf16).
int attn_bwd_impl(const thd_meta* meta, const void* q, const void* k, const void* v,
                  const float* lse, const float* o_f32, const void* d_o, float* dq, void* dk,
                  void* dv, int32_t hq, int32_t hkv, int32_t d_qk, int32_t d_v,
                  float softmax_scale, void* workspace, int64_t workspace_bytes,
                  void* hip_stream, bool kv_bf16) {
  return guarded([&] {
    const MetaEntry& e = entry_of(meta);
    const Plan& p = *e.plan;
    check_heads(hq, hkv);
    if (!bwd_supported(d_qk, d_v))
      fail(THD_EUNSUPPORTED, "no backward kernel for d_qk=" + std::to_string(d_qk) +
                                 ", d_v=" + std::to_string(d_v));
    softmax_scale = resolve_scale(softmax_scale, d_qk);
    const int32_t group = hq / hkv;
    check_bwd_tiles(p, group);
    if (p.pass) fail(THD_EMISMATCH, "metadata is a pass plan, not the full key range");
    if (p.packed)
      fail(THD_EMISMATCH, "metadata is a packed plan, which is forward-only: build it with "
                          "thd_build_metadata for the backward");
    check_ptr(q, "q", 16);
    check_ptr(k, "k", 16);
    check_ptr(v, "v", 16);
    check_ptr(lse, "lse", 16);
    if (o_f32 != nullptr) check_ptr(o_f32, "o_f32", 16);
    check_ptr(d_o, "d_o", 16);
    check_ptr(dq, "dq", 16);
    check_ptr(dk, "dk", 16);
    check_ptr(dv, "dv", 16);
    check_ptr(workspace, "workspace", 16);
    const int64_t need = 2 * bwd_ws_array_bytes(p.local, hq);
    if (workspace_bytes < need)
      fail(THD_EINVAL, "workspace has " + std::to_string(workspace_bytes) + " bytes, needs " +
                           std::to_string(need));
    const DeviceMeta& d = device_meta(e);
    check_kv_bytes(p.total, hkv, d_qk, d_v);
    const int64_t n_tiles = int64_t(p.tiles.size() / 8);
    const int64_t n_kvtiles = int64_t(p.kvtiles.size() / 8);
    if (n_tiles * hkv >= (int64_t(1) << 31) || n_kvtiles * hkv >= (int64_t(1) << 31))
      fail(THD_ERANGE, "grid too large");
    BwdParams bp{};
    bp.q = q;
    bp.k = k;
    bp.v = v;
    bp.lse = lse;
    bp.o_f32 = o_f32;
    bp.d_o = d_o;
    bp.dq = dq;
    bp.dk = dk;
    bp.dv = dv;
    bp.delta = static_cast<float*>(workspace);
    bp.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + bwd_ws_array_bytes(p.local, hq));
    bp.tiles = d.tiles;
    bp.order = d.order;
    bp.kvtiles = d.kvtiles;
    bp.kv_order = d.kv_order;
    bp.kv_row = d.kv_row;
    bp.n_tiles = int32_t(n_tiles);
    bp.n_kvtiles = int32_t(n_kvtiles);
    bp.hq = hq;
    bp.hkv = hkv;
    bp.group = group;
    bp.block_t = p.block_t;
    bp.total = p.total;
    bp.local = p.local;
    bp.kv_bf16 = kv_bf16 ? 1 : 0;
    bp.scale = softmax_scale;
    bp.scale_log2 = softmax_scale * 1.4426950408889634f;
    check_hip(hipError_t(launch_bwd(bp, d_qk, d_v, hip_stream)), "backward launch");
  });
}

}  // namespace
}  // namespace thd

extern "C" {

int thd_attn_bwd(const thd_meta* meta, const void* q, const void* k, const void* v,
                 const float* lse, const float* o_f32, const void* d_o, float* dq, float* dk,
                 float* dv, int32_t hq, int32_t hkv, int32_t d_qk, int32_t d_v,
                 float softmax_scale, void* workspace, int64_t workspace_bytes,
                 void* hip_stream) {
  return attn_bwd_impl(meta, q, k, v, lse, o_f32, d_o, dq, dk, dv, hq, hkv, d_qk, d_v,
                       softmax_scale, workspace, workspace_bytes, hip_stream, false);
}

int thd_attn_bwd_bf16kv(const thd_meta* meta, const void* q, const void* k, const void* v,
                        const float* lse, const float* o_f32, const void* d_o, float* dq,
                        void* dk, void* dv, int32_t hq, int32_t hkv, int32_t d_qk, int32_t d_v,
                        float softmax_scale, void* workspace, int64_t workspace_bytes,
                        void* hip_stream) {
  return attn_bwd_impl(meta, q, k, v, lse, o_f32, d_o, dq, dk, dv, hq, hkv, d_qk, d_v,
                       softmax_scale, workspace, workspace_bytes, hip_stream, true);
}

}  // extern "C"
