// Concurrency stress of the metadata planner and cache through the C ABI,
// built with a sanitizer (ThreadSanitizer, or AddressSanitizer plus
// UndefinedBehaviorSanitizer) by tests/test_host_sanitizers.py. Host-only
// metadata (device = -1): nothing here touches a GPU.
//
// 16 threads build, inspect, copy and release metadata for a small set of
// length lists (so most builds are cache hits and entries are shared), while
// some threads clear the cache. The cases cover plain plans, packed plans
// (also from real lengths, padded), and pass plans. Every copy must equal the
// reference copy made before the threads start. Exit status 0 on success.
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <thread>
#include <vector>

#include "thdattn.h"

namespace {

enum Kind { kPlain, kPacked, kPackedPadded, kPass, kPassPadded };

struct Case {
  std::vector<int32_t> lengths;
  int32_t cp, rank, block_t, block_n, concurrency;
  Kind kind = kPlain;
  uint64_t shards = 0;   // pass plans
};

int build(const Case& c, thd_meta** m) {
  const int32_t n = int32_t(c.lengths.size());
  switch (c.kind) {
    case kPacked:
      return thd_build_packed_metadata(c.lengths.data(), n, c.cp, c.rank, c.block_t, c.block_n,
                                       c.concurrency, 0, -1, m);
    case kPackedPadded:
      return thd_build_packed_metadata(c.lengths.data(), n, c.cp, c.rank, c.block_t, c.block_n,
                                       c.concurrency, 1, -1, m);
    case kPass:
      return thd_build_pass_metadata(c.lengths.data(), n, c.cp, c.rank, c.block_t, c.block_n,
                                     c.shards, -1, m);
    case kPassPadded:
      return thd_build_pass_metadata_padded(c.lengths.data(), n, c.cp, c.rank, c.block_t,
                                            c.block_n, c.shards, -1, m);
    default:
      return thd_build_metadata(c.lengths.data(), n, c.cp, c.rank, c.block_t, c.block_n,
                                c.concurrency, -1, m);
  }
}

std::vector<int32_t> field(const thd_meta* m, int32_t f, int64_t n) {
  std::vector<int32_t> out(size_t(n > 0 ? n : 0));
  if (n > 0 && thd_meta_copy(m, f, out.data(), n) != THD_OK) {
    std::fprintf(stderr, "meta_copy failed: %s\n", thd_last_error());
    std::exit(2);
  }
  return out;
}

struct Snapshot {
  std::vector<int32_t> q_global, kv_row, tiles, kvtiles, items, splits, pack_rows, pack_keys,
      doc_end;
};

Snapshot take(const thd_meta* m) {
  thd_meta_info_t info{};
  if (thd_meta_info(m, &info) != THD_OK) {
    std::fprintf(stderr, "meta_info failed: %s\n", thd_last_error());
    std::exit(2);
  }
  Snapshot s;
  s.q_global = field(m, THD_FIELD_Q_GLOBAL, info.local_tokens);
  s.kv_row = field(m, THD_FIELD_KV_ROW, info.total_tokens);
  s.tiles = field(m, THD_FIELD_TILES, info.n_tiles * 8);
  s.kvtiles = field(m, THD_FIELD_KVTILES, info.n_kvtiles * 8);
  s.items = field(m, THD_FIELD_ITEMS, info.n_items * info.item_ints);
  s.splits = field(m, THD_FIELD_SPLITS, (info.is_pass ? info.n_tiles : info.n_splits) * 4);
  s.pack_rows = field(m, THD_FIELD_PACK_ROWS, info.n_pack_rows * 4);
  s.pack_keys = field(m, THD_FIELD_PACK_KEYS, info.n_pack_keys);
  s.doc_end = field(m, THD_FIELD_DOC_END, info.n_docs);
  return s;
}

bool same(const Snapshot& a, const Snapshot& b) {
  return a.q_global == b.q_global && a.kv_row == b.kv_row && a.tiles == b.tiles &&
         a.kvtiles == b.kvtiles && a.items == b.items && a.splits == b.splits &&
         a.pack_rows == b.pack_rows && a.pack_keys == b.pack_keys && a.doc_end == b.doc_end;
}

}  // namespace

int main() {
  const std::vector<Case> cases = {
      {{256, 512, 256}, 2, 0, 64, 64, 0},
      {{256, 512, 256}, 2, 1, 64, 64, 0},
      {{8, 24, 40, 136, 520}, 4, 1, 32, 64, 64},
      {{1000, 72, 600}, 4, 3, 32, 64, 0},
      {{4096, 96}, 4, 0, 16, 64, 8},
      {{16, 32, 1040, 16, 400}, 8, 3, 8, 64, 0},
      {{16, 48, 8, 80, 16, 8, 32}, 2, 1, 8, 32, 0, kPacked},
      {{16 * 1, 16 * 2, 16 * 3, 16 * 5, 16 * 8, 16 * 13, 16 * 21}, 8, 0, 16, 32, 84, kPacked},
      {{5, 13, 8, 3, 30, 1, 22}, 2, 0, 32, 64, 0, kPackedPadded},
      {{16, 32, 1040, 16, 400}, 8, 3, 32, 64, 0, kPass, 0x9u},
      {{256, 512, 256}, 2, 1, 64, 64, 0, kPass, 0x2u},
      {{17, 1040, 9, 400}, 8, 3, 32, 64, 0, kPassPadded, 0x11u},
  };
  std::vector<Snapshot> ref;
  for (const Case& c : cases) {
    thd_meta* m = nullptr;
    if (build(c, &m) != THD_OK) {
      std::fprintf(stderr, "build failed: %s\n", thd_last_error());
      return 2;
    }
    ref.push_back(take(m));
    thd_meta_release(m);
  }
  std::atomic<int> bad{0};
  std::vector<std::thread> threads;
  for (int t = 0; t < 16; ++t) {
    threads.emplace_back([&, t] {
      for (int it = 0; it < 60; ++it) {
        const size_t k = size_t(t * 7 + it) % cases.size();
        const Case& c = cases[k];
        thd_meta* m = nullptr;
        if (build(c, &m) != THD_OK) {
          ++bad;
          continue;
        }
        if (!same(take(m), ref[k])) ++bad;
        // an error path from every thread: its message is thread-local
        int64_t T = 0, T_local = 0;
        const int32_t odd[2] = {6, 8};
        if (thd_plan_partition(odd, 2, 2, 0, &T, &T_local, nullptr, nullptr, nullptr) != THD_ENOTDIV)
          ++bad;
        thd_meta_release(m);
        if (t % 5 == 0 && it % 10 == 9) thd_cache_clear();
      }
    });
  }
  for (auto& th : threads) th.join();
  if (bad.load() != 0) {
    std::fprintf(stderr, "%d mismatches or failures\n", bad.load());
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
