// Host planner: symmetric EOD-aware partition and per-tile bounds.
//
// Partition ("kvallgather cp thd load balance", Ascend/MindSpeed, section
// "What this PR does / why we need it?"; divisibility rule from "Does this PR
// introduce any user-facing change?"): document i of length L_i is cut into
// 2*cp chunks of c_i = L_i / (2cp) tokens and rank r owns chunks r and
// 2cp-1-r. Local rows run document by document, chunk r first, so document i
// starts at local row cu_i / cp. K/V are gathered rank-major, so global token
// g at offset off = g - cu_i of document i (chunk k = off / c_i, o = off % c_i)
// sits at gathered row owner(k)*T_local + cu_i/cp + slot(k)*c_i + o, where
// owner(k) = min(k, 2cp-1-k) and slot(k) = (k >= cp).
//
// Tiles: a query tile holds up to block_t consecutive tokens of one owned
// chunk, so every row of a tile belongs to the same document and its KV loop
// starts at the document's first key; the loop stops at the last row's own
// position, and only the tiles past the first row's position need the causal
// compare. The arrays are built in one pass with closed forms. The longest
// tiles' key ranges may be split into several forward work items (below).
//
// Packed plans (short-segment packing, after the per-row [start, end) key
// bounds of the FlashMask kernels on "[Optim] FlashMask-4 Overlap support
// part 1 (NVSHMEM backend) - #166"): the last, partial tile of each chunk is
// grouped with its neighbours' into one tile of up to block_t rows, whose key
// slots hold the documents' keys one document after the other and whose rows
// each see one window of slots.
#include <algorithm>
#include <cstring>
#include <numeric>

#include <string>

#include "internal.h"

namespace thd {

[[noreturn]] void fail(int code, const std::string& msg) { throw Error{code, msg}; }

int64_t validate_partition(const int32_t* seqlens, int32_t n_docs, int32_t cp, int32_t rank) {
  if (seqlens == nullptr) fail(THD_EINVAL, "seqlens is NULL");
  if (n_docs < 1) fail(THD_EINVAL, "n_docs must be >= 1");
  if (cp < 1) fail(THD_ERANGE, "cp must be >= 1");
  if (rank < 0 || rank >= cp)
    fail(THD_ERANGE, "rank " + std::to_string(rank) + " outside [0, " + std::to_string(cp) + ")");
  int64_t total = 0;
  for (int32_t i = 0; i < n_docs; ++i) {
    const int64_t len = seqlens[i];
    if (len < 1) fail(THD_EINVAL, "subsequence " + std::to_string(i) + " has length < 1");
    if (len % (2 * int64_t(cp)) != 0)
      fail(THD_ENOTDIV, "subsequence " + std::to_string(i) + " length " + std::to_string(len) +
                            " is not divisible by 2*cp = " + std::to_string(2 * cp));
    total += len;
    if (total >= (int64_t(1) << 31)) fail(THD_ERANGE, "total tokens must be < 2^31");
  }
  return total;
}

void plan_partition(const int32_t* seqlens, int32_t n_docs, int32_t cp, int32_t rank,
                    int32_t* q_global, int32_t* kv_row, int32_t* chunk_off) {
  int64_t total = 0;
  for (int32_t i = 0; i < n_docs; ++i) total += seqlens[i];
  const int64_t local = total / cp;
  int64_t cu = 0;
  for (int32_t i = 0; i < n_docs; ++i) {
    const int64_t c = seqlens[i] / (2 * cp);
    const int64_t local_doc = cu / cp;   // first local row of document i
    if (q_global != nullptr) {
      const int64_t first[2] = {cu + rank * c, cu + (2 * cp - 1 - rank) * c};
      for (int s = 0; s < 2; ++s)
        for (int64_t o = 0; o < c; ++o) q_global[local_doc + s * c + o] = int32_t(first[s] + o);
    }
    for (int32_t k = 0; k < 2 * cp; ++k) {
      const int64_t owner = std::min<int64_t>(k, 2 * cp - 1 - k);
      const int64_t slot = k >= cp ? 1 : 0;
      const int64_t row0 = owner * local + local_doc + slot * c;
      if (chunk_off != nullptr) chunk_off[int64_t(i) * 2 * cp + k] = int32_t(row0);
      if (kv_row != nullptr)
        for (int64_t o = 0; o < c; ++o) kv_row[cu + k * c + o] = int32_t(row0 + o);
    }
    cu += seqlens[i];
  }
}

namespace {

// Replaces the partial tiles of p.tiles (n_rows < block_t) by packed tiles.
// The partial tiles are taken in tile order and grouped greedily: a tile joins
// the open group while the group stays within block_t rows and within
// block_n * K key slots, K = max_kv_tiles, or the plain tiles' kv_split when
// that is positive and smaller (a packed tile is never split, so it must not
// outlast the longest plain tile nor the split parts); a tile of the same
// document as the group's previous member adds only the keys past that
// member's (its keys extend the member's). Groups of
// one tile stay plain. Plain tiles keep their tile order and the packed tiles
// follow in group order as [-1, first pack row, rows, -1, -1, first pack key,
// n_kv, 0]. Each packed row gets [local row, first slot, last slot, real]; a
// document's keys cu_i .. cu_i + K_i - 1 take consecutive slots from the
// document's base, K_i the key count of its last member, and row g of the
// document sees slots base .. base + g - cu_i. The slots are padded to whole
// KV tiles with the last slot's row, which no row sees.
void pack_partial_tiles(Plan& p) {
  const int64_t n = int64_t(p.tiles.size() / 8);
  auto rec = [&](int64_t t) { return &p.tiles[size_t(t) * 8]; };
  auto kv_len = [&](int64_t t) { return int64_t(rec(t)[1]) + rec(t)[2] - rec(t)[5]; };
  int64_t cap_tiles = p.max_kv_tiles;
  if (p.concurrency > 0 && n < 2 * int64_t(p.concurrency)) {
    int64_t total_kv = 0;
    for (int64_t t = 0; t < n; ++t) total_kv += rec(t)[6];
    const int64_t split = std::max<int64_t>((total_kv + p.concurrency - 1) / p.concurrency, 8);
    cap_tiles = std::min(cap_tiles, split);
  }
  const int64_t key_cap = int64_t(p.block_n) * cap_tiles;
  std::vector<std::vector<int64_t>> groups;
  std::vector<int64_t> group;
  int64_t g_rows = 0, g_keys = 0;
  for (int64_t t = 0; t < n; ++t) {
    const int64_t n_rows = rec(t)[2];
    if (n_rows == p.block_t) continue;
    const bool same_doc = !group.empty() && rec(group.back())[3] == rec(t)[3];
    const int64_t add = kv_len(t) - (same_doc ? kv_len(group.back()) : 0);
    if (!group.empty() && g_rows + n_rows <= p.block_t && g_keys + add <= key_cap) {
      group.push_back(t);
      g_rows += n_rows;
      g_keys += add;
      continue;
    }
    if (!group.empty()) groups.push_back(std::move(group));
    group.assign(1, t);
    g_rows = n_rows;
    g_keys = kv_len(t);
  }
  if (!group.empty()) groups.push_back(std::move(group));

  std::vector<char> in_pack(size_t(n), 0);
  for (const auto& g : groups)
    if (g.size() > 1)
      for (int64_t t : g) in_pack[size_t(t)] = 1;
  std::vector<int32_t> out;
  out.reserve(p.tiles.size());
  for (int64_t t = 0; t < n; ++t)
    if (!in_pack[size_t(t)]) out.insert(out.end(), rec(t), rec(t) + 8);
  for (const auto& g : groups) {
    if (g.size() < 2) continue;
    const int64_t row0 = int64_t(p.pack_rows.size() / 4), key0 = int64_t(p.pack_keys.size());
    int64_t base = 0;
    for (size_t m = 0; m < g.size(); ++m) {
      const int32_t* r = rec(g[m]);
      if (m > 0 && rec(g[m - 1])[3] != r[3]) base += kv_len(g[m - 1]);
      const int64_t q_local = r[0], q_glob = r[1], n_rows = r[2], doc = r[3], cu = r[5];
      for (int64_t o = 0; o < n_rows; ++o) {
        const int64_t pos = q_glob + o;
        const int32_t prow[4] = {int32_t(q_local + o), int32_t(base), int32_t(base + pos - cu),
                                 pos < p.doc_end[size_t(doc)] ? 1 : 0};
        p.pack_rows.insert(p.pack_rows.end(), prow, prow + 4);
      }
      // The document's keys, once its last member (which sees the most) is reached.
      if (m + 1 == g.size() || rec(g[m + 1])[3] != r[3])
        p.pack_keys.insert(p.pack_keys.end(), p.kv_row.begin() + cu, p.kv_row.begin() + cu + kv_len(g[m]));
    }
    const int64_t slots = int64_t(p.pack_keys.size()) - key0;
    const int64_t n_kv = (slots + p.block_n - 1) / p.block_n;
    p.pack_keys.resize(size_t(key0 + n_kv * p.block_n), p.pack_keys.back());
    const int32_t prec[8] = {-1, int32_t(row0), int32_t(int64_t(p.pack_rows.size() / 4) - row0),
                             -1, -1, int32_t(key0), int32_t(n_kv), 0};
    out.insert(out.end(), prec, prec + 8);
    ++p.n_packed;
  }
  p.tiles.swap(out);
}

}  // namespace

std::unique_ptr<Plan> build_plan(const int32_t* seqlens, int32_t n_docs, int32_t cp,
                                 int32_t rank, int32_t block_t, int32_t block_n,
                                 int32_t concurrency, const int32_t* real_lengths, bool packed) {
  const int64_t total = validate_partition(seqlens, n_docs, cp, rank);
  if (real_lengths != nullptr)
    for (int32_t i = 0; i < n_docs; ++i)
      if (real_lengths[i] < 1 || real_lengths[i] > seqlens[i])
        fail(THD_EINVAL, "real length " + std::to_string(real_lengths[i]) + " of document " +
                             std::to_string(i) + " is outside [1, " + std::to_string(seqlens[i]) + "]");
  if (block_t < 1 || block_n < 1 || block_t > 4096 || block_n > 4096)
    fail(THD_ERANGE, "tile sizes must be in [1, 4096]");
  if (concurrency < 0) fail(THD_EINVAL, "concurrency must be >= 0");
  auto plan = std::make_unique<Plan>();
  Plan& p = *plan;
  p.seqlens.assign(seqlens, seqlens + n_docs);
  p.real.assign(real_lengths != nullptr ? real_lengths : seqlens,
                (real_lengths != nullptr ? real_lengths : seqlens) + n_docs);
  // One past each document's last real token (the padded layout puts a
  // document's pad tokens after all of its real ones).
  p.doc_end.resize(n_docs);
  {
    int64_t cu_d = 0;
    for (int32_t i = 0; i < n_docs; ++i) {
      p.doc_end[i] = int32_t(cu_d + p.real[i]);
      p.pad_tokens += seqlens[i] - p.real[i];
      cu_d += seqlens[i];
    }
  }
  p.cp = cp;
  p.rank = rank;
  p.block_t = block_t;
  p.block_n = block_n;
  p.concurrency = concurrency;
  p.total = total;
  p.local = total / cp;
  p.q_global.resize(p.local);
  p.kv_row.resize(total);
  p.chunk_off.resize(size_t(n_docs) * 2 * cp);
  plan_partition(seqlens, n_docs, cp, rank, p.q_global.data(), p.kv_row.data(),
                 p.chunk_off.data());

  // Query tiles, natural order: document, slot (chunk r, then 2cp-1-r), offset.
  std::vector<int64_t> doc_first_tile(n_docs), doc_end_tile(n_docs);
  int64_t cu = 0;
  for (int32_t i = 0; i < n_docs; ++i) {
    const int64_t c = seqlens[i] / (2 * cp);
    p.useful_pairs += int64_t(seqlens[i]) * (int64_t(seqlens[i]) + 1) / (2 * cp);
    doc_first_tile[i] = int64_t(p.tiles.size() / 8);
    const int64_t chunks[2] = {rank, 2 * cp - 1 - rank};
    for (int s = 0; s < 2; ++s) {
      for (int64_t t0 = 0; t0 < c; t0 += block_t) {
        const int64_t n_rows = std::min<int64_t>(block_t, c - t0);
        const int64_t q_glob = cu + chunks[s] * c + t0;
        const int64_t kv_len = q_glob + n_rows - cu;
        const int64_t n_kv = (kv_len + block_n - 1) / block_n;
        const int64_t n_full = (q_glob - cu + 1) / block_n;
        const int32_t rec[8] = {int32_t(cu / cp + s * c + t0), int32_t(q_glob), int32_t(n_rows),
                                int32_t(i), int32_t(s), int32_t(cu), int32_t(n_kv),
                                int32_t(n_full)};
        p.tiles.insert(p.tiles.end(), rec, rec + 8);
        p.max_kv_tiles = std::max(p.max_kv_tiles, n_kv);
      }
    }
    doc_end_tile[i] = int64_t(p.tiles.size() / 8);
    cu += seqlens[i];
  }
  if (packed) {
    p.packed = true;
    pack_partial_tiles(p);
  }
  const int64_t n_tiles = int64_t(p.tiles.size() / 8);

  // Largest-first order: stable sort by KV-tile count, descending.
  p.order.resize(n_tiles);
  std::iota(p.order.begin(), p.order.end(), 0);
  std::stable_sort(p.order.begin(), p.order.end(), [&](int32_t a, int32_t b) {
    return p.tiles[size_t(a) * 8 + 6] > p.tiles[size_t(b) * 8 + 6];
  });

  // Backward key tiles cover every key of every document. The query tiles
  // seeing a key tile form a suffix of the document's tiles, found by one
  // forward walk because tile end positions increase within a document; keys
  // past offset (2cp-r)*c_i are seen by no local query (the rank's later chunk
  // is 2cp-1-r), so their tiles get an empty range. (Packed plans are
  // forward-only and have none.)
  cu = 0;
  for (int32_t i = 0; i < n_docs && !p.packed; ++i) {
    const int64_t len = seqlens[i];
    int64_t qb = doc_first_tile[i];
    for (int64_t j = 0; j * block_n < len; ++j) {
      const int64_t ks = cu + j * block_n;
      const int64_t nk = std::min<int64_t>(block_n, len - j * block_n);
      while (qb < doc_end_tile[i] &&
             int64_t(p.tiles[size_t(qb) * 8 + 1]) + p.tiles[size_t(qb) * 8 + 2] - 1 < ks)
        ++qb;
      const int32_t rec[8] = {int32_t(i), int32_t(ks), int32_t(nk), int32_t(qb),
                              int32_t(doc_end_tile[i]), 0, 0, 0};
      p.kvtiles.insert(p.kvtiles.end(), rec, rec + 8);
    }
    cu += seqlens[i];
  }
  // The dK/dV kernel's dispatch order: key tiles by the local query tokens
  // that see them (their query tiles' rows), most first, stable.
  {
    const int64_t n_kv = int64_t(p.kvtiles.size() / 8);
    const int64_t n_q = int64_t(p.tiles.size() / 8);
    std::vector<int64_t> rows_before(size_t(n_q) + 1, 0);   // prefix sums of tile rows
    for (int64_t t = 0; t < n_q; ++t)
      rows_before[size_t(t) + 1] = rows_before[size_t(t)] + p.tiles[size_t(t) * 8 + 2];
    std::vector<int64_t> seen(size_t(n_kv), 0);
    for (int64_t j = 0; j < n_kv; ++j)
      seen[size_t(j)] = rows_before[size_t(p.kvtiles[size_t(j) * 8 + 4])] -
                        rows_before[size_t(p.kvtiles[size_t(j) * 8 + 3])];
    p.kv_order.resize(size_t(n_kv));
    std::iota(p.kv_order.begin(), p.kv_order.end(), 0);
    std::stable_sort(p.kv_order.begin(), p.kv_order.end(),
                     [&](int32_t a, int32_t b) { return seen[size_t(a)] > seen[size_t(b)]; });
  }
  // Forward work items: the key range of the longest tiles is cut into parts
  // when the tiles alone are too few to keep the device busy, so no single
  // workgroup's loop is much longer than the average per workgroup slot. Every
  // part starts with a KV tile all its rows see whole (cuts at or before
  // n_full - 1), so no row of a part is empty.
  int64_t total_kv = 0;
  for (int64_t t = 0; t < n_tiles; ++t) total_kv += p.tiles[size_t(t) * 8 + 6];
  if (concurrency > 0 && n_tiles < 2 * int64_t(concurrency))
    p.kv_split = int32_t(std::max<int64_t>((total_kv + concurrency - 1) / concurrency, 8));
  std::vector<int32_t> natural;
  for (int64_t t = 0; t < n_tiles; ++t) {
    const int64_t n_kv = p.tiles[size_t(t) * 8 + 6];
    const int64_t n_full = p.tiles[size_t(t) * 8 + 7];
    if (p.kv_split == 0 || n_kv <= p.kv_split || n_full < 2) {
      const int32_t rec[4] = {int32_t(t), 0, int32_t(n_kv), -1};
      natural.insert(natural.end(), rec, rec + 4);
      continue;
    }
    const int64_t count = std::min<int64_t>((n_kv + p.kv_split - 1) / p.kv_split, n_full);
    std::vector<int64_t> bounds(count + 1);
    bounds[0] = 0;
    bounds[count] = n_kv;
    for (int64_t i = 1; i < count; ++i) bounds[i] = i * n_kv / count;
    bounds[count - 1] = std::min(bounds[count - 1], n_full - 1);
    for (int64_t i = count - 2; i >= 1; --i) bounds[i] = std::min(bounds[i], bounds[i + 1] - 1);
    const int32_t srec[4] = {int32_t(t), int32_t(p.n_part_slots), int32_t(count), 0};
    p.splits.insert(p.splits.end(), srec, srec + 4);
    for (int64_t i = 0; i < count; ++i) {
      const int32_t rec[4] = {int32_t(t), int32_t(bounds[i]), int32_t(bounds[i + 1]),
                              int32_t(p.n_part_slots++)};
      natural.insert(natural.end(), rec, rec + 4);
    }
  }
  const int64_t n_items = int64_t(natural.size() / 4);
  std::vector<int32_t> rank_of(n_items);
  std::iota(rank_of.begin(), rank_of.end(), 0);
  std::stable_sort(rank_of.begin(), rank_of.end(), [&](int32_t a, int32_t b) {
    return natural[size_t(a) * 4 + 2] - natural[size_t(a) * 4 + 1] >
           natural[size_t(b) * 4 + 2] - natural[size_t(b) * 4 + 1];
  });
  p.items.reserve(natural.size());
  for (int32_t i : rank_of) p.items.insert(p.items.end(), &natural[size_t(i) * 4], &natural[size_t(i) * 4] + 4);
  return plan;
}

std::unique_ptr<Plan> build_pass_plan(const int32_t* seqlens, int32_t n_docs, int32_t cp,
                                      int32_t rank, int32_t block_t, int32_t block_n,
                                      uint64_t shard_mask, const int32_t* real_lengths) {
  validate_partition(seqlens, n_docs, cp, rank);
  if (cp > 64) fail(THD_ERANGE, "pass plans take cp <= 64 (one mask bit per source rank)");
  if (shard_mask == 0 || (cp < 64 && (shard_mask >> cp) != 0))
    fail(THD_EINVAL, "shard_mask must name at least one source rank, and only ranks < cp");
  auto plan = build_plan(seqlens, n_docs, cp, rank, block_t, block_n, 0, real_lengths);
  Plan& p = *plan;
  p.pass = true;
  p.shard_mask = shard_mask;
  p.items.clear();
  p.splits.clear();
  p.n_part_slots = 0;
  p.kv_split = 0;
  // Chunk k of a document is held by source rank min(k, 2cp-1-k). A tile of
  // chunk k's rows sees chunks 0..k; each maximal run [a, b] of those held by
  // a rank in the mask is one work item, from the run's first key to the end
  // of chunk b (or to the tile's last row when b is the rows' own chunk).
  auto held = [&](int64_t chunk) {
    const int64_t owner = std::min<int64_t>(chunk, 2 * int64_t(cp) - 1 - chunk);
    return ((shard_mask >> owner) & 1u) != 0;
  };
  const int64_t n_tiles = int64_t(p.tiles.size() / 8);
  std::vector<int32_t> natural;
  for (int64_t t = 0; t < n_tiles; ++t) {
    const int32_t* rec = &p.tiles[size_t(t) * 8];
    const int64_t q_glob = rec[1], n_rows = rec[2], doc = rec[3], slot = rec[4], cu = rec[5];
    const int64_t c = seqlens[doc] / (2 * int64_t(cp));
    const int64_t k = slot == 0 ? rank : 2 * int64_t(cp) - 1 - rank;
    const int64_t first = p.n_part_slots;
    for (int64_t chunk = 0; chunk <= k; ++chunk) {
      if (!held(chunk)) continue;
      const int64_t a = chunk;
      while (chunk + 1 <= k && held(chunk + 1)) ++chunk;
      const int64_t lo = cu + a * c;
      const int64_t hi = chunk < k ? cu + (chunk + 1) * c : q_glob + n_rows;
      const int64_t n_kv = (hi - lo + block_n - 1) / block_n;
      const int64_t n_full = std::min((q_glob - lo + 1) / block_n, (hi - lo) / block_n);
      const int32_t item[8] = {int32_t(t),    int32_t(lo),   int32_t(hi), int32_t(p.n_part_slots++),
                               int32_t(n_kv), int32_t(n_full), 0,         0};
      natural.insert(natural.end(), item, item + 8);
    }
    const int32_t srec[4] = {int32_t(t), int32_t(first), int32_t(p.n_part_slots - first), 0};
    p.splits.insert(p.splits.end(), srec, srec + 4);
  }
  const int64_t n_items = int64_t(natural.size() / 8);
  std::vector<int32_t> idx(n_items);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) {
    return natural[size_t(a) * 8 + 4] > natural[size_t(b) * 8 + 4];
  });
  p.items.reserve(natural.size());
  for (int32_t i : idx) p.items.insert(p.items.end(), &natural[size_t(i) * 8], &natural[size_t(i) * 8] + 8);
  // The kernel's view: runs in part-slot order (a tile's runs consecutive),
  // and the tiles with runs by their KV tiles, most first (stable), then the
  // tiles without runs (which a first or last pass still visits).
  p.pass_runs = natural;
  std::vector<int64_t> work(size_t(n_tiles), 0);
  for (int64_t i = 0; i < n_items; ++i) work[size_t(natural[size_t(i) * 8])] += natural[size_t(i) * 8 + 4];
  std::vector<int32_t> with, without;
  for (int64_t t = 0; t < n_tiles; ++t) (p.splits[size_t(t) * 4 + 2] > 0 ? with : without).push_back(int32_t(t));
  std::stable_sort(with.begin(), with.end(), [&](int32_t a, int32_t b) { return work[size_t(a)] > work[size_t(b)]; });
  p.n_run_tiles = int64_t(with.size());
  p.pass_order = with;
  p.pass_order.insert(p.pass_order.end(), without.begin(), without.end());
  return plan;
}

}  // namespace thd
