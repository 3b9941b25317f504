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
  if (rank < 0 || rank >= cp) fail(THD_ERANGE, "rank must be in [0, cp)");
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

std::unique_ptr<Plan> build_plan(const int32_t* seqlens, int32_t n_docs, int32_t cp,
                                 int32_t rank, int32_t block_t, int32_t block_n,
                                 int32_t concurrency, const int32_t* real_lengths) {
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
  // is 2cp-1-r), so their tiles get an empty range.
  cu = 0;
  for (int32_t i = 0; i < n_docs; ++i) {
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

}  // namespace thd
