"""Per-tile document and causal bounds for one rank (oracle of the metadata).

Test infrastructure only (see the package docstring).

The subject page ("kvallgather cp thd load balance", section "What this PR does
/ why we need it?") says metadata is cached to avoid repeated computation but
gives no format. The format below is this project's interface contract between
the host planner and the GPU kernels (version 4). It is unique given
(lengths, cp, rank, BT, BN, concurrency), so the host library must reproduce it bit for bit.

Definitions (all integer, floor division of non-negative values):

tiles[n_tiles][8], natural order: for document i, slot s in (0, 1) (chunk
k = r for s = 0, k = 2cp-1-r for s = 1), token offsets t0 = 0, BT, 2BT, ... < c_i:
    n_rows  = min(BT, c_i - t0)
    q_glob  = cu_i + k*c_i + t0                    (global position of row 0)
    kv_len  = q_glob + n_rows - cu_i               (keys the last row sees)
    n_kv    = ceil(kv_len / BN)                    (KV tiles visited, from cu_i)
    n_full  = (q_glob - cu_i + 1) // BN            (KV tiles every row sees whole)
    record  = [cu_i/cp + s*c_i + t0, q_glob, n_rows, i, s, cu_i, n_kv, n_full]
KV tile j of a Q tile covers keys [cu_i + j*BN, cu_i + min((j+1)*BN, kv_len)).

doc_end[n_docs] (version 3): global position one past the last real token of
each document, cu_i + R_i. Without padding R_i = L_i; with padding-tolerant
partitioning (see partition.pad_lengths) R_i is the real length and tokens at
positions >= doc_end are pads.

order[n_tiles]: tile indices sorted by n_kv descending, ties by index
ascending (largest work first). Parity unpinned: it is a scheduling choice with
no truth outside this definition.

Forward work items (key-range splitting for load balance). Given
concurrency C (work items of one kv head the device runs at once; 0 = never
split) and T_kv = sum of n_kv over the tiles:
    kv_split = 0                            if C <= 0 or n_tiles >= 2 C
             = max(ceil(T_kv / C), 8)       otherwise
A tile with kv_split > 0, n_kv > kv_split and n_full >= 2 is cut into
P = min(ceil(n_kv / kv_split), n_full) parts at s_i = floor(i n_kv / P),
i = 1..P-1, then clamped from the last one down: s_{P-1} <= n_full - 1 and
s_i <= s_{i+1} - 1. Part i covers KV tiles [s_i, s_{i+1}) (s_0 = 0,
s_P = n_kv), so every part starts with a KV tile all of its rows see whole.
items[n_items][4] = [tile, kv_begin, kv_end, part slot or -1], listed by tile
then part and sorted by kv_end - kv_begin descending (ties by that listing
order); part slots count up over the split tiles in tile order.
splits[n_split][4] = [tile, first part slot, P, 0] in tile order.
(The items' order, like order above, is parity unpinned.)

kvtiles[m][8] (backward): for document i, j = 0 .. ceil(L_i / BN) - 1:
    ks      = cu_i + j*BN
    n_keys  = min(BN, L_i - j*BN)
    q_begin = first tile of document i (natural index) whose last row's global
              position is >= ks, or q_end if there is none
    q_end   = one past the last tile of document i
    record  = [i, ks, n_keys, q_begin, q_end, 0, 0, 0]
The key tiles cover every key once. Keys of document i at offset >=
(2cp-r)*c_i are seen by no local query (the rank's later chunk is 2cp-1-r), so
tiles made only of such keys get the empty range q_begin = q_end.

Packed forward plans (version 4; short-segment packing, a reading of the
column-wise [start, end) key bounds per row of the FlashMask kernels named on
"[Optim] FlashMask-4 Overlap support part 1 (NVSHMEM backend) - #166"). A
(document, slot) whose chunk length is not a multiple of BT leaves one
partial tile, its last. With key_cap = BN * K, where K is the largest n_kv
over all tiles, or min(K, kv_split) when the split rule above gives the
plain tiles a kv_split > 0 for the plan's concurrency (a packed tile is never
split, so it must not outlast the split parts), the partial tiles are taken
in tile order and grouped greedily. A tile of
document i adds keys add = kv_len - kv_len(prev) when the group's previous
member is also of document i (its keys are then a prefix of this tile's) and
add = kv_len otherwise; it joins the open group while the group's tokens plus
n_rows stay <= BT and the group's keys plus add stay <= key_cap, else the
group closes and a new one opens with it. A group of one tile stays as it is;
each larger group becomes one packed tile. The plan's tiles are the tiles in
no larger group (tile order), then the packed tiles (group order); order and
the work items are then formed over this list as above (a packed tile has
n_full = 0, so it is never split).
A packed tile lays its documents' keys out one document after the other: a
document's block starts at slot base_i and holds keys cu_i .. cu_i + K_i - 1,
K_i the kv_len of its last member. The member's row o (global position
g = q_glob + o) sees slots base_i .. base_i + (g - cu_i), exactly its causal
keys. Both window ends grow along the packed rows. Records:
    packed tile     = [-1, first pack row, tokens, -1, -1, first pack key,
                       n_kv = ceil(slots / BN), 0]
    pack_rows[.][4] = [local row, first visible slot, last visible slot,
                       1 if g < doc_end_i else 0], one per packed row, members
                       in group order
    pack_keys[.]    = gathered row (kv_row) of each slot's key, the tile's
                       slots padded to whole KV tiles with its last slot's
                       row (seen by no row)

Pass plans (all-gather overlap; a reading of "[Optim] FlashMask-4 Overlap
support part 1 (NVSHMEM backend) - #166", feature list, "AG fwd overlap"): a
forward pass over the keys of a set S of source ranks' shards. For each tile
(same tiles as above; document i, chunk k of its rows, q_glob, n_rows), the
chunks 0..k the rows can see are grouped into maximal runs [a, b] of
consecutive chunks whose owner min(chunk, 2cp-1-chunk) is in S. Run [a, b]
gives the work item
    lo     = cu_i + a*c_i
    hi     = cu_i + (b+1)*c_i if b < k else q_glob + n_rows
    n_kv   = ceil((hi - lo) / BN)            (KV tiles from lo)
    n_full = min((q_glob - lo + 1) // BN, (hi - lo) // BN)
    record = [tile, lo, hi, part slot, n_kv, n_full, 0, 0]
with part slots counted up over the runs in tile order. pass_items lists the
records sorted by n_kv descending (ties by that listing; parity unpinned);
pass_tiles[n_tiles][4] = [tile, first part slot, number of runs, 0] for every
tile in natural order (a tile with no run has 0). Every key of a run lies in a
chunk the rows see from its start, so every row sees the first key of each of
its items.
"""
from __future__ import annotations

import numpy as np

from . import partition

VERSION = 4
TILE_FIELDS = ("q_local_start", "q_global_start", "n_rows", "doc", "slot",
               "kv_start", "n_kv_tiles", "n_full_kv_tiles")
KVTILE_FIELDS = ("doc", "kv_global_start", "n_keys", "q_tile_begin", "q_tile_end",
                 "pad0", "pad1", "pad2")


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def tiles(seqlens, cp: int, rank: int, block_t: int, block_n: int) -> np.ndarray:
    lengths = partition.validate(seqlens, cp, rank)
    if block_t < 1 or block_n < 1:
        raise partition.PartitionError("tile sizes must be positive")
    cu = partition.cu_seqlens(lengths)
    rows = []
    for i, length in enumerate(lengths):
        c = length // (2 * cp)
        for s, k in enumerate(partition.owned_chunks(cp, rank)):
            for t0 in range(0, c, block_t):
                n_rows = min(block_t, c - t0)
                q_glob = cu[i] + k * c + t0
                kv_len = q_glob + n_rows - cu[i]
                n_kv = _ceil_div(kv_len, block_n)
                n_full = (q_glob - cu[i] + 1) // block_n
                rows.append([cu[i] // cp + s * c + t0, q_glob, n_rows, i, s, cu[i], n_kv, n_full])
    return np.asarray(rows, dtype=np.int32).reshape(-1, 8)


def doc_end(seqlens, cp: int, real_lengths=None) -> np.ndarray:
    """One past the last real token of each document (padded layout)."""
    lengths = partition.validate(seqlens, cp, 0)
    cu = partition.cu_seqlens(lengths)
    real = lengths if real_lengths is None else [int(x) for x in np.asarray(real_lengths).reshape(-1)]
    if len(real) != len(lengths) or any(not 1 <= r <= length for r, length in zip(real, lengths)):
        raise partition.PartitionError("real lengths must lie in [1, padded length]")
    return np.asarray([cu[i] + real[i] for i in range(len(lengths))], dtype=np.int32)


def order(tile_table: np.ndarray) -> np.ndarray:
    n_kv = [int(x) for x in tile_table[:, 6]]
    idx = sorted(range(len(n_kv)), key=lambda t: (-n_kv[t], t))
    return np.asarray(idx, dtype=np.int32)


def kvtiles(seqlens, cp: int, rank: int, block_t: int, block_n: int) -> np.ndarray:
    lengths = partition.validate(seqlens, cp, rank)
    cu = partition.cu_seqlens(lengths)
    tt = tiles(lengths, cp, rank, block_t, block_n)
    rows = []
    for i, length in enumerate(lengths):
        doc_tiles = [t for t in range(tt.shape[0]) if int(tt[t, 3]) == i]
        q_end = doc_tiles[-1] + 1
        for j in range(_ceil_div(length, block_n)):
            ks = cu[i] + j * block_n
            n_keys = min(block_n, length - j * block_n)
            q_begin = q_end
            for t in doc_tiles:
                if int(tt[t, 1]) + int(tt[t, 2]) - 1 >= ks:
                    q_begin = t
                    break
            rows.append([i, ks, n_keys, q_begin, q_end, 0, 0, 0])
    return np.asarray(rows, dtype=np.int32).reshape(-1, 8)


def useful_pairs_closed_form(seqlens, cp: int) -> int:
    """Sum over documents of L_i (L_i + 1) / (2 cp): the same for every rank.

    Chunk k of a document with chunk size c has c rows, the row at offset o
    seeing k*c + o + 1 keys. Chunks r and 2cp-1-r together see
    (2cp-1) c^2 + c (c+1) = L (L+1) / (2cp) pairs whatever r is.
    """
    total = 0
    for length in seqlens:
        length = int(length)
        total += length * (length + 1) // (2 * cp)
    return total


def kv_split_for(tile_table: np.ndarray, concurrency: int) -> int:
    n_tiles = int(tile_table.shape[0])
    if concurrency <= 0 or n_tiles >= 2 * concurrency:
        return 0
    total = sum(int(x) for x in tile_table[:, 6])
    return max(_ceil_div(total, concurrency), 8)


def _parts(n_kv: int, n_full: int, kv_split: int):
    if kv_split <= 0 or n_kv <= kv_split or n_full < 2:
        return [(0, n_kv)]
    count = min(_ceil_div(n_kv, kv_split), n_full)
    cuts = [i * n_kv // count for i in range(1, count)]
    cuts[-1] = min(cuts[-1], n_full - 1)
    for i in range(len(cuts) - 2, -1, -1):
        cuts[i] = min(cuts[i], cuts[i + 1] - 1)
    bounds = [0] + cuts + [n_kv]
    return [(bounds[i], bounds[i + 1]) for i in range(count)]


def items_and_splits(tile_table: np.ndarray, concurrency: int):
    """(items [n_items][4] in work order, splits [n_split][4])."""
    kv_split = kv_split_for(tile_table, concurrency)
    natural = []
    splits = []
    slot = 0
    for t in range(tile_table.shape[0]):
        parts = _parts(int(tile_table[t, 6]), int(tile_table[t, 7]), kv_split)
        if len(parts) == 1:
            natural.append([t, parts[0][0], parts[0][1], -1])
            continue
        splits.append([t, slot, len(parts), 0])
        for begin, end in parts:
            natural.append([t, begin, end, slot])
            slot += 1
    ranked = sorted(range(len(natural)), key=lambda i: (-(natural[i][2] - natural[i][1]), i))
    items = np.asarray([natural[i] for i in ranked], dtype=np.int32).reshape(-1, 4)
    return items, np.asarray(splits, dtype=np.int32).reshape(-1, 4)


def owner(chunk: int, cp: int) -> int:
    """Source rank whose shard holds a document's chunk (ranks own r, 2cp-1-r)."""
    return min(chunk, 2 * cp - 1 - chunk)


def pass_plan(seqlens, cp: int, rank: int, block_t: int, block_n: int, shards):
    """(pass_items [n][8] in work order, pass_tiles [n_tiles][4]) for the set of
    source ranks ``shards`` (see the module docstring)."""
    lengths = partition.validate(seqlens, cp, rank)
    held = {int(x) for x in shards}
    cu = partition.cu_seqlens(lengths)
    tt = tiles(lengths, cp, rank, block_t, block_n)
    natural = []
    table = []
    slot = 0
    for t in range(tt.shape[0]):
        q_glob, n_rows, i, s = (int(x) for x in tt[t, 1:5])
        c = lengths[i] // (2 * cp)
        k = rank if s == 0 else 2 * cp - 1 - rank
        first = slot
        chunk = 0
        while chunk <= k:
            if owner(chunk, cp) not in held:
                chunk += 1
                continue
            a = chunk
            while chunk + 1 <= k and owner(chunk + 1, cp) in held:
                chunk += 1
            b = chunk
            lo = cu[i] + a * c
            hi = cu[i] + (b + 1) * c if b < k else q_glob + n_rows
            n_kv = _ceil_div(hi - lo, block_n)
            n_full = min((q_glob - lo + 1) // block_n, (hi - lo) // block_n)
            natural.append([t, lo, hi, slot, n_kv, n_full, 0, 0])
            slot += 1
            chunk += 1
        table.append([t, first, slot - first, 0])
    ranked = sorted(range(len(natural)), key=lambda j: (-natural[j][4], j))
    items = np.asarray([natural[j] for j in ranked], dtype=np.int32).reshape(-1, 8)
    return items, np.asarray(table, dtype=np.int32).reshape(-1, 4)


def packed_plan(seqlens, cp: int, rank: int, block_t: int, block_n: int, real_lengths=None,
                concurrency: int = 0):
    """(tiles, pack_rows, pack_keys) of a packed forward plan (module docstring)."""
    lengths = partition.validate(seqlens, cp, rank)
    tt = tiles(lengths, cp, rank, block_t, block_n)
    cu = partition.cu_seqlens(lengths)
    rowmap = partition.kv_row(lengths, cp)
    ends = doc_end(lengths, cp, real_lengths)
    longest = max(int(x) for x in tt[:, 6])
    split = kv_split_for(tt, concurrency)
    key_cap = block_n * (min(longest, split) if split > 0 else longest)

    def kv_len(t):
        return int(tt[t, 1]) + int(tt[t, 2]) - int(tt[t, 5])

    groups, group, g_tok, g_keys = [], [], 0, 0
    for t in range(tt.shape[0]):
        if int(tt[t, 2]) == block_t:
            continue
        same_doc = bool(group) and int(tt[group[-1], 3]) == int(tt[t, 3])
        add = kv_len(t) - (kv_len(group[-1]) if same_doc else 0)
        if group and g_tok + int(tt[t, 2]) <= block_t and g_keys + add <= key_cap:
            group.append(t)
            g_tok += int(tt[t, 2])
            g_keys += add
            continue
        if group:
            groups.append(group)
        group, g_tok, g_keys = [t], int(tt[t, 2]), kv_len(t)
    if group:
        groups.append(group)

    packed = {t for g in groups if len(g) > 1 for t in g}
    out = [[int(x) for x in tt[t]] for t in range(tt.shape[0]) if t not in packed]
    rows, keys = [], []
    for g in groups:
        if len(g) == 1:
            continue
        row0, key0 = len(rows), len(keys)
        docs = []                       # (doc, base slot, K) in order
        for t in g:
            i = int(tt[t, 3])
            if docs and docs[-1][0] == i:
                docs[-1][2] = max(docs[-1][2], kv_len(t))
            else:
                docs.append([i, sum(d[2] for d in docs), kv_len(t)])
        base = {d[0]: d[1] for d in docs}
        for i, _, k_i in docs:
            keys.extend(int(rowmap[cu[i] + x]) for x in range(k_i))
        for t in g:
            q_local, q_glob, n_rows, i = (int(x) for x in tt[t, :4])
            for o in range(n_rows):
                g_pos = q_glob + o
                rows.append([q_local + o, base[i], base[i] + g_pos - cu[i],
                             1 if g_pos < int(ends[i]) else 0])
        slots = len(keys) - key0
        n_kv = _ceil_div(slots, block_n)
        keys.extend([keys[-1]] * (n_kv * block_n - slots))
        out.append([-1, row0, len(rows) - row0, -1, -1, key0, n_kv, 0])
    return (np.asarray(out, dtype=np.int32).reshape(-1, 8),
            np.asarray(rows, dtype=np.int32).reshape(-1, 4),
            np.asarray(keys, dtype=np.int32))


def packed_forward_plan(seqlens, cp: int, rank: int, block_t: int, block_n: int,
                        concurrency: int, real_lengths=None) -> dict:
    """Every table of a packed forward plan: tiles, order, items, splits,
    pack_rows, pack_keys (order and items over the packed tile list)."""
    tt, rows, keys = packed_plan(seqlens, cp, rank, block_t, block_n, real_lengths, concurrency)
    items, splits = items_and_splits(tt, concurrency)
    return {"tiles": tt, "order": order(tt), "items": items, "splits": splits,
            "pack_rows": rows, "pack_keys": keys}
