"""Per-tile document and causal bounds for one rank (oracle of the metadata).

Test infrastructure only (see the package docstring).

The subject page ("kvallgather cp thd load balance", section "What this PR does
/ why we need it?") says metadata is cached to avoid repeated computation but
gives no format. The format below is this project's interface contract between
the host planner and the GPU kernels (version 3). It is unique given
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
"""
from __future__ import annotations

import numpy as np

from . import partition

VERSION = 3
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
