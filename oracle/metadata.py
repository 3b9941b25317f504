"""Per-tile document and causal bounds for one rank (oracle of the metadata).

Test infrastructure only (see the package docstring).

The subject page ("kvallgather cp thd load balance", section "What this PR does
/ why we need it?") says metadata is cached to avoid repeated computation but
gives no format. The format below is this project's interface contract between
the host planner and the GPU kernels (version 1). It is unique given
(lengths, cp, rank, BT, BN), so the host library must reproduce it bit for bit.

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

order[n_tiles]: tile indices sorted by n_kv descending, ties by index
ascending (largest work first). Parity unpinned: it is a scheduling choice with
no truth outside this definition.

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

VERSION = 1
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
