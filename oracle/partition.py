"""Symmetric EOD-aware partition of THD-packed sequences (oracle).

Test infrastructure only (see the package docstring).

Source: "kvallgather cp thd load balance" (Ascend/MindSpeed pull request),
section "What this PR does / why we need it?": EOD-aware symmetric sequence
partitioning with direct rank-major K/V indexing; section "Does this PR
introduce any user-facing change?": every packed subsequence length is
divisible by 2 * context_parallel_size.

Readings taken where the page is silent:
  * chunking is per subsequence (document): document i of length L_i is cut
    into 2*cp chunks of c_i = L_i / (2*cp) tokens; rank r owns chunks r and
    2*cp-1-r ("symmetric");
  * a rank's local rows keep documents in packed order and, inside a
    document, chunk r before chunk 2*cp-1-r, so document i starts at local
    row cu_i / cp;
  * "rank-major" K/V is the all-gather result: rank 0's local shard, then
    rank 1's, ..., each in that rank's own local order.

All loops below are plain Python integer loops over tokens.
"""
from __future__ import annotations

import numpy as np


class PartitionError(ValueError):
    pass


def validate(seqlens, cp: int, rank: int) -> list[int]:
    """Check the divisibility rule and argument ranges; return lengths as ints."""
    lengths = [int(x) for x in np.asarray(seqlens).reshape(-1)]
    if cp < 1:
        raise PartitionError("cp must be >= 1")
    if not 0 <= rank < cp:
        raise PartitionError("rank must be in [0, cp)")
    if len(lengths) == 0:
        raise PartitionError("at least one subsequence is required")
    for length in lengths:
        if length < 1:
            raise PartitionError("subsequence lengths must be positive")
        if length % (2 * cp) != 0:
            raise PartitionError("each subsequence length must be divisible by 2*cp")
    return lengths


def pad_lengths(real_lengths, cp: int) -> list[int]:
    """Padded length of each document: the least multiple of 2*cp holding it.

    Padding-tolerant partitioning (a reading: the subject page requires every
    length to be divisible by 2*cp; this relaxes it). A document of R real
    tokens is stored as L = ceil(R / 2cp) * 2cp tokens, its R real tokens
    first and L - R pad tokens after them, and is partitioned like any other
    document of length L. Every pad token comes after every real token of its
    document, so the causal mask already hides the pads from real queries.
    """
    real = [int(x) for x in np.asarray(real_lengths).reshape(-1)]
    if cp < 1:
        raise PartitionError("cp must be >= 1")
    if len(real) == 0:
        raise PartitionError("at least one subsequence is required")
    out = []
    for r in real:
        if r < 1:
            raise PartitionError("subsequence lengths must be positive")
        out.append(-(-r // (2 * cp)) * (2 * cp))
    return out


def pad_rows(real_lengths, cp: int, rank: int) -> np.ndarray:
    """Bool per local row of the padded layout: True for pad tokens."""
    lengths = pad_lengths(real_lengths, cp)
    cu = cu_seqlens(lengths)
    ends = [cu[i] + int(r) for i, r in enumerate(np.asarray(real_lengths).reshape(-1))]
    docs = doc_of(lengths)
    return np.asarray([g >= ends[int(docs[g])] for g in q_global(lengths, cp, rank).tolist()],
                      dtype=bool)


def cu_seqlens(lengths) -> list[int]:
    """Exclusive prefix sums: cu[0] = 0, cu[i+1] = cu[i] + L_i."""
    cu = [0]
    for length in lengths:
        cu.append(cu[-1] + int(length))
    return cu


def owned_chunks(cp: int, rank: int) -> tuple[int, int]:
    """The two chunk indices rank ``rank`` owns, in local order."""
    return rank, 2 * cp - 1 - rank


def q_global(seqlens, cp: int, rank: int) -> np.ndarray:
    """Global packed position of each of the rank's local query rows.

    Local rows run document by document; inside document i come the c_i
    tokens of chunk r, then the c_i tokens of chunk 2*cp-1-r.
    """
    lengths = validate(seqlens, cp, rank)
    cu = cu_seqlens(lengths)
    out = []
    for i, length in enumerate(lengths):
        c = length // (2 * cp)
        for chunk in owned_chunks(cp, rank):
            for o in range(c):
                out.append(cu[i] + chunk * c + o)
    return np.asarray(out, dtype=np.int32)


def gathered_order(seqlens, cp: int) -> np.ndarray:
    """Global position of every row of the all-gathered (rank-major) K/V.

    The all-gather concatenates the local shards of ranks 0..cp-1 in rank
    order, so row j*T_local + l holds global token q_global(rank j)[l].
    """
    return np.concatenate([q_global(seqlens, cp, j) for j in range(cp)])


def kv_row(seqlens, cp: int) -> np.ndarray:
    """Row of the rank-major gathered K/V that holds each global token.

    The inverse of :func:`gathered_order`; it does not depend on the rank.
    """
    order = gathered_order(seqlens, cp)
    inv = np.full(order.shape[0], -1, dtype=np.int64)
    for row, g in enumerate(order.tolist()):
        inv[g] = row
    return inv.astype(np.int32)


def chunk_off(seqlens, cp: int) -> np.ndarray:
    """Gathered row of the first token of every chunk, [n_docs * 2cp]."""
    lengths = validate(seqlens, cp, 0)
    cu = cu_seqlens(lengths)
    rows = kv_row(lengths, cp)
    out = []
    for i, length in enumerate(lengths):
        c = length // (2 * cp)
        for chunk in range(2 * cp):
            out.append(int(rows[cu[i] + chunk * c]))
    return np.asarray(out, dtype=np.int32)


def doc_of(seqlens) -> np.ndarray:
    """Document index of every global token."""
    out = []
    for i, length in enumerate(seqlens):
        out.extend([i] * int(length))
    return np.asarray(out, dtype=np.int32)


def visible_count(seqlens, cp: int, rank: int) -> int:
    """Number of (local query, key) pairs the causal + EOD mask leaves open.

    Counted token by token: a query at global position g in document i sees
    the keys cu_i .. g, that is g - cu_i + 1 keys.
    """
    lengths = validate(seqlens, cp, rank)
    cu = cu_seqlens(lengths)
    docs = doc_of(lengths)
    total = 0
    for g in q_global(lengths, cp, rank).tolist():
        total += g - cu[int(docs[g])] + 1
    return total
