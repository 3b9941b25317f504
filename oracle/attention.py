"""fp64 causal + EOD-reset attention for one context-parallel rank (oracle).

Test infrastructure only (see the package docstring).

Source: "kvallgather cp thd load balance" (Ascend/MindSpeed pull request). The
section "What this PR does / why we need it?" names the computation (THD
attention over the rank's query shard against all-gathered, rank-major K/V,
MHA / GQA / expanded MLA); the section "Does this PR introduce any user-facing
change?" fixes the mask (causal, reset at every EOD). The page prints no
formula, so the textbook softmax attention is taken:

  for local row l at global position g in document i, and q head h with kv
  head h // G (G = Hq / Hkv, contiguous head groups):
    s_j    = scale * <Q[l, h], K_glob[j, h // G]>     for cu_i <= j <= g
    LSE    = ln sum_j exp(s_j)
    O[l,h] = sum_j exp(s_j - LSE) * V_glob[j, h // G]
  K_glob[j] = K[kv_row[j]] undoes the rank-major all-gather.

Backward, for a given dO, with P = exp(S - LSE) and D = rowsum(dO * O):
    dP = dO V^T,  dS = P * (dP - D),  dQ = scale * dS K,
    dK = scale * dS^T Q,  dV = P^T dO,
  dK and dV summed over the G q heads of each kv head and returned in the
  rank-major gathered layout (keys no local query sees get exact zeros).

Everything is float64 numpy; the caller passes bf16 values widened exactly.
Readings: scale defaults to 1/sqrt(dqk); LSE uses the natural log.
"""
from __future__ import annotations

import math

import numpy as np

from . import partition


def _check(q, k, v, seqlens, cp, rank):
    lengths = partition.validate(seqlens, cp, rank)
    total = sum(lengths)
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3:
        raise ValueError("q, k, v must be [tokens, heads, dim]")
    if q.shape[0] != total // cp or k.shape[0] != total or v.shape[0] != total:
        raise ValueError("token counts do not match the lengths")
    hq, hkv = q.shape[1], k.shape[1]
    if hq % hkv != 0 or v.shape[1] != hkv or q.shape[2] != k.shape[2]:
        raise ValueError("head shapes do not match")
    return lengths, hq // hkv


def to_global(x_gathered: np.ndarray, seqlens, cp: int) -> np.ndarray:
    """Reorder rank-major gathered rows into global packed order."""
    rows = partition.kv_row(seqlens, cp)
    return x_gathered[rows]


def _segments(lengths, cp, rank):
    """(local row start, global row start, chunk size, doc start, chunk) per owned chunk."""
    cu = partition.cu_seqlens(lengths)
    for i, length in enumerate(lengths):
        c = length // (2 * cp)
        for s, chunk in enumerate(partition.owned_chunks(cp, rank)):
            yield cu[i] // cp + s * c, cu[i] + chunk * c, c, cu[i], chunk


def attn_fwd64(q, k, v, seqlens, cp, rank, scale=None):
    """O [T_loc, Hq, dv] and LSE [T_loc, Hq] for every local row (fp64)."""
    q = np.asarray(q, dtype=np.float64)
    lengths, group = _check(q, k, v, seqlens, cp, rank)
    kg = to_global(np.asarray(k, dtype=np.float64), lengths, cp)
    vg = to_global(np.asarray(v, dtype=np.float64), lengths, cp)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[2])
    tl, hq = q.shape[0], q.shape[1]
    out = np.zeros((tl, hq, v.shape[2]))
    lse = np.zeros((tl, hq))
    for lstart, gstart, c, doc_start, chunk in _segments(lengths, cp, rank):
        n_keys = (chunk + 1) * c
        # column j (key doc_start + j) is visible to segment row o iff j <= chunk*c + o
        visible = np.arange(n_keys)[None, :] <= (chunk * c + np.arange(c))[:, None]
        for hk in range(k.shape[1]):
            keys = kg[doc_start:doc_start + n_keys, hk]
            vals = vg[doc_start:doc_start + n_keys, hk]
            for h in range(hk * group, (hk + 1) * group):
                s = scale * (q[lstart:lstart + c, h] @ keys.T)
                s = np.where(visible, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                p = np.exp(s - m)
                denom = p.sum(axis=1, keepdims=True)
                out[lstart:lstart + c, h] = (p @ vals) / denom
                lse[lstart:lstart + c, h] = (m + np.log(denom))[:, 0]
    return out, lse


def attn_fwd64_rows(q, k, v, seqlens, cp, rank, rows, scale=None):
    """O and LSE for the given local rows only, one row at a time (fp64).

    Used to check sampled rows of full-size workloads.
    """
    q = np.asarray(q)
    lengths, group = _check(q, k, v, seqlens, cp, rank)
    cu = partition.cu_seqlens(lengths)
    docs = partition.doc_of(lengths)
    qg = partition.q_global(lengths, cp, rank)
    rowmap = partition.kv_row(lengths, cp)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[2])
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.shape[0], q.shape[1], v.shape[2]))
    lse = np.zeros((rows.shape[0], q.shape[1]))
    for n, row in enumerate(rows.tolist()):
        g = int(qg[row])
        start = cu[int(docs[g])]
        gathered = rowmap[start:g + 1]
        keys = np.asarray(k[gathered], dtype=np.float64)    # [n, Hkv, d]
        vals = np.asarray(v[gathered], dtype=np.float64)
        for h in range(q.shape[1]):
            s = scale * (keys[:, h // group] @ np.asarray(q[row, h], dtype=np.float64))
            m = s.max()
            p = np.exp(s - m)
            out[n, h] = (p @ vals[:, h // group]) / p.sum()
            lse[n, h] = m + math.log(p.sum())
    return out, lse


def attn_bwd64(q, k, v, do, seqlens, cp, rank, scale=None):
    """dQ [T_loc, Hq, dqk], dK [T, Hkv, dqk], dV [T, Hkv, dv] (fp64).

    dK and dV are rank partials in the rank-major gathered layout: a key no
    local query sees gets exact zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    lengths, group = _check(q, k, v, seqlens, cp, rank)
    rowmap = partition.kv_row(lengths, cp)
    kg = np.asarray(k, dtype=np.float64)[rowmap]
    vg = np.asarray(v, dtype=np.float64)[rowmap]
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[2])
    dq = np.zeros_like(q)
    dkg = np.zeros_like(kg)
    dvg = np.zeros_like(vg)
    for lstart, gstart, c, doc_start, chunk in _segments(lengths, cp, rank):
        n_keys = (chunk + 1) * c
        visible = np.arange(n_keys)[None, :] <= (chunk * c + np.arange(c))[:, None]
        for hk in range(k.shape[1]):
            keys = kg[doc_start:doc_start + n_keys, hk]
            vals = vg[doc_start:doc_start + n_keys, hk]
            for h in range(hk * group, (hk + 1) * group):
                qs = q[lstart:lstart + c, h]
                dos = do[lstart:lstart + c, h]
                s = np.where(visible, scale * (qs @ keys.T), -np.inf)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                p = e / e.sum(axis=1, keepdims=True)
                o = p @ vals
                d_row = (dos * o).sum(axis=1, keepdims=True)
                dp = dos @ vals.T
                ds = p * (dp - d_row)
                dq[lstart:lstart + c, h] = scale * (ds @ keys)
                dkg[doc_start:doc_start + n_keys, hk] += scale * (ds.T @ qs)
                dvg[doc_start:doc_start + n_keys, hk] += p.T @ dos
    dk = np.zeros_like(dkg)
    dv = np.zeros_like(dvg)
    dk[rowmap] = dkg
    dv[rowmap] = dvg
    return dq, dk, dv


def attn_fwd64_shards(q, k, v, seqlens, cp, rank, shards, scale=None):
    """O and LSE over the keys held by the given source ranks' shards (fp64).

    Reading for the all-gather overlap of the FlashMask-4 overlap page
    ("[Optim] FlashMask-4 Overlap support part 1 (NVSHMEM backend) - #166",
    feature list, "AG fwd overlap"): the all-gather delivers K/V one source
    rank's shard at a time, rank s's shard holding chunks s and 2cp-1-s of
    every document; a forward pass over the shards that have arrived computes
    the attention of each row restricted to the keys of those shards. With
    every shard it is attn_fwd64. A row that sees no key of the set gets
    O = 0 and LSE = -inf (the log of an empty sum).
    """
    q = np.asarray(q, dtype=np.float64)
    lengths, group = _check(q, k, v, seqlens, cp, rank)
    shards = {int(x) for x in shards}
    kg = to_global(np.asarray(k, dtype=np.float64), lengths, cp)
    vg = to_global(np.asarray(v, dtype=np.float64), lengths, cp)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[2])
    tl, hq = q.shape[0], q.shape[1]
    out = np.zeros((tl, hq, v.shape[2]))
    lse = np.full((tl, hq), -np.inf)
    for lstart, gstart, c, doc_start, chunk in _segments(lengths, cp, rank):
        n_keys = (chunk + 1) * c
        visible = np.arange(n_keys)[None, :] <= (chunk * c + np.arange(c))[:, None]
        # key j of the document lies in chunk j // c, owned by rank min(k, 2cp-1-k)
        owner = np.minimum(np.arange(n_keys) // c, 2 * cp - 1 - np.arange(n_keys) // c)
        held = np.isin(owner, sorted(shards))
        visible = visible & held[None, :]
        seen = visible.any(axis=1)
        if not seen.any():
            continue
        for hk in range(k.shape[1]):
            keys = kg[doc_start:doc_start + n_keys, hk]
            vals = vg[doc_start:doc_start + n_keys, hk]
            for h in range(hk * group, (hk + 1) * group):
                s = scale * (q[lstart:lstart + c, h] @ keys.T)
                s = np.where(visible, s, -np.inf)[seen]
                m = s.max(axis=1, keepdims=True)
                p = np.exp(s - m)
                denom = p.sum(axis=1, keepdims=True)
                rows = lstart + np.nonzero(seen)[0]
                out[rows, h] = (p @ vals) / denom
                lse[rows, h] = (m + np.log(denom))[:, 0]
    return out, lse


def merge_lse(parts):
    """Merge partial softmax results over disjoint key sets (fp64).

    parts: (O_i, LSE_i) pairs, each the attention over its own key set. The
    softmax over the union weights each part by exp(LSE_i - LSE) with
    LSE = ln sum_i exp(LSE_i); parts with LSE = -inf weigh nothing, and a row
    no part covers stays O = 0, LSE = -inf.
    """
    lses = np.stack([np.asarray(l, dtype=np.float64) for _, l in parts])
    m = lses.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.exp(lses - m_safe[None])
    total = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, total, 1.0)), -np.inf)
    out = np.zeros_like(np.asarray(parts[0][0], dtype=np.float64))
    for (o, _), wi in zip(parts, w):
        out += wi[..., None] * np.asarray(o, dtype=np.float64)
    out = np.where(finite[..., None], out / np.where(finite, total, 1.0)[..., None], 0.0)
    return out, lse


def attn_fwd64_padded(q, k, v, real_lengths, cp, rank, scale=None):
    """Forward over the padded layout of partition.pad_lengths (fp64).

    Real rows: the attention above over their document's keys cu_i .. g, all
    real (pads follow every real token). Pad rows (a reading; the pages have no
    padding): O = 0 and LSE = +inf, the log-sum-exp that makes exp(S - LSE)
    vanish, so that a backward built on P = exp(S - LSE) gives them nothing.
    """
    lengths = partition.pad_lengths(real_lengths, cp)
    out, lse = attn_fwd64(q, k, v, lengths, cp, rank, scale)
    pad = partition.pad_rows(real_lengths, cp, rank)
    out[pad] = 0.0
    lse[pad] = np.inf
    return out, lse


def attn_bwd64_padded(q, k, v, do, real_lengths, cp, rank, scale=None):
    """Backward over the padded layout: pad rows take part with P = 0.

    With P = 0 on a pad row its dS is 0 whatever dO holds there, so it adds
    nothing to dK, dV and gets dQ = 0; pad keys are seen by no real row and get
    exact zeros. That is the backward above with dO zeroed on pad rows.
    """
    lengths = partition.pad_lengths(real_lengths, cp)
    do = np.array(do, dtype=np.float64)
    do[partition.pad_rows(real_lengths, cp, rank)] = 0.0
    return attn_bwd64(q, k, v, do, lengths, cp, rank, scale)


def brute_fwd(q, k, v, seqlens, cp, rank, scale=None):
    """Pure Python loops over (row, head, key, dim); tiny inputs only.

    Independent of the numpy path above: it walks tokens with explicit
    document bounds and accumulates the softmax with math.exp.
    """
    lengths, group = _check(np.asarray(q), k, v, seqlens, cp, rank)
    cu = partition.cu_seqlens(lengths)
    docs = partition.doc_of(lengths)
    qg = partition.q_global(lengths, cp, rank)
    rowmap = partition.kv_row(lengths, cp)
    tl, hq, dqk = np.asarray(q).shape
    dv = np.asarray(v).shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    qa = np.asarray(q, dtype=np.float64).tolist()
    ka = np.asarray(k, dtype=np.float64).tolist()
    va = np.asarray(v, dtype=np.float64).tolist()
    out = [[[0.0] * dv for _ in range(hq)] for _ in range(tl)]
    lse = [[0.0] * hq for _ in range(tl)]
    for row in range(tl):
        g = int(qg[row])
        start = cu[int(docs[g])]
        for h in range(hq):
            hk = h // group
            scores = []
            for j in range(start, g + 1):
                kr = ka[int(rowmap[j])][hk]
                acc = 0.0
                for d in range(dqk):
                    acc += qa[row][h][d] * kr[d]
                scores.append(scale * acc)
            m = max(scores)
            weights = [math.exp(s - m) for s in scores]
            total = sum(weights)
            for d in range(dv):
                acc = 0.0
                for w, j in zip(weights, range(start, g + 1)):
                    acc += w * va[int(rowmap[j])][hk][d]
                out[row][h][d] = acc / total
            lse[row][h] = m + math.log(total)
    return np.asarray(out), np.asarray(lse)
