"""Pins of the fp64 attention oracle (CPU only).

The oracle is checked against: a pure-loop brute force, PyTorch's
scaled_dot_product_attention in float64 with an explicit block-diagonal causal
mask on the unpartitioned packed sequence (a library special case), closed
forms (zero queries, document-start rows), plain causal attention for one
document at cp=1, float64 autograd of the library formulation, central finite
differences, and gradient identities that hold for any softmax attention.
"""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import attention, partition


def _case(seed, lengths, cp, rank, hq, hkv, dqk, dv, with_do=False):
    rng = np.random.default_rng(seed)
    total = int(sum(lengths))
    q = rng.standard_normal((total // cp, hq, dqk))
    k = rng.standard_normal((total, hkv, dqk))
    v = rng.standard_normal((total, hkv, dv))
    do = rng.standard_normal((total // cp, hq, dv)) if with_do else None
    return q, k, v, do


def _library_reference(q_loc, k, v, lengths, cp, rank, scale):
    """SDPA(float64) over the unpartitioned sequence, returned for the rank's rows.

    Every rank's queries are needed to rebuild the global Q; other ranks' rows
    are filled with independent noise, which the mask keeps out of this rank's
    outputs.
    """
    total = int(sum(lengths))
    qg = partition.q_global(lengths, cp, rank)
    kg = attention.to_global(k, lengths, cp)
    vg = attention.to_global(v, lengths, cp)
    q_full = np.random.default_rng(999).standard_normal((total,) + q_loc.shape[1:])
    q_full[qg] = q_loc
    docs = partition.doc_of(lengths)
    idx = np.arange(total)
    mask = (docs[:, None] == docs[None, :]) & (idx[None, :] <= idx[:, None])
    group = q_loc.shape[1] // k.shape[1]
    qt = torch.from_numpy(q_full).permute(1, 0, 2)
    kt = torch.from_numpy(kg).repeat_interleave(group, dim=1).permute(1, 0, 2)
    vt = torch.from_numpy(vg).repeat_interleave(group, dim=1).permute(1, 0, 2)
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.from_numpy(mask), scale=scale)
    return out.permute(1, 0, 2).numpy()[qg]


@pytest.mark.parametrize("lengths,cp,rank,hq,hkv,dqk,dv", [
    ([8, 16, 8], 2, 0, 2, 1, 8, 4),
    ([8, 16, 8], 2, 1, 4, 2, 6, 6),
    ([12, 24], 3, 2, 3, 3, 5, 7),
    ([8], 4, 3, 2, 2, 4, 4),
])
def test_numpy_oracle_matches_brute_force(lengths, cp, rank, hq, hkv, dqk, dv):
    q, k, v, _ = _case(1, lengths, cp, rank, hq, hkv, dqk, dv)
    o, lse = attention.attn_fwd64(q, k, v, lengths, cp, rank)
    ob, lseb = attention.brute_fwd(q, k, v, lengths, cp, rank)
    assert np.max(np.abs(o - ob)) <= 1e-12
    assert np.max(np.abs(lse - lseb)) <= 1e-12
    rows = np.arange(q.shape[0])
    orr, lser = attention.attn_fwd64_rows(q, k, v, lengths, cp, rank, rows)
    assert np.max(np.abs(o - orr)) <= 1e-12
    assert np.max(np.abs(lse - lser)) <= 1e-12


@pytest.mark.parametrize("lengths,cp,rank,hq,hkv,dqk,dv", [
    ([64, 128, 64], 2, 0, 4, 4, 16, 16),
    ([64, 128, 64], 2, 1, 8, 2, 16, 8),
    ([48, 16, 96, 32], 4, 2, 4, 1, 24, 16),
    ([80, 240], 8, 5, 2, 2, 12, 8),
])
def test_oracle_matches_library_sdpa(lengths, cp, rank, hq, hkv, dqk, dv):
    q, k, v, _ = _case(2, lengths, cp, rank, hq, hkv, dqk, dv)
    scale = 0.37
    o, _ = attention.attn_fwd64(q, k, v, lengths, cp, rank, scale=scale)
    ref = _library_reference(q, k, v, lengths, cp, rank, scale)
    assert np.max(np.abs(o - ref)) <= 1e-12


def test_single_document_cp1_is_plain_causal_attention():
    q, k, v, _ = _case(3, [96], 1, 0, 4, 2, 16, 16)
    o, _ = attention.attn_fwd64(q, k, v, [96], 1, 0)
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).repeat_interleave(2, dim=1).permute(1, 0, 2)
    vt = torch.from_numpy(v).repeat_interleave(2, dim=1).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    assert np.max(np.abs(o - ref.permute(1, 0, 2).numpy())) <= 1e-12


def test_zero_queries_give_prefix_means_and_log_counts():
    lengths, cp, rank = [16, 32, 8], 2, 1
    q, k, v, _ = _case(4, lengths, cp, rank, 4, 2, 8, 8)
    q[:] = 0.0
    o, lse = attention.attn_fwd64(q, k, v, lengths, cp, rank)
    cu = partition.cu_seqlens(lengths)
    docs = partition.doc_of(lengths)
    vg = attention.to_global(v, lengths, cp)
    for row, g in enumerate(partition.q_global(lengths, cp, rank).tolist()):
        start = cu[int(docs[g])]
        mean = vg[start:g + 1].mean(axis=0)              # [Hkv, dv]
        for h in range(4):
            assert np.allclose(o[row, h], mean[h // 2], rtol=0, atol=1e-13)
            assert abs(lse[row, h] - math.log(g - start + 1)) <= 1e-13


def test_document_start_rows_copy_v_exactly():
    lengths, cp = [16, 32, 8], 2
    q, k, v, _ = _case(5, lengths, cp, 0, 4, 4, 8, 8)
    o, lse = attention.attn_fwd64(q, k, v, lengths, cp, 0)
    cu = partition.cu_seqlens(lengths)
    qg = partition.q_global(lengths, cp, 0).tolist()
    vg = attention.to_global(v, lengths, cp)
    for start in cu[:-1]:
        row = qg.index(start)
        assert np.array_equal(o[row], vg[start])


def test_eod_isolation_and_causality():
    """Changing another document's K/V, or a later key, leaves a row unchanged."""
    lengths, cp, rank = [16, 32, 16], 2, 0
    q, k, v, _ = _case(6, lengths, cp, rank, 2, 2, 8, 8)
    o, _ = attention.attn_fwd64(q, k, v, lengths, cp, rank)
    rows = partition.kv_row(lengths, cp)
    k2, v2 = k.copy(), v.copy()
    k2[rows[:16]] += 5.0          # document 0's keys
    v2[rows[:16]] -= 3.0
    o2, _ = attention.attn_fwd64(q, k2, v2, lengths, cp, rank)
    qg = partition.q_global(lengths, cp, rank)
    other = qg >= 16
    assert np.array_equal(o[other], o2[other])
    assert not np.allclose(o[~other], o2[~other])
    k3 = k.copy()
    k3[rows[40:48]] += 7.0        # keys 40..47 of document 1
    o3, _ = attention.attn_fwd64(q, k3, v, lengths, cp, rank)
    before = qg < 40
    assert np.array_equal(o[before], o3[before])


def _library_grads(q_loc, k, v, do, lengths, cp, rank, scale):
    total = int(sum(lengths))
    qg = partition.q_global(lengths, cp, rank)
    rows = partition.kv_row(lengths, cp)
    docs = partition.doc_of(lengths)
    idx = np.arange(total)
    mask = torch.from_numpy((docs[:, None] == docs[None, :]) & (idx[None, :] <= idx[:, None]))
    group = q_loc.shape[1] // k.shape[1]
    q_full = np.zeros((total,) + q_loc.shape[1:])
    q_full[qg] = q_loc
    qt = torch.from_numpy(q_full).requires_grad_()
    kt = torch.from_numpy(k[rows]).requires_grad_()
    vt = torch.from_numpy(v[rows]).requires_grad_()
    out = torch.nn.functional.scaled_dot_product_attention(
        qt.permute(1, 0, 2), kt.repeat_interleave(group, dim=1).permute(1, 0, 2),
        vt.repeat_interleave(group, dim=1).permute(1, 0, 2), attn_mask=mask, scale=scale)
    out = out.permute(1, 0, 2)[torch.from_numpy(qg.astype(np.int64))]
    (out * torch.from_numpy(do)).sum().backward()
    dq = qt.grad.numpy()[qg]
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dk[rows] = kt.grad.numpy()
    dv[rows] = vt.grad.numpy()
    return dq, dk, dv


@pytest.mark.parametrize("lengths,cp,rank,hq,hkv,dqk,dv", [
    ([32, 64, 32], 2, 0, 4, 2, 16, 8),
    ([32, 64, 32], 2, 1, 4, 4, 8, 16),
    ([48, 16, 96], 4, 3, 6, 2, 12, 8),
])
def test_backward_matches_library_autograd(lengths, cp, rank, hq, hkv, dqk, dv):
    q, k, v, do = _case(7, lengths, cp, rank, hq, hkv, dqk, dv, with_do=True)
    scale = 0.29
    dq, dk, dvv = attention.attn_bwd64(q, k, v, do, lengths, cp, rank, scale=scale)
    rq, rk, rv = _library_grads(q, k, v, do, lengths, cp, rank, scale)
    for a, b in ((dq, rq), (dk, rk), (dvv, rv)):
        assert np.max(np.abs(a - b)) <= 1e-11


def test_backward_finite_differences():
    lengths, cp, rank = [16, 32], 2, 1
    q, k, v, do = _case(8, lengths, cp, rank, 4, 2, 8, 8, with_do=True)
    dq, dk, dv = attention.attn_bwd64(q, k, v, do, lengths, cp, rank)

    def loss(qq, kk, vv):
        return float((attention.attn_fwd64(qq, kk, vv, lengths, cp, rank)[0] * do).sum())

    eps = 1e-6
    rows = partition.kv_row(lengths, cp)
    for arr, grad, idx in ((q, dq, (3, 1, 2)), (q, dq, (20, 3, 7)),
                           (k, dk, (int(rows[17]), 1, 4)), (v, dv, (int(rows[9]), 0, 5))):
        plus = arr.copy(); plus[idx] += eps
        minus = arr.copy(); minus[idx] -= eps
        args_p = [plus if arr is x else x for x in (q, k, v)]
        args_m = [minus if arr is x else x for x in (q, k, v)]
        fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd))


def test_backward_identities():
    lengths, cp, rank = [24, 48, 24], 3, 1
    hq, hkv = 6, 2
    q, k, v, do = _case(9, lengths, cp, rank, hq, hkv, 8, 8, with_do=True)
    dq, dk, dv = attention.attn_bwd64(q, k, v, do, lengths, cp, rank)
    group = hq // hkv
    # rows of P sum to one: the keys' dV add up to the rows' dO, per kv head
    for hk in range(hkv):
        assert np.allclose(dv[:, hk].sum(0), do[:, hk * group:(hk + 1) * group].sum((0, 1)), atol=1e-12)
        # rows of dS sum to zero, so the keys' dK add up to zero
        assert np.allclose(dk[:, hk].sum(0), 0.0, atol=1e-12)
    # keys no local query sees get exact zeros: offsets >= (2cp-r)*c in each document
    cu = partition.cu_seqlens(lengths)
    rows = partition.kv_row(lengths, cp)
    unseen = []
    for i, length in enumerate(lengths):
        c = length // (2 * cp)
        unseen.extend(range(cu[i] + (2 * cp - rank) * c, cu[i + 1]))
    assert unseen
    assert np.all(dk[rows[unseen]] == 0.0) and np.all(dv[rows[unseen]] == 0.0)
    # constant keys give uniform weights and a zero query gradient
    k_const = np.broadcast_to(k[:1], k.shape).copy()
    dq0, _, _ = attention.attn_bwd64(q, k_const, v, do, lengths, cp, rank)
    assert np.max(np.abs(dq0)) <= 1e-12


def test_workload_shapes_tiny_runs():
    w = workloads.BY_NAME["tiny"]
    b = workloads.make_batch(w)
    q = b.q.double().numpy()
    rows = np.arange(0, q.shape[0], 37)
    o, lse = attention.attn_fwd64_rows(q, b.k.double().numpy(), b.v.double().numpy(),
                                       b.lengths, w.cp, w.rank, rows)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


# ---------------------------------------------------------------- padding
# Pins of the padded layout (documents of any length, padded at their end to
# a multiple of 2*cp): real rows against PyTorch on the unpadded sequence of
# real tokens alone, which knows nothing of the partition or the pads.

def _padded_case(seed, real, cp, hq, hkv, dqk, dv):
    rng = np.random.default_rng(seed)
    total = int(sum(partition.pad_lengths(real, cp)))
    q = rng.standard_normal((total // cp, hq, dqk))
    k = rng.standard_normal((total, hkv, dqk))
    v = rng.standard_normal((total, hkv, dv))
    do = rng.standard_normal((total // cp, hq, dv))
    return q, k, v, do


def _real_sequence(real, cp):
    """Padded global position of every real token, in order; document of each."""
    lengths = partition.pad_lengths(real, cp)
    cu = partition.cu_seqlens(lengths)
    pos, doc = [], []
    for i, r in enumerate(real):
        pos.extend(range(cu[i], cu[i] + r))
        doc.extend([i] * r)
    return np.asarray(pos), np.asarray(doc)


def _unpadded_library(q_loc, k, v, do, real, cp, rank, scale):
    """O, LSE and gradients from float64 PyTorch on the real tokens only."""
    lengths = partition.pad_lengths(real, cp)
    pos, doc = _real_sequence(real, cp)
    n = pos.shape[0]
    qg = partition.q_global(lengths, cp, rank)
    rows = partition.kv_row(lengths, cp)
    where = {int(g): j for j, g in enumerate(pos.tolist())}
    local_real = [l for l, g in enumerate(qg.tolist()) if int(g) in where]
    real_idx = [where[int(qg[l])] for l in local_real]
    group = q_loc.shape[1] // k.shape[1]
    q_full = np.random.default_rng(5).standard_normal((n,) + q_loc.shape[1:])
    q_full[real_idx] = q_loc[local_real]
    idx = np.arange(n)
    mask = (doc[:, None] == doc[None, :]) & (idx[None, :] <= idx[:, None])
    qt = torch.from_numpy(q_full).requires_grad_()
    kt = torch.from_numpy(k[rows[pos]]).requires_grad_()
    vt = torch.from_numpy(v[rows[pos]]).requires_grad_()
    s = scale * torch.einsum("ihd,jhd->hij", qt, kt.repeat_interleave(group, dim=1))
    s = s.masked_fill(~torch.from_numpy(mask)[None], -math.inf)
    lse = torch.logsumexp(s, dim=2)                           # [h, n]
    out = torch.einsum("hij,jhd->ihd", torch.exp(s - lse[:, :, None]),
                       vt.repeat_interleave(group, dim=1))
    sel = torch.from_numpy(np.asarray(real_idx, dtype=np.int64))
    (out[sel] * torch.from_numpy(do[local_real])).sum().backward()
    dq = np.zeros_like(q_loc)
    dq[local_real] = qt.grad.numpy()[real_idx]
    dk = np.zeros_like(k)
    dvv = np.zeros_like(v)
    dk[rows[pos]] = kt.grad.numpy()
    dvv[rows[pos]] = vt.grad.numpy()
    o = np.zeros((q_loc.shape[0], q_loc.shape[1], v.shape[2]))
    o[local_real] = out.detach().numpy()[real_idx]
    lse_loc = np.full(q_loc.shape[:2], np.inf)
    lse_loc[local_real] = lse.detach().numpy().T[real_idx]
    return o, lse_loc, dq, dk, dvv


@pytest.mark.parametrize("real,cp,rank,hq,hkv,dqk,dv", [
    ([5, 13, 8], 2, 0, 2, 1, 8, 4),      # pads inside the last chunk
    ([1, 3, 30], 4, 3, 4, 2, 6, 6),      # a 1-token document: pads span 7 chunks
    ([7, 9, 2], 3, 1, 3, 3, 5, 7),
    ([16, 4], 2, 1, 2, 2, 4, 4),         # one document needs no pad
])
def test_padded_layout_matches_unpadded_library(real, cp, rank, hq, hkv, dqk, dv):
    q, k, v, do = _padded_case(31, real, cp, hq, hkv, dqk, dv)
    scale = 0.37
    o, lse = attention.attn_fwd64_padded(q, k, v, real, cp, rank, scale=scale)
    dq, dk, dvv = attention.attn_bwd64_padded(q, k, v, do, real, cp, rank, scale=scale)
    ro, rlse, rdq, rdk, rdv = _unpadded_library(q, k, v, do, real, cp, rank, scale)
    pad = partition.pad_rows(real, cp, rank)
    assert np.max(np.abs(o - ro)) <= 1e-12
    assert np.all(np.isinf(lse[pad])) and np.all(lse[pad] > 0)
    assert np.max(np.abs(lse[~pad] - rlse[~pad])) <= 1e-12
    assert np.all(o[pad] == 0.0) and np.all(dq[pad] == 0.0)
    for a, b in ((dq, rdq), (dk, rdk), (dvv, rdv)):
        assert np.max(np.abs(a - b)) <= 1e-11
    # pad keys get exact zeros, whatever dO holds on pad rows
    lengths = partition.pad_lengths(real, cp)
    pos, _ = _real_sequence(real, cp)
    is_real = np.zeros(sum(lengths), dtype=bool)
    is_real[pos] = True
    pad_keys = partition.kv_row(lengths, cp)[~is_real]
    assert np.all(dk[pad_keys] == 0.0) and np.all(dvv[pad_keys] == 0.0)


def test_padding_without_pads_is_the_plain_oracle():
    real, cp, rank = [8, 16, 8], 2, 1
    q, k, v, do = _padded_case(32, real, cp, 4, 2, 8, 8)
    o, lse = attention.attn_fwd64_padded(q, k, v, real, cp, rank)
    o2, lse2 = attention.attn_fwd64(q, k, v, real, cp, rank)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


# --- attention over a subset of source ranks' shards (all-gather overlap) ---

def _library_shards(q_loc, k, v, lengths, cp, rank, shards, scale):
    """SDPA(float64) and a torch log-sum-exp over the unpartitioned sequence,
    with the causal + EOD mask narrowed to keys whose gathered row lies in a
    listed rank's block of the rank-major K/V (row // T_local = holding rank).
    Returns O, LSE and the rank's rows that see at least one key."""
    total = int(sum(lengths))
    t_loc = total // cp
    qg = partition.q_global(lengths, cp, rank)
    kg = attention.to_global(k, lengths, cp)
    vg = attention.to_global(v, lengths, cp)
    holder = partition.kv_row(lengths, cp) // t_loc          # rank holding each global key
    q_full = np.random.default_rng(998).standard_normal((total,) + q_loc.shape[1:])
    q_full[qg] = q_loc
    docs = partition.doc_of(lengths)
    idx = np.arange(total)
    mask = (docs[:, None] == docs[None, :]) & (idx[None, :] <= idx[:, None])
    mask &= np.isin(holder, list(shards))[None, :]
    seen = mask[qg].any(axis=1)
    group = q_loc.shape[1] // k.shape[1]
    qt = torch.from_numpy(q_full).permute(1, 0, 2)
    kt = torch.from_numpy(kg).repeat_interleave(group, dim=1).permute(1, 0, 2)
    vt = torch.from_numpy(vg).repeat_interleave(group, dim=1).permute(1, 0, 2)
    mt = torch.from_numpy(mask)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt, scale=scale)
    s = (qt @ kt.transpose(1, 2)) * scale
    lse = torch.logsumexp(s.masked_fill(~mt, float("-inf")), dim=-1)
    return out.permute(1, 0, 2).numpy()[qg], lse.permute(1, 0).numpy()[qg], seen


@pytest.mark.parametrize("lengths,cp,rank,shards", [
    ([16, 32, 16], 2, 0, {1}),
    ([16, 32, 16], 2, 1, {0}),
    ([48, 16, 96, 32], 4, 2, {2}),
    ([48, 16, 96, 32], 4, 2, {0, 3}),
    ([48, 16, 96, 32], 4, 1, {1, 2, 3}),
    ([80, 240], 8, 5, {0, 5, 7}),
])
def test_shard_subset_oracle_matches_library(lengths, cp, rank, shards):
    """Attention restricted to some shards against SDPA with the narrowed mask
    (holder taken from the rank-major gathered row, not from the chunk formula)."""
    q, k, v, _ = _case(41, lengths, cp, rank, 4, 2, 12, 8)
    scale = 0.29
    o, lse = attention.attn_fwd64_shards(q, k, v, lengths, cp, rank, shards, scale=scale)
    ref_o, ref_lse, seen = _library_shards(q, k, v, lengths, cp, rank, shards, scale)
    assert seen.any()
    assert np.max(np.abs(o[seen] - ref_o[seen])) <= 1e-12
    assert np.max(np.abs(lse[seen] - ref_lse[seen])) <= 1e-12
    # rows that see none of the shards' keys: empty softmax
    assert np.all(o[~seen] == 0.0) and np.all(np.isneginf(lse[~seen]))


def test_shard_passes_merge_to_full_attention():
    """One pass per shard, merged by log-sum-exp weights, is the whole forward;
    so is the pass over every shard at once. For rank r the rows of chunk r see
    no key of a shard s > r (its chunks s and 2cp-1-s both follow chunk r)."""
    lengths, cp, rank = [32, 64, 16, 48], 4, 1
    q, k, v, _ = _case(42, lengths, cp, rank, 4, 2, 8, 8)
    full_o, full_lse = attention.attn_fwd64(q, k, v, lengths, cp, rank)
    all_o, all_lse = attention.attn_fwd64_shards(q, k, v, lengths, cp, rank, range(cp))
    assert np.max(np.abs(all_o - full_o)) <= 1e-12 and np.max(np.abs(all_lse - full_lse)) <= 1e-12
    parts = [attention.attn_fwd64_shards(q, k, v, lengths, cp, rank, [s]) for s in range(cp)]
    m_o, m_lse = attention.merge_lse(parts)
    assert np.max(np.abs(m_o - full_o)) <= 1e-12 and np.max(np.abs(m_lse - full_lse)) <= 1e-12
    # merging in another grouping gives the same result
    m2 = attention.merge_lse([attention.merge_lse(parts[:2]), attention.merge_lse(parts[2:])])
    assert np.max(np.abs(m2[0] - full_o)) <= 1e-12
    chunk_r_rows = []
    cu = partition.cu_seqlens(lengths)
    qg = partition.q_global(lengths, cp, rank)
    for i, L in enumerate(lengths):
        c = L // (2 * cp)
        chunk_r_rows += [row for row, g in enumerate(qg.tolist())
                         if cu[i] + rank * c <= g < cu[i] + (rank + 1) * c]
    for s in range(rank + 1, cp):
        assert np.all(np.isneginf(parts[s][1][chunk_r_rows]))
