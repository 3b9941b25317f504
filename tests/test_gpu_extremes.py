"""Extreme score distributions on an MI355X, against the fp64 oracle.

- Scores that grow along every document (a shared direction added to Q, and to
  each key in proportion to its place in its document): a row's maximum rises
  by a large factor (2^9 to 2^36 across a 64-key tile here) on nearly every
  KV tile, so the running maximum and the accumulator are rescaled on nearly
  every tile.
- Scores that fall along every document: the first keys dominate and later
  probabilities underflow to zero.
- A large softmax scale (nearly one-hot rows).
- Zero queries: every visible key weighs the same, so O is the mean of the
  visible values and LSE = ln(number of visible keys), a closed form.
Forward with 64- and 32-key tiles, split and unsplit, and the backward on both
D paths, every element.
"""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as oatt
from oracle import partition as opart
from parity import LSE_ABS, assert_close, device, to64

pytestmark = pytest.mark.gpu

thd = pytest.importorskip("packed_sequence_causal_amd")

CASES = [
    # (seed, lengths, cp, rank, hq, hkv, dqk, dv)
    (9301, [1024, 512, 2048], 2, 1, 16, 4, 128, 128),
    (9302, [256, 1536, 768], 4, 0, 16, 16, 192, 128),
    (9303, [96, 1024, 64, 352], 4, 3, 8, 8, 64, 64),
]


def _place(lengths, cp):
    """Place of each gathered K/V row in its document, over the document's length."""
    order = opart.gathered_order(lengths, cp)          # global token of each gathered row
    cu = np.asarray(opart.cu_seqlens(lengths))
    doc = opart.doc_of(lengths)[order]
    return (order - cu[doc]) / np.asarray(lengths)[doc]


def _shaped(case, trend):
    """The case's batch with a trend along each document (+1 growing, -1 falling)."""
    seed, lengths, cp, rank, hq, hkv, dqk, dv = case
    b = workloads.small_case(seed, lengths, cp, hq, hkv, dqk, dv, backward=True, rank=rank)
    q = b.q.float()
    k = b.k.float()
    q[:, :, 0] += 48.0
    k[:, :, 0] += torch.from_numpy(trend * 48.0 * _place(lengths, cp)).float()[:, None]
    b.q, b.k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    return b


def _check(case, b, scale=None):
    seed, lengths, cp, rank, hq, hkv, dqk, dv = case
    dev = device()
    q, k, v, do = (t.to(dev) for t in (b.q, b.k, b.v, b.do))
    want_o, want_lse = oatt.attn_fwd64(to64(b.q), to64(b.k), to64(b.v), lengths, cp, rank, scale=scale)
    for bn in (64, 32):
        if bn == 32 and dqk > 128:
            continue                      # no 32-key kernel at d_qk = 192
        for conc in (0, 64):
            bt, _ = thd.preferred_tiles(hq=hq, hkv=hkv, d_qk=dqk, d_v=dv)
            meta = thd.build_metadata(seqlens=b.lengths, cp=cp, rank=rank, block_t=bt, block_n=bn,
                                      concurrency=conc, device=0)
            print(f"[extremes] seed={seed} block_n={bn} concurrency={conc} "
                  f"splits={meta.info()['n_splits']}", flush=True)
            o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=cp, rank=rank,
                                  softmax_scale=scale, meta=meta)
            torch.cuda.synchronize()
            assert_close(to64(o), want_o, f"O bn={bn} conc={conc}")
            assert_close(lse.cpu().double().numpy(), want_lse, f"LSE bn={bn} conc={conc}",
                         max_abs=LSE_ABS, mean_abs=LSE_ABS)
    want = oatt.attn_bwd64(to64(b.q), to64(b.k), to64(b.v), to64(b.do), lengths, cp, rank,
                           scale=scale)
    for exact_o in (False, True):
        print(f"[extremes] seed={seed} backward exact_o={exact_o}", flush=True)
        o32 = torch.empty((q.shape[0], hq, dv), dtype=torch.float32, device=dev) if exact_o else None
        o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=cp, rank=rank,
                              softmax_scale=scale, out_f32=o32)
        got = thd.attn_bwd(q=q, k=k, v=v, lse=lse, d_o=do, seqlens=b.lengths, cp=cp, rank=rank,
                           softmax_scale=scale, o_f32=o32)
        torch.cuda.synchronize()
        for name, g, e in zip(("dQ", "dK", "dV"), got, want):
            assert_close(g.cpu().double().numpy(), e, f"{name} exact_o={exact_o}")


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c[0]}")
def test_growing_scores_rescale_on_every_tile(case):
    _check(case, _shaped(case, +1.0))


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c[0]}")
def test_falling_scores_underflow(case):
    _check(case, _shaped(case, -1.0))


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c[0]}")
def test_large_scale_nearly_one_hot(case):
    seed, lengths, cp, rank, hq, hkv, dqk, dv = case
    b = workloads.small_case(seed, lengths, cp, hq, hkv, dqk, dv, backward=True, rank=rank)
    _check(case, b, scale=1.5)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c[0]}")
def test_zero_queries_give_prefix_means(case):
    seed, lengths, cp, rank, hq, hkv, dqk, dv = case
    b = workloads.small_case(seed, lengths, cp, hq, hkv, dqk, dv, rank=rank)
    b.q = torch.zeros_like(b.q)
    dev = device()
    print(f"[extremes] seed={seed} zero queries", flush=True)
    o, lse = thd.attn_fwd(q=b.q.to(dev), k=b.k.to(dev), v=b.v.to(dev), seqlens=b.lengths,
                          cp=cp, rank=rank)
    torch.cuda.synchronize()
    # closed form: row at global position g of a document starting at s sees
    # the keys s..g, all with the same weight
    qg = opart.q_global(lengths, cp, rank)
    cu = np.asarray(opart.cu_seqlens(lengths))
    start = cu[opart.doc_of(lengths)[qg]]
    v_glob = to64(b.v)[opart.kv_row(lengths, cp)]          # values in global order
    csum = np.concatenate([np.zeros((1,) + v_glob.shape[1:]), np.cumsum(v_glob, axis=0)])
    count = (qg - start + 1).astype(np.float64)
    mean = (csum[qg + 1] - csum[start]) / count[:, None, None]          # [T_local, Hkv, dv]
    want_o = np.repeat(mean, hq // hkv, axis=1)
    want_lse = np.repeat(np.log(count)[:, None], hq, axis=1)
    assert_close(to64(o), want_o, "O")
    assert_close(lse.cpu().double().numpy(), want_lse, "LSE", max_abs=LSE_ABS, mean_abs=LSE_ABS)
