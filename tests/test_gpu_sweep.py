"""Seeded sweep of random shapes on an MI355X against the fp64 oracle.

Each case draws a context-parallel size and rank, a handful of document
lengths (from a single token per chunk up to several KV tiles), a head layout
(MHA, GQA with groups 2 to 8, expanded MLA) and a split concurrency, then
checks on every element: the forward (the plan's own tiles), the packed-plan
forward, the backward on both D paths, and a forward run shard by shard.
The draws come from numpy's generator seeded by the case number, so every
case is fixed and printed before it runs. Fixed cases with 32 to 128 q heads
per kv head (query tiles of 4 tokens down to one) follow, then context-parallel
sizes of 16 to 100 (chunks of a few tokens; shard passes up to cp = 64).
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import attention as oatt
from parity import LSE_ABS, assert_close, device, to64

pytestmark = pytest.mark.gpu

thd = pytest.importorskip("packed_sequence_causal_amd")

HEADS = [(8, 8, 64, 64), (16, 4, 128, 128), (12, 4, 128, 128), (32, 8, 128, 128),
         (4, 1, 64, 64), (6, 2, 128, 128), (8, 8, 192, 128), (64, 8, 128, 128)]


def _draw(case):
    rng = np.random.default_rng(9000 + case)
    cp = int(rng.choice([1, 2, 3, 4, 8]))
    rank = int(rng.integers(0, cp))
    hq, hkv, dqk, dv = HEADS[case % len(HEADS)]     # every layout twelve times
    n = int(rng.integers(1, 7))
    # chunk lengths from 1 token to a few hundred, total at most ~4k tokens
    chunk = rng.choice([1, 2, 3, 8, 17, 40, 64, 100, 255], size=n)
    lengths = [int(2 * cp * c) for c in chunk]
    while sum(lengths) > 4096:
        lengths.pop()
    concurrency = int(rng.choice([0, 8, 64]))
    return cp, rank, hq, hkv, dqk, dv, lengths, concurrency


@pytest.mark.parametrize("case", range(96))
def test_random_shapes(case):
    cp, rank, hq, hkv, dqk, dv, lengths, concurrency = _draw(case)
    print(f"[sweep] case={case} cp={cp} rank={rank} hq={hq} hkv={hkv} dqk={dqk} dv={dv} "
          f"lengths={lengths} concurrency={concurrency}", flush=True)
    b = workloads.small_case(9000 + case, lengths, cp, hq, hkv, dqk, dv, backward=True, rank=rank)
    dev = device()
    q, k, v, do = (t.to(dev) for t in (b.q, b.k, b.v, b.do))
    want_o, want_lse = oatt.attn_fwd64(to64(b.q), to64(b.k), to64(b.v), lengths, cp, rank)

    # forward, plain plan (the batch's preferred tile sizes), then packed
    for packed in (False, True):
        meta = thd.device_metadata(seqlens=b.lengths, cp=cp, rank=rank, hq=hq, hkv=hkv, d_qk=dqk,
                                   d_v=dv, device=0, concurrency=concurrency, forward=True,
                                   packed=packed)
        o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=cp, rank=rank, meta=meta)
        torch.cuda.synchronize()
        assert_close(to64(o), want_o, f"O packed={packed}")
        assert_close(lse.cpu().double().numpy(), want_lse, f"LSE packed={packed}",
                     max_abs=LSE_ABS, mean_abs=LSE_ABS)

    # backward, D from the scores and D from the exact fp32 O
    want = oatt.attn_bwd64(to64(b.q), to64(b.k), to64(b.v), to64(b.do), lengths, cp, rank)
    for exact_o in (False, True):
        o32 = torch.empty((q.shape[0], hq, dv), dtype=torch.float32, device=dev) if exact_o else None
        o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=cp, rank=rank, out_f32=o32)
        got = thd.attn_bwd(q=q, k=k, v=v, lse=lse, d_o=do, seqlens=b.lengths, cp=cp, rank=rank,
                           o_f32=o32)
        torch.cuda.synchronize()
        for name, g, e in zip(("dQ", "dK", "dV"), got, want):
            assert_close(g.cpu().double().numpy(), e, f"{name} exact_o={exact_o}")

    # shard by shard, local shard first
    bt, _ = thd.preferred_tiles(hq=hq, hkv=hkv, d_qk=dqk, d_v=dv)
    order = [rank] + [s for s in range(cp) if s != rank]
    state = None
    for i, s in enumerate(order):
        meta = thd.build_pass_metadata(seqlens=b.lengths, cp=cp, rank=rank, block_t=bt,
                                       block_n=64, shards=[s], device=0)
        if state is None:
            state = thd.pass_state(meta=meta, hq=hq, hkv=hkv, d_v=dv, device=dev)
        res = thd.attn_fwd_pass(q=q, k=k, v=v, meta=meta, state=state, first=i == 0,
                                last=i == len(order) - 1)
    torch.cuda.synchronize()
    o, lse = res
    assert_close(to64(o), want_o, "O shard by shard")
    assert_close(lse.cpu().double().numpy(), want_lse, "LSE shard by shard",
                 max_abs=LSE_ABS, mean_abs=LSE_ABS)


LARGE_GROUPS = [
    # (seed, lengths, cp, rank, hq, hkv, dqk, dv): 32 to 128 q heads per kv head,
    # so a query tile holds 4 tokens down to a single one, and dK, dV sum over
    # that many heads
    (9101, [64, 200, 40], 2, 1, 32, 1, 128, 128),
    (9102, [16, 96, 8, 48], 4, 2, 64, 1, 64, 64),
    (9103, [24, 120, 8], 2, 0, 128, 1, 128, 128),
    (9104, [48, 16, 80], 4, 3, 128, 2, 128, 128),
    (9105, [32, 96], 2, 1, 64, 1, 192, 128),
]


@pytest.mark.parametrize("case", LARGE_GROUPS, ids=lambda c: f"seed{c[0]}")
def test_large_groups(case):
    seed, lengths, cp, rank, hq, hkv, dqk, dv = case
    print(f"[large groups] seed={seed} G={hq // hkv} lengths={lengths} cp={cp} rank={rank} "
          f"dqk={dqk}", flush=True)
    b = workloads.small_case(seed, lengths, cp, hq, hkv, dqk, dv, backward=True, rank=rank)
    dev = device()
    q, k, v, do = (t.to(dev) for t in (b.q, b.k, b.v, b.do))
    want_o, want_lse = oatt.attn_fwd64(to64(b.q), to64(b.k), to64(b.v), lengths, cp, rank)
    for packed in (False, True):
        o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=cp, rank=rank, packed=packed)
        torch.cuda.synchronize()
        assert_close(to64(o), want_o, f"O packed={packed}")
        assert_close(lse.cpu().double().numpy(), want_lse, f"LSE packed={packed}",
                     max_abs=LSE_ABS, mean_abs=LSE_ABS)
    want = oatt.attn_bwd64(to64(b.q), to64(b.k), to64(b.v), to64(b.do), lengths, cp, rank)
    for exact_o in (False, True):
        o32 = torch.empty((q.shape[0], hq, dv), dtype=torch.float32, device=dev) if exact_o else None
        o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=cp, rank=rank, out_f32=o32)
        got = thd.attn_bwd(q=q, k=k, v=v, lse=lse, d_o=do, seqlens=b.lengths, cp=cp, rank=rank,
                           o_f32=o32)
        torch.cuda.synchronize()
        for name, g, e in zip(("dQ", "dK", "dV"), got, want):
            assert_close(g.cpu().double().numpy(), e, f"{name} exact_o={exact_o}")


LARGE_CP = [
    # (seed, lengths, cp, rank, hq, hkv, dqk, dv): chunks of one to a few
    # tokens; cp = 64 is the largest the shard-pass plans take
    (9201, [32, 96, 320, 64], 16, 5, 8, 2, 128, 128),
    (9202, [128, 256, 1280], 64, 0, 8, 8, 64, 64),
    (9203, [128, 384, 1280, 128], 64, 63, 16, 4, 128, 128),
    (9204, [128, 256, 1408], 64, 31, 16, 16, 192, 128),
    (9205, [200, 1000, 2600], 100, 37, 8, 2, 128, 128),
]


@pytest.mark.parametrize("case", LARGE_CP, ids=lambda c: f"cp{c[2]}_rank{c[3]}")
def test_large_cp(case):
    seed, lengths, cp, rank, hq, hkv, dqk, dv = case
    print(f"[large cp] seed={seed} cp={cp} rank={rank} lengths={lengths} hq={hq} hkv={hkv} "
          f"dqk={dqk}", flush=True)
    b = workloads.small_case(seed, lengths, cp, hq, hkv, dqk, dv, backward=True, rank=rank)
    dev = device()
    q, k, v, do = (t.to(dev) for t in (b.q, b.k, b.v, b.do))
    want_o, want_lse = oatt.attn_fwd64(to64(b.q), to64(b.k), to64(b.v), lengths, cp, rank)
    for packed in (False, True):
        o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=cp, rank=rank, packed=packed)
        torch.cuda.synchronize()
        assert_close(to64(o), want_o, f"O packed={packed}")
        assert_close(lse.cpu().double().numpy(), want_lse, f"LSE packed={packed}",
                     max_abs=LSE_ABS, mean_abs=LSE_ABS)
    want = oatt.attn_bwd64(to64(b.q), to64(b.k), to64(b.v), to64(b.do), lengths, cp, rank)
    for exact_o in (False, True):
        o32 = torch.empty((q.shape[0], hq, dv), dtype=torch.float32, device=dev) if exact_o else None
        o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=cp, rank=rank, out_f32=o32)
        got = thd.attn_bwd(q=q, k=k, v=v, lse=lse, d_o=do, seqlens=b.lengths, cp=cp, rank=rank,
                           o_f32=o32)
        torch.cuda.synchronize()
        for name, g, e in zip(("dQ", "dK", "dV"), got, want):
            assert_close(g.cpu().double().numpy(), e, f"{name} exact_o={exact_o}")
    if cp > 64:
        return
    # shard by shard in four groups of sources, the local shard's group first
    bt, _ = thd.preferred_tiles(hq=hq, hkv=hkv, d_qk=dqk, d_v=dv)
    groups = [list(range(g, cp, 4)) for g in range(4)]
    groups.sort(key=lambda s: rank not in s)
    state = None
    for i, shards in enumerate(groups):
        meta = thd.build_pass_metadata(seqlens=b.lengths, cp=cp, rank=rank, block_t=bt,
                                       block_n=64, shards=shards, device=0)
        if state is None:
            state = thd.pass_state(meta=meta, hq=hq, hkv=hkv, d_v=dv, device=dev)
        res = thd.attn_fwd_pass(q=q, k=k, v=v, meta=meta, state=state, first=i == 0,
                                last=i == len(groups) - 1)
    torch.cuda.synchronize()
    o, lse = res
    assert_close(to64(o), want_o, "O shard groups")
    assert_close(lse.cpu().double().numpy(), want_lse, "LSE shard groups",
                 max_abs=LSE_ABS, mean_abs=LSE_ABS)
