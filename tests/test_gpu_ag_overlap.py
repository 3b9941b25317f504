"""Shard-by-shard forward (all-gather overlap) on an MI355X, against the fp64
oracle: passes over single shards (or sets of shards) merged through the
running state, each pass started by the event that delivered its shard."""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as oatt
from parity import LSE_ABS, assert_close, device, to64

pytestmark = pytest.mark.gpu

thd = pytest.importorskip("packed_sequence_causal_amd")

CASES = [
    # (seed, lengths, cp, rank, hq, hkv, dqk, dv)
    (61, [256, 512, 256], 2, 0, 8, 8, 64, 64),
    (62, [8, 24, 40, 136, 520], 4, 1, 32, 8, 128, 128),
    (63, [16, 32, 1040, 16, 400], 8, 3, 16, 16, 192, 128),
    (64, [1000, 72, 600], 4, 2, 32, 8, 128, 128),
    (65, [36, 300, 84], 3, 2, 12, 4, 128, 128),
]


def _pass_meta(b, cp, rank, hq, hkv, dqk, dv, shards):
    bt, _ = thd.preferred_tiles(hq=hq, hkv=hkv, d_qk=dqk, d_v=dv)
    return thd.build_pass_metadata(seqlens=b.lengths, cp=cp, rank=rank, block_t=bt, block_n=64,
                                   shards=shards, device=0)


def _state_views(state, t_loc, hq, dv):
    n = t_loc * hq * dv
    return state[:n].view(t_loc, hq, dv), state[n:].view(t_loc, hq)


def _order(kind, cp, rank):
    if kind == "local_first":
        return [rank] + [s for s in range(cp) if s != rank][::-1]
    if kind == "ascending":     # the last shard may hold no key of a tile's rows
        return list(range(cp))
    return list(range(cp))[::-1]   # descending: so may the first


@pytest.mark.parametrize("order_kind", ["local_first", "ascending", "descending"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c[0]}")
def test_shards_one_at_a_time_match_oracle(case, order_kind):
    """Shard s is copied into a NaN-filled gathered K/V only after the pass
    before it has run, so a pass reading any row outside its shard would turn
    its rows into NaN. After each pass the state is the attention over the
    shards delivered so far; after the last, o and lse are the forward's. The
    orders make first and last passes in which some tiles have no run (their
    rows' state must still be set, and read out)."""
    seed, lengths, cp, rank, hq, hkv, dqk, dv = case
    b = workloads.small_case(seed, lengths, cp, hq, hkv, dqk, dv, rank=rank)
    dev = device()
    t_loc = b.q.shape[0]
    q, k_src, v_src = b.q.to(dev), b.k.to(dev), b.v.to(dev)
    k = torch.full_like(k_src, float("nan"))
    v = torch.full_like(v_src, float("nan"))
    order = _order(order_kind, cp, rank)
    print(f"[ag] seed={seed} cp={cp} rank={rank} order={order}", flush=True)
    copy = torch.cuda.Stream(device=dev)
    compute = torch.cuda.current_stream(dev)
    state = None
    q64, k64, v64 = to64(b.q), to64(b.k), to64(b.v)
    for i, s in enumerate(order):
        copy.wait_stream(compute)                  # the previous pass is done
        with torch.cuda.stream(copy):
            k[s * t_loc:(s + 1) * t_loc].copy_(k_src[s * t_loc:(s + 1) * t_loc])
            v[s * t_loc:(s + 1) * t_loc].copy_(v_src[s * t_loc:(s + 1) * t_loc])
            ready = torch.cuda.Event()
            ready.record(copy)
        compute.wait_event(ready)
        meta = _pass_meta(b, cp, rank, hq, hkv, dqk, dv, [s])
        if state is None:
            state = thd.pass_state(meta=meta, hq=hq, hkv=hkv, d_v=dv, device=dev)
            state.fill_(float("nan"))              # THD_PASS_FIRST ignores the contents
        res = thd.attn_fwd_pass(q=q, k=k, v=v, meta=meta, state=state, first=i == 0,
                                last=i == cp - 1)
        torch.cuda.synchronize()
        want_o, want_lse = oatt.attn_fwd64_shards(q64, k64, v64, lengths, cp, rank, order[:i + 1])
        if res is None:
            so, sl = _state_views(state, t_loc, hq, dv)
            so, sl = to64(so), sl.double().cpu().numpy() * math.log(2.0)
            seen = np.isfinite(want_lse)
            assert np.all(np.isneginf(sl[~seen]))
            # P enters P.V in bf16, so the fp32 state carries the O tolerance
            assert_close(so[seen], want_o[seen], f"state O after {i + 1} shards")
            assert_close(sl[seen], want_lse[seen], f"state LSE after {i + 1} shards",
                         max_abs=LSE_ABS, mean_abs=LSE_ABS)
        else:
            o, lse = res
            assert_close(to64(o), want_o, "O")
            assert_close(lse.double().cpu().numpy(), want_lse, "LSE", max_abs=LSE_ABS,
                         mean_abs=LSE_ABS)
            o1, lse1 = thd.attn_fwd(q=q, k=k_src, v=v_src, seqlens=b.lengths, cp=cp, rank=rank)
            torch.cuda.synchronize()
            # different summation order only; a bf16 ulp of O is up to 2^-6 near |O| = 4
            assert (o.float() - o1.float()).abs().max().item() <= 2e-2
            assert (lse - lse1).abs().max().item() <= 1e-4


@pytest.mark.parametrize("case", CASES[1:3], ids=lambda c: f"seed{c[0]}")
def test_overlapped_delivery_and_grouped_passes(case):
    """All copies enqueued at once on a side stream, each pass waiting only on
    its shard's event (the overlapped schedule); then a two-pass schedule:
    the local shard, then every other shard at once."""
    seed, lengths, cp, rank, hq, hkv, dqk, dv = case
    b = workloads.small_case(seed, lengths, cp, hq, hkv, dqk, dv, rank=rank)
    dev = device()
    t_loc = b.q.shape[0]
    q, k_src, v_src = b.q.to(dev), b.k.to(dev), b.v.to(dev)
    want_o, want_lse = oatt.attn_fwd64(to64(b.q), to64(b.k), to64(b.v), lengths, cp, rank)
    schedules = [[[s] for s in [rank] + [x for x in range(cp) if x != rank]],
                 [[rank], [x for x in range(cp) if x != rank]]]
    for groups in schedules:
        print(f"[ag overlap] seed={seed} groups={groups}", flush=True)
        k = torch.full_like(k_src, float("nan"))
        v = torch.full_like(v_src, float("nan"))
        torch.cuda.synchronize()
        copy = torch.cuda.Stream(device=dev)
        compute = torch.cuda.current_stream(dev)
        events = []
        with torch.cuda.stream(copy):
            for group in groups:
                for s in group:
                    k[s * t_loc:(s + 1) * t_loc].copy_(k_src[s * t_loc:(s + 1) * t_loc])
                    v[s * t_loc:(s + 1) * t_loc].copy_(v_src[s * t_loc:(s + 1) * t_loc])
                ev = torch.cuda.Event()
                ev.record(copy)
                events.append(ev)
        metas = [_pass_meta(b, cp, rank, hq, hkv, dqk, dv, g) for g in groups]
        state = thd.pass_state(meta=metas[0], hq=hq, hkv=hkv, d_v=dv, device=dev)
        res = None
        for i, (meta, ev) in enumerate(zip(metas, events)):
            compute.wait_event(ev)
            res = thd.attn_fwd_pass(q=q, k=k, v=v, meta=meta, state=state, first=i == 0,
                                    last=i == len(groups) - 1)
        torch.cuda.synchronize()
        o, lse = res
        assert_close(to64(o), want_o, "O")
        assert_close(lse.double().cpu().numpy(), want_lse, "LSE", max_abs=LSE_ABS,
                     mean_abs=LSE_ABS)


@pytest.mark.parametrize("name", ["gqa_mid", "mla", "short"])
def test_full_size_shard_passes(name):
    """The full-size forward workloads (gqa_mid: cp 4; mla and short: cp 8)
    shard by shard, the local shard first: every element of O and LSE against
    the oracle."""
    w = workloads.BY_NAME[name]
    print(f"[ag full] {name} cp={w.cp} rank={w.rank}", flush=True)
    b = workloads.make_batch(w)
    dev = device()
    q, k, v = b.q.to(dev), b.k.to(dev), b.v.to(dev)
    order = [w.rank] + [s for s in range(w.cp) if s != w.rank]
    state = None
    res = None
    for i, s in enumerate(order):
        meta = _pass_meta(b, w.cp, w.rank, w.hq, w.hkv, w.d_qk, w.d_v, [s])
        if state is None:
            state = thd.pass_state(meta=meta, hq=w.hq, hkv=w.hkv, d_v=w.d_v, device=dev)
        res = thd.attn_fwd_pass(q=q, k=k, v=v, meta=meta, state=state, first=i == 0,
                                last=i == w.cp - 1)
    torch.cuda.synchronize()
    o, lse = res
    want_o, want_lse = oatt.attn_fwd64(to64(b.q), to64(b.k), to64(b.v), b.lengths, w.cp, w.rank)
    assert_close(to64(o), want_o, "O")
    assert_close(lse.double().cpu().numpy(), want_lse, "LSE", max_abs=LSE_ABS, mean_abs=LSE_ABS)
