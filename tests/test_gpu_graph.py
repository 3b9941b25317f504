"""HIP graphs (torch.cuda.graph) on an MI355X. The forward that allocates
nothing, captured alone: replays over inputs rewritten in place, with eager
calls on other inputs in between (they overwrite the library's static array of
partial results), must equal the eager forward bit for bit on every replay, and
the oracle within the bound; a split plan puts both the forward and the combine
kernel into the graph. A training step (forward with the fp32 O, backward)
captured whole: every replay equals the eager step bit for bit."""
import pytest
import torch

import workloads
from oracle import attention as oatt
from parity import LSE_ABS, assert_close, device, to64

pytestmark = pytest.mark.gpu

thd = pytest.importorskip("packed_sequence_causal_amd")

CASES = [
    # (seed, lengths, cp, rank, hq, hkv, dqk, dv, concurrency)
    (9501, [2048, 512, 1024], 2, 1, 16, 4, 128, 128, 64),     # split key ranges + combine
    (9502, [16, 32, 1040, 16, 400], 8, 3, 16, 16, 192, 128, 0),
    (9503, [256, 512, 256], 2, 0, 8, 8, 64, 64, 0),
]
REPLAYS = 3


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c[0]}")
def test_noalloc_forward_replays_in_a_graph(case):
    seed, lengths, cp, rank, hq, hkv, dqk, dv, conc = case
    dev = device()
    b = workloads.small_case(seed, lengths, cp, hq, hkv, dqk, dv, rank=rank)
    q, k, v = b.q.to(dev), b.k.to(dev), b.v.to(dev)
    meta = thd.device_metadata(seqlens=b.lengths, cp=cp, rank=rank, hq=hq, hkv=hkv, d_qk=dqk,
                               d_v=dv, device=0, concurrency=conc)
    print(f"[graph] seed={seed} splits={meta.info()['n_splits']}", flush=True)
    out = torch.empty((q.shape[0], hq, dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((q.shape[0], hq), dtype=torch.float32, device=dev)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # first call (sets up the static array) outside capture
        thd.attn_fwd_noalloc(q=q, k=k, v=v, out=out, lse=lse, meta=meta)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        thd.attn_fwd_noalloc(q=q, k=k, v=v, out=out, lse=lse, meta=meta)
    other = workloads.small_case(seed + 50, lengths, cp, hq, hkv, dqk, dv, rank=rank)
    oq, ok_, ov = other.q.to(dev), other.k.to(dev), other.v.to(dev)
    o_other = torch.empty_like(out)
    l_other = torch.empty_like(lse)
    for rep in range(REPLAYS):
        fresh = workloads.small_case(seed + 100 + rep, lengths, cp, hq, hkv, dqk, dv, rank=rank)
        q.copy_(fresh.q.to(dev))
        k.copy_(fresh.k.to(dev))
        v.copy_(fresh.v.to(dev))
        # eager work on other inputs: overwrites the static array's partial results
        thd.attn_fwd_noalloc(q=oq, k=ok_, v=ov, out=o_other, lse=l_other, meta=meta)
        torch.cuda.synchronize()
        print(f"[graph] seed={seed} replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        want_o, want_lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=cp, rank=rank,
                                        meta=meta)
        torch.cuda.synchronize()
        assert torch.equal(out, want_o) and torch.equal(lse, want_lse), rep
        if rep == REPLAYS - 1:
            o64, lse64 = oatt.attn_fwd64(to64(fresh.q), to64(fresh.k), to64(fresh.v), lengths,
                                         cp, rank)
            assert_close(to64(out), o64, "O")
            assert_close(lse.cpu().double().numpy(), lse64, "LSE", max_abs=LSE_ABS,
                         mean_abs=LSE_ABS)


def test_training_step_replays_in_a_graph():
    """Forward (with the fp32 O) and backward captured together; their outputs
    and workspaces come from the graph's memory pool. Every replay over
    rewritten inputs equals the eager step bit for bit."""
    seed, lengths, cp, rank, hq, hkv, dqk, dv = 9511, [1000, 72, 600], 4, 2, 32, 8, 128, 128
    dev = device()
    b = workloads.small_case(seed, lengths, cp, hq, hkv, dqk, dv, backward=True, rank=rank)
    q, k, v, do = (t.to(dev) for t in (b.q, b.k, b.v, b.do))
    meta = thd.device_metadata(seqlens=b.lengths, cp=cp, rank=rank, hq=hq, hkv=hkv, d_qk=dqk,
                               d_v=dv, device=0)

    def step():
        o32 = torch.empty((q.shape[0], hq, dv), dtype=torch.float32, device=dev)
        o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=cp, rank=rank, out_f32=o32,
                              meta=meta)
        return (o, lse) + tuple(thd.attn_bwd(q=q, k=k, v=v, lse=lse, d_o=do, seqlens=b.lengths,
                                             cp=cp, rank=rank, o_f32=o32, meta=meta))

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = step()
    for rep in range(REPLAYS):
        fresh = workloads.small_case(seed + 100 + rep, lengths, cp, hq, hkv, dqk, dv,
                                     backward=True, rank=rank)
        for dst, src in zip((q, k, v, do), (fresh.q, fresh.k, fresh.v, fresh.do)):
            dst.copy_(src.to(dev))
        torch.cuda.synchronize()
        print(f"[graph] training step replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        want = step()
        torch.cuda.synchronize()
        for name, g, e in zip(("O", "LSE", "dQ", "dK", "dV"), captured, want):
            assert torch.equal(g, e), (rep, name)
