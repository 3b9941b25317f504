"""The forward entry point that allocates nothing (thd_attn_fwd_noalloc),
called through the C ABI, against thd_attn_fwd with a caller workspace on the
same inputs: two calls in a row on the library's per-device static array, the
second with a smaller input, and a plan with no split tile."""
import pytest
import torch

import workloads
from parity import device

pytestmark = pytest.mark.gpu

thd = pytest.importorskip("packed_sequence_causal_amd")

CASES = [
    # (seed, lengths, cp, rank, hq, hkv, dqk, dv, concurrency): split plans
    # first, so the static array holds partial results; the second is smaller
    (91, [2048, 512, 1024], 2, 1, 16, 4, 128, 128, 64),
    (92, [1024, 96], 2, 0, 16, 4, 128, 128, 64),
    (93, [3072, 1040], 8, 3, 16, 16, 192, 128, 64),
    (94, [256, 512, 256], 2, 0, 8, 8, 64, 64, 0),
]


def _inputs(case):
    seed, lengths, cp, rank, hq, hkv, dqk, dv, conc = case
    b = workloads.small_case(seed, lengths, cp, hq, hkv, dqk, dv, rank=rank)
    dev = device()
    q, k, v = b.q.to(dev), b.k.to(dev), b.v.to(dev)
    meta = thd.device_metadata(seqlens=b.lengths, cp=cp, rank=rank, hq=hq, hkv=hkv, d_qk=dqk,
                               d_v=dv, device=0, concurrency=conc)
    return b, q, k, v, meta


def test_noalloc_forward_matches_workspace_forward():
    for case in CASES:
        b, q, k, v, meta = _inputs(case)
        info = meta.info()
        print(f"[noalloc] seed={case[0]} splits={info['n_splits']} parts={info['n_part_slots']}",
              flush=True)
        assert (info["n_splits"] > 0) == (case[-1] > 0)
        hq, dv = q.shape[1], v.shape[2]
        want_o, want_lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=case[2],
                                        rank=case[3], meta=meta)
        o = torch.full((q.shape[0], hq, dv), float("nan"), dtype=torch.bfloat16, device=q.device)
        lse = torch.full((q.shape[0], hq), float("nan"), dtype=torch.float32, device=q.device)
        o32 = torch.full((q.shape[0], hq, dv), float("nan"), dtype=torch.float32,
                         device=q.device)
        thd.attn_fwd_noalloc(q=q, k=k, v=v, out=o, lse=lse, meta=meta)
        torch.cuda.synchronize()
        # same kernels and partial-result layout: bit-identical to the workspace path
        assert torch.equal(o, want_o) and torch.equal(lse, want_lse)
        # and the exact-O path, whose combine also writes the fp32 O
        want32 = torch.empty_like(o32)
        thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=case[2], rank=case[3], meta=meta,
                     out_f32=want32)
        thd.attn_fwd_noalloc(q=q, k=k, v=v, out=o, lse=lse, out_f32=o32, meta=meta)
        torch.cuda.synchronize()
        assert torch.equal(o32, want32)
