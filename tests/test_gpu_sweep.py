"""Edge shapes of the HIP path against the fp64 oracle, on an MI355X.

The other GPU tests cover the workloads' shapes; this grid covers the rest of
the supported space: group sizes from 1 to the maximum 128 (a query tile of a
single token), groups that do not divide 128 or the 32-row backward blocks,
context-parallel sizes 1 to 16 with first, middle and last ranks, documents of
the minimum length 2*cp (one row per chunk) beside long ones, and every
supported head-dimension pair. Each case runs the forward (bf16 P, and split
probabilities with the fp32 O), the forward with the finest split of long key
ranges the planner makes, and the backward along both D paths, and compares
every output element with the oracle.
"""
import pytest
import torch

import workloads
from oracle import attention as oatt
from parity import LSE_ABS, assert_close, device, to64

pytestmark = pytest.mark.gpu

thd = pytest.importorskip("packed_sequence_causal_amd")

GRID = [
    # (seed, lengths, cp, rank, hq, hkv, dqk, dv)
    (91, [4, 12, 36], 2, 1, 128, 1, 64, 64),                 # group 128: one token per tile
    (92, [8, 40, 4], 2, 0, 64, 1, 128, 128),                 # group 64: two 32-row blocks a token
    (93, [8, 64, 200], 4, 3, 64, 2, 128, 128),               # group 32, last rank
    (94, [10, 70, 330], 5, 4, 16, 8, 128, 128),              # group 2, cp 5
    (95, [12, 36, 600], 6, 2, 10, 2, 64, 64),                # group 5: 125-row tiles
    (96, [14, 140, 546], 7, 5, 14, 2, 192, 128),             # group 7, expanded-MLA dims
    (97, [6, 6, 6, 6, 6, 600], 3, 0, 24, 4, 128, 128),       # group 6, one-row chunks
    (98, [2, 2, 1022], 1, 0, 4, 4, 192, 128),                # cp 1, group 1
    (99, [16] * 10 + [512], 8, 7, 64, 8, 128, 128),          # cp 8, last rank, minimal documents
    (100, [32, 96, 640], 16, 9, 16, 4, 128, 128),            # cp 16: chunks of 1 to 20 tokens
]


def _ids(c):
    return f"seed{c[0]}-g{c[4] // c[5]}-cp{c[2]}r{c[3]}-d{c[6]}"


@pytest.mark.parametrize("case", GRID, ids=_ids)
def test_edge_shapes_forward_and_backward(case):
    seed, lengths, cp, rank, hq, hkv, dqk, dv = case
    b = workloads.small_case(seed, lengths, cp, hq, hkv, dqk, dv, backward=True, rank=rank)
    dev = device()
    q, k, v, do = (t.to(dev) for t in (b.q, b.k, b.v, b.do))
    print(f"[sweep] seed={seed} lengths={lengths} cp={cp} rank={rank} hq={hq} hkv={hkv} "
          f"dqk={dqk} dv={dv}", flush=True)
    want_o, want_lse = oatt.attn_fwd64(to64(b.q), to64(b.k), to64(b.v), lengths, cp, rank)

    o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=lengths, cp=cp, rank=rank)
    torch.cuda.synchronize()
    assert_close(to64(o), want_o, "O")
    assert_close(to64(lse), want_lse, "LSE", max_abs=LSE_ABS, mean_abs=LSE_ABS)

    # As many work items as the planner will make: tiles with more than eight
    # key tiles are cut into parts that the combine kernel merges.
    o_s, lse_s = thd.attn_fwd(q=q, k=k, v=v, seqlens=lengths, cp=cp, rank=rank,
                              concurrency=1 << 20)
    torch.cuda.synchronize()
    assert_close(to64(o_s), want_o, "O (split)")
    assert_close(to64(lse_s), want_lse, "LSE (split)", max_abs=LSE_ABS, mean_abs=LSE_ABS)

    o32 = torch.empty((q.shape[0], hq, dv), dtype=torch.float32, device=dev)
    o_x, lse_x = thd.attn_fwd(q=q, k=k, v=v, seqlens=lengths, cp=cp, rank=rank, out_f32=o32)
    torch.cuda.synchronize()
    assert_close(to64(o32), want_o, "O32", max_abs=2e-4, mean_abs=2e-5)
    assert_close(to64(lse_x), want_lse, "LSE (exact)", max_abs=LSE_ABS, mean_abs=LSE_ABS)

    want = oatt.attn_bwd64(to64(b.q), to64(b.k), to64(b.v), to64(b.do), lengths, cp, rank)
    for o_f32 in (None, o32):
        got = thd.attn_bwd(q=q, k=k, v=v, lse=lse_x, d_o=do, seqlens=lengths, cp=cp, rank=rank,
                           o_f32=o_f32)
        torch.cuda.synchronize()
        path = "D from scores" if o_f32 is None else "D from O32"
        for name, g, e in zip(("dQ", "dK", "dV"), got, want):
            assert_close(to64(g), e, f"{name} ({path})")
