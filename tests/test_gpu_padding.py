"""Padding-tolerant partitioning on an MI355X: documents of any length, each
padded at its end to a multiple of 2*cp, against the fp64 oracle.

Real rows must match the oracle to the usual bf16 bounds; pad rows get O = 0,
LSE = +inf and dQ = 0 exactly, and pad keys dK = dV = 0 exactly, whatever dO
holds on pad rows (the cases draw it at random there).
"""
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
    # (seed, real lengths, cp, rank, hq, hkv, dqk, dv)
    (61, [5, 13, 8], 2, 0, 8, 8, 64, 64),
    (62, [1, 3, 300, 77], 4, 3, 32, 8, 128, 128),   # a 1-token document: pads span 7 chunks
    (63, [1000, 37, 601], 4, 0, 32, 8, 128, 128),
    (64, [17, 1040, 9, 400], 8, 3, 16, 16, 192, 128),
    (65, [129, 2, 250], 3, 1, 12, 4, 128, 128),     # group 3
]


def _batch(case, backward=False):
    seed, real, cp, rank, hq, hkv, dqk, dv = case
    lengths = opart.pad_lengths(real, cp)
    return workloads.small_case(seed, lengths, cp, hq, hkv, dqk, dv, backward=backward, rank=rank)


def _pad_keys(real, cp):
    lengths = opart.pad_lengths(real, cp)
    cu = opart.cu_seqlens(lengths)
    is_pad = np.zeros(sum(lengths), dtype=bool)
    for i, r in enumerate(real):
        is_pad[cu[i] + r:cu[i + 1]] = True
    return opart.kv_row(lengths, cp)[is_pad]


@pytest.mark.parametrize("concurrency", [None, 100000], ids=["default", "split"])
@pytest.mark.parametrize("exact", [False, True], ids=["bf16P", "exactO"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c[0]}")
def test_padded_forward_matches_oracle(case, exact, concurrency):
    seed, real, cp, rank, hq, hkv, dqk, dv = case
    b = _batch(case)
    dev = device()
    q, k, v = b.q.to(dev), b.k.to(dev), b.v.to(dev)
    print(f"[pad fwd] seed={seed} real={real} cp={cp} rank={rank} exact={exact} "
          f"concurrency={concurrency}", flush=True)
    o32 = torch.empty((q.shape[0], hq, dv), dtype=torch.float32, device=dev) if exact else None
    o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=real, cp=cp, rank=rank, padded=True,
                          out_f32=o32, concurrency=concurrency)
    torch.cuda.synchronize()
    want_o, want_lse = oatt.attn_fwd64_padded(to64(b.q), to64(b.k), to64(b.v), real, cp, rank)
    pad = opart.pad_rows(real, cp, rank)
    got_o = to64(o)
    got_lse = lse.cpu().double().numpy()
    assert pad.any()
    assert np.all(got_o[pad] == 0.0)
    assert np.all(np.isposinf(got_lse[pad]))
    assert_close(got_o[~pad], want_o[~pad], "O")
    assert_close(got_lse[~pad], want_lse[~pad], "LSE", max_abs=LSE_ABS, mean_abs=LSE_ABS)
    if exact:
        got32 = o32.cpu().double().numpy()
        assert np.all(got32[pad] == 0.0)
        assert np.max(np.abs(got32[~pad] - want_o[~pad])) <= 2e-4


@pytest.mark.parametrize("exact_o", [False, True], ids=["D_from_scores", "D_from_o32"])
@pytest.mark.parametrize("case", CASES[:4], ids=lambda c: f"seed{c[0]}")
def test_padded_backward_matches_oracle(case, exact_o):
    seed, real, cp, rank, hq, hkv, dqk, dv = case
    b = _batch(case, backward=True)
    dev = device()
    q, k, v, do = (t.to(dev) for t in (b.q, b.k, b.v, b.do))
    print(f"[pad bwd] seed={seed} real={real} cp={cp} rank={rank} exact_o={exact_o}", flush=True)
    o32 = torch.empty((q.shape[0], hq, dv), dtype=torch.float32, device=dev) if exact_o else None
    o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=real, cp=cp, rank=rank, padded=True, out_f32=o32)
    dq, dk, dvv = thd.attn_bwd(q=q, k=k, v=v, lse=lse, d_o=do, seqlens=real, cp=cp, rank=rank,
                               padded=True, o_f32=o32)
    torch.cuda.synchronize()
    want = oatt.attn_bwd64_padded(to64(b.q), to64(b.k), to64(b.v), to64(b.do), real, cp, rank)
    pad = opart.pad_rows(real, cp, rank)
    pad_keys = _pad_keys(real, cp)
    got = [t.cpu().double().numpy() for t in (dq, dk, dvv)]
    assert np.all(got[0][pad] == 0.0)
    assert np.all(got[1][pad_keys] == 0.0) and np.all(got[2][pad_keys] == 0.0)
    for name, g, e in zip(("dQ", "dK", "dV"), got, want):
        assert_close(g, e, f"padded {name}")
