"""Inputs at the boundary's size limit, on an MI355X.

The kernels address the gathered K and V with 32-bit byte offsets, and the
boundary refuses K or V of 4 GiB or more. Here K and V are each 32 KiB short
of that (T = 2^21 - 16 tokens, 8 kv heads of dimension 128, cp = 8), and the
forward and the backward run on the whole batch. A document's outputs and
gradients depend on its own tokens only (the mask resets at every EOD), so
the first and the last document, whose K/V rows lie at the lowest and the
highest offsets of the rank-major layout, are compared element by element
with the fp64 oracle run on that document alone.
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

CP, RANK = 8, 0
HQ, HKV, D = 16, 8, 128
# 511 documents of 4096 tokens and one of 4080: K and V take 2^32 - 32 KiB each
LENGTHS = [4096] * 511 + [4080]
DOCS = (0, len(LENGTHS) - 1)


@pytest.fixture(scope="module")
def big():
    dev = device()
    total = sum(LENGTHS)
    tl = total // CP
    print(f"[limits] drawing T={total} cp={CP} rank={RANK} hq={HQ} hkv={HKV} d={D}", flush=True)
    q = workloads.device_normal(31001, (tl, HQ, D), dev)
    k = workloads.device_normal(31002, (total, HKV, D), dev)
    v = workloads.device_normal(31003, (total, HKV, D), dev)
    do = workloads.device_normal(31004, (tl, HQ, D), dev)
    assert (1 << 32) - k.numel() * 2 == 32 * 1024 and v.numel() == k.numel()
    qg = opart.q_global(LENGTHS, CP, RANK)
    kvr = opart.kv_row(LENGTHS, CP)
    cu = opart.cu_seqlens(LENGTHS)
    docs = {}
    for d in DOCS:
        lo, hi = cu[d], cu[d + 1]
        local = np.nonzero((qg >= lo) & (qg < hi))[0]           # the rank's rows, in order
        small_len = [hi - lo]
        assert np.array_equal(qg[local] - lo, opart.q_global(small_len, CP, RANK))
        rows_big = kvr[lo:hi]                                   # gathered row of each token
        rows_small = opart.kv_row(small_len, CP)
        docs[d] = (local, rows_big, rows_small, small_len)
    batch = dict(q=q, k=k, v=v, do=do, docs=docs)
    del q, k, v, do
    yield batch
    batch.clear()
    torch.cuda.empty_cache()


def _alone(b, d):
    """The document's own Q, K, V, dO as a one-document batch (fp64, host)."""
    local, rows_big, rows_small, small_len = b["docs"][d]
    idx_q = torch.as_tensor(local, device=b["q"].device)
    idx_k = torch.as_tensor(rows_big.astype(np.int64), device=b["k"].device)
    inv = np.empty_like(rows_small)
    inv[rows_small] = np.arange(rows_small.shape[0])          # small row -> token
    order = torch.as_tensor(inv.astype(np.int64), device=b["k"].device)
    q = to64(b["q"][idx_q])
    do = to64(b["do"][idx_q])
    k = to64(b["k"][idx_k][order])
    v = to64(b["v"][idx_k][order])
    return q, k, v, do, small_len


def test_forward_at_the_kv_size_limit(big):
    print("[limits] forward, whole batch", flush=True)
    o, lse = thd.attn_fwd(q=big["q"], k=big["k"], v=big["v"], seqlens=LENGTHS, cp=CP, rank=RANK)
    torch.cuda.synchronize()
    for d in DOCS:
        local, rows_big, rows_small, small_len = big["docs"][d]
        print(f"[limits] forward, document {d}: {len(local)} rows, gathered rows "
              f"{int(rows_big.min())}..{int(rows_big.max())}", flush=True)
        q, k, v, _, small_len = _alone(big, d)
        want_o, want_lse = oatt.attn_fwd64(q, k, v, small_len, CP, RANK)
        idx = torch.as_tensor(local, device=o.device)
        assert_close(to64(o[idx]), want_o, f"O doc {d}")
        assert_close(lse[idx].cpu().double().numpy(), want_lse, f"LSE doc {d}",
                     max_abs=LSE_ABS, mean_abs=LSE_ABS)


@pytest.mark.parametrize("exact_o", [False, True])
def test_backward_at_the_kv_size_limit(big, exact_o):
    dev = big["q"].device
    print(f"[limits] backward, whole batch, exact_o={exact_o}", flush=True)
    o32 = torch.empty((big["q"].shape[0], HQ, D), dtype=torch.float32, device=dev) if exact_o else None
    o, lse = thd.attn_fwd(q=big["q"], k=big["k"], v=big["v"], seqlens=LENGTHS, cp=CP, rank=RANK,
                          out_f32=o32)
    dq, dk, dv = thd.attn_bwd(q=big["q"], k=big["k"], v=big["v"], lse=lse, d_o=big["do"],
                              seqlens=LENGTHS, cp=CP, rank=RANK, o_f32=o32)
    torch.cuda.synchronize()
    del o, o32
    for d in DOCS:
        local, rows_big, rows_small, small_len = big["docs"][d]
        print(f"[limits] backward, document {d}", flush=True)
        q, k, v, do, small_len = _alone(big, d)
        want_dq, want_dk, want_dv = oatt.attn_bwd64(q, k, v, do, small_len, CP, RANK)
        idx_q = torch.as_tensor(local, device=dev)
        idx_k = torch.as_tensor(rows_big.astype(np.int64), device=dev)
        # the oracle's gradients are in the one-document batch's gathered order
        assert_close(dq[idx_q].cpu().double().numpy(), want_dq, f"dQ doc {d}")
        assert_close(dk[idx_k].cpu().double().numpy(), want_dk[rows_small], f"dK doc {d}")
        assert_close(dv[idx_k].cpu().double().numpy(), want_dv[rows_small], f"dV doc {d}")
    del dq, dk, dv
    torch.cuda.empty_cache()
