"""Backward parity of the HIP path against the fp64 oracle, on an MI355X.

dQ, dK, dV are compared element by element with the oracle's gradients for
the same inputs (the GPU backward consumes its own forward's O and LSE).
The full fwd+bwd workload is compared in full; small ragged cases cover the
edge shapes. Unseen keys must get exact zeros, and runs are bitwise
reproducible.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import attention as oatt
from oracle import partition as opart
from parity import assert_close, device, to64

pytestmark = pytest.mark.gpu

thd = pytest.importorskip("packed_sequence_causal_amd")


def _run(batch, rank=None, scale=None, exact_o=False):
    """Forward then backward on the GPU. exact_o: the forward also writes its
    fp32 O and the backward takes D from it (two backward launches instead of
    three)."""
    w = batch.workload
    r = w.rank if rank is None else rank
    dev = device()
    q, k, v, do = (t.to(dev) for t in (batch.q, batch.k, batch.v, batch.do))
    print(f"[bwd] case={w.name} n={len(batch.lengths)} cp={w.cp} rank={r} hq={w.hq} hkv={w.hkv} "
          f"dqk={w.d_qk} dv={w.d_v} exact_o={exact_o}", flush=True)
    o32 = torch.empty((q.shape[0], w.hq, w.d_v), dtype=torch.float32, device=dev) if exact_o else None
    o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=batch.lengths, cp=w.cp, rank=r, softmax_scale=scale,
                          out_f32=o32)
    dq, dk, dv = thd.attn_bwd(q=q, k=k, v=v, lse=lse, d_o=do, seqlens=batch.lengths, cp=w.cp,
                              rank=r, softmax_scale=scale, o_f32=o32)
    torch.cuda.synchronize()
    return dq, dk, dv


def _check(batch, got, rank=None, scale=None):
    w = batch.workload
    r = w.rank if rank is None else rank
    want = oatt.attn_bwd64(to64(batch.q), to64(batch.k), to64(batch.v), to64(batch.do),
                           batch.lengths, w.cp, r, scale=scale)
    errs = []
    for name, g, e in zip(("dQ", "dK", "dV"), got, want):
        d = np.abs(g.cpu().double().numpy() - e)
        errs.append(f"{name} max-abs {d.max():.3g} mean-abs {d.mean():.3g} (|ref| max {np.abs(e).max():.3g})")
    print(f"[bwd] {w.name}: " + "; ".join(errs), flush=True)
    for name, g, e in zip(("dQ", "dK", "dV"), got, want):
        assert_close(g.cpu().double().numpy(), e, f"{w.name} {name}")
    return want


SMALL = [
    # (seed, lengths, cp, rank, hq, hkv, dqk, dv)
    (51, [256, 512, 256], 2, 0, 8, 8, 64, 64),
    (52, [8, 24, 40, 136, 520], 4, 1, 32, 8, 128, 128),
    (53, [16 * x for x in (1, 2, 3, 5, 8, 13, 21, 32)], 8, 0, 64, 8, 128, 128),
    (54, [1000, 72, 600], 4, 3, 32, 8, 128, 128),
    (55, [36, 300, 84], 3, 2, 12, 4, 128, 128),
    (56, [16, 32, 1040, 16], 8, 3, 16, 16, 192, 128),
    (57, [2, 4, 6, 2], 1, 0, 4, 2, 128, 128),
]


@pytest.mark.parametrize("exact_o", [False, True], ids=["D_from_scores", "D_from_o32"])
@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"seed{c[0]}")
def test_backward_matches_oracle_small(case, exact_o):
    seed, lengths, cp, rank, hq, hkv, dqk, dv = case
    b = workloads.small_case(seed, lengths, cp, hq, hkv, dqk, dv, backward=True, rank=rank)
    got = _run(b, exact_o=exact_o)
    _check(b, got)


@pytest.mark.parametrize("exact_o", [False, True], ids=["D_from_scores", "D_from_o32"])
def test_backward_custom_scale(exact_o):
    b = workloads.small_case(58, [64, 192], 2, 8, 2, 128, 128, backward=True, rank=1)
    got = _run(b, scale=0.2, exact_o=exact_o)
    _check(b, got, scale=0.2)


def test_backward_paths_agree():
    """D from the scores and D from the exact fp32 O give the same gradients
    up to fp32 rounding."""
    b = workloads.small_case(53, [16 * x for x in (1, 2, 3, 5, 8, 13, 21, 32)], 8, 64, 8, 128, 128,
                             backward=True, rank=0)
    g0 = _run(b, exact_o=False)
    g1 = _run(b, exact_o=True)
    for name, a, c in zip(("dQ", "dK", "dV"), g0, g1):
        diff = (a - c).abs().max().item()
        print(f"[bwd] paths {name} max diff {diff:.3g}", flush=True)
        assert diff <= 1e-4


@pytest.mark.parametrize("exact_o", [False, True], ids=["D_from_scores", "D_from_o32"])
def test_backward_fwdbwd_workload_full(exact_o):
    w = workloads.BY_NAME["fwdbwd"]
    b = workloads.make_batch(w)
    dq, dk, dv = _run(b, exact_o=exact_o)
    _check(b, (dq, dk, dv))
    # keys no local query sees (offsets >= (2cp - r) c in each document) are exact zeros
    cu = opart.cu_seqlens(b.lengths)
    rows = opart.kv_row(b.lengths, w.cp)
    unseen = np.concatenate([rows[cu[i] + (2 * w.cp - w.rank) * (int(L) // (2 * w.cp)):cu[i + 1]]
                             for i, L in enumerate(b.lengths)]).astype(np.int64)
    assert unseen.size > 0
    idx = torch.from_numpy(unseen).to(dk.device)
    assert torch.count_nonzero(dk[idx]).item() == 0 and torch.count_nonzero(dv[idx]).item() == 0
    # bitwise reproducible (no atomics)
    dq2, dk2, dv2 = _run(b, exact_o=exact_o)
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)


@pytest.mark.parametrize("rank", [0, 1, 3])
def test_backward_fwdbwd_workload_other_ranks(rank):
    """The full training workload at the other ranks of its group (the batch's
    Q and dO stand in for that rank's share), training path (D from the fp32
    O): every element of dQ, dK, dV against the oracle, unseen keys zero."""
    w = workloads.BY_NAME["fwdbwd"]
    b = workloads.make_batch(w)
    dq, dk, dv = _run(b, rank=rank, exact_o=True)
    _check(b, (dq, dk, dv), rank=rank)
    cu = opart.cu_seqlens(b.lengths)
    rows = opart.kv_row(b.lengths, w.cp)
    unseen = np.concatenate([rows[cu[i] + (2 * w.cp - rank) * (int(L) // (2 * w.cp)):cu[i + 1]]
                             for i, L in enumerate(b.lengths)]).astype(np.int64)
    if unseen.size:
        idx = torch.from_numpy(unseen).to(dk.device)
        assert torch.count_nonzero(dk[idx]).item() == 0 and torch.count_nonzero(dv[idx]).item() == 0


def test_backward_gradient_identities_on_gpu():
    lengths, cp, rank, hq, hkv = [96, 480, 192], 4, 1, 16, 4
    b = workloads.small_case(59, lengths, cp, hq, hkv, 128, 128, backward=True, rank=rank)
    dq, dk, dv = _run(b)
    group = hq // hkv
    do = b.do.double()
    for hk in range(hkv):
        want = do[:, hk * group:(hk + 1) * group].sum((0, 1))
        got = dv[:, hk].double().sum(0).cpu()
        assert torch.allclose(got, want, atol=5e-2, rtol=1e-3)
        assert dk[:, hk].double().sum(0).abs().max().item() < 5e-2


BF16_KV = [SMALL[1], SMALL[4], SMALL[5], SMALL[6]]


@pytest.mark.parametrize("exact_o", [False, True], ids=["D_from_scores", "D_from_o32"])
@pytest.mark.parametrize("case", BF16_KV + ["fwdbwd"], ids=lambda c: c if isinstance(c, str) else f"seed{c[0]}")
def test_backward_bf16_dkdv_are_the_fp32_results_rounded(case, exact_o):
    """thd_attn_bwd_bf16kv: dk and dv are the fp32 path's values rounded to
    nearest even, bit for bit, and dq is the fp32 path's, bit for bit; against
    the oracle they stay within the bound plus one bf16 rounding."""
    if case == "fwdbwd":
        w = workloads.BY_NAME[case]
        b = workloads.make_batch(w)
    else:
        seed, lengths, cp, rank, hq, hkv, dqk, dv = case
        b = workloads.small_case(seed, lengths, cp, hq, hkv, dqk, dv, backward=True, rank=rank)
        w = b.workload
    dev = device()
    q, k, v, do = (t.to(dev) for t in (b.q, b.k, b.v, b.do))
    print(f"[bwd bf16 dk/dv] case={w.name} cp={w.cp} rank={w.rank} hq={w.hq} hkv={w.hkv} "
          f"dqk={w.d_qk} exact_o={exact_o}", flush=True)
    o32 = torch.empty((q.shape[0], w.hq, w.d_v), dtype=torch.float32, device=dev) if exact_o else None
    o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=w.cp, rank=w.rank, out_f32=o32)
    args = dict(q=q, k=k, v=v, lse=lse, d_o=do, seqlens=b.lengths, cp=w.cp, rank=w.rank, o_f32=o32)
    dq32, dk32, dv32 = thd.attn_bwd(**args)
    dq, dk, dv = thd.attn_bwd(**args, dkdv_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert dk.dtype == torch.bfloat16 and dv.dtype == torch.bfloat16 and dq.dtype == torch.float32
    assert torch.equal(dq, dq32)
    assert torch.equal(dk, dk32.to(torch.bfloat16)) and torch.equal(dv, dv32.to(torch.bfloat16))
    want = oatt.attn_bwd64(to64(b.q), to64(b.k), to64(b.v), to64(b.do), b.lengths, w.cp, w.rank)
    for name, g, e in zip(("dK", "dV"), (dk, dv), want[1:]):
        err = np.abs(to64(g) - e)
        print(f"[bwd bf16 dk/dv] {name} max-abs {err.max():.3g} (|ref| max {np.abs(e).max():.3g})",
              flush=True)
        assert np.all(err <= 2e-2 + 2.0 ** -8 * np.abs(e)), name
