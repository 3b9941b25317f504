"""Short-segment packing on an MI355X: forward plans whose partial query
tiles of several documents share one tile (per-row key-slot windows), against
the fp64 oracle, element by element over every output.

Packing changes which rows share a workgroup, never what a row attends to, so
every case must match the oracle to the same bounds as the plain plan; pad
rows of packed tiles still get O = 0 and LSE = +inf exactly, and document-start
rows still equal their first key's V bit for bit.
"""
import functools

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as oatt
from oracle import partition as opart
from parity import LSE_ABS, assert_close, device, to64

pytestmark = pytest.mark.gpu

thd = pytest.importorskip("packed_sequence_causal_amd")

O32_ABS = 2e-4

CASES = [
    # (seed, lengths, cp, rank, hq, hkv, dqk, dv); every case leaves partial
    # tiles in many documents for the forward's block_t = 128 // group
    (81, [16 * x for x in (1, 2, 3, 5, 8, 13, 21, 32, 7, 4)], 8, 0, 64, 8, 128, 128),
    (82, [8, 24, 40, 136, 520, 24, 8], 4, 1, 32, 8, 128, 128),
    (83, [16, 32, 1040, 16, 400, 48], 8, 3, 16, 16, 192, 128),     # expanded MLA shape
    (84, [36, 300, 84, 12, 6], 3, 2, 12, 4, 128, 128),              # group 3: 42-token tiles
    (85, [2, 4, 6, 2, 10, 14], 1, 0, 4, 2, 128, 128),               # cp = 1
    (86, [256, 40, 72, 8, 512, 24], 2, 1, 8, 8, 64, 64),
]


@functools.lru_cache(maxsize=None)
def _case(seed):
    case = next(c for c in CASES if c[0] == seed)
    _, lengths, cp, rank, hq, hkv, dqk, dv = case
    b = workloads.small_case(seed, lengths, cp, hq, hkv, dqk, dv, rank=rank)
    want = oatt.attn_fwd64(to64(b.q), to64(b.k), to64(b.v), lengths, cp, rank)
    return case, b, want


def _params():
    out = []
    for c in CASES:
        for bn in (32, 64):
            if bn == 32 and c[6] > 128:
                continue   # no 32-key kernel for d_qk = 192
            for conc in (0, 64):
                out.append(pytest.param(c[0], bn, conc, id=f"seed{c[0]}-bn{bn}-c{conc}"))
    return out


@pytest.mark.parametrize("seed,block_n,concurrency", _params())
def test_packed_forward_matches_oracle(seed, block_n, concurrency):
    """Both P paths (bf16 P; the exact fp32 O with split P) and the plain
    tiles' split key ranges, with packed tiles in the same launch."""
    (_, lengths, cp, rank, hq, hkv, dqk, dv), b, (want_o, want_lse) = _case(seed)
    dev = device()
    q, k, v = b.q.to(dev), b.k.to(dev), b.v.to(dev)
    bt = thd.preferred_tiles(hq=hq, hkv=hkv, d_qk=dqk, d_v=dv)[0]
    meta = thd.build_metadata(seqlens=b.lengths, cp=cp, rank=rank, block_t=bt, block_n=block_n,
                              concurrency=concurrency, device=0, packed=True)
    info = meta.info()
    print(f"[packed fwd] seed={seed} block_t={bt} block_n={block_n} concurrency={concurrency} "
          f"tiles={info['n_tiles']} packed={info['n_packed_tiles']} splits={info['n_splits']}",
          flush=True)
    assert info["n_packed_tiles"] > 0
    o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=cp, rank=rank, meta=meta)
    o32 = torch.full((q.shape[0], hq, dv), float("nan"), dtype=torch.float32, device=dev)
    o_x, _ = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=cp, rank=rank, meta=meta,
                          out_f32=o32)
    torch.cuda.synchronize()
    assert_close(to64(o), want_o, "O")
    assert_close(lse.cpu().double().numpy(), want_lse, "LSE", max_abs=LSE_ABS, mean_abs=LSE_ABS)
    assert_close(to64(o32), want_o, "O32", max_abs=O32_ABS, mean_abs=O32_ABS / 10)
    assert_close(to64(o_x), want_o, "O (exact path)")


PAD_CASES = [
    # (seed, real lengths, cp, rank, hq, hkv, dqk, dv)
    (91, [5, 13, 8, 3, 30, 1, 22], 2, 0, 32, 8, 128, 128),
    (92, [1, 3, 300, 77, 9, 14], 4, 3, 32, 8, 128, 128),
    (93, [17, 1040, 9, 400, 5], 8, 3, 16, 16, 192, 128),
]


@pytest.mark.parametrize("case", PAD_CASES, ids=lambda c: f"seed{c[0]}")
def test_packed_padded_forward_matches_oracle(case):
    seed, real, cp, rank, hq, hkv, dqk, dv = case
    lengths = opart.pad_lengths(real, cp)
    b = workloads.small_case(seed, lengths, cp, hq, hkv, dqk, dv, rank=rank)
    dev = device()
    q, k, v = b.q.to(dev), b.k.to(dev), b.v.to(dev)
    meta = thd.device_metadata(seqlens=real, cp=cp, rank=rank, hq=hq, hkv=hkv, d_qk=dqk, d_v=dv,
                               device=0, padded=True, forward=True, packed=True)
    info = meta.info()
    print(f"[packed pad fwd] seed={seed} real={real} block_n={info['block_n']} "
          f"packed={info['n_packed_tiles']}", flush=True)
    assert info["n_packed_tiles"] > 0
    rows = meta.field("pack_rows")
    assert (rows[:, 3] == 0).any()           # some pad rows sit in packed tiles
    o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=real, cp=cp, rank=rank, padded=True, meta=meta)
    torch.cuda.synchronize()
    want_o, want_lse = oatt.attn_fwd64_padded(to64(b.q), to64(b.k), to64(b.v), real, cp, rank)
    pad = opart.pad_rows(real, cp, rank)
    got_o, got_lse = to64(o), lse.cpu().double().numpy()
    assert np.all(got_o[pad] == 0.0)
    assert np.all(np.isposinf(got_lse[pad]))
    assert_close(got_o[~pad], want_o[~pad], "O")
    assert_close(got_lse[~pad], want_lse[~pad], "LSE", max_abs=LSE_ABS, mean_abs=LSE_ABS)


@pytest.mark.parametrize("name", ["short", "gqa_mid"])
def test_packed_forward_full_size_every_element(name):
    """The full-size workload with a packed plan in the forward's tile sizes
    and the device's split plan: every element of O and LSE against the
    oracle, and document-start rows equal to their first key's V bit for bit."""
    w = workloads.BY_NAME[name]
    b = workloads.make_batch(w)
    dev = device()
    q, k, v = b.q.to(dev), b.k.to(dev), b.v.to(dev)
    meta = thd.device_metadata(seqlens=b.lengths, cp=w.cp, rank=w.rank, hq=w.hq, hkv=w.hkv,
                               d_qk=w.d_qk, d_v=w.d_v, device=0, forward=True, packed=True)
    info = meta.info()
    print(f"[packed fwd full] {name} block_n={info['block_n']} tiles={info['n_tiles']} "
          f"packed={info['n_packed_tiles']} items={info['n_items']}", flush=True)
    assert info["n_packed_tiles"] > 0
    o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=w.cp, rank=w.rank, meta=meta)
    torch.cuda.synchronize()
    want_o, want_lse = oatt.attn_fwd64(to64(b.q), to64(b.k), to64(b.v), b.lengths, w.cp, w.rank)
    mx, mean = assert_close(to64(o), want_o, f"{name} O")
    lmx, _ = assert_close(lse.cpu().double().numpy(), want_lse, f"{name} LSE",
                          max_abs=LSE_ABS, mean_abs=LSE_ABS)
    print(f"[packed fwd full] {name} O max-abs {mx:.3g} mean-abs {mean:.3g} LSE max-abs {lmx:.3g}",
          flush=True)
    qg = opart.q_global(b.lengths, w.cp, w.rank)
    cu = opart.cu_seqlens(b.lengths)
    pos = {g: i for i, g in enumerate(qg.tolist())}
    starts = [pos[c] for c in cu[:-1] if c in pos]
    if starts:
        firsts = [c for c in cu[:-1] if c in pos]
        rows_v = opart.kv_row(b.lengths, w.cp)[firsts]
        group = w.hq // w.hkv
        got = o[torch.tensor(starts, device=o.device)].cpu()
        want = b.v[torch.from_numpy(rows_v.astype(np.int64))].repeat_interleave(group, dim=1)
        assert torch.equal(got, want)
