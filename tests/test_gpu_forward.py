"""Forward parity of the HIP path against the fp64 oracle, on an MI355X.

Every case, the full-size workloads included, is compared element by element
over every output; properties that hold at any size are checked besides
(document-start rows, EOD isolation, causality, determinism, union over
ranks).
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


def _run(batch, rank=None, scale=None):
    w = batch.workload
    r = w.rank if rank is None else rank
    dev = device()
    q = batch.q.to(dev)
    k = batch.k.to(dev)
    v = batch.v.to(dev)
    print(f"[fwd] case={w.name} lengths[:4]={batch.lengths[:4].tolist()} n={len(batch.lengths)} "
          f"cp={w.cp} rank={r} hq={w.hq} hkv={w.hkv} dqk={w.d_qk} dv={w.d_v}", flush=True)
    o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=batch.lengths, cp=w.cp, rank=r,
                          softmax_scale=scale)
    torch.cuda.synchronize()
    return o, lse


SMALL = [
    # (seed, lengths, cp, rank, hq, hkv, dqk, dv)
    (11, [256, 512, 256], 2, 0, 8, 8, 64, 64),
    (12, [256, 512, 256], 2, 1, 8, 8, 64, 64),
    (13, [8, 24, 40, 136, 520], 4, 1, 32, 8, 128, 128),
    (14, [16, 32, 1040, 16, 400], 8, 3, 16, 16, 192, 128),
    (15, [16 * x for x in (1, 2, 3, 5, 8, 13, 21, 32, 7, 4)], 8, 0, 64, 8, 128, 128),
    (16, [1000, 72, 600], 4, 2, 32, 8, 128, 128),
    (17, [36, 300, 84], 3, 2, 12, 4, 128, 128),        # group 3: 126 of 128 rows used
    (18, [2, 4, 6, 2], 1, 0, 4, 2, 128, 128),          # cp = 1, documents shorter than a tile
    (19, [4096], 2, 1, 4, 1, 64, 64),                  # one long document, group 4, MQA-like
    (20, [32, 64], 2, 1, 32, 2, 128, 128),             # group 16: 8 tokens per tile
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"seed{c[0]}")
def test_forward_matches_oracle_small(case):
    seed, lengths, cp, rank, hq, hkv, dqk, dv = case
    b = workloads.small_case(seed, lengths, cp, hq, hkv, dqk, dv, rank=rank)
    o, lse = _run(b)
    want_o, want_lse = oatt.attn_fwd64(to64(b.q), to64(b.k), to64(b.v), lengths, cp, rank)
    assert_close(to64(o), want_o, "O")
    assert_close(lse.cpu().double().numpy(), want_lse, "LSE", max_abs=LSE_ABS, mean_abs=LSE_ABS)


SPLIT = [
    # (seed, lengths, cp, rank, hq, hkv, dqk, dv): long documents, so the
    # key ranges of the late chunk's tiles are cut into several parts
    (71, [2048, 512, 1024], 2, 1, 16, 4, 128, 128),
    (72, [4096, 96], 4, 0, 8, 8, 64, 64),
    (73, [3072, 1040], 8, 3, 16, 16, 192, 128),
    (74, [1512, 300], 3, 1, 12, 4, 128, 128),      # group 3: 126-row tiles
]


@pytest.mark.parametrize("case", SPLIT, ids=lambda c: f"seed{c[0]}")
@pytest.mark.parametrize("concurrency", [64, 100000])
def test_forward_split_key_ranges_match_oracle(case, concurrency):
    seed, lengths, cp, rank, hq, hkv, dqk, dv = case
    b = workloads.small_case(seed, lengths, cp, hq, hkv, dqk, dv, rank=rank)
    dev = device()
    q, k, v = b.q.to(dev), b.k.to(dev), b.v.to(dev)
    meta = thd.device_metadata(seqlens=b.lengths, cp=cp, rank=rank, hq=hq, hkv=hkv, d_qk=dqk,
                               d_v=dv, device=0, concurrency=concurrency)
    info = meta.info()
    print(f"[fwd split] seed={seed} concurrency={concurrency} kv_split={info['kv_split']} "
          f"splits={info['n_splits']} parts={info['n_part_slots']}", flush=True)
    assert info["n_splits"] > 0
    o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=cp, rank=rank, meta=meta)
    torch.cuda.synchronize()
    want_o, want_lse = oatt.attn_fwd64(to64(b.q), to64(b.k), to64(b.v), lengths, cp, rank)
    assert_close(to64(o), want_o, "O")
    assert_close(lse.cpu().double().numpy(), want_lse, "LSE", max_abs=LSE_ABS, mean_abs=LSE_ABS)
    # the same rows without splitting agree closely (different summation order only)
    o1, lse1 = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=cp, rank=rank, concurrency=0)
    torch.cuda.synchronize()
    assert (o.float() - o1.float()).abs().max().item() <= 1e-2
    assert (lse - lse1).abs().max().item() <= 1e-4


@pytest.mark.parametrize("case", [c for c in SMALL + SPLIT if c[6] <= 128], ids=lambda c: f"seed{c[0]}")
@pytest.mark.parametrize("concurrency", [0, 64])
def test_forward_short_tiles_match_oracle(case, concurrency):
    """The 32-key-tile kernels (three workgroups per CU), with and without split
    key ranges, in both P paths: O, LSE and the exact fp32 O against the oracle."""
    seed, lengths, cp, rank, hq, hkv, dqk, dv = case
    b = workloads.small_case(seed, lengths, cp, hq, hkv, dqk, dv, rank=rank)
    dev = device()
    q, k, v = b.q.to(dev), b.k.to(dev), b.v.to(dev)
    bt = thd.preferred_tiles(hq=hq, hkv=hkv, d_qk=dqk, d_v=dv)[0]
    meta = thd.build_metadata(seqlens=b.lengths, cp=cp, rank=rank, block_t=bt, block_n=32,
                              concurrency=concurrency, device=0)
    print(f"[fwd short tiles] seed={seed} concurrency={concurrency} "
          f"splits={meta.info()['n_splits']}", flush=True)
    want_o, want_lse = oatt.attn_fwd64(to64(b.q), to64(b.k), to64(b.v), lengths, cp, rank)
    o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=cp, rank=rank, meta=meta)
    o32 = torch.full((q.shape[0], hq, dv), float("nan"), dtype=torch.float32, device=dev)
    o_x, lse_x = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=cp, rank=rank, meta=meta,
                              out_f32=o32)
    torch.cuda.synchronize()
    assert_close(to64(o), want_o, "O")
    assert_close(lse.cpu().double().numpy(), want_lse, "LSE", max_abs=LSE_ABS, mean_abs=LSE_ABS)
    assert_close(to64(o32), want_o, "O32", max_abs=O32_ABS, mean_abs=O32_ABS / 10)
    assert_close(to64(o_x), want_o, "O (exact path)")


def test_split_forward_and_backward_on_side_streams():
    """Calls on two side streams at once (split forward, whose partial results
    need a workspace, then the backward) give bit-identical results to the same
    calls on the current stream: per-call workspaces are never shared."""
    seed, lengths, cp, rank, hq, hkv, dqk, dv = SPLIT[0]
    b = workloads.small_case(seed, lengths, cp, hq, hkv, dqk, dv, backward=True, rank=rank)
    dev = device()
    q, k, v, do = (t.to(dev) for t in (b.q, b.k, b.v, b.do))
    meta = thd.device_metadata(seqlens=b.lengths, cp=cp, rank=rank, hq=hq, hkv=hkv, d_qk=dqk,
                               d_v=dv, device=0, concurrency=64)
    assert meta.info()["n_splits"] > 0
    print(f"[fwd streams] seed={seed}", flush=True)

    def run(stream):
        o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=cp, rank=rank, meta=meta,
                              stream=stream)
        g = thd.attn_bwd(q=q, k=k, v=v, lse=lse, d_o=do, seqlens=b.lengths, cp=cp, rank=rank,
                         meta=meta, stream=stream)
        return (o, lse) + g

    want = run(None)
    torch.cuda.synchronize()
    side = [torch.cuda.Stream(device=dev) for _ in range(2)]
    for s in side:
        s.wait_stream(torch.cuda.current_stream(dev))
    got = [run(s) for s in side]
    torch.cuda.synchronize()
    for res in got:
        for name, a, w in zip(("O", "LSE", "dQ", "dK", "dV"), res, want):
            assert torch.equal(a, w), name


EXACT = [
    # (seed, lengths, cp, rank, hq, hkv, dqk, dv, concurrency)
    (81, [256, 512, 256], 2, 0, 8, 8, 64, 64, 0),
    (82, [8, 24, 40, 136, 520], 4, 1, 32, 8, 128, 128, 0),
    (83, [16, 32, 1040, 16, 400], 8, 3, 16, 16, 192, 128, 0),
    (84, [2048, 512, 1024], 2, 1, 16, 4, 128, 128, 64),    # split key ranges: combine writes O32
    (85, [36, 300, 84], 3, 2, 12, 4, 128, 128, 0),
]
O32_ABS = 2e-4   # split probabilities: O limited by fp32 accumulation


@pytest.mark.parametrize("case", EXACT, ids=lambda c: f"seed{c[0]}")
def test_forward_fp32_output_is_exact(case):
    """With out_f32, P enters P.V as a bf16 pair: the fp32 O matches the fp64
    oracle far inside the bf16 tolerance, and o and lse still match."""
    seed, lengths, cp, rank, hq, hkv, dqk, dv, conc = case
    b = workloads.small_case(seed, lengths, cp, hq, hkv, dqk, dv, rank=rank)
    dev = device()
    q, k, v = b.q.to(dev), b.k.to(dev), b.v.to(dev)
    print(f"[fwd] exact case seed={seed} cp={cp} rank={rank} dqk={dqk} concurrency={conc}", flush=True)
    meta = thd.device_metadata(seqlens=b.lengths, cp=cp, rank=rank, hq=hq, hkv=hkv, d_qk=dqk,
                               d_v=dv, device=0, concurrency=conc)
    o32 = torch.full((q.shape[0], hq, dv), float("nan"), dtype=torch.float32, device=dev)
    o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=cp, rank=rank, out_f32=o32,
                          meta=meta)
    torch.cuda.synchronize()
    want_o, want_lse = oatt.attn_fwd64(to64(b.q), to64(b.k), to64(b.v), lengths, cp, rank)
    assert_close(to64(o), want_o, "O")
    assert_close(lse.cpu().double().numpy(), want_lse, "LSE", max_abs=LSE_ABS, mean_abs=LSE_ABS)
    err = np.abs(o32.cpu().double().numpy() - want_o)
    print(f"[fwd] O32 max-abs {err.max():.3g} mean-abs {err.mean():.3g}", flush=True)
    assert err.max() <= O32_ABS
    # the bf16 output is the fp32 one rounded to nearest even
    assert torch.equal(o, o32.to(torch.bfloat16))


def test_forward_custom_scale():
    b = workloads.small_case(21, [64, 192], 2, 8, 2, 128, 128, rank=1)
    o, lse = _run(b, scale=0.3)
    want_o, want_lse = oatt.attn_fwd64(to64(b.q), to64(b.k), to64(b.v), b.lengths, 2, 1, scale=0.3)
    assert_close(to64(o), want_o, "O")
    assert_close(lse.cpu().double().numpy(), want_lse, "LSE", max_abs=LSE_ABS, mean_abs=LSE_ABS)
    # the library's default scale is 1/sqrt(d_qk), rounded to fp32
    o_def, lse_def = _run(b)
    o_exp, lse_exp = _run(b, scale=float(np.float32(1.0 / np.sqrt(128.0))))
    assert torch.equal(o_def, o_exp) and torch.equal(lse_def, lse_exp)


@pytest.mark.parametrize("w", workloads.WORKLOADS, ids=lambda w: w.name)
def test_forward_full_size_every_element(w):
    """Each workload at its full size, in the launch configuration the
    benchmark times (the forward's tile choice for the batch and the device's
    split plan): every element of O and LSE against the fp64 oracle."""
    b = workloads.make_batch(w)
    dev = device()
    q, k, v = b.q.to(dev), b.k.to(dev), b.v.to(dev)
    meta = thd.device_metadata(seqlens=b.lengths, cp=w.cp, rank=w.rank, hq=w.hq, hkv=w.hkv,
                               d_qk=w.d_qk, d_v=w.d_v, device=0, forward=True)
    info = meta.info()
    print(f"[fwd full] {w.name} block_n={info['block_n']} items={info['n_items']} "
          f"splits={info['n_splits']}", flush=True)
    # the paths the benchmark runs on these workloads are the ones compared here
    if w.name == "mla":
        assert info["n_splits"] > 0          # split key ranges plus the combine pass
    if w.name == "short":
        assert info["block_n"] == 32         # the 32-key tile kernel
    o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=w.cp, rank=w.rank, meta=meta)
    torch.cuda.synchronize()
    want_o, want_lse = oatt.attn_fwd64(to64(b.q), to64(b.k), to64(b.v), b.lengths, w.cp, w.rank)
    mx, mean = assert_close(to64(o), want_o, f"{w.name} O")
    lmx, _ = assert_close(lse.cpu().double().numpy(), want_lse, f"{w.name} LSE",
                          max_abs=LSE_ABS, mean_abs=LSE_ABS)
    print(f"[fwd full] {w.name} O max-abs {mx:.3g} mean-abs {mean:.3g} LSE max-abs {lmx:.3g}",
          flush=True)
    # rows that are a document's first token see one key: O equals V exactly
    if w.rank == 0:
        qg = opart.q_global(b.lengths, w.cp, w.rank)
        cu = opart.cu_seqlens(b.lengths)
        pos = {g: i for i, g in enumerate(qg.tolist())}
        starts = [pos[c] for c in cu[:-1]]
        rows_v = opart.kv_row(b.lengths, w.cp)[cu[:-1]]
        group = w.hq // w.hkv
        got = o[torch.tensor(starts, device=o.device)].cpu()
        want = b.v[torch.from_numpy(rows_v.astype(np.int64))].repeat_interleave(group, dim=1)
        assert torch.equal(got, want)


OTHER_RANKS = [(name, r) for name in ("gqa_mid", "mla", "short")
               for r in range(workloads.BY_NAME[name].cp) if r != workloads.BY_NAME[name].rank]


@functools.lru_cache(maxsize=1)
def _full_batch(name):
    """One workload's batch, on the host and on the device, drawn once for all its ranks."""
    b = workloads.make_batch(workloads.BY_NAME[name])
    dev = device()
    return b, (b.q.to(dev), b.k.to(dev), b.v.to(dev)), (to64(b.q), to64(b.k), to64(b.v))


@pytest.mark.parametrize("name,rank", OTHER_RANKS, ids=lambda x: str(x))
def test_forward_full_size_every_rank(name, rank):
    """The full-size forward workloads at every other rank of their
    context-parallel group (same batch, that rank's share and plan): every
    element of O and LSE against the fp64 oracle."""
    w = workloads.BY_NAME[name]
    # the batch's Q is drawn for the workload's own rank; any rank's share has
    # the same shape, and these values stand in for it
    b, (q, k, v), (q64, k64, v64) = _full_batch(name)
    meta = thd.device_metadata(seqlens=b.lengths, cp=w.cp, rank=rank, hq=w.hq, hkv=w.hkv,
                               d_qk=w.d_qk, d_v=w.d_v, device=0, forward=True)
    info = meta.info()
    print(f"[fwd rank] {name} rank={rank} block_n={info['block_n']} items={info['n_items']} "
          f"splits={info['n_splits']}", flush=True)
    o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=b.lengths, cp=w.cp, rank=rank, meta=meta)
    torch.cuda.synchronize()
    want_o, want_lse = oatt.attn_fwd64(q64, k64, v64, b.lengths, w.cp, rank)
    assert_close(to64(o), want_o, f"{name} rank {rank} O")
    assert_close(lse.cpu().double().numpy(), want_lse, f"{name} rank {rank} LSE",
                 max_abs=LSE_ABS, mean_abs=LSE_ABS)


def test_forward_tiny_full_compare():
    w = workloads.BY_NAME["tiny"]
    b = workloads.make_batch(w)
    o, lse = _run(b)
    want_o, want_lse = oatt.attn_fwd64(to64(b.q), to64(b.k), to64(b.v), b.lengths, w.cp, w.rank)
    assert_close(to64(o), want_o, "O")
    assert_close(lse.cpu().double().numpy(), want_lse, "LSE", max_abs=LSE_ABS, mean_abs=LSE_ABS)


def test_forward_deterministic_and_isolated():
    lengths, cp, rank = [64, 320, 128], 2, 0
    b = workloads.small_case(30, lengths, cp, 32, 8, 128, 128, rank=rank)
    o1, l1 = _run(b)
    o2, l2 = _run(b)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # EOD isolation: NaN in every other document's K/V leaves document 1's rows bit-identical
    rows = opart.kv_row(lengths, cp)
    cu = opart.cu_seqlens(lengths)
    others = np.concatenate([rows[cu[0]:cu[1]], rows[cu[2]:cu[3]]]).astype(np.int64)
    k2, v2 = b.k.clone(), b.v.clone()
    k2[torch.from_numpy(others)] = float("nan")
    v2[torch.from_numpy(others)] = float("nan")
    b2 = workloads.Batch(b.workload, b.lengths, b.q, k2, v2)
    o3, l3 = _run(b2)
    qg = opart.q_global(lengths, cp, rank)
    mine = torch.from_numpy(np.nonzero((qg >= cu[1]) & (qg < cu[2]))[0]).to(o1.device)
    assert torch.equal(o3[mine], o1[mine]) and torch.equal(l3[mine], l1[mine])
    # causality: changing keys after position 330 (inside a query tile of rank 0's
    # chunk [304, 384)) leaves rows at or before 330 bit-identical
    k4, v4 = b.k.clone(), b.v.clone()
    later = torch.from_numpy(rows[331:cu[2]].astype(np.int64))
    k4[later] = -k4[later] * 3
    v4[later] = v4[later] + 1
    o4, l4 = _run(workloads.Batch(b.workload, b.lengths, b.q, k4, v4))
    early = torch.from_numpy(np.nonzero(qg <= 330)[0]).to(o1.device)
    assert torch.equal(o4[early], o1[early]) and torch.equal(l4[early], l1[early])


def test_union_over_ranks_is_unpartitioned_attention():
    lengths, cp, hq, hkv = [64, 256, 128, 32], 4, 16, 4
    total = sum(lengths)
    rng = np.random.default_rng(31)
    qglob = workloads.bf16_normal(rng, (total, hq, 128))
    kglob = workloads.bf16_normal(rng, (total, hkv, 128))
    vglob = workloads.bf16_normal(rng, (total, hkv, 128))
    order = torch.from_numpy(opart.gathered_order(lengths, cp).astype(np.int64))
    k = kglob[order].contiguous()
    v = vglob[order].contiguous()
    out = torch.zeros((total, hq, 128), dtype=torch.float64)
    for r in range(cp):
        qg = torch.from_numpy(opart.q_global(lengths, cp, r).astype(np.int64))
        w = workloads.Workload("union", 31, total, cp, r, hq, hkv, 128, 128, "fixed",
                               fixed=tuple(lengths))
        o, _ = _run(workloads.Batch(w, np.asarray(lengths, np.int32), qglob[qg].contiguous(), k, v))
        out[qg] = o.double().cpu()
    # cp = 1 is the unpartitioned sequence: global order for Q, K and V
    want, _ = oatt.attn_fwd64(to64(qglob), to64(kglob), to64(vglob), lengths, 1, 0)
    assert_close(out.numpy(), want, "union O")


def test_forward_reports_errors_from_device_path():
    b = workloads.small_case(40, [64], 2, 8, 8, 128, 128, rank=0)
    dev = device()
    q, k, v = b.q.to(dev), b.k.to(dev), b.v.to(dev)
    # metadata built for another group size is refused before launch
    meta = thd.build_metadata(seqlens=b.lengths, cp=2, rank=0, block_t=128, block_n=64, device=0)
    with pytest.raises(thd.ThdError) as err:
        thd.attn_fwd(q=q[:, :8].contiguous(), k=k[:, :1].contiguous(), v=v[:, :1].contiguous(),
                     seqlens=b.lengths, cp=2, rank=0, meta=meta)
    assert err.value.status == "THD_EMISMATCH"
    with pytest.raises(thd.ThdError):
        thd.attn_fwd(q=q, k=k[:-2], v=v[:-2], seqlens=b.lengths, cp=2, rank=0)


def test_binding_refuses_mismatched_tensors_before_launch():
    """Every tensor is checked (dtype, device, contiguity, exact shape) before
    the library is called: the kernels size their loads and stores from the
    head counts and dims, so a wrong tensor must fail as ThdError, not as a
    device fault."""
    b = workloads.small_case(41, [64, 128], 2, 8, 2, 128, 128, backward=True, rank=1)
    dev = device()
    q, k, v, do = (t.to(dev) for t in (b.q, b.k, b.v, b.do))
    kw = dict(seqlens=b.lengths, cp=2, rank=1)
    t_loc, hq, dv = q.shape[0], q.shape[1], v.shape[2]
    bad_fwd = [
        dict(v=v[:, :1].contiguous()),                                 # Hkv of v != Hkv of k
        dict(k=k[:, :, :64].contiguous()),                             # d_qk of k != d_qk of q
        dict(v=v[:-2]),                                                # too few K/V rows
        dict(q=q.transpose(0, 1)),                                     # not contiguous
        dict(k=k.float()),                                             # wrong dtype
        dict(out=torch.empty((t_loc, hq, dv - 8), dtype=torch.bfloat16, device=dev)),
        dict(out=torch.empty((t_loc, hq, dv), dtype=torch.float32, device=dev)),
        dict(lse=torch.empty((t_loc, hq), dtype=torch.float32)),       # host tensor
        dict(lse=torch.empty((t_loc, hq + 1), dtype=torch.float32, device=dev)),
        dict(out_f32=torch.empty((t_loc, hq, dv), dtype=torch.bfloat16, device=dev)),
    ]
    for change in bad_fwd:
        args = dict(q=q, k=k, v=v)
        args.update(change)
        with pytest.raises(thd.ThdError):
            thd.attn_fwd(**args, **kw)
    o, lse = thd.attn_fwd(q=q, k=k, v=v, **kw)
    bad_bwd = [
        dict(v=v[:-2]),
        dict(v=v[:, :1].contiguous()),
        dict(lse=lse.cpu()),
        dict(lse=lse[:-1]),
        dict(d_o=do[:, :, :64].contiguous()),
        dict(d_o=do.float()),
        dict(o_f32=torch.empty((t_loc, hq, dv), dtype=torch.bfloat16, device=dev)),
        dict(workspace=torch.empty(16, dtype=torch.uint8, device=dev)),   # too small
        dict(workspace=torch.empty(1 << 20, dtype=torch.uint8)),          # host tensor
    ]
    for change in bad_bwd:
        args = dict(q=q, k=k, v=v, lse=lse, d_o=do)
        args.update(change)
        with pytest.raises(thd.ThdError):
            thd.attn_bwd(**args, **kw)
    torch.cuda.synchronize()
