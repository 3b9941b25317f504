"""Benchmark: useful-FLOP throughput of causal + EOD-reset THD attention for
one context-parallel rank on one MI355X.

A step is one pass of the whole path over one synthetic packed batch that is
already resident in HBM: metadata lookup (cached after the first step, as the
planner's cache is meant to be used), then the forward kernel (and, for the
fwdbwd workload, the backward kernels, with the forward also writing its fp32
O for the backward's D, as a training step would). Useful FLOPs count only unmasked
(query, key) pairs: pairs x Hq x 2 (dqk + dv) forward, pairs x Hq x
(6 dqk + 4 dv) backward.

Prints one JSON line. Besides the contract fields it carries
  roofline      the forward kernel's achieved TFLOP/s (useful FLOPs per launch
                over its mean duration, timed with HIP events on the launch
                stream) against the dense bf16 MFMA peak, and the HBM traffic
                per launch measured with rocprofv3 counters when the committed
                counter summary matches the current kernel source;
  timing        the forward kernel's median and minimum launch time with warm
                caches and with cold caches (512 MiB written between launches),
                and its median time for every rank of the configuration (same
                tensors, that rank's metadata) with their max/min ratio;
  cpu_baseline  the fp64 oracle timed on this host's cores on the same
                workload (reported, not a target).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
FWD_SOURCE = os.path.join(ROOT, "packed_sequence_causal_amd", "csrc", "thd_fwd.hip")
METRIC = "masked-attention fwd TFLOP/s (useful FLOPs) on 1 MI355X; % of bf16 MFMA peak"


def _kernel_sha() -> str:
    with open(FWD_SOURCE, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def _traffic(workload: str):
    """HBM bytes per forward launch from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"thd_fwd_kernel_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.startswith("- "):
                key, val = line[2:].split(":", 1)
                fields[key.strip()] = val.strip().strip("`")
    if fields.get("kernel_source_sha256") != _kernel_sha():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _cpu_baseline(w, batch, budget_s: float = 10.0):
    """Time the fp64 oracle on the same workload (repeated until budget_s)."""
    from threadpoolctl import threadpool_info

    from oracle import attention, metadata

    q = batch.q.double().numpy()
    k = batch.k.double().numpy()
    v = batch.v.double().numpy()
    flops = metadata.useful_pairs_closed_form(batch.lengths, w.cp) * w.hq * 2 * (w.d_qk + w.d_v)
    reps = 0
    t0 = time.perf_counter()
    while True:
        attention.attn_fwd64(q, k, v, batch.lengths, w.cp, w.rank)
        reps += 1
        elapsed = time.perf_counter() - t0
        if elapsed >= budget_s or elapsed * (reps + 1) / reps > 3 * budget_s:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": round(flops * reps / elapsed / 1e12, 6), "unit": "TFLOP/s",
            "cores": int(threads), "kind": "oracle",
            "sample": f"full {w.name} forward (all {w.hq} q heads, {w.t_local} rows) "
                      f"x{reps} in {elapsed:.1f} s, numpy fp64"}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # The GPU's clock ramps up over the first ~20-40 ms of sustained work (the
    # forward runs ~15% slower during the first ~200 launches), so the default
    # warm-up is long enough for every workload to reach its steady state.
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="gqa_mid")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true",
                    help="skip the parity gate (used only for profiler passes)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel(), "launches": 3}))
        return 0

    import packed_sequence_causal_amd as thd
    import workloads
    from oracle import metadata as ometa

    w = workloads.BY_NAME[args.workload]
    dev = torch.device("cuda", 0)
    batch = workloads.make_batch(w)
    q, k, v = batch.q.to(dev), batch.k.to(dev), batch.v.to(dev)
    do = batch.do.to(dev) if batch.do is not None else None
    pairs = ometa.useful_pairs_closed_form(batch.lengths, w.cp)
    fwd_flops = pairs * w.hq * 2 * (w.d_qk + w.d_v)
    bwd_flops = pairs * w.hq * (6 * w.d_qk + 4 * w.d_v) if w.backward else 0
    o = torch.empty((w.t_local, w.hq, w.d_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.t_local, w.hq), dtype=torch.float32, device=dev)

    # Training step (fwdbwd): the forward also writes its fp32 O, from which
    # the backward takes D (the path a training loop would use).
    o32 = (torch.empty((w.t_local, w.hq, w.d_v), dtype=torch.float32, device=dev)
           if w.backward else None)

    def step():
        # The forward's tile sizes depend on the batch (32-key tiles for short
        # documents); the backward's are fixed per head shape.
        meta = thd.device_metadata(seqlens=batch.lengths, cp=w.cp, rank=w.rank, hq=w.hq,
                                   hkv=w.hkv, d_qk=w.d_qk, d_v=w.d_v, device=0, forward=True)
        thd.attn_fwd(q=q, k=k, v=v, seqlens=batch.lengths, cp=w.cp, rank=w.rank, out=o, lse=lse,
                     out_f32=o32, meta=meta)
        if w.backward:
            meta_b = thd.device_metadata(seqlens=batch.lengths, cp=w.cp, rank=w.rank, hq=w.hq,
                                         hkv=w.hkv, d_qk=w.d_qk, d_v=w.d_v, device=0)
            thd.attn_bwd(q=q, k=k, v=v, lse=lse, d_o=do, seqlens=batch.lengths, cp=w.cp,
                         rank=w.rank, o_f32=o32, meta=meta_b)

    # Parity gate: no throughput is reported for a path that disagrees with the oracle.
    step()
    torch.cuda.synchronize()
    if not args.no_check:
        from oracle import attention
        rows = np.unique(np.linspace(0, w.t_local - 1, 24).astype(np.int64))
        want, _ = attention.attn_fwd64_rows(batch.q.float().numpy(), batch.k.float().numpy(),
                                           batch.v.float().numpy(), batch.lengths, w.cp, w.rank,
                                           rows)
        got = o[torch.from_numpy(rows).to(dev)].double().cpu().numpy()
        err = np.abs(got - want)
        if not (err.max() <= 2e-2 and err.mean() <= 2e-3):
            print(f"parity gate failed: max-abs {err.max():.3g}", file=sys.stderr)
            return 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = (fwd_flops + bwd_flops) * args.steps / elapsed / 1e12

    # Forward kernel duration: HIP events around each launch on the launch stream
    # (for the training workload, the forward the step runs: it also writes the
    # fp32 O the backward takes D from).
    stream = torch.cuda.current_stream(dev)
    meta = thd.device_metadata(seqlens=batch.lengths, cp=w.cp, rank=w.rank, hq=w.hq, hkv=w.hkv,
                               d_qk=w.d_qk, d_v=w.d_v, device=0, forward=True)
    n_ev = max(10, min(args.steps, 100))
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    for i in range(n_ev):
        starts[i].record(stream)
        thd.attn_fwd(q=q, k=k, v=v, seqlens=batch.lengths, cp=w.cp, rank=w.rank, out=o, lse=lse,
                     out_f32=o32, meta=meta, stream=stream)
        ends[i].record(stream)
    torch.cuda.synchronize()
    warm = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    kern_ms = float(np.mean(warm))

    # Cold caches: a 512 MiB write (larger than L2 plus the 256 MB MALL)
    # before each launch, on the same stream; median and minimum reported.
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(10):
        scratch.fill_(i & 0xFF)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        thd.attn_fwd(q=q, k=k, v=v, seqlens=batch.lengths, cp=w.cp, rank=w.rank, out=o, lse=lse,
                     out_f32=o32, meta=meta, stream=stream)
        s1.record(stream)
        s1.synchronize()
        cold.append(s0.elapsed_time(s1))
    del scratch

    # Every rank of the configuration on this GPU (same tensors, that rank's
    # metadata): equal useful work per rank should give near-equal times, the
    # one-GPU view of the partition's load balance.
    per_rank = []
    for r in range(w.cp):
        meta_r = thd.device_metadata(seqlens=batch.lengths, cp=w.cp, rank=r, hq=w.hq, hkv=w.hkv,
                                     d_qk=w.d_qk, d_v=w.d_v, device=0, forward=True)
        for _ in range(3):
            thd.attn_fwd(q=q, k=k, v=v, seqlens=batch.lengths, cp=w.cp, rank=r, out=o, lse=lse,
                         out_f32=o32, meta=meta_r, stream=stream)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(10)]
        for s0, s1 in evs:
            s0.record(stream)
            thd.attn_fwd(q=q, k=k, v=v, seqlens=batch.lengths, cp=w.cp, rank=r, out=o, lse=lse,
                         out_f32=o32, meta=meta_r, stream=stream)
            s1.record(stream)
        torch.cuda.synchronize()
        per_rank.append(float(np.median([s0.elapsed_time(s1) for s0, s1 in evs])))
    # Algorithmic bytes per launch: Q once, every K/V row some local query sees
    # once (keys of document i up to the end of chunk 2cp-1-r), O and LSE once.
    seen_keys = sum((2 * w.cp - w.rank) * (int(L) // (2 * w.cp)) for L in batch.lengths)
    # Q, every visible K/V row once, O (bf16, plus the fp32 copy the training
    # forward writes for the backward), LSE.
    o_bytes = (2 + (4 if w.backward else 0)) * w.t_local * w.hq * w.d_v
    alg_bytes = (2 * w.t_local * w.hq * w.d_qk + 2 * w.hkv * (w.d_qk + w.d_v) * seen_keys
                 + o_bytes + 4 * w.t_local * w.hq)
    intensity = fwd_flops / alg_bytes
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    traffic = _traffic(w.name)
    if intensity >= ridge:
        roof = {"bound": "mfma", "achieved": round(fwd_flops / (kern_ms * 1e-3) / 1e12, 3),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(alg_bytes / (kern_ms * 1e-3) / 1e9, 3),
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof.update({"traffic": traffic, "kernel": "thd_fwd_kernel", "kernel_ms": round(kern_ms, 5),
                 "algorithmic_bytes": int(alg_bytes), "useful_flops": int(fwd_flops),
                 "intensity_flop_per_byte": round(intensity, 1),
                 "mfma_frac": round(fwd_flops / (kern_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)})
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.total, "cp": w.cp, "rank": w.rank, "hq": w.hq,
                   "hkv": w.hkv, "d_qk": w.d_qk, "d_v": w.d_v, "n_docs": int(len(batch.lengths)),
                   "lengths_sha16": workloads.lengths_digest(batch.lengths),
                   "useful_pairs": int(pairs), "backward": bool(w.backward),
                   "fwd_block_t": int(meta.info()["block_t"]),
                   "fwd_block_n": int(meta.info()["block_n"])},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": roof,
        "timing": {"fwd_kernel_ms_median_warm": round(float(np.median(warm)), 5),
                   "fwd_kernel_ms_min_warm": round(float(np.min(warm)), 5),
                   "fwd_kernel_ms_median_cold": round(float(np.median(cold)), 5),
                   "fwd_kernel_ms_min_cold": round(float(np.min(cold)), 5),
                   "fwd_kernel_ms_per_rank": [round(t, 5) for t in per_rank],
                   "rank_spread": round(max(per_rank) / min(per_rank), 4)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = _cpu_baseline(w, batch)
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
