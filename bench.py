"""Benchmark: useful-FLOP throughput of causal + EOD-reset THD attention for
one context-parallel rank on one MI355X.

A step is one pass of the whole path over one synthetic packed batch that is
already resident in HBM: metadata lookup (cached after the first step, as the
planner's cache is meant to be used), then the forward (the main kernel, plus
the combine pass when the plan splits key ranges; for the fwdbwd workload also
the backward kernels, with the forward writing its fp32 O for the backward's
D, as a training step would). Useful FLOPs count only unmasked (query, key)
pairs: pairs x Hq x 2 (dqk + dv) forward, pairs x Hq x (6 dqk + 4 dv)
backward.

The headline is the GQA-mid workload (T 16384, cp 4, rank 1, 32 q / 8 kv
heads, d 128). The expanded-MLA and many-short-documents workloads, the two
other forward targets, are measured the same way and reported as sub-records
under "workloads" of the same JSON line.

Per workload, in this order:
  parity gate   every element of O and LSE against the fp64 oracle (no number
                is reported for a path that disagrees), for the plain plan and
                for the packed one;
  settle        the step repeated, untimed, until the GPU has run it for
                about 150 ms: the shader clock ramps up over the first tens of
                ms of sustained load, and every measurement below is taken at
                the steady clock a training loop runs at;
  side timings  the forward with cold caches (512 MiB written between
                launches), for every rank of the configuration, as shard
                passes, and with the packed plan;
  warm-up       W untimed steps;
  timed region  exactly K steps, between a synchronize and a synchronize, with
                HIP events recorded on the launch stream at both ends: the
                events give the GPU time of the same K launches, so the
                kernel time behind `roofline` can never exceed ms_per_step.

Fields besides the contract's:
  roofline      the forward's achieved TFLOP/s (useful FLOPs per launch over
                its event-timed duration in the timed region) against the
                dense bf16 MFMA peak, or its algorithmic bytes per second
                against 8 TB/s when the workload's intensity is below the
                ridge; `traffic` = HBM bytes per launch from rocprofv3 counters
                while the committed counter summary matches the current
                kernel source;
  timing        cold-cache median and minimum, and the median for every rank
                with their max/min ratio;
  metadata      cold build (plan plus upload) and warm lookup times;
  ag_overlap    the forward as one pass per source rank's shard (all-gather
                overlap) against the one-pass time;
  packing       the forward with a packed plan (short-segment packing; same
                parity gate) against the plain plan, timed back to back;
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
HEADLINE = "gqa_mid"
SUB_WORKLOADS = ("mla", "short")
SETTLE_MS = 150.0


def _kernel_sha() -> str:
    with open(FWD_SOURCE, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def _traffic(workload: str, block_n: int):
    """HBM bytes per forward launch from the committed counter summary, if it
    was taken on the current kernel source and on the KV tile size this run
    uses; else None."""
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
    if fields.get("kernel_block_n") != str(block_n):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_baseline(w, batch, budget_s: float):
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
                      f"x{reps} in {elapsed:.1f} s, numpy fp64 on {_cpu_model()}"}


def _oracle(w, batch):
    from oracle import attention

    return attention.attn_fwd64(batch.q.double().numpy(), batch.k.double().numpy(),
                                batch.v.double().numpy(), batch.lengths, w.cp, w.rank)


def _parity(want, o, lse):
    """Every element of O and LSE against the fp64 oracle's (want_o, want_lse)."""
    import numpy as np

    want_o, want_lse = want
    err = np.abs(o.double().cpu().numpy() - want_o)
    lerr = np.abs(lse.double().cpu().numpy() - want_lse)
    res = {"elements": int(err.size), "o_max_abs": float(f"{err.max():.4g}"),
           "o_mean_abs": float(f"{err.mean():.4g}"), "lse_max_abs": float(f"{lerr.max():.4g}")}
    res["ok"] = bool(np.all(np.isfinite(err)) and err.max() <= 2e-2 and err.mean() <= 2e-3
                     and lerr.max() <= 1e-3)
    return res


def measure(w, args, dev, cpu_budget_s: float):
    """One workload's record (see the module docstring), or raises SystemExit
    when its parity gate fails."""
    import numpy as np
    import torch

    import packed_sequence_causal_amd as thd
    import workloads
    from oracle import metadata as ometa

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
    stream = torch.cuda.current_stream(dev)

    def fwd_meta(rank=w.rank):
        return thd.device_metadata(seqlens=batch.lengths, cp=w.cp, rank=rank, hq=w.hq,
                                   hkv=w.hkv, d_qk=w.d_qk, d_v=w.d_v, device=dev.index,
                                   forward=True)

    # Metadata: cold build (planner plus one upload) and warm lookup.
    thd.cache_clear()
    t0 = time.perf_counter()
    fwd_meta()
    build_ms = (time.perf_counter() - t0) * 1e3
    t0 = time.perf_counter()
    for _ in range(100):
        fwd_meta()
    lookup_us = (time.perf_counter() - t0) * 1e4

    def step():
        # The forward's tile sizes depend on the batch (32-key tiles for short
        # documents); the backward's are fixed per head shape.
        meta = fwd_meta()
        thd.attn_fwd(q=q, k=k, v=v, seqlens=batch.lengths, cp=w.cp, rank=w.rank, out=o, lse=lse,
                     out_f32=o32, meta=meta, stream=stream)
        if w.backward:
            meta_b = thd.device_metadata(seqlens=batch.lengths, cp=w.cp, rank=w.rank, hq=w.hq,
                                         hkv=w.hkv, d_qk=w.d_qk, d_v=w.d_v, device=dev.index)
            thd.attn_bwd(q=q, k=k, v=v, lse=lse, d_o=do, seqlens=batch.lengths, cp=w.cp,
                         rank=w.rank, o_f32=o32, meta=meta_b, stream=stream)

    def fwd_only(meta, rank=w.rank):
        thd.attn_fwd(q=q, k=k, v=v, seqlens=batch.lengths, cp=w.cp, rank=rank, out=o, lse=lse,
                     out_f32=o32, meta=meta, stream=stream)

    # Parity gate: no throughput is reported for a path that disagrees with the oracle.
    step()
    torch.cuda.synchronize()
    parity = {"skipped": True}
    want = None
    if not args.no_check:
        want = _oracle(w, batch)
        parity = _parity(want, o, lse)
        if not parity["ok"]:
            print(f"parity gate failed on {w.name}: {parity}", file=sys.stderr)
            raise SystemExit(1)

    # Short-segment packing: the same forward with a packed plan (the partial
    # query tiles of several documents share a tile), held to the same parity
    # gate (here) and timed against the plain plan (below).
    packing = None
    pmeta = None
    if not w.backward:
        pmeta = thd.device_metadata(seqlens=batch.lengths, cp=w.cp, rank=w.rank, hq=w.hq,
                                    hkv=w.hkv, d_qk=w.d_qk, d_v=w.d_v, device=dev.index,
                                    forward=True, packed=True)
        pinfo = pmeta.info()
        fwd_only(pmeta)
        torch.cuda.synchronize()
        p_parity = {"skipped": True}
        if want is not None:
            p_parity = _parity(want, o, lse)
            if not p_parity["ok"]:
                print(f"parity gate failed on {w.name} (packed plan): {p_parity}", file=sys.stderr)
                raise SystemExit(1)
    # Settle the clock: repeat the step until ~SETTLE_MS of GPU time has run.
    settled = 0.0
    while settled < SETTLE_MS:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(50):
            step()
        e1.record(stream)
        e1.synchronize()
        settled += e0.elapsed_time(e1)

    meta = fwd_meta()
    # Cold caches: a 512 MiB write (larger than L2 plus the 256 MB MALL)
    # before each launch, on the same stream; median and minimum reported.
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(10):
        scratch.fill_(i & 0xFF)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        fwd_only(meta)
        s1.record(stream)
        s1.synchronize()
        cold.append(s0.elapsed_time(s1))
    del scratch

    # Every rank of the configuration on this GPU (same tensors, that rank's
    # metadata): equal useful work per rank should give near-equal times, the
    # one-GPU view of the partition's load balance.
    per_rank = []
    for r in range(w.cp):
        meta_r = fwd_meta(r)
        for _ in range(20):
            fwd_only(meta_r, r)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for _ in range(20):
            fwd_only(meta_r, r)
        s1.record(stream)
        s1.synchronize()
        per_rank.append(s0.elapsed_time(s1) / 20)

    def timed(fn, n=20):
        for _ in range(3):
            fn()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(n):
            fn()
        a1.record(stream)
        a1.synchronize()
        return a0.elapsed_time(a1) / n

    # All-gather overlap: the same forward as cp passes, one per source rank's
    # shard, local shard first (K/V resident): what splitting the forward into
    # shard passes costs against the one-pass time, and the share of the work
    # the local shard's pass does before any remote shard is needed.
    ag = None
    if not w.backward:
        bt = thd.preferred_tiles(hq=w.hq, hkv=w.hkv, d_qk=w.d_qk, d_v=w.d_v)[0]
        order = [w.rank] + [s_ for s_ in range(w.cp) if s_ != w.rank]
        metas = [thd.build_pass_metadata(seqlens=batch.lengths, cp=w.cp, rank=w.rank, block_t=bt,
                                         block_n=64, shards=[s_], device=dev.index)
                 for s_ in order]
        state = thd.pass_state(meta=metas[0], hq=w.hq, hkv=w.hkv, d_v=w.d_v, device=dev)

        def passes(upto=None):
            ms = metas if upto is None else metas[:upto]
            for i, m in enumerate(ms):
                thd.attn_fwd_pass(q=q, k=k, v=v, meta=m, state=state, first=i == 0,
                                  last=i == len(metas) - 1, out=o, lse=lse, stream=stream)

        all_ms = timed(passes)
        local_ms = timed(lambda: passes(1))
        ag = {"passes": w.cp, "all_passes_ms": round(all_ms, 5), "local_pass_ms": round(local_ms, 5)}

    info = meta.info()
    if pmeta is not None:
        # The two plans alternate, so both see the same clock.
        rounds = {"plain": [], "packed": []}
        for _ in range(3):
            rounds["plain"].append(timed(lambda: fwd_only(meta), n=max(args.steps, 20)))
            rounds["packed"].append(timed(lambda: fwd_only(pmeta), n=max(args.steps, 20)))
        plain_ms = float(np.median(rounds["plain"]))
        packed_ms = float(np.median(rounds["packed"]))
        packing = {"tiles": int(info["n_tiles"]), "packed_plan_tiles": int(pinfo["n_tiles"]),
                   "packed_tiles": int(pinfo["n_packed_tiles"]), "plain_ms": round(plain_ms, 5),
                   "packed_ms": round(packed_ms, 5), "ratio": round(packed_ms / plain_ms, 4),
                   "parity": p_parity}

    # Timed region last, so that the last K launches of the forward kernel in
    # a profiler's trace are exactly the ones timed here.
    for _ in range(args.warmup):
        step()
    # Timed region: exactly K steps; the events on the launch stream bracket
    # the same K steps the wall clock does.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    gpu_ms = ev0.elapsed_time(ev1) / args.steps
    value = (fwd_flops + bwd_flops) * args.steps / elapsed / 1e12

    # The forward's share of the timed region: the whole step for the forward
    # workloads; for the training workload it is timed the same way on its own.
    if w.backward:
        for _ in range(args.warmup):
            fwd_only(meta)
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record(stream)
        for _ in range(args.steps):
            fwd_only(meta)
        f1.record(stream)
        torch.cuda.synchronize()
        kern_ms = f0.elapsed_time(f1) / args.steps
    else:
        kern_ms = gpu_ms
    if ag is not None:
        ag.update({"one_pass_ms": round(kern_ms, 5), "overhead": round(ag["all_passes_ms"] / kern_ms, 4)})

    # Algorithmic bytes per launch: Q once, every K/V row some local query sees
    # once (keys of document i up to the end of chunk 2cp-1-r), O (bf16, plus
    # the fp32 copy the training forward writes for the backward) and LSE once.
    seen_keys = sum((2 * w.cp - w.rank) * (int(L) // (2 * w.cp)) for L in batch.lengths)
    o_bytes = (2 + (4 if w.backward else 0)) * w.t_local * w.hq * w.d_v
    alg_bytes = (2 * w.t_local * w.hq * w.d_qk + 2 * w.hkv * (w.d_qk + w.d_v) * seen_keys
                 + o_bytes + 4 * w.t_local * w.hq)
    intensity = fwd_flops / alg_bytes
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if intensity >= ridge:
        roof = {"bound": "mfma", "achieved": round(fwd_flops / (kern_ms * 1e-3) / 1e12, 3),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(alg_bytes / (kern_ms * 1e-3) / 1e9, 3),
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    kernels = "thd_fwd_kernel" + (" + thd_fwd_combine_kernel" if info["n_splits"] > 0 else "")
    roof.update({"traffic": _traffic(w.name, int(info["block_n"])), "kernel": kernels, "kernel_ms": round(kern_ms, 5),
                 "algorithmic_bytes": int(alg_bytes), "useful_flops": int(fwd_flops),
                 "intensity_flop_per_byte": round(intensity, 1),
                 "mfma_frac": round(fwd_flops / (kern_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)})
    rec = {
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "ms_per_step": round(ms_per_step, 5),
        "gpu_ms_per_step": round(gpu_ms, 5),
        "config": {"workload": w.name, "T": w.total, "cp": w.cp, "rank": w.rank, "hq": w.hq,
                   "hkv": w.hkv, "d_qk": w.d_qk, "d_v": w.d_v, "n_docs": int(len(batch.lengths)),
                   "lengths_sha16": workloads.lengths_digest(batch.lengths),
                   "useful_pairs": int(pairs), "backward": bool(w.backward),
                   "fwd_block_t": int(info["block_t"]), "fwd_block_n": int(info["block_n"]),
                   "fwd_items": int(info["n_items"]), "fwd_split_tiles": int(info["n_splits"])},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": roof,
        "timing": {"fwd_ms_median_cold": round(float(np.median(cold)), 5),
                   "fwd_ms_min_cold": round(float(np.min(cold)), 5),
                   "fwd_ms_per_rank": [round(t, 5) for t in per_rank],
                   "rank_spread": round(max(per_rank) / min(per_rank), 4),
                   "settle_ms": round(settled, 1)},
        "metadata": {"build_ms_cold": round(build_ms, 3), "lookup_us_warm": round(lookup_us, 2)},
        "parity": parity,
    }
    if ag is not None:
        rec["ag_overlap"] = ag
    if packing is not None:
        rec["packing"] = packing
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = _cpu_baseline(w, batch, cpu_budget_s)
    return rec


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE,
                    help="headline workload; with the default, mla and short are added as "
                         "sub-records")
    ap.add_argument("--only", action="store_true", help="measure the headline workload only")
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

    import workloads

    dev = torch.device("cuda", 0)
    head = measure(workloads.BY_NAME[args.workload], args, dev, cpu_budget_s=10.0)
    subs = {}
    if args.workload == HEADLINE and not args.only:
        for name in SUB_WORKLOADS:
            subs[name] = measure(workloads.BY_NAME[name], args, dev, cpu_budget_s=5.0)
    result = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
    }
    for key in ("config", "pct_of_bf16_peak", "roofline", "gpu_ms_per_step", "timing", "metadata",
                "parity", "ag_overlap", "packing", "cpu_baseline"):
        if key in head:
            result[key] = head[key]
    result["host"] = {"cpu_model": _cpu_model(), "cpus": len(os.sched_getaffinity(0))}
    if subs:
        result["workloads"] = subs
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
