"""Seeded synthetic inputs for packed-sequence causal attention.

This module is shared by the tests, the benchmark and the oracle's callers.
It holds no part of the attention method: it only draws packed document
lengths and bf16 tensors of the shapes one context-parallel rank consumes.

Workloads (the pages print no dataset; these stand in for the packed batches
the subject page, Ascend/MindSpeed "kvallgather cp thd load balance", trains
on):

  tiny      T=1024, lengths [256,512,256], cp=2, rank 0, MHA 8 heads x 64
  gqa_mid   T=16384, lognormal lengths (mean 2048) in multiples of 8, cp=4,
            rank 1, 32 q / 8 kv heads x 128
  mla       T=32768, lengths uniform in [1024,8192] in multiples of 16, cp=8,
            rank 3, 16 heads, qk 192 / v 128 (expanded MLA)
  short     T=65536, lengths uniform in [16,512] in multiples of 16, cp=8,
            rank 0, 64 q / 8 kv heads x 128
  fwdbwd    T=32768, gqa_mid's heads, dims and length law, cp=4, rank 2,
            forward and backward

Recipe (seed = workload index): numpy ``default_rng(seed)``; lengths are drawn
first, one at a time, until their sum reaches T, and the last one is cut to the
remainder. Lognormal lengths use sigma=1 and mu = ln(2048) - 1/2 (mean 2048),
rounded to the nearest multiple of 2*cp, at least 2*cp. Uniform lengths are
uniform over {a, a+16, ..., b}. Then Q_local, K, V (and dO) are drawn as
float32 standard normals in their consumed layouts and rounded to bf16 (round
to nearest even): Q_local [T/cp, Hq, dqk], K [T, Hkv, dqk] and V [T, Hkv, dv]
(already gathered, rank-major), dO [T/cp, Hq, dv].
"""
from __future__ import annotations

import dataclasses
import hashlib
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    total: int          # T, packed tokens over all ranks
    cp: int
    rank: int
    hq: int
    hkv: int
    d_qk: int
    d_v: int
    law: str            # "fixed" | "lognormal" | "uniform"
    lo: int = 0
    hi: int = 0
    fixed: tuple = ()
    backward: bool = False

    @property
    def t_local(self) -> int:
        return self.total // self.cp


WORKLOADS = [
    Workload("tiny", 0, 1024, 2, 0, 8, 8, 64, 64, "fixed", fixed=(256, 512, 256)),
    Workload("gqa_mid", 1, 16384, 4, 1, 32, 8, 128, 128, "lognormal"),
    Workload("mla", 2, 32768, 8, 3, 16, 16, 192, 128, "uniform", lo=1024, hi=8192),
    Workload("short", 3, 65536, 8, 0, 64, 8, 128, 128, "uniform", lo=16, hi=512),
    Workload("fwdbwd", 4, 32768, 4, 2, 32, 8, 128, 128, "lognormal", backward=True),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def draw_lengths(w: Workload, rng: np.random.Generator) -> np.ndarray:
    """Packed document lengths for workload ``w`` (int32, summing to T)."""
    if w.law == "fixed":
        return np.asarray(w.fixed, dtype=np.int32)
    step = 2 * w.cp if w.law == "lognormal" else 16
    out = []
    total = 0
    mu = math.log(2048.0) - 0.5
    while total < w.total:
        if w.law == "lognormal":
            x = rng.lognormal(mean=mu, sigma=1.0)
            length = max(step, int(round(x / step)) * step)
        else:
            length = int(rng.integers(w.lo // 16, w.hi // 16 + 1)) * 16
        length = min(length, w.total - total)
        out.append(length)
        total += length
    return np.asarray(out, dtype=np.int32)


def lengths_digest(lengths: np.ndarray) -> str:
    """First 16 hex digits of sha256 over the int32 little-endian lengths."""
    return hashlib.sha256(np.asarray(lengths, dtype="<i4").tobytes()).hexdigest()[:16]


def random_lengths(rng: np.random.Generator, n: int, cp: int, max_chunk: int) -> np.ndarray:
    """n lengths, each 2*cp times a uniform integer in [1, max_chunk]."""
    return (rng.integers(1, max_chunk + 1, size=n) * 2 * cp).astype(np.int32)


def bf16_normal(rng: np.random.Generator, shape, device="cpu"):
    """float32 standard normal rounded to bf16 (round to nearest even)."""
    import torch

    x = rng.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).to(device)


def device_normal(seed: int, shape, device):
    """bf16 standard normal drawn on the device by torch's generator seeded with
    ``seed``: for batches too large to draw on the host."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.randn(shape, generator=gen, device=device, dtype=torch.bfloat16)


@dataclasses.dataclass
class Batch:
    workload: Workload
    lengths: np.ndarray
    q: object           # torch bf16 [T/cp, Hq, dqk]
    k: object           # torch bf16 [T, Hkv, dqk], gathered, rank-major
    v: object           # torch bf16 [T, Hkv, dv], gathered, rank-major
    do: object = None   # torch bf16 [T/cp, Hq, dv]


def make_batch(w: Workload, device="cpu", lengths=None, seed=None) -> Batch:
    """Draw one batch of ``w`` (seed defaults to the workload index)."""
    rng = np.random.default_rng(w.index if seed is None else seed)
    drawn = draw_lengths(w, rng)
    if lengths is None:
        lengths = drawn
    lengths = np.asarray(lengths, dtype=np.int32)
    total = int(lengths.sum())
    tl = total // w.cp
    q = bf16_normal(rng, (tl, w.hq, w.d_qk), device)
    k = bf16_normal(rng, (total, w.hkv, w.d_qk), device)
    v = bf16_normal(rng, (total, w.hkv, w.d_v), device)
    do = bf16_normal(rng, (tl, w.hq, w.d_v), device) if w.backward else None
    return Batch(w, lengths, q, k, v, do)


def small_case(seed: int, lengths, cp: int, hq: int, hkv: int, d_qk: int, d_v: int,
               backward: bool = False, device="cpu", rank: int = 0) -> Batch:
    """A batch of arbitrary small shape for parity and edge-case tests."""
    lengths = np.asarray(lengths, dtype=np.int32)
    w = Workload(f"case{seed}", seed, int(lengths.sum()), cp, rank, hq, hkv, d_qk, d_v,
                 "fixed", fixed=tuple(int(x) for x in lengths), backward=backward)
    return make_batch(w, device=device, lengths=lengths, seed=seed)
