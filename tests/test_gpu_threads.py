"""Concurrent callers on an MI355X: the C ABI is thread-safe.

Eight host threads, each on its own HIP stream, run forward and backward over
their own batches at once, with the metadata cache cleared first so that
concurrent misses build and upload entries (some threads share lengths, so
they also race for the same entry). Every result must equal, bit for bit, the
same call made alone on the default stream (the kernels are deterministic),
and each thread's refused call must report its own message (the last-error
text is per thread).
"""
import threading

import pytest
import torch

import workloads
from parity import device

pytestmark = pytest.mark.gpu

thd = pytest.importorskip("packed_sequence_causal_amd")

CASES = [
    # (seed, lengths, cp, rank, hq, hkv, dqk, dv); pairs share their lengths
    (9401, [256, 512, 256], 2, 0, 8, 8, 64, 64),
    (9402, [256, 512, 256], 2, 1, 8, 8, 64, 64),
    (9403, [1000, 72, 600], 4, 2, 32, 8, 128, 128),
    (9404, [1000, 72, 600], 4, 2, 32, 8, 128, 128),
    (9405, [16, 32, 1040, 16, 400], 8, 3, 16, 16, 192, 128),
    (9406, [48, 2048, 96], 4, 1, 16, 4, 128, 128),
    (9407, [36, 300, 84], 3, 2, 12, 4, 128, 128),
    (9408, [8, 24, 40, 136, 520], 4, 1, 32, 8, 128, 128),
]
REPEATS = 3


def _inputs(case, dev):
    seed, lengths, cp, rank, hq, hkv, dqk, dv = case
    b = workloads.small_case(seed, lengths, cp, hq, hkv, dqk, dv, backward=True, rank=rank)
    return [t.to(dev) for t in (b.q, b.k, b.v, b.do)], b.lengths


def _run(case, tensors, lengths):
    seed, _, cp, rank, hq, hkv, dqk, dv = case
    q, k, v, do = tensors
    o32 = torch.empty((q.shape[0], hq, dv), dtype=torch.float32, device=q.device)
    o, lse = thd.attn_fwd(q=q, k=k, v=v, seqlens=lengths, cp=cp, rank=rank, out_f32=o32)
    grads = thd.attn_bwd(q=q, k=k, v=v, lse=lse, d_o=do, seqlens=lengths, cp=cp, rank=rank,
                         o_f32=o32)
    return (o, lse, o32) + tuple(grads)


def test_concurrent_callers_match_single_calls():
    dev = device()
    inputs = [_inputs(c, dev) for c in CASES]
    print("[threads] reference runs, one at a time", flush=True)
    want = [_run(c, t, l) for c, (t, l) in zip(CASES, inputs)]
    torch.cuda.synchronize()
    thd.cache_clear()

    results = [None] * len(CASES)
    errors = [None] * len(CASES)
    failures = []
    barrier = threading.Barrier(len(CASES), timeout=60)

    def worker(i):
        try:
            stream = torch.cuda.Stream(device=dev)
            tensors, lengths = inputs[i]
            barrier.wait()
            with torch.cuda.stream(stream):
                for tensor in tensors:
                    tensor.record_stream(stream)
                outs = [_run(CASES[i], tensors, lengths) for _ in range(REPEATS)]
                # a refused call: the message names this thread's own rank
                try:
                    thd.build_metadata(seqlens=[64], cp=2, rank=100 + i, block_t=32, block_n=64)
                except thd.ThdError as e:
                    errors[i] = str(e)
            stream.synchronize()
            results[i] = outs
        except Exception as e:          # reported below, from the main thread
            failures.append((i, repr(e)))

    print(f"[threads] {len(CASES)} threads x {REPEATS} forward+backward calls", flush=True)
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(CASES))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not failures, failures
    names = ("O", "LSE", "O32", "dQ", "dK", "dV")
    for i, outs in enumerate(results):
        for rep, got in enumerate(outs):
            for name, g, w in zip(names, got, want[i]):
                assert torch.equal(g, w), (CASES[i][0], rep, name)
        assert errors[i] is not None and str(100 + i) in errors[i], (i, errors[i])
    stats = thd.cache_stats()
    print(f"[threads] cache {stats}", flush=True)
