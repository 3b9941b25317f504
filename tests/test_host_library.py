"""The C-ABI library on the CPU: exports, host planner, metadata cache.

No device compute runs here; metadata is built host-only (device = -1).
The planner must match the oracle bit for bit.
"""
import ctypes
import os
import re
import threading

import numpy as np
import pytest

import packed_sequence_causal_amd as thd
import workloads
from oracle import metadata as ometa
from oracle import partition as opart

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "thdattn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(thd_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    declared = _declared_functions()
    assert len(declared) >= 12
    lib = ctypes.CDLL(thd.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(thd.EXPORTS) == declared


def _compare_plan(lengths, cp, rank, bt, bn, concurrency=0):
    m = thd.build_metadata(seqlens=lengths, cp=cp, rank=rank, block_t=bt, block_n=bn,
                           concurrency=concurrency)
    assert np.array_equal(m.field("q_global"), opart.q_global(lengths, cp, rank))
    assert np.array_equal(m.field("kv_row"), opart.kv_row(lengths, cp))
    assert np.array_equal(m.field("chunk_off"), opart.chunk_off(lengths, cp))
    tt = ometa.tiles(lengths, cp, rank, bt, bn)
    assert np.array_equal(m.field("tiles"), tt)
    assert np.array_equal(m.field("order"), ometa.order(tt))
    assert np.array_equal(m.field("kvtiles"), ometa.kvtiles(lengths, cp, rank, bt, bn))
    items, splits = ometa.items_and_splits(tt, concurrency)
    assert np.array_equal(m.field("items"), items)
    assert np.array_equal(m.field("splits"), splits)
    info = m.info()
    assert info["kv_split"] == ometa.kv_split_for(tt, concurrency)
    assert info["n_part_slots"] == int(splits[:, 2].sum()) if splits.size else info["n_part_slots"] == 0
    assert info["useful_pairs"] == ometa.useful_pairs_closed_form(lengths, cp)
    assert info["max_kv_tiles"] == int(tt[:, 6].max())
    assert info["version"] == ometa.VERSION == thd.META_VERSION
    assert np.array_equal(m.field("doc_end"), ometa.doc_end(lengths, cp))
    assert info["pad_tokens"] == 0
    plan = thd.plan_partition(seqlens=lengths, cp=cp, rank=rank)
    assert np.array_equal(plan["q_global"], m.field("q_global"))
    assert np.array_equal(plan["kv_row"], m.field("kv_row"))
    assert np.array_equal(plan["chunk_off"], m.field("chunk_off"))


@pytest.mark.parametrize("w", workloads.WORKLOADS, ids=lambda w: w.name)
def test_metadata_bit_exact_on_workloads(w):
    lengths = workloads.draw_lengths(w, np.random.default_rng(w.index))
    bt, bn = thd.preferred_tiles(hq=w.hq, hkv=w.hkv, d_qk=w.d_qk, d_v=w.d_v)
    ranks = sorted({w.rank, 0, w.cp - 1})
    for rank in ranks:
        for concurrency in (0, 512 // w.hkv, 7):
            _compare_plan(lengths, w.cp, rank, bt, bn, concurrency)


@pytest.mark.parametrize("seed", range(12))
def test_metadata_bit_exact_random(seed):
    rng = np.random.default_rng(1000 + seed)
    cp = int(rng.choice([1, 2, 3, 4, 8]))
    lengths = workloads.random_lengths(rng, int(rng.integers(1, 9)), cp, 40)
    bt = int(rng.choice([1, 3, 16, 32, 128]))
    bn = int(rng.choice([1, 5, 64]))
    _compare_plan(lengths, cp, int(rng.integers(0, cp)), bt, bn, int(rng.choice([0, 1, 4, 50])))


@pytest.mark.parametrize("seed", range(4))
def test_metadata_bit_exact_large_cp(seed):
    """Context-parallel sizes beyond the workloads' (16 to 64), where a document's chunks
    are a few tokens long and most tiles hold a single chunk."""
    rng = np.random.default_rng(2000 + seed)
    cp = int(rng.choice([16, 32, 64]))
    lengths = workloads.random_lengths(rng, int(rng.integers(1, 6)), cp, 12)
    bt = int(rng.choice([1, 4, 16, 32]))
    _compare_plan(lengths, cp, int(rng.integers(0, cp)), bt, 64, int(rng.choice([0, 4, 50])))


def test_preferred_tiles():
    assert thd.preferred_tiles(hq=32, hkv=8, d_qk=128, d_v=128) == (32, 64)
    assert thd.preferred_tiles(hq=64, hkv=8, d_qk=128, d_v=128) == (16, 64)
    assert thd.preferred_tiles(hq=16, hkv=16, d_qk=192, d_v=128) == (128, 64)
    assert thd.preferred_tiles(hq=8, hkv=8, d_qk=64, d_v=64) == (128, 64)
    assert thd.preferred_tiles(hq=12, hkv=4, d_qk=128, d_v=128) == (42, 64)


def _key_slots(lengths, cp, rank, bt, bn):
    """Key slots a forward with bn-key tiles computes: each query tile visits
    its document's keys up to its last row, in whole KV tiles."""
    total = 0
    for length in lengths:
        c = length // (2 * cp)
        for k in (rank, 2 * cp - 1 - rank):
            for t0 in range(0, c, bt):
                kv_len = k * c + t0 + min(bt, c - t0)
                total += -(-kv_len // bn) * bn
    return total


def test_preferred_fwd_tiles_pick_short_tiles_when_they_save_key_slots():
    """32-key tiles when they compute at least 7% fewer key slots than 64-key
    tiles (d_qk <= 128 only); block_t as for the general tile sizes."""
    rng = np.random.default_rng(77)
    for _ in range(40):
        cp = int(rng.choice([1, 2, 4, 8]))
        lengths = workloads.random_lengths(rng, int(rng.integers(1, 12)), cp, 48)
        rank = int(rng.integers(0, cp))
        g = int(rng.choice([1, 4, 8]))
        bt = 128 // g
        want = 32 if 100 * _key_slots(lengths, cp, rank, bt, 32) <= 93 * _key_slots(
            lengths, cp, rank, bt, 64) else 64
        got = thd.preferred_fwd_tiles(seqlens=lengths, cp=cp, rank=rank, hq=8 * g, hkv=8,
                                      d_qk=128, d_v=128)
        assert got == (bt, want), (lengths, cp, rank, g)
    heads = dict(hq=64, hkv=8, d_qk=128, d_v=128)
    # a one-token chunk next to a 32-token one: most of each 64-key tile is masked
    assert thd.preferred_fwd_tiles(seqlens=[512, 16], cp=8, rank=0, **heads) == (16, 32)
    # chunks of whole 64-key tiles save nothing
    assert thd.preferred_fwd_tiles(seqlens=[512] * 4, cp=4, rank=2, hq=32, hkv=8, d_qk=128,
                                   d_v=128) == (32, 64)
    # of the workloads only the short-document one takes 32-key tiles
    for w in workloads.WORKLOADS:
        lengths = workloads.draw_lengths(w, np.random.default_rng(w.index))
        bt, bn = thd.preferred_fwd_tiles(seqlens=lengths, cp=w.cp, rank=w.rank, hq=w.hq,
                                         hkv=w.hkv, d_qk=w.d_qk, d_v=w.d_v)
        assert bt == thd.preferred_tiles(hq=w.hq, hkv=w.hkv, d_qk=w.d_qk, d_v=w.d_v)[0]
        assert bn == (32 if w.name == "short" else 64), w.name
    # no 32-key kernel for d_qk = 192
    assert thd.preferred_fwd_tiles(seqlens=[512, 16], cp=8, rank=0, hq=16, hkv=16, d_qk=192,
                                   d_v=128) == (128, 64)
    # padded layout: the padded lengths count (17 real tokens -> 32 with cp 8)
    assert thd.preferred_fwd_tiles(seqlens=[512, 1], cp=8, rank=0, padded=True,
                                   **heads) == (16, 32)
    with pytest.raises(thd.ThdError) as err:
        thd.preferred_fwd_tiles(seqlens=[6], cp=2, rank=0, **heads)
    assert err.value.status == "THD_ENOTDIV"


def test_preferred_fwd_tiles_take_short_tiles_for_large_grids_of_short_query_tiles():
    """Given the 32-key concurrency C, 32-key tiles also when query tiles hold
    at most 32 tokens (4+ q heads per kv head) and there are at least 2C of
    them (no key range would be split); never for longer query tiles."""
    rng = np.random.default_rng(78)
    for _ in range(40):
        cp = int(rng.choice([1, 2, 4, 8]))
        lengths = workloads.random_lengths(rng, int(rng.integers(1, 12)), cp, 48)
        rank = int(rng.integers(0, cp))
        g = int(rng.choice([1, 2, 4, 8]))
        bt = 128 // g
        conc = int(rng.choice([1, 4, 16, 84]))
        n_tiles = ometa.tiles(lengths, cp, rank, bt, 64).shape[0]
        saves = 100 * _key_slots(lengths, cp, rank, bt, 32) <= 93 * _key_slots(
            lengths, cp, rank, bt, 64)
        want = 32 if saves or (bt <= 32 and n_tiles >= 2 * conc) else 64
        got = thd.preferred_fwd_tiles(seqlens=lengths, cp=cp, rank=rank, hq=8 * g, hkv=8,
                                      d_qk=128, d_v=128, concurrency32=conc)
        assert got == (bt, want), (lengths, cp, rank, g, conc)
    # the training workload (272 tiles of 32 tokens) at the 32-key concurrency
    # of 256 CUs, three workgroups each, 7/8, over 8 kv heads: 32-key tiles;
    # gqa_mid (134 tiles) would split them and keeps 64
    conc = 256 * 3 * 7 // (8 * 8)
    for name, bn in (("fwdbwd", 32), ("gqa_mid", 64), ("short", 32), ("mla", 64)):
        w = workloads.BY_NAME[name]
        lengths = workloads.draw_lengths(w, np.random.default_rng(w.index))
        got = thd.preferred_fwd_tiles(seqlens=lengths, cp=w.cp, rank=w.rank, hq=w.hq, hkv=w.hkv,
                                      d_qk=w.d_qk, d_v=w.d_v, concurrency32=conc)
        assert got[1] == bn, name
    with pytest.raises(thd.ThdError) as err:
        thd.preferred_fwd_tiles(seqlens=[512], cp=1, rank=0, hq=8, hkv=8, d_qk=128, d_v=128,
                                concurrency32=-1)
    assert err.value.status == "THD_EINVAL"


def test_short_tile_metadata_is_refused_where_it_has_no_kernel():
    """Metadata with 32-key tiles serves the forward for d_qk <= 128 only: the
    backward and the d_qk = 192 forward refuse it before any device check."""
    m = thd.build_metadata(seqlens=[256], cp=1, rank=0, block_t=32, block_n=32)
    buf = ctypes.create_string_buffer(1 << 16)
    ptr = (ctypes.addressof(buf) + 15) // 16 * 16
    lib = thd._lib
    assert lib.thd_attn_bwd(m.handle, ptr, ptr, ptr, ptr, None, ptr, ptr, ptr, ptr, 32, 8, 128,
                            128, 0.1, ptr, 1 << 16, None) == -5
    assert b"block_n" in lib.thd_last_error()
    m192 = thd.build_metadata(seqlens=[256], cp=1, rank=0, block_t=128, block_n=32)
    assert lib.thd_attn_fwd(m192.handle, ptr, ptr, ptr, ptr, ptr, None, 16, 16, 192, 128, 0.1,
                            None, 0, None) == -5
    # 32-key metadata reaches the device check for d_qk = 128 (host-only copy here)
    assert lib.thd_attn_fwd(m.handle, ptr, ptr, ptr, ptr, ptr, None, 32, 8, 128, 128, 0.1,
                            None, 0, None) == -5
    assert b"device copy" in lib.thd_last_error()
    c = ctypes.c_int32()
    assert lib.thd_fwd_concurrency(0, 8, 48, ctypes.byref(c)) == -1
    assert lib.thd_fwd_concurrency(0, 0, 64, ctypes.byref(c)) == -1


def test_bf16_dkdv_backward_checks_its_arguments_as_the_fp32_one():
    """thd_attn_bwd_bf16kv shares thd_attn_bwd's checks: each bad argument
    gets the same status from both, before any device work."""
    m = thd.build_metadata(seqlens=[256], cp=1, rank=0, block_t=32, block_n=64)
    m32 = thd.build_metadata(seqlens=[256], cp=1, rank=0, block_t=32, block_n=32)
    buf = ctypes.create_string_buffer(1 << 16)
    ptr = (ctypes.addressof(buf) + 15) // 16 * 16
    lib = thd._lib
    cases = [
        ((m.handle, ptr, ptr, ptr, ptr, None, ptr, ptr, ptr, ptr), (32, 8, 96, 96, 0.1), -8),
        ((m.handle, ptr, ptr, ptr, ptr, None, ptr, ptr, ptr, ptr), (32, 8, 128, 128, -1.0), -1),
        ((m.handle, ptr, ptr, ptr, ptr, None, ptr, ptr, ptr, ptr), (30, 8, 128, 128, 0.1), -1),
        ((m32.handle, ptr, ptr, ptr, ptr, None, ptr, ptr, ptr, ptr), (32, 8, 128, 128, 0.1), -5),
        ((m.handle, ptr, ptr, ptr, ptr, None, ptr, ptr, ptr + 2, ptr), (32, 8, 128, 128, 0.1), -4),
        ((m.handle, ptr, ptr, ptr, ptr, None, ptr, ptr, ptr, None), (32, 8, 128, 128, 0.1), -1),
        ((m.handle, ptr, ptr, ptr, ptr, None, ptr, ptr, ptr, ptr), (32, 8, 128, 128, 0.1), -5),
    ]
    for ptrs, dims, status in cases:
        for fn in (lib.thd_attn_bwd, lib.thd_attn_bwd_bf16kv):
            assert fn(*ptrs, *dims, ptr, 1 << 16, None) == status, (fn.__name__, dims, status)
    assert b"device" in lib.thd_last_error()   # host-only metadata cannot launch


@pytest.mark.parametrize("kwargs,status", [
    (dict(seqlens=[6, 8], cp=2, rank=0), "THD_ENOTDIV"),
    (dict(seqlens=[8], cp=2, rank=2), "THD_ERANGE"),
    (dict(seqlens=[8], cp=2, rank=-1), "THD_ERANGE"),
    (dict(seqlens=[8], cp=0, rank=0), "THD_ERANGE"),
    (dict(seqlens=[0, 8], cp=2, rank=0), "THD_EINVAL"),
    (dict(seqlens=[-4], cp=2, rank=0), "THD_EINVAL"),
    (dict(seqlens=[], cp=1, rank=0), "THD_EINVAL"),
    (dict(seqlens=[2 ** 30, 2 ** 30], cp=1, rank=0), "THD_ERANGE"),
])
def test_partition_errors(kwargs, status):
    with pytest.raises(thd.ThdError) as err:
        thd.plan_partition(**kwargs)
    assert err.value.status == status
    assert str(err.value)
    with pytest.raises(thd.ThdError) as err:
        thd.build_metadata(block_t=4, block_n=4, **kwargs)
    assert err.value.status == status


def test_metadata_argument_errors():
    for bt, bn in ((0, 4), (4, 0), (4, 5000)):
        with pytest.raises(thd.ThdError) as err:
            thd.build_metadata(seqlens=[8], cp=1, rank=0, block_t=bt, block_n=bn)
        assert err.value.status == "THD_ERANGE"
    with pytest.raises(thd.ThdError) as err:
        thd.build_metadata(seqlens=[8], cp=1, rank=0, block_t=4, block_n=4, device=-2)
    assert err.value.status == "THD_EINVAL"
    for kw, status in ((dict(hq=12, hkv=5), "THD_EINVAL"), (dict(hq=0, hkv=1), "THD_EINVAL"),
                       (dict(hq=256, hkv=1), "THD_EUNSUPPORTED")):
        with pytest.raises(thd.ThdError) as err:
            thd.preferred_tiles(d_qk=128, d_v=128, **kw)
        assert err.value.status == status
    with pytest.raises(thd.ThdError) as err:
        thd.preferred_tiles(hq=8, hkv=8, d_qk=96, d_v=96)
    assert err.value.status == "THD_EUNSUPPORTED"


def test_null_pointers_return_errors():
    lib = thd._lib
    assert lib.thd_plan_partition(None, 1, 1, 0, None, None, None, None, None) == -1
    assert lib.thd_build_metadata(None, 1, 1, 0, 1, 1, 0, -1, None) == -1
    assert lib.thd_meta_info(None, None) == -1
    assert lib.thd_meta_copy(None, 0, None, 0) == -1
    lib.thd_meta_release(None)
    assert lib.thd_attn_fwd(None, None, None, None, None, None, None, 1, 1, 128, 128, 1.0, None,
                            0, None) == -1
    assert b"NULL" in lib.thd_last_error()
    m = thd.build_metadata(seqlens=[8], cp=1, rank=0, block_t=4, block_n=64)
    n = ctypes.c_int32()
    # wrong count and unknown field
    assert lib.thd_meta_copy(m.handle, 0, ctypes.byref(n), 1) == -1
    assert lib.thd_meta_copy(m.handle, 9, ctypes.byref(n), 1) == -1


def test_forward_rejects_host_only_metadata_and_bad_arguments():
    m = thd.build_metadata(seqlens=[256], cp=1, rank=0, block_t=32, block_n=64)
    buf = ctypes.create_string_buffer(1 << 16)
    ptr = (ctypes.addressof(buf) + 15) // 16 * 16
    lib = thd._lib
    args = [m.handle, ptr, ptr, ptr, ptr, ptr, None]
    tail = [None, 0, None]
    # unsupported head dims are refused before any device check
    assert lib.thd_attn_fwd(*args, 32, 8, 96, 96, 0.1, *tail) == -8
    # bad scale (0 selects 1/sqrt(d_qk) and so passes this check)
    assert lib.thd_attn_fwd(*args, 32, 8, 128, 128, -0.5, *tail) == -1
    assert lib.thd_attn_fwd(*args, 32, 8, 128, 128, float("nan"), *tail) == -1
    assert lib.thd_attn_fwd(*args, 32, 8, 128, 128, float("inf"), *tail) == -1
    assert b"softmax_scale" in lib.thd_last_error()
    assert lib.thd_attn_fwd(*args, 32, 8, 128, 128, 0.0, *tail) == -5
    # tile sizes that do not fit the group size
    assert lib.thd_attn_fwd(*args, 64, 8, 128, 128, 0.1, *tail) == -5
    # misaligned pointer
    assert lib.thd_attn_fwd(m.handle, ptr + 2, ptr, ptr, ptr, ptr, None, 32, 8, 128, 128, 0.1,
                            *tail) == -4
    # misaligned optional fp32 output
    assert lib.thd_attn_fwd(m.handle, ptr, ptr, ptr, ptr, ptr, ptr + 4, 32, 8, 128, 128, 0.1,
                            *tail) == -4
    # host-only metadata cannot launch
    assert lib.thd_attn_fwd(*args, 32, 8, 128, 128, 0.1, *tail) == -5
    assert b"device" in lib.thd_last_error()
    # a split plan needs its workspace
    ms = thd.build_metadata(seqlens=[4096], cp=1, rank=0, block_t=32, block_n=64, concurrency=256)
    assert ms.info()["n_part_slots"] > 0
    assert lib.thd_attn_fwd(ms.handle, ptr, ptr, ptr, ptr, ptr, None, 32, 8, 128, 128, 0.1,
                            *tail) == -1
    assert b"workspace" in lib.thd_last_error()


def test_noalloc_forward_refuses_plans_beyond_its_static_array():
    """thd_attn_fwd_noalloc checks the split tiles' need against its fixed
    per-device array before anything touches a device."""
    lib = thd._lib
    buf = ctypes.create_string_buffer(1 << 16)
    ptr = (ctypes.addressof(buf) + 15) // 16 * 16
    big = thd.build_metadata(seqlens=[65536], cp=1, rank=0, block_t=128, block_n=64,
                             concurrency=1000)
    assert big.fwd_workspace_bytes(16, 16, 128) > (64 << 20)
    assert lib.thd_attn_fwd_noalloc(big.handle, ptr, ptr, ptr, ptr, ptr, None, 16, 16, 128, 128,
                                    0.0, None) == -3
    assert b"no-allocation" in lib.thd_last_error()
    # a plan that fits gets past the size check to the device check (host-only metadata)
    small = thd.build_metadata(seqlens=[2048, 512, 1024], cp=2, rank=1, block_t=32, block_n=64,
                               concurrency=64)
    assert 0 < small.fwd_workspace_bytes(16, 4, 128) <= (64 << 20)
    assert lib.thd_attn_fwd_noalloc(small.handle, ptr, ptr, ptr, ptr, ptr, None, 16, 4, 128, 128,
                                    0.0, None) == -5
    assert b"device" in lib.thd_last_error()
    # the usual argument checks apply
    assert lib.thd_attn_fwd_noalloc(small.handle, ptr + 2, ptr, ptr, ptr, ptr, None, 16, 4, 128,
                                    128, 0.0, None) == -4
    assert lib.thd_attn_fwd_noalloc(None, ptr, ptr, ptr, ptr, ptr, None, 16, 4, 128, 128, 0.0,
                                    None) == -1


def test_cache_hits_and_key_completeness():
    thd.cache_clear()
    a = thd.build_metadata(seqlens=[8, 16, 8], cp=2, rank=0, block_t=4, block_n=8)
    b = thd.build_metadata(seqlens=[8, 16, 8], cp=2, rank=0, block_t=4, block_n=8)
    assert a.info()["cache_hit"] == 0 and b.info()["cache_hit"] == 1
    # same T and document count, different lengths: must miss and differ
    c = thd.build_metadata(seqlens=[16, 8, 8], cp=2, rank=0, block_t=4, block_n=8)
    assert c.info()["cache_hit"] == 0
    assert not np.array_equal(a.field("q_global"), c.field("q_global"))
    for kw in (dict(rank=1), dict(block_t=2), dict(block_n=4), dict(concurrency=3)):
        args = dict(seqlens=[8, 16, 8], cp=2, rank=0, block_t=4, block_n=8)
        args.update(kw)
        assert thd.build_metadata(**args).info()["cache_hit"] == 0
    st = thd.cache_stats()
    assert st["hits"] == 1 and st["misses"] == 6 and st["uploads"] == 0
    # a handle outlives the cache entry it came from
    thd.cache_clear()
    assert np.array_equal(a.field("tiles"), ometa.tiles([8, 16, 8], 2, 0, 4, 8))
    a.release()
    a.release()


def test_cache_eviction_keeps_results_exact():
    thd.cache_clear()
    held = []
    for i in range(80):
        lengths = [8 * (1 + i % 7), 8 * (1 + i % 5)]
        held.append((lengths, thd.build_metadata(seqlens=lengths, cp=2, rank=i % 2, block_t=4,
                                                 block_n=8)))
    assert thd.cache_stats()["entries"] <= 64
    for i, (lengths, m) in enumerate(held):
        assert np.array_equal(m.field("tiles"), ometa.tiles(lengths, 2, i % 2, 4, 8))


def test_concurrent_builds_agree():
    thd.cache_clear()
    rng = np.random.default_rng(5)
    cases = [workloads.random_lengths(rng, 6, 4, 30) for _ in range(4)]
    errors = []
    results = {}

    def worker(tid):
        try:
            for rep in range(25):
                idx = (tid + rep) % len(cases)
                m = thd.build_metadata(seqlens=cases[idx], cp=4, rank=tid % 4, block_t=16,
                                       block_n=64)
                tiles = m.field("tiles")
                results.setdefault((idx, tid % 4), tiles)
                if not np.array_equal(results[(idx, tid % 4)], tiles):
                    errors.append("mismatch")
                m.release()
        except Exception as exc:  # pragma: no cover - reported below
            errors.append(repr(exc))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(16)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors
    st = thd.cache_stats()
    assert st["misses"] == len({(i, r) for i in range(4) for r in range(4)} & set(results))
    for (idx, rank), tiles in results.items():
        assert np.array_equal(tiles, ometa.tiles(cases[idx], 4, rank, 16, 64))


# ---------------------------------------------------------------- padding

@pytest.mark.parametrize("real,cp,rank", [
    ([5, 13, 8], 2, 0), ([1, 3, 30], 4, 3), ([7, 9, 2], 3, 1), ([1], 8, 5),
    ([100, 250, 31, 7, 64], 8, 2),
])
def test_padded_metadata_matches_the_oracle(real, cp, rank):
    lengths = opart.pad_lengths(real, cp)
    assert thd.pad_lengths(seqlens=real, cp=cp).tolist() == lengths
    bt, bn = 16, 32
    m = thd.build_metadata(seqlens=real, cp=cp, rank=rank, block_t=bt, block_n=bn, padded=True)
    plain = thd.build_metadata(seqlens=lengths, cp=cp, rank=rank, block_t=bt, block_n=bn)
    for name in ("q_global", "kv_row", "chunk_off", "tiles", "order", "kvtiles", "items", "splits"):
        assert np.array_equal(m.field(name), plain.field(name)), name
    assert np.array_equal(m.field("doc_end"), ometa.doc_end(lengths, cp, real))
    assert np.array_equal(plain.field("doc_end"), ometa.doc_end(lengths, cp))
    assert m.info()["pad_tokens"] == sum(lengths) - sum(real)
    assert m.info()["total_tokens"] == sum(lengths)


def test_padded_metadata_cache_key_holds_the_real_lengths():
    a = thd.build_metadata(seqlens=[5, 8], cp=2, rank=0, block_t=8, block_n=16, padded=True)
    b = thd.build_metadata(seqlens=[6, 8], cp=2, rank=0, block_t=8, block_n=16, padded=True)
    c = thd.build_metadata(seqlens=[8, 8], cp=2, rank=0, block_t=8, block_n=16)
    assert a.field("doc_end").tolist() == [5, 16]
    assert b.field("doc_end").tolist() == [6, 16]
    assert c.field("doc_end").tolist() == [8, 16]
    again = thd.build_metadata(seqlens=[5, 8], cp=2, rank=0, block_t=8, block_n=16, padded=True)
    assert again.info()["cache_hit"] == 1 and not b.info()["cache_hit"]


@pytest.mark.parametrize("kwargs,status", [
    ({"seqlens": [3, 0], "cp": 2}, "THD_EINVAL"),
    ({"seqlens": [3], "cp": 0}, "THD_ERANGE"),
    ({"seqlens": [2**31 - 1], "cp": 2}, "THD_ERANGE"),
])
def test_pad_lengths_errors(kwargs, status):
    with pytest.raises(thd.ThdError) as e:
        thd.pad_lengths(**kwargs)
    assert e.value.status == status
    with pytest.raises(thd.ThdError):
        thd.build_metadata(block_t=8, block_n=16, rank=0, padded=True, **kwargs)


@pytest.mark.parametrize("seed", range(8))
def test_pass_plans_match_oracle_bit_for_bit(seed):
    rng = np.random.default_rng(500 + seed)
    cp = int(rng.choice([1, 2, 3, 4, 8]))
    rank = int(rng.integers(0, cp))
    lengths = [2 * cp * int(x) for x in rng.integers(1, 40, size=int(rng.integers(1, 9)))]
    bt = int(rng.choice([4, 16, 32, 128]))
    bn = 64
    shards = sorted({int(x) for x in rng.integers(0, cp, size=int(rng.integers(1, cp + 1)))})
    m = thd.build_pass_metadata(seqlens=lengths, cp=cp, rank=rank, block_t=bt, block_n=bn,
                                shards=shards)
    info = m.info()
    assert info["is_pass"] == 1 and info["item_ints"] == 8
    assert info["shard_mask"] == sum(1 << s for s in shards)
    want_items, want_tiles = ometa.pass_plan(lengths, cp, rank, bt, bn, shards)
    assert np.array_equal(m.field("items"), want_items)
    assert np.array_equal(m.field("splits"), want_tiles)
    assert np.array_equal(m.field("tiles"), ometa.tiles(lengths, cp, rank, bt, bn))
    assert info["n_part_slots"] == want_items.shape[0]
    # the mask is part of the cache key
    other = thd.build_pass_metadata(seqlens=lengths, cp=cp, rank=rank, block_t=bt, block_n=bn,
                                    shards=[s for s in range(cp) if s not in shards] or shards)
    if set(shards) != set(range(cp)):
        assert other.info()["shard_mask"] != info["shard_mask"]


def test_pass_metadata_errors():
    lib = thd._lib
    for shards in ([], [2]):   # no shard; a shard beyond cp
        with pytest.raises(thd.ThdError) as err:
            thd.build_pass_metadata(seqlens=[8, 16], cp=2, rank=0, block_t=4, block_n=64,
                                    shards=shards)
        assert err.value.status == "THD_EINVAL"
    with pytest.raises(thd.ThdError) as err:
        thd.build_pass_metadata(seqlens=[6], cp=2, rank=0, block_t=4, block_n=64, shards=[0])
    assert err.value.status == "THD_ENOTDIV"
    # a pass plan is refused by the one-pass entry points, and the reverse
    buf = ctypes.create_string_buffer(1 << 16)
    ptr = (ctypes.addressof(buf) + 15) // 16 * 16
    mp = thd.build_pass_metadata(seqlens=[256], cp=1, rank=0, block_t=32, block_n=64, shards=[0])
    assert lib.thd_attn_fwd(mp.handle, ptr, ptr, ptr, ptr, ptr, None, 32, 8, 128, 128, 0.0, None,
                            0, None) == -5
    assert b"pass" in lib.thd_last_error()
    m = thd.build_metadata(seqlens=[256], cp=1, rank=0, block_t=32, block_n=64)
    assert lib.thd_attn_fwd_pass(m.handle, ptr, ptr, ptr, ptr, ptr, ptr, 3, 32, 8, 128, 128, 0.0,
                                 None) == -5
    assert lib.thd_attn_fwd_pass(mp.handle, ptr, ptr, ptr, ptr, ptr, ptr, 4, 32, 8, 128, 128, 0.0,
                                 None) == -1
    n = ctypes.c_int64()
    assert lib.thd_attn_fwd_pass_state_bytes(m.handle, 32, 8, 128, ctypes.byref(n)) == -5


def _compare_packed(lengths, cp, rank, bt, bn, concurrency, real=None):
    m = thd.build_metadata(seqlens=real if real is not None else lengths, cp=cp, rank=rank,
                           block_t=bt, block_n=bn, concurrency=concurrency,
                           padded=real is not None, packed=True)
    info = m.info()
    want = ometa.packed_forward_plan(lengths, cp, rank, bt, bn, concurrency, real_lengths=real)
    assert info["is_packed"] == 1 and info["is_pass"] == 0 and info["n_kvtiles"] == 0
    assert info["n_packed_tiles"] == int((want["tiles"][:, 0] < 0).sum())
    for name in ("tiles", "order", "items", "splits", "pack_rows", "pack_keys"):
        got, ref = m.field(name), want[name]
        assert got.size == ref.size and np.array_equal(got.reshape(-1), ref.reshape(-1)), name
    return m


@pytest.mark.parametrize("seed", range(8))
def test_packed_plans_match_oracle_bit_for_bit(seed):
    rng = np.random.default_rng(700 + seed)
    cp = int(rng.choice([1, 2, 3, 4, 8]))
    rank = int(rng.integers(0, cp))
    real = [int(x) for x in rng.integers(1, 60 * cp, size=int(rng.integers(1, 12)))]
    bt = int(rng.choice([2, 4, 8, 16, 32]))
    bn = int(rng.choice([32, 64]))
    concurrency = int(rng.choice([0, 2, 8]))
    lengths = opart.pad_lengths(real, cp)
    _compare_packed(lengths, cp, rank, bt, bn, concurrency)
    _compare_packed(lengths, cp, rank, bt, bn, concurrency, real=real)


@pytest.mark.parametrize("name", ["tiny", "gqa_mid", "mla", "short", "fwdbwd"])
def test_packed_plans_of_the_workloads_match_oracle(name):
    w = workloads.BY_NAME[name]
    lengths = workloads.draw_lengths(w, np.random.default_rng(w.index))
    g = w.hq // w.hkv
    _compare_packed(lengths, w.cp, w.rank, 128 // g, 32 if w.d_qk <= 128 else 64, 0)


def test_packed_metadata_errors_and_refusals():
    lib = thd._lib
    h = ctypes.c_void_p()
    lens = np.asarray([8, 16], np.int32)
    assert lib.thd_build_packed_metadata(thd._ptr32(lens), 2, 2, 0, 4, 64, 0, 2, -1,
                                         ctypes.byref(h)) == -1
    assert b"padded" in lib.thd_last_error()
    with pytest.raises(thd.ThdError) as err:
        thd.build_metadata(seqlens=[6], cp=2, rank=0, block_t=4, block_n=64, packed=True)
    assert err.value.status == "THD_ENOTDIV"
    # the packed flag is part of the cache key
    plain = thd.build_metadata(seqlens=[8, 16, 8], cp=2, rank=0, block_t=4, block_n=64)
    packed = thd.build_metadata(seqlens=[8, 16, 8], cp=2, rank=0, block_t=4, block_n=64,
                                packed=True)
    assert plain.info()["is_packed"] == 0 and packed.info()["is_packed"] == 1
    assert packed.info()["n_packed_tiles"] > 0
    # the backward refuses a packed plan before touching any pointer
    buf = ctypes.create_string_buffer(1 << 16)
    ptr = (ctypes.addressof(buf) + 15) // 16 * 16
    mp = thd.build_metadata(seqlens=[256, 64], cp=1, rank=0, block_t=32, block_n=64, packed=True)
    assert lib.thd_attn_bwd(mp.handle, ptr, ptr, ptr, ptr, None, ptr, ptr, ptr, ptr, 32, 8, 128,
                            128, 0.0, ptr, 1 << 16, None) == -5
    assert b"packed" in lib.thd_last_error()
    with pytest.raises(thd.ThdError):
        thd.device_metadata(seqlens=[256], cp=1, rank=0, hq=32, hkv=8, d_qk=128, d_v=128,
                            device=0, packed=True)
