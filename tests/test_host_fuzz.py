"""Property-based sweep of the host planner against the oracle (CPU only).

Hypothesis draws context-parallel sizes, ranks, document lengths (real lengths
of any size, padded to multiples of 2cp where a plan takes them), tile sizes,
split concurrencies and shard sets, and every plan kind the library builds
(plain, padded, packed, packed padded, shard pass, padded shard pass) must equal the oracle's
tables bit for bit. The draws are derandomised, so a run is reproducible.
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import packed_sequence_causal_amd as thd
from oracle import metadata as ometa
from oracle import partition as opart

SETTINGS = settings(max_examples=250, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow])


@st.composite
def problems(draw, max_cp=16, max_docs=10, max_chunk=48):
    cp = draw(st.integers(1, max_cp))
    rank = draw(st.integers(0, cp - 1))
    n = draw(st.integers(1, max_docs))
    real = draw(st.lists(st.integers(1, 2 * cp * max_chunk), min_size=n, max_size=n))
    return cp, rank, real


def _fields(m, names):
    return {name: m.field(name) for name in names}


def _check_plain(lengths, cp, rank, bt, bn, concurrency):
    m = thd.build_metadata(seqlens=lengths, cp=cp, rank=rank, block_t=bt, block_n=bn,
                           concurrency=concurrency)
    assert np.array_equal(m.field("q_global"), opart.q_global(lengths, cp, rank))
    assert np.array_equal(m.field("kv_row"), opart.kv_row(lengths, cp))
    tt = ometa.tiles(lengths, cp, rank, bt, bn)
    assert np.array_equal(m.field("tiles"), tt)
    assert np.array_equal(m.field("order"), ometa.order(tt))
    assert np.array_equal(m.field("kvtiles"), ometa.kvtiles(lengths, cp, rank, bt, bn))
    items, splits = ometa.items_and_splits(tt, concurrency)
    assert np.array_equal(m.field("items"), items)
    assert np.array_equal(m.field("splits"), splits)
    assert np.array_equal(m.field("doc_end"), ometa.doc_end(lengths, cp))
    assert m.info()["useful_pairs"] == ometa.useful_pairs_closed_form(lengths, cp)
    return m


@SETTINGS
@given(problems(), st.sampled_from([1, 2, 5, 16, 32, 64, 128]), st.sampled_from([1, 3, 32, 64]),
       st.sampled_from([0, 1, 3, 8, 40]))
def test_plain_and_padded_plans(problem, bt, bn, concurrency):
    cp, rank, real = problem
    lengths = opart.pad_lengths(real, cp)
    plain = _check_plain(lengths, cp, rank, bt, bn, concurrency)
    # the padded plan of the real lengths is the plain plan of the padded
    # lengths plus the real document ends
    m = thd.build_metadata(seqlens=real, cp=cp, rank=rank, block_t=bt, block_n=bn,
                           concurrency=concurrency, padded=True)
    names = ("q_global", "kv_row", "chunk_off", "tiles", "order", "kvtiles", "items", "splits")
    got, want = _fields(m, names), _fields(plain, names)
    for name in names:
        assert np.array_equal(got[name], want[name]), name
    assert np.array_equal(m.field("doc_end"), ometa.doc_end(lengths, cp, real))
    assert m.info()["pad_tokens"] == sum(lengths) - sum(real)


@SETTINGS
@given(problems(), st.sampled_from([1, 2, 4, 8, 16, 32, 128]), st.sampled_from([32, 64]),
       st.sampled_from([0, 2, 8, 30]), st.booleans())
def test_packed_plans(problem, bt, bn, concurrency, padded):
    cp, rank, real = problem
    lengths = opart.pad_lengths(real, cp)
    m = thd.build_metadata(seqlens=real if padded else lengths, cp=cp, rank=rank, block_t=bt,
                           block_n=bn, concurrency=concurrency, padded=padded, packed=True)
    want = ometa.packed_forward_plan(lengths, cp, rank, bt, bn, concurrency,
                                     real_lengths=real if padded else None)
    for name in ("tiles", "order", "items", "splits", "pack_rows", "pack_keys"):
        got, ref = m.field(name), want[name]
        assert got.size == ref.size and np.array_equal(got.reshape(-1), ref.reshape(-1)), name
    info = m.info()
    assert info["is_packed"] == 1 and info["n_kvtiles"] == 0
    assert info["n_packed_tiles"] == int((want["tiles"][:, 0] < 0).sum())


@SETTINGS
@given(problems(max_cp=8), st.sampled_from([1, 4, 16, 32, 128]), st.data())
def test_pass_plans(problem, bt, data):
    cp, rank, real = problem
    lengths = opart.pad_lengths(real, cp)
    shards = sorted(data.draw(st.sets(st.integers(0, cp - 1), min_size=1, max_size=cp)))
    m = thd.build_pass_metadata(seqlens=lengths, cp=cp, rank=rank, block_t=bt, block_n=64,
                                shards=shards)
    want_items, want_tiles = ometa.pass_plan(lengths, cp, rank, bt, 64, shards)
    assert np.array_equal(m.field("items"), want_items)
    assert np.array_equal(m.field("splits"), want_tiles)
    assert np.array_equal(m.field("tiles"), ometa.tiles(lengths, cp, rank, bt, 64))
    assert m.info()["shard_mask"] == sum(1 << s for s in shards)
    # the padded pass plan of the real lengths: the same tables, real document ends
    mp = thd.build_pass_metadata(seqlens=real, cp=cp, rank=rank, block_t=bt, block_n=64,
                                 shards=shards, padded=True)
    for name in ("q_global", "kv_row", "tiles", "items", "splits"):
        assert np.array_equal(mp.field(name), m.field(name)), name
    assert np.array_equal(mp.field("doc_end"), ometa.doc_end(lengths, cp, real))
    assert mp.info()["is_pass"] == 1 and mp.info()["pad_tokens"] == sum(lengths) - sum(real)


@pytest.mark.parametrize("cp", [1, 3, 8])
def test_single_shard_passes_partition_every_tiles_keys(cp):
    """The cp single-shard passes of a forward split each tile's keys between
    them: their runs, together, cover [document start, last row] once, with
    no gap and no overlap, and each run lies inside its pass's shard."""
    rng = np.random.default_rng(cp)
    lengths = [2 * cp * int(x) for x in rng.integers(1, 30, size=6)]
    t_local = sum(lengths) // cp
    kv_row = opart.kv_row(lengths, cp)
    for rank in range(cp):
        tt = ometa.tiles(lengths, cp, rank, 16, 64)
        runs = {t: [] for t in range(tt.shape[0])}
        for s in range(cp):
            m = thd.build_pass_metadata(seqlens=lengths, cp=cp, rank=rank, block_t=16,
                                        block_n=64, shards=[s])
            for run in m.field("items").reshape(-1, 8):
                keys = np.arange(int(run[1]), int(run[2]))
                assert np.all(kv_row[keys] // t_local == s), (rank, s)
                runs[int(run[0])].append((int(run[1]), int(run[2])))
        for t, rs in runs.items():
            covered = [k for lo, hi in sorted(rs) for k in range(lo, hi)]
            assert covered == list(range(int(tt[t, 5]), int(tt[t, 1] + tt[t, 2]))), (rank, t)
