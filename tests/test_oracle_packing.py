"""Pins of the oracle's packed forward plans (short-segment packing; CPU only).

A hand-derived fixture fixes the grouping rule and the table layouts; a
brute-force enumeration shows that the packed tables give every real local
row exactly its causal, same-document keys; and attention evaluated through
the tables (the way a kernel reads them) equals the oracle's attention.
"""
import math

import numpy as np
import pytest

from golden_io import read_records
from oracle import attention, metadata, partition


def test_packed_plans_match_hand_derived_fixture():
    g = read_records("packed_plan_small.txt")
    tt, rows, keys = metadata.packed_plan([8, 12, 4, 20], 2, 0, 4, 4)
    assert tt.tolist() == g["tileA"]
    assert rows.tolist() == g["rowA"]
    assert keys.tolist() == [x for rec in g["keyA"] for x in rec]
    tt_b, rows_b, keys_b = metadata.packed_plan([8, 12, 4, 20], 2, 0, 4, 4,
                                                real_lengths=[8, 12, 3, 17])
    assert tt_b.tolist() == g["tileA"] and keys_b.tolist() == keys.tolist()
    assert rows_b.tolist() == g["rowB"]


def _random_case(seed):
    rng = np.random.default_rng(500 + seed)
    cp = int(rng.choice([1, 2, 3, 4]))
    rank = int(rng.integers(0, cp))
    real = [int(x) for x in rng.integers(1, 14 * cp, size=int(rng.integers(1, 9)))]
    lengths = partition.pad_lengths(real, cp)
    bt = int(rng.choice([2, 3, 4, 8]))
    bn = int(rng.choice([1, 2, 4, 8]))
    return lengths, real, cp, rank, bt, bn


@pytest.mark.parametrize("seed", range(10))
def test_packed_plan_gives_each_row_exactly_its_causal_keys(seed):
    """Every local row lies in exactly one tile; a plain tile's row sees keys
    kv_start .. its own position, a packed row the gathered rows of its slot
    window; both must equal kv_row of the document's keys up to the row's
    position (nothing of another document, nothing later, no pad slot). The
    grouping limits hold: at most BT rows and BN * max n_kv slots per tile."""
    lengths, real, cp, rank, bt, bn = _random_case(seed)
    plain = metadata.tiles(lengths, cp, rank, bt, bn)
    tt, rows, keys = metadata.packed_plan(lengths, cp, rank, bt, bn, real_lengths=real)
    kvr = partition.kv_row(lengths, cp)
    cu = partition.cu_seqlens(lengths)
    docs = partition.doc_of(lengths)
    qg = partition.q_global(lengths, cp, rank)
    pads = partition.pad_rows(real, cp, rank)
    cap = bn * int(plain[:, 6].max())
    seen = {}
    used_rows = 0
    for rec in tt.tolist():
        q_local, q_glob, n_rows, doc, slot, kv_start, n_kv, n_full = rec
        assert 1 <= n_rows <= bt and n_kv <= int(plain[:, 6].max())
        if q_local >= 0:
            for o in range(n_rows):
                seen.setdefault(q_local + o, []).append(
                    sorted(int(kvr[x]) for x in range(kv_start, q_glob + o + 1)))
            continue
        assert n_full == 0 and doc == -1 and slot == -1
        assert q_glob == used_rows     # packed rows are listed tile by tile
        used_rows += n_rows
        window = keys[kv_start:kv_start + n_kv * bn]
        assert len(window) == n_kv * bn
        hi_max = -1
        for local, lo, hi, is_real in rows[q_glob:q_glob + n_rows].tolist():
            assert 0 <= lo <= hi < cap
            hi_max = max(hi_max, hi)
            assert is_real == (0 if pads[local] else 1)
            seen.setdefault(local, []).append(sorted(int(x) for x in window[lo:hi + 1]))
        assert -(-(hi_max + 1) // bn) == n_kv   # pad slots only fill the last KV tile
    assert used_rows == rows.shape[0]
    assert sorted(seen) == list(range(len(qg)))
    for local, lists in seen.items():
        assert len(lists) == 1, local
        g = int(qg[local])
        want = sorted(int(kvr[x]) for x in range(cu[int(docs[g])], g + 1))
        assert lists[0] == want, (local, g)


def test_packing_groups_partial_tiles_and_keeps_full_ones():
    """Short documents: every tile with BT rows stays plain, and packing
    strictly lowers the tile count when several documents end in short
    partial tiles."""
    lengths = [16, 24, 8, 40, 16, 8, 32]
    cp, rank, bt, bn = 2, 1, 8, 4
    plain = metadata.tiles(lengths, cp, rank, bt, bn)
    tt, rows, _ = metadata.packed_plan(lengths, cp, rank, bt, bn)
    full = [r for r in plain.tolist() if r[2] == bt]
    assert [r for r in tt.tolist() if r[0] >= 0 and r[2] == bt] == full
    assert len(tt) < len(plain)
    assert rows.shape[0] == sum(r[2] for r in plain.tolist() if r[2] < bt) - sum(
        r[2] for r in tt.tolist() if r[0] >= 0 and r[2] < bt)


@pytest.mark.parametrize("seed", range(4))
def test_attention_through_packed_tables_equals_oracle(seed):
    """fp64 attention evaluated row by row through the packed tables (query
    row from pack_rows, keys from the slot window through pack_keys) equals
    the oracle's attention, pad rows aside (O = 0, LSE = +inf)."""
    lengths, real, cp, rank, bt, bn = _random_case(seed)
    rng = np.random.default_rng(seed)
    hkv, group, d = 2, 2, 8
    t = sum(lengths)
    q = rng.standard_normal((t // cp, hkv * group, d))
    k = rng.standard_normal((t, hkv, d))
    v = rng.standard_normal((t, hkv, d))
    want_o, want_lse = attention.attn_fwd64_padded(q, k, v, real, cp, rank)
    tt, rows, keys = metadata.packed_plan(lengths, cp, rank, bt, bn, real_lengths=real)
    kvr = partition.kv_row(lengths, cp)
    scale = 1.0 / math.sqrt(d)
    ends = metadata.doc_end(lengths, cp, real)
    got_o = np.full_like(want_o, np.nan)
    got_lse = np.full_like(want_lse, np.nan)

    def put(local, gathered, is_real):
        for h in range(hkv * group):
            kh = h // group
            if not is_real:
                got_o[local, h], got_lse[local, h] = 0.0, np.inf
                continue
            s = scale * (k[gathered, kh] @ q[local, h])
            m = s.max()
            p = np.exp(s - m)
            got_o[local, h] = (p @ v[gathered, kh]) / p.sum()
            got_lse[local, h] = m + math.log(p.sum())

    for q_local, q_glob, n_rows, doc, _, kv_start, n_kv, _ in tt.tolist():
        if q_local >= 0:
            for o in range(n_rows):
                put(q_local + o, kvr[kv_start:q_glob + o + 1], q_glob + o < int(ends[doc]))
            continue
        for local, lo, hi, is_real in rows[q_glob:q_glob + n_rows].tolist():
            put(local, keys[kv_start + lo:kv_start + hi + 1], is_real == 1)
    np.testing.assert_allclose(got_o, want_o, rtol=0, atol=1e-12)
    assert np.array_equal(np.isinf(got_lse), np.isinf(want_lse))
    fin = np.isfinite(want_lse)
    np.testing.assert_allclose(got_lse[fin], want_lse[fin], rtol=0, atol=1e-12)


def test_packed_forward_plan_items_cover_every_tile_once():
    lengths, real, cp, rank, bt, bn = _random_case(3)
    plan = metadata.packed_forward_plan(lengths, cp, rank, bt, bn, 4, real_lengths=real)
    tt = plan["tiles"]
    assert sorted(plan["order"].tolist()) == list(range(len(tt)))
    cover = {}
    for tile, begin, end, _ in plan["items"].tolist():
        for j in range(begin, end):
            cover[(tile, j)] = cover.get((tile, j), 0) + 1
    want = {(t, j) for t in range(len(tt)) for j in range(int(tt[t, 6]))}
    assert set(cover) == want and all(c == 1 for c in cover.values())
    for tile, *_ in plan["splits"].tolist():
        assert int(tt[tile, 0]) >= 0   # packed tiles (n_full = 0) are never split


@pytest.mark.parametrize("concurrency", [20, 50, 100])
def test_packed_tiles_never_outlast_the_split_parts(concurrency):
    """With a concurrency that splits the plain tiles (fewer than 2C tiles), a
    packed tile (never split itself) holds at most kv_split KV tiles; the
    packing still gives every row its causal keys (checked above)."""
    lengths = [16, 24, 8, 40, 16, 8, 32, 200, 8, 24]
    cp, rank, bt, bn = 2, 0, 8, 4
    plain = metadata.tiles(lengths, cp, rank, bt, bn)
    split = metadata.kv_split_for(plain, concurrency)
    assert split > 0
    cap = min(int(plain[:, 6].max()), split)
    tt, rows, _ = metadata.packed_plan(lengths, cp, rank, bt, bn, concurrency=concurrency)
    packed = tt[tt[:, 0] < 0]
    assert packed.shape[0] > 0 and int(packed[:, 6].max()) <= cap
    if concurrency == 100:
        free, _, _ = metadata.packed_plan(lengths, cp, rank, bt, bn)
        assert int(free[free[:, 0] < 0][:, 6].max()) > cap   # the cap binds here
