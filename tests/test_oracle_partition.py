"""Pins of the oracle's partition and metadata (CPU only).

Each test checks the oracle against something other than itself: a
hand-derived fixture, a closed form, or a brute-force enumeration.
"""
import numpy as np
import pytest

import workloads
from golden_io import read_records, runs_to_positions
from oracle import metadata, partition


def test_tiny_partition_matches_hand_derivation():
    g = read_records("partition_tiny.txt")
    lengths = g["lengths"][0]
    cp = g["cp"][0][0]
    assert partition.q_global(lengths, cp, 0).tolist() == runs_to_positions(g["runs0"][0])
    assert partition.q_global(lengths, cp, 1).tolist() == runs_to_positions(g["runs1"][0])
    rows = partition.kv_row(lengths, cp)
    for tok, row in g["kv_row"][0]:
        assert int(rows[tok]) == row, tok
    for r in range(cp):
        assert partition.visible_count(lengths, cp, r) == g["pairs"][0][0]


@pytest.mark.parametrize("cp", [1, 2, 3, 4, 8])
def test_partition_invariants_random(cp):
    rng = np.random.default_rng(100 + cp)
    lengths = workloads.random_lengths(rng, 7, cp, 9)
    total = int(lengths.sum())
    cu = partition.cu_seqlens(lengths)
    allq = np.concatenate([partition.q_global(lengths, cp, r) for r in range(cp)])
    # the ranks' query maps partition [0, T)
    assert sorted(allq.tolist()) == list(range(total))
    # kv_row is the inverse of the gathered (rank-major) order
    rows = partition.kv_row(lengths, cp)
    assert sorted(rows.tolist()) == list(range(total))
    assert np.array_equal(rows[allq], np.arange(total))
    # symmetric ownership: within each document rank r holds exactly chunks r and 2cp-1-r
    for r in range(cp):
        qg = partition.q_global(lengths, cp, r)
        for i, length in enumerate(lengths.tolist()):
            c = length // (2 * cp)
            mine = [g for g in qg.tolist() if cu[i] <= g < cu[i + 1]]
            assert sorted({(g - cu[i]) // c for g in mine}) == sorted({r, 2 * cp - 1 - r})
            assert len(mine) == 2 * c
    # chunk_off is the gathered row of every chunk's first token, and chunks are contiguous there
    offs = partition.chunk_off(lengths, cp)
    for i, length in enumerate(lengths.tolist()):
        c = length // (2 * cp)
        for k in range(2 * cp):
            start = cu[i] + k * c
            assert list(rows[start:start + c]) == list(range(offs[i * 2 * cp + k], offs[i * 2 * cp + k] + c))


@pytest.mark.parametrize("cp", [1, 2, 4, 8])
def test_load_balance_closed_form(cp):
    rng = np.random.default_rng(7 * cp)
    lengths = workloads.random_lengths(rng, 5, cp, 12)
    closed = metadata.useful_pairs_closed_form(lengths, cp)
    for r in range(cp):
        assert partition.visible_count(lengths, cp, r) == closed


def test_partition_rejects_bad_input():
    with pytest.raises(partition.PartitionError):
        partition.q_global([6, 8], 2, 0)       # 6 % 4 != 0
    with pytest.raises(partition.PartitionError):
        partition.q_global([8], 2, 2)          # rank >= cp
    with pytest.raises(partition.PartitionError):
        partition.q_global([], 1, 0)
    with pytest.raises(partition.PartitionError):
        partition.q_global([0, 4], 1, 0)


def test_small_tiles_match_hand_derivation():
    g = read_records("tiles_small.txt")
    lengths, cp, rank, bt, bn = [8, 16], 2, 1, 2, 4
    tt = metadata.tiles(lengths, cp, rank, bt, bn)
    assert tt.tolist() == g["tile"]
    assert metadata.order(tt).tolist() == g["order"][0]
    assert metadata.kvtiles(lengths, cp, rank, bt, bn).tolist() == g["kvtile"]


def _visible_pairs(lengths, cp, rank):
    """Brute force: all (local row, global key) pairs the mask leaves open."""
    cu = partition.cu_seqlens(lengths)
    docs = partition.doc_of(lengths)
    out = set()
    for row, g in enumerate(partition.q_global(lengths, cp, rank).tolist()):
        for key in range(cu[int(docs[g])], g + 1):
            out.add((row, key))
    return out


@pytest.mark.parametrize("lengths,cp", [([8, 16, 8, 24], 1), ([8, 16, 8, 24], 2), ([8, 16, 8, 24], 4),
                                        ([24, 8], 2), ([16], 4)])
@pytest.mark.parametrize("bt,bn", [(1, 1), (2, 3), (3, 2), (4, 8), (8, 4)])
def test_tiles_cover_visible_pairs_exactly(lengths, cp, bt, bn):
    for rank in range(cp):
        want = _visible_pairs(lengths, cp, rank)
        tt = metadata.tiles(lengths, cp, rank, bt, bn)
        seen = []
        for q0, qg0, nr, doc, slot, kv0, n_kv, n_full in tt.tolist():
            assert 1 <= nr <= bt
            for j in range(n_kv):
                keys = range(kv0 + j * bn, kv0 + min((j + 1) * bn, qg0 + nr - kv0))
                pairs = [(q0 + o, key) for o in range(nr) for key in keys if key <= qg0 + o]
                assert pairs, "a visited KV tile must hold a visible pair"
                if j < n_full:
                    assert len(pairs) == nr * len(keys), "a full tile needs no mask"
                seen.extend(pairs)
        assert len(seen) == len(set(seen)) == len(want)
        assert set(seen) == want
        order = metadata.order(tt)
        assert sorted(order.tolist()) == list(range(tt.shape[0]))
        n_kv = tt[order, 6]
        assert all(n_kv[:-1] >= n_kv[1:])
        # backward tiles: each visible pair covered once by (kv tile, q tile in [begin, end))
        seen_b = []
        for doc, ks, nk, qb, qe, *_ in metadata.kvtiles(lengths, cp, rank, bt, bn).tolist():
            for t in range(qb, qe):
                q0, qg0, nr = tt[t, 0], tt[t, 1], tt[t, 2]
                assert tt[t, 3] == doc
                seen_b.extend((q0 + o, key) for o in range(nr) for key in range(ks, ks + nk)
                              if key <= qg0 + o)
        assert len(seen_b) == len(set(seen_b)) == len(want)
        assert set(seen_b) == want


def test_kvtiles_cover_every_key_once():
    lengths, cp = [16, 32, 8], 2
    cu = partition.cu_seqlens(lengths)
    for rank in range(cp):
        tt = metadata.tiles(lengths, cp, rank, 2, 4)
        kt = metadata.kvtiles(lengths, cp, rank, 2, 4)
        keys_seen = {key for _, key in _visible_pairs(lengths, cp, rank)}
        covered = [key for doc, ks, nk, *_ in kt.tolist() for key in range(ks, ks + nk)]
        assert covered == list(range(cu[-1]))
        for doc, ks, nk, qb, qe, *_ in kt.tolist():
            assert cu[doc] <= ks and ks + nk <= cu[doc + 1]
            if qb == qe:
                # an empty range only for keys no local query sees
                assert not keys_seen & set(range(ks, ks + nk))
                continue
            # the first q tile listed sees the tile's first key, the one before it does not
            assert tt[qb, 1] + tt[qb, 2] - 1 >= ks
            if qb > 0 and tt[qb - 1, 3] == doc:
                assert tt[qb - 1, 1] + tt[qb - 1, 2] - 1 < ks


@pytest.mark.parametrize("w", workloads.WORKLOADS, ids=lambda w: w.name)
def test_workload_lengths_are_valid(w):
    lengths = workloads.draw_lengths(w, np.random.default_rng(w.index))
    assert int(lengths.sum()) == w.total
    assert all(int(x) % (2 * w.cp) == 0 and int(x) > 0 for x in lengths)


def test_work_items_match_hand_derivation():
    g = read_records("items_small.txt")
    tt = metadata.tiles([64], 1, 0, 8, 4)
    items, splits = metadata.items_and_splits(tt, 8)
    assert items.tolist() == g["itemA"] and splits.tolist() == g["splitA"]
    tt = metadata.tiles([256], 1, 0, 128, 4)
    items, splits = metadata.items_and_splits(tt, 12)
    assert items.tolist() == g["itemB"] and splits.tolist() == g["splitB"]


@pytest.mark.parametrize("concurrency", [0, 1, 3, 16, 64, 1000])
def test_work_items_cover_each_tile_once(concurrency):
    rng = np.random.default_rng(concurrency)
    for cp in (1, 2, 4):
        lengths = workloads.random_lengths(rng, 5, cp, 60)
        for rank in range(cp):
            tt = metadata.tiles(lengths, cp, rank, 8, 4)
            items, splits = metadata.items_and_splits(tt, concurrency)
            lens = items[:, 2] - items[:, 1]
            assert all(lens[:-1] >= lens[1:])
            split_tiles = {int(r[0]): r for r in splits.tolist()}
            slots = []
            for t in range(tt.shape[0]):
                mine = sorted((int(b), int(e), int(s)) for tile, b, e, s in items.tolist() if tile == t)
                # the parts tile [0, n_kv) exactly, in order
                assert mine[0][0] == 0 and mine[-1][1] == tt[t, 6]
                assert all(mine[i][1] == mine[i + 1][0] for i in range(len(mine) - 1))
                if len(mine) == 1:
                    assert mine[0][2] == -1 and t not in split_tiles
                    continue
                first, count = split_tiles[t][1], split_tiles[t][2]
                assert [m[2] for m in mine] == list(range(first, first + count))
                slots.extend(m[2] for m in mine)
                # every part starts with a KV tile all rows see whole
                assert all(m[0] <= tt[t, 7] - 1 for m in mine)
            assert sorted(slots) == list(range(len(slots)))


def test_pad_lengths_closed_form():
    rng = np.random.default_rng(3)
    for cp in (1, 2, 3, 8):
        real = rng.integers(1, 200, size=40).tolist()
        padded = partition.pad_lengths(real, cp)
        for r, length in zip(real, padded):
            assert length % (2 * cp) == 0 and r <= length < r + 2 * cp
    assert partition.pad_lengths([1, 4, 5], 2) == [4, 4, 8]
    with pytest.raises(partition.PartitionError):
        partition.pad_lengths([3, 0], 2)


def test_pad_rows_are_the_tokens_past_each_real_end():
    real, cp = [1, 5, 8, 21], 2
    lengths = partition.pad_lengths(real, cp)
    cu = partition.cu_seqlens(lengths)
    total_pads = 0
    for rank in range(cp):
        pad = partition.pad_rows(real, cp, rank)
        qg = partition.q_global(lengths, cp, rank)
        docs = partition.doc_of(lengths)
        for l, g in enumerate(qg.tolist()):
            assert pad[l] == (g >= cu[int(docs[g])] + real[int(docs[g])])
        total_pads += int(pad.sum())
    assert total_pads == sum(lengths) - sum(real)
    ends = metadata.doc_end(lengths, cp, real)
    assert ends.tolist() == [cu[i] + real[i] for i in range(len(real))]
    assert metadata.doc_end(lengths, cp).tolist() == cu[1:]


def test_pass_plans_match_hand_derived_fixture():
    g = read_records("pass_plan_small.txt")
    cases = {"A": ([16, 32, 16], 2, 0, 4, 4, [1]), "B": ([16], 2, 1, 2, 2, [0, 1]),
             "C": ([16], 2, 1, 2, 2, [0])}
    for name, (lengths, cp, rank, bt, bn, shards) in cases.items():
        items, table = metadata.pass_plan(lengths, cp, rank, bt, bn, shards)
        assert items.tolist() == g["item" + name], name
        assert table.tolist() == g["tile" + name], name


@pytest.mark.parametrize("seed", range(6))
def test_pass_plan_covers_each_visible_pair_of_the_shards_once(seed):
    """Brute force: every (local row, key) pair the causal + EOD mask leaves
    open and whose key lies in a listed shard is covered by exactly one KV tile
    of exactly one item; no item reaches a key outside the listed shards; the
    first n_full KV tiles of an item are wholly visible to all of its rows and
    every row sees the first key of each of its items."""
    rng = np.random.default_rng(300 + seed)
    cp = int(rng.choice([1, 2, 3, 4]))
    rank = int(rng.integers(0, cp))
    lengths = [2 * cp * int(x) for x in rng.integers(1, 7, size=int(rng.integers(1, 5)))]
    bt, bn = int(rng.choice([1, 2, 3, 5])), int(rng.choice([1, 2, 3, 4, 8]))
    shards = sorted({int(x) for x in rng.integers(0, cp, size=int(rng.integers(1, cp + 1)))})
    items, table = metadata.pass_plan(lengths, cp, rank, bt, bn, shards)
    tt = metadata.tiles(lengths, cp, rank, bt, bn)
    holder = partition.kv_row(lengths, cp) // (sum(lengths) // cp)
    cu = partition.cu_seqlens(lengths)
    docs = partition.doc_of(lengths)
    covered = {}
    for tile, lo, hi, slot, n_kv, n_full, _, _ in items.tolist():
        q_glob, n_rows = int(tt[tile, 1]), int(tt[tile, 2])
        assert n_kv == -(-(hi - lo) // bn) and 0 <= n_full <= n_kv
        for row_pos in range(q_glob, q_glob + n_rows):
            assert lo <= row_pos    # every row sees the item's first key
        for j in range(n_kv):
            for key in range(lo + j * bn, min(lo + (j + 1) * bn, hi)):
                assert int(holder[key]) in shards
                for row_pos in range(q_glob, q_glob + n_rows):
                    if j < n_full:
                        assert key <= row_pos
                    if key <= row_pos:
                        covered[(row_pos, key)] = covered.get((row_pos, key), 0) + 1
    want = set()
    for row_pos in partition.q_global(lengths, cp, rank).tolist():
        start = cu[int(docs[row_pos])]
        for key in range(start, row_pos + 1):
            if int(holder[key]) in shards:
                want.add((row_pos, key))
    assert set(covered) == want and all(c == 1 for c in covered.values())
    # the per-tile table lists each tile's part slots
    slots = sorted(int(x) for x in items[:, 3]) if items.size else []
    assert slots == list(range(len(slots)))
    for tile, first, n_parts, _ in table.tolist():
        mine = sorted(int(s) for t, _, _, s, *_ in items.tolist() if t == tile)
        assert mine == list(range(first, first + n_parts))
