"""Paged cache page tables (host, CPU): the library's table builder against the
oracle's, byte for byte, over token-by-token growth across block starts with a
free-page stack; invariants (every record one page, pages unique and inside the
pool, released pages exactly those dropped) and argument validation."""
import numpy as np
import pytest

import oracle

tria = pytest.importorskip("block_sparse_mixed_head_amd")


def _grow(b, hq, hk, d, blk, hi, keep, ctx0, steps, n_pages, seed):
    dd = tria.make_dims(b, hq, hk, d, blk, ctx0 + steps + 1)
    rng = np.random.default_rng(seed)
    free = list(rng.permutation(n_pages).astype(np.int32))   # stack: front = next page handed out
    old = old_ref = None
    for ctx in range(ctx0, ctx0 + steps + 1):
        t, used, rel = tria.build_paged_table(dd, hi, keep, ctx, n_pages, free, old)
        r, rused, rrel = oracle.paged_table(b, hq, hk, d, blk, ctx, hi, keep, n_pages, old_ref, free)
        assert np.array_equal(t, r), ctx
        assert used == rused and np.array_equal(rel, rrel), ctx
        P, rmax = b * hk, (ctx - 1) // blk + 1
        pages = t[64 + 64 * P:].view(np.int32).reshape(P, rmax)
        held = pages[pages >= 0]
        assert len(np.unique(held)) == held.size and held.max() < n_pages
        if old is not None:
            oP = old[64 + 64 * P:].view(np.int32)
            assert set(oP[oP >= 0]) - set(held) == set(rel.tolist())
        free = free[used:] + list(rel)
        old, old_ref = t, r
    return dd


@pytest.mark.parametrize("case", [
    (2, 8, 2, 128, 64, [1, 3], [4, 9], 60, 200, 400),
    (1, 4, 4, 64, 128, [0, 2, 5, 0], [0, 6, 5, 30], 1, 300, 200),
    (1, 2, 1, 64, 64, [40], [40], 1, 130, 10),
])
def test_paged_table_matches_oracle_while_growing(case):
    b, hq, hk, d, blk, hi, keep, ctx0, steps, n_pages = case
    _grow(b, hq, hk, d, blk, np.array(hi, np.int32), np.array(keep, np.int32), ctx0, steps, n_pages, seed=5)


def test_paged_table_validation():
    from block_sparse_mixed_head_amd import TriaError
    dd = tria.make_dims(1, 4, 2, 64, 64, 1000)
    hi, keep = np.array([1, 2], np.int32), np.array([4, 4], np.int32)
    t, used, rel = tria.build_paged_table(dd, hi, keep, 300, 64, np.arange(64, dtype=np.int32))
    assert used > 0 and rel.size == 0
    with pytest.raises(TriaError):   # too few free pages
        tria.build_paged_table(dd, hi, keep, 300, 64, np.arange(2, dtype=np.int32))
    with pytest.raises(TriaError):   # a free page outside the pool
        tria.build_paged_table(dd, hi, keep, 300, 8, np.arange(20, dtype=np.int32))
    with pytest.raises(TriaError):   # a free page given twice
        tria.build_paged_table(dd, hi, keep, 300, 64, np.zeros(20, np.int32))
    with pytest.raises(TriaError):   # a free page the old table still holds
        tria.build_paged_table(dd, hi, keep, 321, 64, np.arange(64, dtype=np.int32), t)
    with pytest.raises(TriaError):   # another policy than the old table's
        tria.build_paged_table(dd, np.array([2, 2], np.int32), keep, 321, 64, np.arange(used, 64, dtype=np.int32), t)
    bad = t.copy()
    bad[0] = 0
    with pytest.raises(TriaError):   # not a page table
        tria.build_paged_table(dd, hi, keep, 321, 64, np.arange(used, 64, dtype=np.int32), bad)


def test_varlen_paged_table_matches_oracle():
    """Sequences of one batch advance at their own pace (continuous batching): each step
    a random subset grows by one token, and now and then a slot starts a new sequence,
    shorter or longer than the one it held, under a new sequence id (its old pages all
    released, none reused).  Library table == oracle table every step."""
    b, hq, hk, d, blk = 4, 8, 2, 64, 64
    hi, keep = np.array([1, 2], np.int32), np.array([5, 9], np.int32)
    dd = tria.make_dims(b, hq, hk, d, blk, 2000)
    rng = np.random.default_rng(17)
    n_pages = 400
    free = list(rng.permutation(n_pages).astype(np.int32))
    lens = np.array([1, 60, 64, 300], np.int64)
    ids = np.arange(b, dtype=np.int64)
    P = b * hk
    old = old_ref = None
    restarted = None
    n_longer = 0
    for step in range(260):
        t, used, rel = tria.build_paged_table(dd, hi, keep, lens, n_pages, free, old, seq_ids=ids)
        r, rused, rrel = oracle.paged_table(b, hq, hk, d, blk, lens, hi, keep, n_pages, old_ref, free, seq_ids=ids)
        assert np.array_equal(t, r), step
        assert used == rused and np.array_equal(rel, rrel), step
        ents = t[64:64 + 64 * P].reshape(P, 64)
        assert np.array_equal(ents[:, 48:56].view(np.int64)[:, 0], np.repeat(ids, hk)), step
        if restarted is not None:   # the restarted slot's pairs hold none of their old pages
            rm, orm = t[:64].view(np.int32)[6], old[:64].view(np.int32)[6]
            new_pages = t[64 + 64 * P:].view(np.int32).reshape(P, rm)
            old_pages = old[64 + 64 * P:].view(np.int32).reshape(P, orm)
            for p in range(restarted * hk, (restarted + 1) * hk):
                held, before = set(new_pages[p][new_pages[p] >= 0]), set(old_pages[p][old_pages[p] >= 0])
                assert not held & before and before <= set(rel.tolist()), (step, p)
            restarted = None
        free = free[used:] + list(rel)
        old, old_ref = t, r
        grow = rng.random(b) < 0.7
        lens = lens + grow
        if step % 37 == 36:
            lens[step % b] = 1 + step % 50        # a new, shorter sequence in this slot
            ids[step % b] += 100
            restarted = step % b
        elif step % 29 == 28 and lens[(step + 1) % b] < 1700:
            restarted = (step + 1) % b            # a new, longer sequence in this slot
            lens[restarted] += 1 + int(rng.integers(1, 250))
            ids[restarted] += 1000
            n_longer += 1
    assert n_longer >= 5
    hdr = t[:64].view(np.int32)
    assert hdr[7] == -1 and t[32:40].view(np.int64)[0] == 0
