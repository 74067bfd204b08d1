"""GPU parity of the paged compressed cache: the pool the packer writes equals the
oracle's (every stored record of the contiguous cache at its page), byte for byte,
when packed fresh and while growing one token at a time across block starts with
pages recycled; decode over the paged cache equals tria_decode over the contiguous
cache bit for bit and the oracle's decode within tolerance."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from test_gpu_parity import assert_close, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tria():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_sparse_mixed_head_amd as t
    return t


def _held_pages(table: np.ndarray, P: int, rmax: int):
    pages = table[64 + 64 * P:].view(np.int32).reshape(P, rmax)
    return pages[pages >= 0]


def _pool_matches(pool_gpu: torch.Tensor, pool_ref: np.ndarray, pages, page: int):
    got = pool_gpu.cpu().numpy().reshape(-1, page)
    ref = pool_ref.reshape(-1, page)
    for pg in pages:
        assert np.array_equal(got[pg], ref[pg]), f"page {pg}"


def _records_match(pool_gpu: torch.Tensor, pool_ref: np.ndarray, table: np.ndarray, P: int, blk: int, d: int,
                   page: int):
    """Held records equal, each over its own length (an int4 record fills only part of
    its page; the rest of a recycled page is not part of the cache)."""
    got = pool_gpu.cpu().numpy().reshape(-1, page)
    ref = pool_ref.reshape(-1, page)
    rmax = table[:64].view(np.int32)[6]
    ent = table[64:64 + 64 * P].view(np.int32).reshape(P, 16)
    pages = table[64 + 64 * P:].view(np.int32).reshape(P, rmax)
    for p in range(P):
        n8, n4 = int(ent[p, 2]), int(ent[p, 3])
        for j in range(n8 + n4):
            pg = pages[p, j]
            ln = 2 * blk * d + 8 * blk if j < n8 else blk * d + 8 * blk
            bad = np.nonzero(got[pg, :ln] != ref[pg, :ln])[0]
            assert bad.size == 0, f"pair {p} record {j} (n8 {n8}) page {pg}: first bad byte {bad[:1]}"


PAGED = [
    # (b, hq, hk, d, n, blk, ctx, hi, keep)
    (2, 8, 2, 128, 1300, 128, 1300, [0, 2], [3, 10]),
    (3, 7, 1, 128, 700, 64, 650, [2], [4]),
    (1, 32, 1, 128, 512, 128, 500, [1], [2]),
    (2, 4, 2, 64, 900, 64, 897, [1, 0], [5, 9]),
    (1, 2, 2, 64, 64, 64, 1, [0, 0], [0, 0]),
]


@pytest.mark.parametrize("case", PAGED, ids=[f"b{c[0]}h{c[1]}k{c[2]}d{c[3]}ctx{c[6]}B{c[5]}" for c in PAGED])
def test_paged_pack_and_decode(tria, case):
    print(f"[case] paged {case}", flush=True)
    b, hq, hk, d, n, blk, ctx, hi, keep = case
    cfg = synth.Config("paged", b, hq, hk, d, n, blk, seed=71, decode=True)
    k, v, q = synth.make_decode_inputs(cfg)
    hi, keep = np.array(hi, np.int32), np.array(keep, np.int32)
    dd = tria.make_dims(b, hq, hk, d, blk, n)
    page = tria.paged_page_bytes(dd)
    P, rmax = b * hk, (ctx - 1) // blk + 1
    n_pages = P * rmax + 7
    free = np.random.default_rng(3).permutation(n_pages).astype(np.int32)   # scattered pages
    table, used, _ = tria.build_paged_table(dd, hi, keep, ctx, n_pages, free)
    pool = torch.zeros(n_pages * page, dtype=torch.uint8, device="cuda")
    kd, vd = dev(k), dev(v)
    tdev = torch.from_numpy(table).cuda()
    tria.pack_kv_cache_paged(dd, hi, keep, ctx, kd, vd, tdev, pool)
    sm = 1.0 / math.sqrt(d)
    out = tria.decode_paged(dd, tdev, pool, ctx, dev(q), sm)
    cache = tria.pack_kv_cache(dd, hi, keep, ctx, kd, vd)
    plain = tria.decode(dd, cache, ctx, dev(q), sm)
    torch.cuda.synchronize()
    ref_pool = oracle.pack_paged(k, v, hi, keep, hq, blk, ctx, table, np.zeros(n_pages * page, np.uint8))
    _pool_matches(pool, ref_pool, _held_pages(table, P, rmax), page)
    assert torch.equal(out, plain)
    assert_close(out.cpu().numpy(), oracle.decode(k, v, q, hi, keep, blk, ctx, sm), f"paged decode {case}")


@pytest.mark.parametrize("case", [
    (2, 8, 2, 128, 1200, 128, 250, 140, [1, 3], [4, 9]),
    (1, 4, 4, 64, 700, 64, 1, 200, [0, 2, 5, 0], [0, 6, 5, 30]),
], ids=["b2k2d128B128", "b1k4d64B64"])
def test_paged_growth_token_by_token(tria, case):
    """One token at a time: the host rebuilds the table from the previous one (pages
    recycled through a free stack), the packer writes only what changed, and after
    every step the held pages equal the oracle's records and decode equals the
    contiguous decode bit for bit."""
    b, hq, hk, d, n, blk, ctx0, steps, hi, keep = case
    print(f"[case] paged growth {case}", flush=True)
    cfg = synth.Config("paged-grow", b, hq, hk, d, n, blk, seed=73, decode=True)
    k, v, q = synth.make_decode_inputs(cfg)
    hi, keep = np.array(hi, np.int32), np.array(keep, np.int32)
    dd = tria.make_dims(b, hq, hk, d, blk, n)
    page = tria.paged_page_bytes(dd)
    P = b * hk
    n_pages = P * ((ctx0 + steps - 1) // blk + 1) + 5
    free = list(np.random.default_rng(9).permutation(n_pages).astype(np.int32))
    pool = torch.zeros(n_pages * page, dtype=torch.uint8, device="cuda")
    kd, vd, qd = dev(k), dev(v), dev(q)
    sm = 1.0 / math.sqrt(d)
    old, old_dev = None, None
    for ctx in range(ctx0, ctx0 + steps):
        table, used, rel = tria.build_paged_table(dd, hi, keep, ctx, n_pages, np.array(free, np.int32), old)
        free = free[used:] + list(rel)
        tdev = torch.from_numpy(table).cuda()
        tria.pack_kv_cache_paged(dd, hi, keep, ctx, kd, vd, tdev, pool, old_table=old_dev)
        out = tria.decode_paged(dd, tdev, pool, ctx, qd, sm)
        plain = tria.decode(dd, tria.pack_kv_cache(dd, hi, keep, ctx, kd, vd), ctx, qd, sm)
        torch.cuda.synchronize()
        assert torch.equal(out, plain), ctx
        c = (ctx - 1) // blk
        if ctx == ctx0 + steps - 1 or (ctx - 1) % blk == 0:   # block starts and the last step
            rmax = c + 1
            ref_pool = oracle.pack_paged(k, v, hi, keep, hq, blk, ctx, table, np.zeros(n_pages * page, np.uint8))
            _pool_matches(pool, ref_pool, _held_pages(table, P, rmax), page)
        old, old_dev = table, tdev


def test_paged_growth_in_jumps(tria):
    """Growth by several tokens at a time (within a block, across one, at a block's
    end): the old table's partly filled current block keeps its page but is rewritten,
    so after every step the held pages equal the oracle's records and decode equals
    the contiguous decode bit for bit."""
    b, hq, hk, d, n, blk = 2, 8, 2, 128, 700, 64
    hi, keep = np.array([1, 2], np.int32), np.array([5, 4], np.int32)
    cfg = synth.Config("paged-jumps", b, hq, hk, d, n, blk, seed=77, decode=True)
    k, v, q = synth.make_decode_inputs(cfg)
    dd = tria.make_dims(b, hq, hk, d, blk, n)
    page = tria.paged_page_bytes(dd)
    P = b * hk
    n_pages = P * ((n - 1) // blk + 1) + 5
    free = list(np.random.default_rng(11).permutation(n_pages).astype(np.int32))
    pool = torch.zeros(n_pages * page, dtype=torch.uint8, device="cuda")
    kd, vd, qd = dev(k), dev(v), dev(q)
    sm = 1.0 / math.sqrt(d)
    old, old_dev = None, None
    for ctx in (70, 100, 128, 129, 190, 300, 320, 321, 700):
        print(f"[case] paged jumps ctx {ctx}", flush=True)
        table, used, rel = tria.build_paged_table(dd, hi, keep, ctx, n_pages, np.array(free, np.int32), old)
        free = free[used:] + list(rel)
        tdev = torch.from_numpy(table).cuda()
        tria.pack_kv_cache_paged(dd, hi, keep, ctx, kd, vd, tdev, pool, old_table=old_dev)
        out = tria.decode_paged(dd, tdev, pool, ctx, qd, sm)
        plain = tria.decode(dd, tria.pack_kv_cache(dd, hi, keep, ctx, kd, vd), ctx, qd, sm)
        torch.cuda.synchronize()
        assert torch.equal(out, plain), ctx
        ref_pool = oracle.pack_paged(k, v, hi, keep, hq, blk, ctx, table, np.zeros(n_pages * page, np.uint8))
        _records_match(pool, ref_pool, table, P, blk, d, page)
        old, old_dev = table, tdev


def test_paged_decode_rejects_bad_table(tria):
    """A page outside the pool makes its pair's query heads NaN (the wavefronts that
    meet it poison their sums); a table whose header does not match gives NaN
    everywhere and reads no record."""
    b, hq, hk, d, n, blk, ctx, hi, keep = PAGED[0]
    cfg = synth.Config("paged", b, hq, hk, d, n, blk, seed=71, decode=True)
    k, v, q = synth.make_decode_inputs(cfg)
    hi, keep = np.array(hi, np.int32), np.array(keep, np.int32)
    dd = tria.make_dims(b, hq, hk, d, blk, n)
    page = tria.paged_page_bytes(dd)
    P, rmax = b * hk, (ctx - 1) // blk + 1
    n_pages = P * rmax
    table, _, _ = tria.build_paged_table(dd, hi, keep, ctx, n_pages, np.arange(n_pages, dtype=np.int32))
    pool = torch.zeros(n_pages * page, dtype=torch.uint8, device="cuda")
    tdev = torch.from_numpy(table).cuda()
    tria.pack_kv_cache_paged(dd, hi, keep, ctx, dev(k), dev(v), tdev, pool)
    bad = table.copy()
    bad[64 + 64 * P:64 + 64 * P + 4] = np.frombuffer(np.int32(n_pages + 3).tobytes(), np.uint8)  # page past the pool
    o = tria.decode_paged(dd, torch.from_numpy(bad).cuda(), pool, ctx, dev(q), 0.125)
    torch.cuda.synchronize()
    G = hq // hk
    assert torch.isnan(o[0, :G]).all().item()          # pair (0, 0): its heads are NaN
    assert torch.isfinite(o[0, G:]).all().item() and torch.isfinite(o[1]).all().item()
    bad = table.copy()
    bad[0] = 0   # magic
    o = tria.decode_paged(dd, torch.from_numpy(bad).cuda(), pool, ctx, dev(q), 0.125)
    torch.cuda.synchronize()
    assert torch.isnan(o).all().item()


def test_paged_full_size(tria):
    """The decode workload (b16, 32/8 heads, d128, ctx 32768, block 128) in pages handed
    out in a scattered order: every held page equals the oracle's record byte for byte,
    and the paged decode equals the contiguous decode bit for bit."""
    cfg = synth.CONFIGS["decode_b16"]
    print("[case] paged full-size decode workload", flush=True)
    k, v, q = synth.make_decode_inputs(cfg)
    hi, keep = cfg.policy()
    dd = tria.make_dims(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.block, cfg.seq_len)
    ctx, page = cfg.seq_len, tria.paged_page_bytes(dd)
    P, rmax = cfg.batch * cfg.n_kv_heads, (ctx - 1) // cfg.block + 1
    n_pages = P * rmax
    free = np.random.default_rng(11).permutation(n_pages).astype(np.int32)
    table, used, _ = tria.build_paged_table(dd, hi, keep, ctx, n_pages, free)
    pool = torch.zeros(n_pages * page, dtype=torch.uint8, device="cuda")
    kd, vd = dev(k), dev(v)
    tdev = torch.from_numpy(table).cuda()
    tria.pack_kv_cache_paged(dd, hi, keep, ctx, kd, vd, tdev, pool)
    sm = 1.0 / math.sqrt(cfg.head_dim)
    out = tria.decode_paged(dd, tdev, pool, ctx, dev(q), sm)
    plain = tria.decode(dd, tria.pack_kv_cache(dd, hi, keep, ctx, kd, vd), ctx, dev(q), sm)
    torch.cuda.synchronize()
    assert torch.equal(out, plain)
    ref_pool = oracle.pack_paged(k, v, hi, keep, cfg.n_q_heads, cfg.block, ctx, table, np.zeros(n_pages * page, np.uint8))
    _pool_matches(pool, ref_pool, _held_pages(table, P, rmax), page)


def test_varlen_paged_continuous_batching(tria):
    """Three sequences in one paged cache advance at their own pace (a random subset
    grows by one token per step) and a slot now and then starts a new sequence with
    other keys and values, shorter or longer than the one it held, under a new
    sequence id.  Each step: host table from the previous one, the packer writes only
    what changed, and decode equals the contiguous variable-length decode of the same
    lengths and contents bit for bit; every 25 steps the held pages equal the oracle's
    records."""
    b, hq, hk, d, n, blk = 3, 8, 2, 128, 700, 64
    cfg = synth.Config("paged-varlen", b, hq, hk, d, n, blk, seed=79, decode=True)
    k, v, q = synth.make_decode_inputs(cfg)
    k_alt, v_alt, _ = synth.make_decode_inputs(cfg.scaled(seed=80))   # contents of new sequences
    hi, keep = np.array([1, 3], np.int32), np.array([4, 8], np.int32)
    dd = tria.make_dims(b, hq, hk, d, blk, n)
    page = tria.paged_page_bytes(dd)
    P = b * hk
    n_pages = P * ((n - 1) // blk + 1)
    rng = np.random.default_rng(23)
    free = list(rng.permutation(n_pages).astype(np.int32))
    pool = torch.zeros(n_pages * page, dtype=torch.uint8, device="cuda")
    kd, vd, qd = dev(k), dev(v), dev(q)
    sm = 1.0 / math.sqrt(d)
    lens = np.array([1, 100, 250], np.int64)
    ids = np.arange(b, dtype=np.int64)
    k, v = k.copy(), v.copy()      # the slots' current contents (host copies for the oracle)

    def restart(slot, length):
        """A new sequence in `slot`: other keys and values, a new id."""
        k[slot], k_alt[slot] = k_alt[slot].copy(), k[slot].copy()
        v[slot], v_alt[slot] = v_alt[slot].copy(), v[slot].copy()
        kd[slot].copy_(dev(k[slot:slot + 1])[0])
        vd[slot].copy_(dev(v[slot:slot + 1])[0])
        ids[slot] += 10
        lens[slot] = length

    old, old_dev = None, None
    for step in range(150):
        if step % 25 == 0:
            print(f"[case] paged varlen step {step} lens {lens.tolist()}", flush=True)
        table, used, rel = tria.build_paged_table(dd, hi, keep, lens, n_pages, np.array(free, np.int32), old,
                                                  seq_ids=ids)
        free = free[used:] + list(rel)
        tdev = torch.from_numpy(table).cuda()
        tria.pack_kv_cache_paged(dd, hi, keep, lens, kd, vd, tdev, pool, old_table=old_dev)
        out = tria.decode_paged_varlen(dd, tdev, pool, qd, sm)
        cont = tria.pack_kv_cache_varlen(dd, hi, keep, lens, kd, vd)
        ref = tria.decode_varlen(dd, cont, qd, sm)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), step
        if step % 25 == 24:
            rmax = int((lens.max() - 1) // blk + 1)
            ref_pool = oracle.pack_paged(k, v, hi, keep, hq, blk, lens, table, np.zeros(n_pages * page, np.uint8))
            _pool_matches(pool, ref_pool, _held_pages(table, P, rmax), page)
        old, old_dev = table, tdev
        last = (lens.copy(), out.cpu().numpy())
        lens = np.minimum(lens + (rng.random(b) < 0.7), n)
        if step in (60, 110):
            restart(step % b, 5 + step % 40)                    # a new, shorter sequence
        if step in (40, 90):
            slot = int(np.argmin(lens))
            restart(slot, min(n, int(lens[slot]) + 150))         # a new, longer sequence
    # the last step against the oracle's decode of each sequence alone
    for i in range(b):
        r = oracle.decode(k[i:i + 1], v[i:i + 1], q[i:i + 1], hi, keep, blk, int(last[0][i]), sm)
        assert_close(last[1][i:i + 1], r, f"paged varlen sequence {i}")
