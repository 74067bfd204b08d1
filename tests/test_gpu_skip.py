"""GPU parity of dynamic block skipping in decode (ETA page, rit.work: section on how
the model decides which part of the context to read): the statistics index
byte-exact against the oracle's, the keep bits bit-exact, and the skipping decode
against the oracle's masked decode.  Inputs: seeded keys with one magnitude per
(batch, KV head, block) and per-head thresholds gamma * ||q|| (synth)."""
import math
import os

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


def parse_summaries(buf: torch.Tensor, pairs: int, rmax: int, d: int):
    b = buf.cpu().numpy()
    hdr, h64 = b[:64].view(np.int32), b[:64].view(np.int64)
    S = 2 * d + 16
    body = b[64:64 + pairs * rmax * S].reshape(pairs, rmax, S)
    lo = body[:, :, :d].view(np.int8)
    hi = body[:, :, d:2 * d].view(np.int8)
    smax = np.ascontiguousarray(body[:, :, 2 * d:2 * d + 4]).view(np.float32)[..., 0]
    pad = np.ascontiguousarray(body[:, :, 2 * d + 4:2 * d + 8]).view(np.int32)[..., 0]
    nmax = np.ascontiguousarray(body[:, :, 2 * d + 8:2 * d + 16]).view(np.float64)[..., 0]
    return hdr, h64, lo, hi, smax, pad, nmax


def expected_stamps(cache: torch.Tensor, pairs: int, rmax: int, blk: int, ctx_of_pair) -> np.ndarray:
    """The index's per-slot stamps: the pair's current block + 1 on its stored records
    (n8 + n4 from the cache directory), 0 on unused slots."""
    dirs = cache[:64 + 64 * pairs].cpu().numpy()
    st = np.zeros((pairs, rmax), np.int32)
    for p in range(pairs):
        n8, n4 = (int(x) for x in dirs[64 + 64 * p + 8:64 + 64 * p + 16].view(np.int32))
        st[p, :n8 + n4] = (int(ctx_of_pair(p)) - 1) // blk + 1
    return st


SKIP_CASES = [
    # (b, hq, hk, d, n, blk, ctx, hi, keep)  policies per KV head
    (2, 8, 2, 128, 1300, 128, 1300, [0, 2], [3, 10]),
    (2, 4, 2, 64, 900, 64, 897, [1, 0], [5, 9]),
    (1, 32, 1, 128, 1100, 128, 1050, [1], [8]),              # G = 32: two row groups
    (3, 12, 4, 128, 700, 64, 650, [2, 0, 1, 5], [4, 9, 9, 5]),  # G = 3: lanes padded to 4
    (1, 4, 2, 128, 9000, 128, 8955, [3, 1], [40, 70]),       # 70 records per pair
    (1, 2, 2, 64, 64, 64, 1, [0, 0], [0, 0]),                 # a single token
    # more records than one pass of the plan stages in LDS (256 slots at G = 4, d = 128;
    # 512 at G = 1, d = 64, where lanes past the stage idle)
    (1, 4, 1, 128, 128 * 300, 128, 128 * 300 - 5, [3], [290]),
    (1, 2, 2, 64, 64 * 600, 64, 64 * 600 - 3, [5, 2], [560, 590]),
]
IDS = [f"b{c[0]}h{c[1]}k{c[2]}d{c[3]}ctx{c[6]}B{c[5]}" for c in SKIP_CASES]


def _setup(tria, case, seed=61):
    b, hq, hk, d, n, blk, ctx, hi, keep = case
    cfg = synth.Config("skip", b, hq, hk, d, n, blk, seed=seed, decode=True)
    k, v, q, th = synth.make_skip_decode_inputs(cfg)
    hi, keep = np.array(hi, np.int32), np.array(keep, np.int32)
    dd = tria.make_dims(b, hq, hk, d, blk, n)
    cache = tria.pack_kv_cache(dd, hi, keep, ctx, dev(k), dev(v))
    sums = tria.build_block_summaries(dd, cache, ctx)
    torch.cuda.synchronize()
    return k, v, q, th, hi, keep, dd, cache, sums


@pytest.mark.parametrize("case", SKIP_CASES, ids=IDS)
def test_summaries_and_masks_match_oracle(tria, case):
    print(f"[case] skip index + masks {case}", flush=True)
    b, hq, hk, d, n, blk, ctx = case[:7]
    k, v, q, th, hi, keep, dd, cache, sums = _setup(tria, case)
    rmax = (ctx - 1) // blk + 1
    assert sums.numel() == 64 + b * hk * rmax * (2 * d + 16)
    hdr, h64, lo, up, smax, pad, nmax = parse_summaries(sums, b * hk, rmax, d)
    assert list(hdr[:8]) == [0x4D534254, 2, b * hk, rmax, d, blk, rmax - 1, 0]
    assert h64[4] == cache.numel() and not h64[5:].any()
    rlo, rup, rsmax, rnmax = oracle.block_summaries(k, hi, keep, hq, blk, ctx)
    assert np.array_equal(lo, rlo) and np.array_equal(up, rup)
    assert np.array_equal(smax, rsmax) and np.array_equal(nmax, rnmax)
    assert np.array_equal(pad, expected_stamps(cache, b * hk, rmax, blk, lambda p: ctx))
    sm = 1.0 / math.sqrt(d)
    thd = torch.from_numpy(th).cuda()
    masks = tria.skip_masks(dd, cache, ctx, sums, dev(q), thd, sm).cpu().numpy().view(np.uint32)
    ref = oracle.skip_masks(k, q, hi, keep, blk, ctx, th, sm)
    assert np.array_equal(masks, ref)
    G = hq // hk
    full = (1 << G) - 1
    kept = [int(m) for m in ref.ravel() if m]
    print(f"[skip] records kept by every head {sum(m == full for m in kept)}, by some {len(kept)} "
          f"of {int((ref != 0).sum())} stored", flush=True)


@pytest.mark.parametrize("case", SKIP_CASES, ids=IDS)
def test_decode_skip_matches_oracle(tria, case):
    print(f"[case] skip decode {case}", flush=True)
    b, hq, hk, d, n, blk, ctx = case[:7]
    k, v, q, th, hi, keep, dd, cache, sums = _setup(tria, case)
    sm = 1.0 / math.sqrt(d)
    thd = torch.from_numpy(th).cuda()
    out = tria.decode_skip(dd, cache, ctx, sums, dev(q), thd, sm)
    torch.cuda.synchronize()
    ref = oracle.decode_skip(k, v, q, hi, keep, blk, ctx, th, sm)
    assert_close(out.cpu().numpy(), ref, f"skip decode {case}")
    # thresholds <= 0 keep everything: the plain decode, bit for bit
    zero = tria.decode_skip(dd, cache, ctx, sums, dev(q), torch.zeros_like(thd), sm)
    plain = tria.decode(dd, cache, ctx, dev(q), sm)
    torch.cuda.synchronize()
    assert torch.equal(zero, plain)
    # +inf keeps only the first and the current block
    inf = tria.decode_skip(dd, cache, ctx, sums, dev(q), torch.full_like(thd, float("inf")), sm)
    torch.cuda.synchronize()
    ref_inf = oracle.decode(k, v, q, np.zeros_like(hi), np.zeros_like(keep), blk, ctx, sm)
    assert_close(inf.cpu().numpy(), ref_inf, f"skip decode +inf {case}")


@pytest.mark.parametrize("grid", [1, 3])
def test_decode_skip_long_segments(tria, grid, monkeypatch):
    """Few work groups: each wavefront walks many kept records (several 64-entry
    windows of the kept list), in both the skipping and the plain decode."""
    case = (2, 8, 2, 128, 128 * 300, 128, 128 * 300 - 17, [4, 2], [150, 299])
    print(f"[case] skip decode grid {grid} {case}", flush=True)
    b, hq, hk, d, n, blk, ctx = case[:7]
    k, v, q, th, hi, keep, dd, cache, sums = _setup(tria, case)
    sm = 1.0 / math.sqrt(d)
    thd = torch.from_numpy(th * 0.8).cuda()   # more records kept
    monkeypatch.setenv("TRIA_DECODE_GRID", str(grid))
    out = tria.decode_skip(dd, cache, ctx, sums, dev(q), thd, sm)
    plain = tria.decode(dd, cache, ctx, dev(q), sm)
    torch.cuda.synchronize()
    monkeypatch.delenv("TRIA_DECODE_GRID")
    ref = oracle.decode_skip(k, v, q, hi, keep, blk, ctx, th * np.float32(0.8), sm)
    assert_close(out.cpu().numpy(), ref, f"skip decode grid {grid}")
    assert_close(plain.cpu().numpy(), oracle.decode(k, v, q, hi, keep, blk, ctx, sm), f"decode grid {grid}")


def test_decode_skip_rejects_stale_index(tria):
    case = SKIP_CASES[0]
    k, v, q, th, hi, keep, dd, cache, sums = _setup(tria, case)
    ctx, d = case[6], case[3]
    thd = torch.from_numpy(th).cuda()
    bad = sums.clone()
    bad[24:28] = torch.tensor([0, 0, 0, 0], dtype=torch.uint8)   # current block 0 instead of its own
    o = tria.decode_skip(dd, cache, ctx, bad, dev(q), thd, 1.0 / math.sqrt(d))
    torch.cuda.synchronize()
    assert torch.isnan(o).all().item()
    badc = cache.clone()
    badc[64 + 8:64 + 12] = torch.tensor([255, 255, 0, 0], dtype=torch.uint8)  # n8 of pair 0
    o = tria.decode_skip(dd, badc, ctx, sums, dev(q), thd, 1.0 / math.sqrt(d))
    torch.cuda.synchronize()
    assert torch.isnan(o).all().item()


def test_decode_skip_full_size(tria):
    """The decode workload (b16, 32/8 heads, d128, ctx 32768, block 128) with block
    structure in the keys: index and keep bits exact, outputs vs the oracle."""
    cfg = synth.CONFIGS["decode_b16"]
    print("[case] skip decode full-size decode workload", flush=True)
    k, v, q, th = synth.make_skip_decode_inputs(cfg)
    hi, keep = cfg.policy()
    dd = tria.make_dims(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.block, cfg.seq_len)
    ctx, d = cfg.seq_len, cfg.head_dim
    sm = 1.0 / math.sqrt(d)
    cache = tria.pack_kv_cache(dd, hi, keep, ctx, dev(k), dev(v))
    sums = tria.build_block_summaries(dd, cache, ctx)
    thd = torch.from_numpy(th).cuda()
    masks = tria.skip_masks(dd, cache, ctx, sums, dev(q), thd, sm)
    out = tria.decode_skip(dd, cache, ctx, sums, dev(q), thd, sm)
    torch.cuda.synchronize()
    ref_masks = oracle.skip_masks(k, q, hi, keep, cfg.block, ctx, th, sm)
    assert np.array_equal(masks.cpu().numpy().view(np.uint32), ref_masks)
    ref = oracle.decode_skip(k, v, q, hi, keep, cfg.block, ctx, th, sm)
    assert_close(out.cpu().numpy(), ref, "skip decode full size")


@pytest.mark.parametrize("case", SKIP_CASES[:5], ids=IDS[:5])
def test_skip_over_paged_cache_equals_contiguous(tria, case):
    """The same cache in scattered pages: its statistics index equals the contiguous
    cache's record for record (the header differs only in the size it names), and the
    skipping decode over the pages equals the contiguous one bit for bit."""
    print(f"[case] paged skip {case}", flush=True)
    b, hq, hk, d, n, blk, ctx = case[:7]
    k, v, q, th, hi, keep, dd, cache, sums = _setup(tria, case)
    page = tria.paged_page_bytes(dd)
    P, rmax = b * hk, (ctx - 1) // blk + 1
    n_pages = P * rmax + 3
    free = np.random.default_rng(5).permutation(n_pages).astype(np.int32)
    table, _, _ = tria.build_paged_table(dd, hi, keep, ctx, n_pages, free)
    pool = torch.zeros(n_pages * page, dtype=torch.uint8, device="cuda")
    tdev = torch.from_numpy(table).cuda()
    tria.pack_kv_cache_paged(dd, hi, keep, ctx, dev(k), dev(v), tdev, pool)
    psums = tria.build_block_summaries_paged(dd, tdev, pool, ctx)
    sm = 1.0 / math.sqrt(d)
    thd = torch.from_numpy(th).cuda()
    out_p = tria.decode_skip_paged(dd, tdev, pool, ctx, psums, dev(q), thd, sm)
    out_c = tria.decode_skip(dd, cache, ctx, sums, dev(q), thd, sm)
    torch.cuda.synchronize()
    a, c = psums.cpu().numpy(), sums.cpu().numpy()
    assert np.array_equal(a[64:], c[64:]) and np.array_equal(a[:32], c[:32])
    assert a[32:40].view(np.int64)[0] == table.size
    assert torch.equal(out_p, out_c)
    zero = tria.decode_skip_paged(dd, tdev, pool, ctx, psums, dev(q), torch.zeros_like(thd), sm)
    torch.cuda.synchronize()
    assert torch.equal(zero, tria.decode_paged(dd, tdev, pool, ctx, dev(q), sm))


def test_skip_over_varlen_cache(tria):
    """A variable-length batch (sequences at 1 to 1300 tokens): each sequence's index
    records equal the oracle's statistics of that sequence alone, and the skipping
    decode of each sequence equals the oracle's masked decode of it alone."""
    b, hq, hk, d, n, blk = 4, 8, 2, 128, 1300, 128
    lens = np.array([1300, 1, 700, 257], np.int64)
    cfg = synth.Config("skip varlen", b, hq, hk, d, n, blk, seed=67, decode=True)
    k, v, q, th = synth.make_skip_decode_inputs(cfg)
    hi, keep = np.array([1, 2], np.int32), np.array([4, 9], np.int32)
    dd = tria.make_dims(b, hq, hk, d, blk, n)
    cache = tria.pack_kv_cache_varlen(dd, hi, keep, lens, dev(k), dev(v))
    sums = tria.build_block_summaries_varlen(dd, cache)
    sm = 1.0 / math.sqrt(d)
    out = tria.decode_skip_varlen(dd, cache, sums, dev(q), torch.from_numpy(th).cuda(), sm)
    torch.cuda.synchronize()
    rmax = (n - 1) // blk + 1
    hdr, h64, lo, up, smax, pad, nmax = parse_summaries(sums, b * hk, rmax, d)
    assert hdr[6] == -1
    assert np.array_equal(pad, expected_stamps(cache, b * hk, rmax, blk, lambda p: lens[p // hk]))
    for i in range(b):
        ctx = int(lens[i])
        rlo, rup, rsmax, rnmax = oracle.block_summaries(k[i:i + 1], hi, keep, hq, blk, ctx)
        rr = rlo.shape[1]
        sl = slice(i * hk, (i + 1) * hk)
        assert np.array_equal(lo[sl, :rr], rlo) and np.array_equal(up[sl, :rr], rup), i
        assert np.array_equal(smax[sl, :rr], rsmax) and np.array_equal(nmax[sl, :rr], rnmax), i
        ref = oracle.decode_skip(k[i:i + 1], v[i:i + 1], q[i:i + 1], hi, keep, blk, ctx, th[i:i + 1], sm)
        assert_close(out[i:i + 1].cpu().numpy(), ref, f"varlen skip sequence {i} (ctx {ctx})")


def test_stale_varlen_index_gives_nan(tria):
    """A variable-length index reused after a sequence that is not the longest moved to
    another block with the same record count (so the cache's size is unchanged): the
    stamps of that sequence's slots no longer match, so the index does not validate
    and the whole output is NaN, as for any index that does not validate; with a
    fresh index every output is finite."""
    b, hq, hk, d, n, blk = 4, 8, 2, 128, 1300, 128
    hi, keep = np.array([1, 1], np.int32), np.array([1, 1], np.int32)   # int8 {0, c-1, c} for c >= 2
    cfg = synth.Config("skip stale", b, hq, hk, d, n, blk, seed=69, decode=True)
    k, v, q, th = synth.make_skip_decode_inputs(cfg)
    dd = tria.make_dims(b, hq, hk, d, blk, n)
    sm = 1.0 / math.sqrt(d)
    thd = torch.from_numpy(th).cuda()
    kd, vd, qd = dev(k), dev(v), dev(q)
    for old_lens, new_lens, moved in (([1300, 300, 700, 257], [1300, 400, 700, 257], 1),   # 300 -> 400: block 2 -> 3
                                      ([1300, 300, 700, 257], [1300, 300, 450, 257], 2)):  # restart 700 -> 450: 5 -> 3
        print(f"[case] stale varlen index {old_lens} -> {new_lens}", flush=True)
        c_old = tria.pack_kv_cache_varlen(dd, hi, keep, np.array(old_lens, np.int64), kd, vd)
        stale = tria.build_block_summaries_varlen(dd, c_old)
        c_new = tria.pack_kv_cache_varlen(dd, hi, keep, np.array(new_lens, np.int64), kd, vd)
        assert c_new.numel() == c_old.numel()
        fresh = tria.build_block_summaries_varlen(dd, c_new)
        got = tria.decode_skip_varlen(dd, c_new, stale, qd, thd, sm)
        want = tria.decode_skip_varlen(dd, c_new, fresh, qd, thd, sm)
        torch.cuda.synchronize()
        got, want = got.cpu().numpy(), want.cpu().numpy()
        assert np.isnan(got).all(), moved
        assert np.isfinite(want).all()
        for i in range(b):   # the fresh index against the oracle, sequence by sequence
            ctx = int(new_lens[i])
            ref = oracle.decode_skip(k[i:i + 1], v[i:i + 1], q[i:i + 1], hi, keep, blk, ctx, th[i:i + 1], sm)
            assert_close(want[i:i + 1], ref, f"fresh index, sequence {i} (ctx {ctx})")


def test_skip_over_varlen_paged_cache(tria):
    """A variable-length batch in scattered pages, grown over a few steps (one
    sequence restarting shorter): its statistics index equals the contiguous
    variable-length cache's record for record, the skipping decode equals the
    contiguous one bit for bit, and with zero thresholds it equals the plain paged
    decode."""
    b, hq, hk, d, n, blk = 4, 8, 2, 128, 1300, 128
    cfg = synth.Config("skip paged varlen", b, hq, hk, d, n, blk, seed=71, decode=True)
    k, v, q, th = synth.make_skip_decode_inputs(cfg)
    hi, keep = np.array([1, 2], np.int32), np.array([4, 9], np.int32)
    dd = tria.make_dims(b, hq, hk, d, blk, n)
    page = tria.paged_page_bytes(dd)
    n_pages = b * hk * ((n - 1) // blk + 1)
    free = list(np.random.default_rng(13).permutation(n_pages).astype(np.int32))
    pool = torch.zeros(n_pages * page, dtype=torch.uint8, device="cuda")
    kd, vd, qd, thd = dev(k), dev(v), dev(q), torch.from_numpy(th).cuda()
    sm = 1.0 / math.sqrt(d)
    old, old_dev = None, None
    for lens in ([1280, 1, 700, 256], [1281, 2, 701, 257], [1282, 3, 5, 258], [1300, 129, 6, 259]):
        lens = np.array(lens, np.int64)
        print(f"[case] skip paged varlen lens {lens.tolist()}", flush=True)
        table, used, rel = tria.build_paged_table(dd, hi, keep, lens, n_pages, np.array(free, np.int32), old)
        free = free[used:] + list(rel)
        tdev = torch.from_numpy(table).cuda()
        tria.pack_kv_cache_paged(dd, hi, keep, lens, kd, vd, tdev, pool, old_table=old_dev)
        old, old_dev = table, tdev
        psums = tria.build_block_summaries_paged_varlen(dd, tdev, pool)
        out_p = tria.decode_skip_paged_varlen(dd, tdev, pool, psums, qd, thd, sm)
        cache = tria.pack_kv_cache_varlen(dd, hi, keep, lens, kd, vd)
        sums = tria.build_block_summaries_varlen(dd, cache)
        out_c = tria.decode_skip_varlen(dd, cache, sums, qd, thd, sm)
        zero = tria.decode_skip_paged_varlen(dd, tdev, pool, psums, qd, torch.zeros_like(thd), sm)
        plain = tria.decode_paged_varlen(dd, tdev, pool, qd, sm)
        torch.cuda.synchronize()
        a, c = psums.cpu().numpy(), sums.cpu().numpy()
        assert np.array_equal(a[64:], c[64:]) and np.array_equal(a[:32], c[:32])
        assert a[32:40].view(np.int64)[0] == table.size
        assert torch.equal(out_p, out_c)
        assert torch.equal(zero, plain)
