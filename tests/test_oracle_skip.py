"""Pins of the oracle's dynamic block skipping (CPU).

ETA page (rit.work, section on how the model decides which part of the context to
read): per-block statistics give an upper bound on the block's scores and a block
below the head's threshold is not read.  The oracle's reading: a box bound from the
per-coordinate code range and a norm bound from the largest key norm; a block is
skipped for a head iff either bound is below the threshold; the first key block and
the current block are never skipped.  These tests pin it against facts that do not
depend on its code: the bound never drops a block that holds a score at or above
the threshold (brute force over every key), the bounds are tight where the
geometry makes them so (hand-derived closed forms), the extremes of the threshold
reduce to the plain decode, and the masked decode equals dense attention over the
kept keys.
"""
import math

import numpy as np
import pytest

import oracle
from synth import gen

pytestmark = pytest.mark.filterwarnings("ignore")


def _bits(x):
    return gen.float32_to_bf16_bits(np.asarray(x, np.float32))


def _records(ctx, block, hi, keep):
    """Stored blocks in record order (int8 ascending, then int4) from the tile rule."""
    c = (ctx - 1) // block
    acts = [oracle.tile_action(c, kb, hi, keep) for kb in range(c + 1)]
    b8 = [kb for kb, a in enumerate(acts) if a == 8]
    b4 = [kb for kb, a in enumerate(acts) if a == 4]
    return [(kb, 127) for kb in b8] + [(kb, 7) for kb in b4]


def _small(seed=11, d=64, block=16, ctx=200, hq=4, hk=1, b=1):
    cfg = gen.Config("skip pin", b, hq, hk, d, ctx, block, seed=seed, decode=True)
    return gen.make_skip_decode_inputs(cfg)


def _codes(rows, qmax):
    rows = np.ascontiguousarray(rows, np.uint16)
    return oracle.quantize_rows(rows, qmax)


def test_summaries_are_code_ranges_of_each_record():
    k, v, q, th = _small()
    block, ctx, hi, keep = 16, 200, 2, 8
    lo, up, smax, nmax = oracle.block_summaries(k, np.array([hi]), np.array([keep]), 4, block, ctx)
    recs = _records(ctx, block, hi, keep)
    for r, (kb, qmax) in enumerate(recs):
        rows = k[0, 0, kb * block:(kb + 1) * block]
        codes, scales = _codes(rows, qmax)
        valid = min(block, ctx - kb * block)
        codes = np.concatenate([codes[:valid], np.zeros((block - valid, codes.shape[1]), np.int8)])
        scales = np.concatenate([scales[:valid], np.zeros(block - valid, np.float32)])
        assert np.array_equal(lo[0, r], codes.min(axis=0)), r
        assert np.array_equal(up[0, r], codes.max(axis=0)), r
        assert smax[0, r] == scales.max()
        n2 = (codes.astype(np.int64) ** 2).sum(axis=1)
        assert nmax[0, r] == max((float(s) * float(s)) * float(t) for s, t in zip(scales, n2))
    assert not lo[0, len(recs):].any() and not smax[0, len(recs):].any()


def _exact_max_scores(k, q, block, ctx, hi, keep, sm):
    """Brute force: per record and head, the largest score over the record's keys,
    as the decode computes it (quantised codes, double)."""
    recs = _records(ctx, block, hi, keep)
    G = q.shape[1]
    out = np.full((len(recs), G), -np.inf)
    for r, (kb, qmax) in enumerate(recs):
        valid = min(block, ctx - kb * block)
        kc, ks = _codes(k[0, 0, kb * block:kb * block + valid], qmax)
        qc, qs = _codes(q[0], qmax)
        dots = qc.astype(np.int64) @ kc.astype(np.int64).T       # [G][rows]
        s = dots.astype(np.float64) * qs[:, None].astype(np.float64) * ks[None, :].astype(np.float64) * sm
        out[r] = s.max(axis=1)
    return recs, out


def test_bound_never_skips_a_block_holding_a_score_above_threshold():
    block, ctx, hi, keep, d = 16, 200, 2, 8, 64
    sm = 1.0 / math.sqrt(d)
    for seed in (11, 12, 13):
        k, v, q, _ = _small(seed=seed)
        recs, mx = _exact_max_scores(k, q, block, ctx, hi, keep, sm)
        for r in range(len(recs)):
            if (mx[r] <= 0).any():
                continue
            # every head's threshold at (just below) this record's largest score
            th = np.nextafter(mx[r].astype(np.float32), np.float32(0)).reshape(1, -1)
            masks = oracle.skip_masks(k, q, np.array([hi]), np.array([keep]), block, ctx, th, sm)
            assert masks[0, r] == 0xF, (seed, r, hex(int(masks[0, r])))


def test_bounds_are_tight_in_closed_form():
    """d = 64, block 16, three blocks, query at the last token.  Block 1 holds the
    one-hot rows 127 e0 and 127 e1 (codes equal values: amax 127 gives scale 1);
    the query is 127 (e0 + e1).  Exact largest score: sm * 127^2.  Box bound:
    sm * (127*127 + 127*127) = 2 sm 127^2.  Norm bound: sm * 127 sqrt(2) * 127.
    So a threshold of 1.40 sm 127^2 keeps block 1 and 1.42 sm 127^2 skips it, by
    the norm bound alone (the box bound is above both)."""
    d, block, ctx, sm = 64, 16, 48, 0.125
    kf = np.zeros((1, 1, ctx, d), np.float32)
    kf[0, 0, :, 5] = 1.0                   # blocks 0 and 2: anything
    kf[0, 0, 16:32, :] = 0.0
    kf[0, 0, 16:24, 0] = 127.0
    kf[0, 0, 24:32, 1] = 127.0
    qf = np.zeros((1, 1, d), np.float32)
    qf[0, 0, :2] = 127.0
    k, q = _bits(kf), _bits(qf)
    unit = sm * 127.0 * 127.0
    for f, kept in ((1.40, 1), (1.42, 0)):
        masks = oracle.skip_masks(k, q, np.array([8]), np.array([8]), block, ctx, np.array([[f * unit]]), sm)
        assert masks[0, 1] == kept, f
        assert masks[0, 0] == 1 and masks[0, 2] == 1     # protected: first and current block
    # the box bound alone: rows all 127 (e0 + e1) -> every score equals the bound
    kf[0, 0, 16:32, :2] = 127.0
    k = _bits(kf)
    for f, kept in ((1.0 - 1e-6, 1), (1.0 + 1e-6, 0)):
        masks = oracle.skip_masks(k, q, np.array([8]), np.array([8]), block, ctx, np.array([[2 * f * unit]]), sm)
        assert masks[0, 1] == kept, f
    # int4 block (hi 0, keep 8): codes 7, scales 127/7 -> the same scores
    for f, kept in ((1.0 - 1e-6, 1), (1.0 + 1e-6, 0)):
        masks = oracle.skip_masks(k, q, np.array([0]), np.array([8]), block, ctx, np.array([[2 * f * unit]]), sm)
        recs = _records(ctx, block, 0, 8)
        assert recs[2] == (1, 7)
        assert masks[0, 2] == kept, f


def test_threshold_extremes_reduce_to_plain_decode():
    k, v, q, th = _small(seed=21, hq=8, hk=2, b=2)
    block, ctx, sm = 16, 200, 0.125
    hi, keep = np.array([2, 1]), np.array([8, 12])
    base = oracle.decode(k, v, q, hi, keep, block, ctx, sm)
    nothing = oracle.decode_skip(k, v, q, hi, keep, block, ctx, np.zeros((2, 8), np.float32), sm)
    assert np.array_equal(base, nothing)
    only = oracle.decode_skip(k, v, q, hi, keep, block, ctx, np.full((2, 8), np.inf, np.float32), sm)
    prot = oracle.decode(k, v, q, np.zeros(2, np.int32), np.zeros(2, np.int32), block, ctx, sm)
    assert np.array_equal(only, prot)
    assert not np.array_equal(only, base)


def test_masked_decode_is_dense_attention_over_kept_keys():
    """int8 only (hi = keep): the masked decode equals dense softmax attention of
    the dequantised codes over the keys of the blocks each head keeps."""
    d, block, ctx, hq, sm = 64, 16, 200, 4, 0.125
    k, v, q, th = _small(seed=31, d=d, block=block, ctx=ctx, hq=hq)
    hi = keep = np.array([6])
    masks = oracle.skip_masks(k, q, hi, keep, block, ctx, th, sm)
    recs = _records(ctx, block, 6, 6)
    assert 0 < sum(bin(int(m)).count("1") for m in masks[0, :len(recs)]) < hq * len(recs)   # some skipped
    out = oracle.decode_skip(k, v, q, hi, keep, block, ctx, th, sm)
    kc, ks = _codes(k[0, 0, :ctx], 127)
    vc, vs = _codes(v[0, 0, :ctx], 127)
    qc, qs = _codes(q[0], 127)
    kd = kc.astype(np.float64) * ks[:, None]
    vd = vc.astype(np.float64) * vs[:, None]
    qd = qc.astype(np.float64) * qs[:, None]
    keepmask = np.zeros((hq, ctx), np.uint8)
    for r, (kb, _) in enumerate(recs):
        for h in range(hq):
            if (int(masks[0, r]) >> h) & 1:
                keepmask[h, kb * block:min(ctx, (kb + 1) * block)] = 1
    ref = oracle.dense_attention(qd, kd, vd, keepmask, sm)
    assert np.abs(out[0] - ref).max() < 1e-6
