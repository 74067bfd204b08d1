"""Pins of the CPU oracle against facts fixed outside it (no GPU).

Each test checks the oracle against something it does not contain: the worked
numbers printed on the pages, dense softmax attention (itself checked against
torch's CPU attention), hand-counted tile maps, library rounding routines, or
invariants of the method.  They are chosen so that a plausible slip in the oracle
(an exclusive boundary, a dropped protected block, the wrong codes in an int4
tile, a transposed operand, a wrong scale) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from synth import float32_to_bf16_bits, bf16_bits_to_float32, normal_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LOG2E = 1.4426950408889634


def bits(a):
    return float32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def int_rows(rng, shape, amax):
    """Integer rows in [-amax, amax], each row containing +-amax (scale exactly 1
    at qmax = amax)."""
    x = rng.integers(-amax, amax + 1, size=shape).astype(np.float32)
    idx = rng.integers(0, shape[-1], size=shape[:-1])
    sign = rng.choice([-1.0, 1.0], size=shape[:-1])
    np.put_along_axis(x, idx[..., None], (sign * amax)[..., None], axis=-1)
    return x


# ---------------------------------------------------------------- page formula
def test_kv_formula_matches_page_examples():
    g = json.load(open(os.path.join(GOLDEN, "kv_cache_bytes.json")))
    for ex in g["examples"]:
        v = oracle.kv_formula_bytes(ex["L"], ex["h"], ex["d_h"], ex["n"], ex["b"], ex["p"])
        if "exact" in ex:
            assert v == ex["exact"]
            assert round(v / 2 ** 30, 2) == ex["printed_gib"]
        else:
            printed = ex["printed"]
            val = v / ex["unit"]
            # the page prints rounded (10.7, 1.34) or truncated (167) figures
            assert printed - 1e-9 <= val + ex["printed_rounding"] and abs(val - printed) <= ex["printed_rounding"], (ex, val)
    for e in g["per_token_per_layer_elements"]:
        assert oracle.kv_formula_bytes(1, e["h"], e["d_h"], 1, 1, 1) == e["value"]


# ---------------------------------------------------------------- policy
def test_tile_map_tiny_config_hand_count():
    # nb = 8, (hi, keep) = (2, 4): counted by hand from the distance rule with
    # inclusive boundaries and the two protected blocks.
    # qb:    0  1  2  3  4  5  6  7
    # int8:  1  2  3  4  4  4  4  4   -> 26 (8 of them diagonal)
    # int4:  0  0  0  0  1  2  2  2   -> 7
    # skip:  0  0  0  0  0  0  1  2   -> 3
    counts = {8: 0, 4: 0, 0: 0}
    for qb in range(8):
        for kb in range(qb + 1):
            counts[oracle.tile_action(qb, kb, 2, 4)] += 1
    assert counts == {8: 26, 4: 7, 0: 3}
    assert all(oracle.tile_action(qb, kb, 2, 4) == -1 for qb in range(8) for kb in range(qb + 1, 8))


@pytest.mark.parametrize("nb", [1, 2, 5, 9])
def test_tile_map_edge_policies(nb):
    top = nb - 1
    for qb in range(nb):
        for kb in range(qb + 1):
            # all-int8 (hi = keep = max)
            assert oracle.tile_action(qb, kb, top, top) == 8
            # protected-only (hi = keep = 0): block 0 and the diagonal survive
            assert oracle.tile_action(qb, kb, 0, 0) == (8 if kb in (0, qb) else 0)
            # all-int4 beyond the diagonal (hi = 0, keep = max)
            assert oracle.tile_action(qb, kb, 0, top) == (8 if kb in (0, qb) else 4)


def test_tile_map_monotone_in_distance():
    # precision never rises with distance from the diagonal (block 0 excepted),
    # and widening a boundary never drops a tile
    rank = {8: 2, 4: 1, 0: 0}
    for hi in range(0, 6):
        for keep in range(hi, 8):
            for qb in range(10):
                acts = [oracle.tile_action(qb, kb, hi, keep) for kb in range(1, qb + 1)]
                r = [rank[a] for a in acts]
                assert r == sorted(r), (hi, keep, qb)
                for kb in range(qb + 1):
                    assert rank[oracle.tile_action(qb, kb, hi, keep + 1)] >= rank[oracle.tile_action(qb, kb, hi, keep)]
                    assert rank[oracle.tile_action(qb, kb, hi + 1, max(keep, hi + 1))] >= rank[oracle.tile_action(qb, kb, hi, keep)]


def test_schedule_round_trips_the_tile_map():
    rng = np.random.default_rng(0)
    for trial in range(20):
        nb = int(rng.integers(1, 14))
        block = 64
        hq, hk, b = 4, 2, 2
        hi = rng.integers(0, nb + 1, size=hq).astype(np.int32)
        keep = (hi + rng.integers(0, nb + 1, size=hq)).astype(np.int32)
        n = nb * block - int(rng.integers(0, block))
        s = oracle.build_schedule(b, hq, hk, 128, block, n, hi, keep)
        assert s[0] == 0x48435354 and s[1] == 1 and s[8] == b * hq * nb
        units = s[16:].reshape(-1, 8)
        seen = set()
        for (bb, h, qb, lo8, lo4, hi4, sink, nt) in units:
            seen.add((bb, h, qb))
            kept = set(range(lo8, qb + 1)) | ({0} if sink else set())
            four = set(range(lo4, hi4 + 1))
            for kb in range(qb + 1):
                a = oracle.tile_action(qb, kb, hi[h], keep[h])
                assert (a == 8) == (kb in kept) and (a == 4) == (kb in four)
            assert nt == len(kept) + len(four)
            assert not (sink and lo8 == 0)
        assert len(seen) == b * hq * nb
        # longest work first, ties in (b, h, qb) order
        key = [(-u[7], u[0], u[1], u[2]) for u in units]
        assert key == sorted(key)


# ---------------------------------------------------------------- quantiser
def test_quantizer_properties():
    rng = np.random.default_rng(1)
    x = bits(rng.standard_normal((512, 128)) * rng.uniform(0.01, 100, size=(512, 1)))
    xf = bf16_bits_to_float32(x).astype(np.float64)
    for qmax in (127, 7):
        codes, scales = oracle.quantize_rows(x, qmax)
        assert codes.min() >= -qmax and codes.max() <= qmax
        err = np.abs(xf - scales[:, None].astype(np.float64) * codes)
        # half a step, plus the fp32 rounding of scale and of qmax/amax (a few ulps of qmax)
        assert np.all(err <= scales[:, None] * (0.5 + qmax * 2.0 ** -21))
        amax = np.abs(xf).max(axis=1)
        assert np.allclose(scales, amax / qmax, rtol=1e-7)
        arg = np.abs(xf).argmax(axis=1)
        assert np.all(np.abs(codes[np.arange(512), arg]) == qmax)
    # constant row, zero row, integer row with amax = 127 (scale exactly 1)
    c, s = oracle.quantize_rows(bits(np.full((1, 64), -3.5)), 127)
    assert np.all(c == -127) and s[0] == np.float32(3.5 / 127)
    c, s = oracle.quantize_rows(np.zeros((2, 64), np.uint16), 7)
    assert np.all(c == 0) and np.all(s == 0)
    ints = int_rows(rng, (64, 128), 127)
    c, s = oracle.quantize_rows(bits(ints), 127)
    assert np.all(s == 1.0) and np.array_equal(c, ints.astype(np.int8))
    ints = int_rows(rng, (64, 64), 7)
    c, s = oracle.quantize_rows(bits(ints), 7)
    assert np.all(s == 1.0) and np.array_equal(c, ints.astype(np.int8))


def test_quantizer_rounds_half_to_even():
    # x * (127/amax) lands exactly on .5 for these rows: 127 * (k + 0.5) / 127
    row = np.zeros((1, 64), np.float32)
    row[0, 0] = 127.0
    row[0, 1:6] = [0.5, 1.5, 2.5, -0.5, -2.5]
    c, s = oracle.quantize_rows(bits(row), 127)
    assert s[0] == 1.0 and list(c[0, :6]) == [127, 0, 2, 2, 0, -2]


def test_nibble_packing_round_trip():
    rng = np.random.default_rng(2)
    codes = rng.integers(-7, 8, size=(10, 64)).astype(np.int8)
    packed = oracle.pack_nibbles(codes)
    lo = (packed & 0xF).astype(np.int8)
    hi = (packed >> 4).astype(np.int8)
    lo[lo > 7] -= 16
    hi[hi > 7] -= 16
    assert np.array_equal(lo, codes[:, 0::2]) and np.array_equal(hi, codes[:, 1::2])


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(3)
    f = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, 3.0e38])]).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mine = np.array([oracle.float_to_bf16(float(v)) for v in f], dtype=np.uint16)
    assert np.array_equal(mine, ref)


# ---------------------------------------------------------------- dense reference
def test_dense_attention_matches_torch_sdpa():
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((37, 16)) for _ in range(3))
    mask = np.tril(np.ones((37, 37), np.uint8))
    out = oracle.dense_attention(q, k, v, mask, 0.25)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        is_causal=True, scale=0.25)[0].numpy()
    assert np.abs(out - ref).max() < 1e-12


# ---------------------------------------------------------------- prefill
def _dequant(x_bits, qmax):
    c, s = oracle.quantize_rows(x_bits, qmax)
    return c.astype(np.float64) * s[..., None].astype(np.float64)


def _augmented_reference(q, k, v, hi, keep, block, sm_scale, G):
    """Dense softmax over augmented vectors: a key of an int8 tile is [k8, 0], of
    an int4 tile [0, k4]; the query is [q8, q4].  Scores then equal the
    precision-selected products, and dense attention over the kept-key mask
    gives the exact (unrounded-weight) method output."""
    b, hq, n, d = q.shape
    q8, q4 = _dequant(q, 127), _dequant(q, 7)
    k8, k4 = _dequant(k, 127), _dequant(k, 7)
    vf = bf16_bits_to_float32(v).astype(np.float64)
    out = np.zeros(q.shape)
    for bb in range(b):
        for h in range(hq):
            g = h // G
            qa = np.concatenate([q8[bb, h], q4[bb, h]], axis=1)
            act = np.array([[oracle.tile_action(i // block, j // block, hi[h], keep[h]) if j <= i else -1
                             for j in range(n)] for i in range(n)])
            # one augmented key row per (query-independent) precision; build two
            # copies of the key set and mask the unused copy
            ka = np.concatenate([np.concatenate([k8[bb, g], np.zeros((n, d))], axis=1),
                                 np.concatenate([np.zeros((n, d)), k4[bb, g]], axis=1)], axis=0)
            va = np.concatenate([vf[bb, g], vf[bb, g]], axis=0)
            mask = np.concatenate([(act == 8), (act == 4)], axis=1).astype(np.uint8)
            out[bb, h] = oracle.dense_attention(qa, ka, va, mask, sm_scale)
    return out


def test_prefill_all_kept_equals_dense_attention():
    # everything int8 and integer rows with amax 127: codes are the values, so the
    # method must reproduce plain causal softmax attention (reference mode)
    rng = np.random.default_rng(5)
    b, hq, hk, n, d, B = 1, 2, 1, 200, 64, 64
    q, k = bits(int_rows(rng, (b, hq, n, d), 127)), bits(int_rows(rng, (b, hk, n, d), 127))
    v = bits(rng.integers(-100, 100, size=(b, hk, n, d)))
    nb = (n + B - 1) // B
    hi = keep = np.full(hq, nb - 1, np.int32)
    sm = 1.0 / 4096
    out = oracle.prefill(q, k, v, hi, keep, B, sm, reference_mode=True)
    qf, kf, vf = (bf16_bits_to_float32(x).astype(np.float64) for x in (q, k, v))
    mask = np.tril(np.ones((n, n), np.uint8))
    for h in range(hq):
        ref = oracle.dense_attention(qf[0, h], kf[0, 0], vf[0, 0], mask, sm)
        # identical up to the fp32 rounding of the emitted output
        assert np.all(np.abs(out[0, h] - ref) <= 2.0 ** -23 * np.abs(ref) + 1e-12), h


def test_prefill_protected_only_is_sink_plus_diagonal():
    rng = np.random.default_rng(6)
    b, hq, hk, n, d, B = 1, 1, 1, 300, 64, 64
    q, k = bits(int_rows(rng, (b, hq, n, d), 127)), bits(int_rows(rng, (b, hk, n, d), 127))
    v = bits(rng.integers(-100, 100, size=(b, hk, n, d)))
    out = oracle.prefill(q, k, v, [0], [0], B, 1.0 / 4096, reference_mode=True)
    qf, kf, vf = (bf16_bits_to_float32(x).astype(np.float64) for x in (q, k, v))
    mask = np.zeros((n, n), np.uint8)
    for i in range(n):
        qb = i // B
        mask[i, :min(B, i + 1)] = 1
        mask[i, qb * B:i + 1] = 1
    ref = oracle.dense_attention(qf[0, 0], kf[0, 0], vf[0, 0], mask, 1.0 / 4096)
    assert np.abs(out[0, 0] - ref).max() < 2e-5


@pytest.mark.parametrize("hi,keep", [(0, 99), (1, 2), (2, 3), (0, 0)])
def test_prefill_equals_augmented_dense(hi, keep):
    # N(0,1) inputs: quantisation is lossy, and int8 vs int4 codes differ; the
    # reference selects the codes per tile through augmented vectors
    b, hq, hk, n, d, B = 1, 2, 1, 330, 64, 64
    G = hq // hk
    q = normal_bf16(11, 1, b * hq * n * d).reshape(b, hq, n, d)
    k = normal_bf16(11, 2, b * hk * n * d).reshape(b, hk, n, d)
    v = normal_bf16(11, 3, b * hk * n * d).reshape(b, hk, n, d)
    his = np.array([hi, min(hi + 1, keep)], np.int32)
    keeps = np.array([keep, keep], np.int32)
    sm = 1.0 / math.sqrt(d)
    out = oracle.prefill(q, k, v, his, keeps, B, sm, reference_mode=True)
    ref = _augmented_reference(q, k, v, his, keeps, B, sm, G)
    assert np.abs(out - ref).max() < 2e-6


def test_prefill_bf16_weights_close_to_exact_and_rows_normalised():
    b, hq, hk, n, d, B = 1, 2, 1, 256, 64, 64
    q = normal_bf16(12, 1, b * hq * n * d).reshape(b, hq, n, d)
    k = normal_bf16(12, 2, b * hk * n * d).reshape(b, hk, n, d)
    v = normal_bf16(12, 3, b * hk * n * d).reshape(b, hk, n, d)
    hi, keep = np.array([1, 0], np.int32), np.array([2, 3], np.int32)
    exact, lse_e = oracle.prefill(q, k, v, hi, keep, B, 0.125, reference_mode=True, with_lse=True)
    rounded, lse_r = oracle.prefill(q, k, v, hi, keep, B, 0.125, with_lse=True)
    # bf16 weights: per-weight relative error <= 2^-9, so the normalised output moves
    # by at most ~2^-8 of the value scale
    assert np.abs(rounded - exact).max() < 2 ** -7
    assert np.abs(rounded - exact).mean() > 0  # the rounding is really applied
    assert np.abs(lse_r - lse_e).max() < 2 ** -7
    # with V = 1 every normalised row is exactly 1 in both modes (weights sum to l)
    ones = bits(np.ones_like(bf16_bits_to_float32(v)))
    for mode in (True, False):
        o = oracle.prefill(q, k, ones, hi, keep, B, 0.125, reference_mode=mode)
        assert np.abs(o - 1.0).max() < 1e-6


def test_prefill_lse_matches_dense_logsumexp():
    rng = np.random.default_rng(7)
    b, hq, hk, n, d, B = 1, 1, 1, 130, 64, 64
    q, k = bits(int_rows(rng, (b, hq, n, d), 127)), bits(int_rows(rng, (b, hk, n, d), 127))
    v = bits(rng.integers(-9, 9, size=(b, hk, n, d)))
    sm = 1.0 / 8192
    _, lse = oracle.prefill(q, k, v, [9], [9], B, sm, reference_mode=True, with_lse=True)
    qf, kf = (bf16_bits_to_float32(x).astype(np.float64)[0, 0] for x in (q, k))
    s = (qf @ kf.T) * sm * LOG2E
    for i in range(n):
        ref = np.log2(np.sum(np.exp2(s[i, :i + 1])))
        assert abs(lse[0, 0, i] - ref) < 1e-5


def test_prefill_never_reads_skipped_or_masked_keys():
    b, hq, hk, n, d, B = 1, 2, 1, 400, 64, 64
    q = normal_bf16(13, 1, b * hq * n * d).reshape(b, hq, n, d)
    k = normal_bf16(13, 2, b * hk * n * d).reshape(b, hk, n, d)
    v = normal_bf16(13, 3, b * hk * n * d).reshape(b, hk, n, d)
    hi, keep = np.array([1, 1], np.int32), np.array([2, 2], np.int32)
    base = oracle.prefill(q, k, v, hi, keep, B, 0.125)
    # block 2 is skipped for query blocks >= 5: poison it and test only those rows
    k2, v2 = k.copy(), v.copy()
    k2[..., 2 * B:3 * B, :] = 0x7FC0  # NaN
    v2[..., 2 * B:3 * B, :] = 0x7FC0
    units = [(0, h, qb) for h in range(hq) for qb in range(5, 7)]
    pois = oracle.prefill(q, k2, v2, hi, keep, B, 0.125, units=units)
    rows = slice(5 * B, n)
    assert np.array_equal(pois[:, :, rows], base[:, :, rows])


@pytest.mark.parametrize("hq,hk", [(4, 4), (4, 1)])
def test_prefill_gqa_equals_independent_heads(hq, hk):
    b, n, d, B = 1, 200, 64, 64
    q = normal_bf16(14, 1, b * hq * n * d).reshape(b, hq, n, d)
    k = normal_bf16(14, 2, b * hk * n * d).reshape(b, hk, n, d)
    v = normal_bf16(14, 3, b * hk * n * d).reshape(b, hk, n, d)
    hi, keep = np.array([0, 1, 2, 0], np.int32), np.array([1, 1, 3, 3], np.int32)
    out = oracle.prefill(q, k, v, hi, keep, B, 0.125)
    G = hq // hk
    for h in range(hq):
        one = oracle.prefill(q[:, h:h + 1], k[:, h // G:h // G + 1], v[:, h // G:h // G + 1],
                             hi[h:h + 1], keep[h:h + 1], B, 0.125)
        assert np.array_equal(one[:, 0], out[:, h])


# ---------------------------------------------------------------- cache
def test_cache_bytes_against_page_formula():
    b, hk, d, B, n = 2, 4, 128, 128, 4096
    nb = n // B
    top = np.full(hk, nb - 1, np.int32)
    header = (64 + 64 * b * hk + 255) // 256 * 256
    # all stored at int8: the page's formula with p = 1 byte, plus fp32 row scales
    codes = oracle.kv_formula_bytes(1, hk, d, n, b, 1)
    scales = 2 * hk * n * b * 4
    assert oracle.cache_bytes(b, hk, hk, d, B, n, top, top) == header + codes + scales
    # protected-only: block 0 and the current block
    zero = np.zeros(hk, np.int32)
    assert oracle.cache_bytes(b, hk, hk, d, B, n, zero, zero) == header + b * hk * 2 * (2 * B * d + 8 * B)
    # everything int4 but the protected blocks: half a byte per element
    assert oracle.cache_bytes(b, hk, hk, d, B, n, zero, top) == header + b * hk * (
        2 * (2 * B * d + 8 * B) + (nb - 2) * (B * d + 8 * B))


def _unpack_nibbles(a):
    """uint8 [..., m] -> int8 [..., 2m], low nibble first, two's complement."""
    lo, hi = (a & 0xF).astype(np.int8), (a >> 4).astype(np.int8)
    out = np.stack([lo, hi], axis=-1).reshape(*a.shape[:-1], 2 * a.shape[-1])
    out[out > 7] -= 16
    return out


def _read_record(rec, B, d, int4):
    """Parses one record of the documented cache layout: 32-token chunks of a K part,
    a V part (both sequences of 16-byte lane units, lane = r + 16q) and the scales."""
    ksl, part = d // 64, (16 if int4 else 32) * d
    kc, vc = np.zeros((B, d), np.int8), np.zeros((B, d), np.int8)
    ks, vs = np.zeros(B, np.float32), np.zeros(B, np.float32)
    tok = np.array([[16 * (p // 4) + 4 * q + (p % 4) for p in range(8)] for q in range(4)])  # [q][p]
    for c in range(B // 32):
        ch = rec[c * (2 * part + 256):(c + 1) * (2 * part + 256)]
        kp, vp, sp = ch[:part], ch[part:2 * part], ch[2 * part:]
        if not int4:  # units (s, ks, q, r): dims 64ks + 16q + i of token 16s + r
            kk = kp.view(np.int8).reshape(2, ksl, 4, 16, 16)
            kc[32 * c:32 * c + 32] = kk.transpose(0, 3, 1, 2, 4).reshape(32, d)
        else:         # units (s, q, r), ks inside: packed dims 64ks + 16q + i
            kk = _unpack_nibbles(kp.reshape(2, 4, 16, ksl, 8))  # [s][q][r][ks][16]
            kc[32 * c:32 * c + 32] = kk.transpose(0, 2, 3, 1, 4).reshape(32, d)
        per = 4 if int4 else 2  # dim groups per unit
        if not int4:
            vv = vp.view(np.int8).reshape(d // 16 // per, 4, 16, per, 8)  # [m][q][r][t][p]
        else:
            vv = _unpack_nibbles(vp.reshape(d // 16 // per, 4, 16, per, 4))
        for m in range(d // 16 // per):
            for t in range(per):
                dt = per * m + t
                for q in range(4):
                    vc[32 * c + tok[q], 16 * dt:16 * dt + 16] = vv[m, q, :, t, :].T  # [p][r]
        ks[32 * c:32 * c + 32] = sp[:128].view(np.float32)
        vs[32 * c:32 * c + 32] = sp[128:256].view(np.float32)
    return kc, vc, ks, vs


@pytest.mark.parametrize("d,B", [(64, 64), (128, 128)])
def test_packed_cache_holds_quantizer_codes(d, B):
    b, hk, hq, n = 2, 2, 4, 700
    ctx = 650
    k = normal_bf16(15, 2, b * hk * n * d).reshape(b, hk, n, d)
    v = normal_bf16(15, 3, b * hk * n * d).reshape(b, hk, n, d)
    hi, keep = np.array([1, 3], np.int32), np.array([4, 5], np.int32)
    blob = oracle.pack_cache(k, v, hi, keep, hq, B, ctx)
    hdr = blob[:64].view(np.int32)
    assert hdr[0] == 0x43564B54 and hdr[1] == 2 and hdr[2] == b and hdr[3] == hk and hdr[7] == (ctx - 1) // B
    assert blob[:64].view(np.int64)[4] == ctx and blob[:64].view(np.int64)[5] == blob.size
    c = (ctx - 1) // B
    k8c, k8s = oracle.quantize_rows(k, 127)
    k4c, k4s = oracle.quantize_rows(k, 7)
    v8c, v8s = oracle.quantize_rows(v, 127)
    v4c, v4s = oracle.quantize_rows(v, 7)
    for bb in range(b):
        for g in range(hk):
            e = blob[64 + 64 * (bb * hk + g):][:64]
            off = int(e[:8].view(np.int64)[0])
            n8, n4, hh, kk, lo8, sink, lo4, hi4 = e[8:40].view(np.int32)
            assert (hh, kk) == (hi[g], keep[g])
            b8 = ([0] if sink else []) + list(range(lo8, c + 1))
            b4 = list(range(lo4, hi4 + 1))
            assert n8 == len(b8) and n4 == len(b4)
            assert set(b8) == {kb for kb in range(c + 1) if oracle.tile_action(c, kb, hi[g], keep[g]) == 8}
            assert set(b4) == {kb for kb in range(c + 1) if oracle.tile_action(c, kb, hi[g], keep[g]) == 4}
            for blocks, qm in ((b8, 127), (b4, 7)):
                kbytes = B * d if qm == 127 else B * d // 2
                for kb in blocks:
                    rec = blob[off:off + 2 * kbytes + 8 * B]
                    toks = np.arange(kb * B, kb * B + B)
                    valid = toks < ctx
                    kc_ref = (k8c if qm == 127 else k4c)[bb, g, np.minimum(toks, n - 1)]
                    ks_ref = (k8s if qm == 127 else k4s)[bb, g, np.minimum(toks, n - 1)]
                    vc_ref = (v8c if qm == 127 else v4c)[bb, g, np.minimum(toks, n - 1)]
                    vs_ref = (v8s if qm == 127 else v4s)[bb, g, np.minimum(toks, n - 1)]
                    kc_ref[~valid] = 0
                    vc_ref[~valid] = 0
                    ks_ref = np.where(valid, ks_ref, 0)
                    vs_ref = np.where(valid, vs_ref, 0)
                    kc, vc, ks, vs = _read_record(rec, B, d, qm == 7)
                    assert np.array_equal(kc, kc_ref)
                    assert np.array_equal(vc, vc_ref)
                    assert np.array_equal(ks, ks_ref)
                    assert np.array_equal(vs, vs_ref)
                    off += 2 * kbytes + 8 * B
            assert off == (int(blob[64 + 64 * (bb * hk + g) + 64:][:8].view(np.int64)[0])
                           if bb * hk + g + 1 < b * hk else blob.size)


# ---------------------------------------------------------------- decode
def test_decode_all_int8_equals_dense():
    rng = np.random.default_rng(8)
    b, hk, hq, n, d, B = 2, 2, 4, 300, 64, 64
    ctx = 290
    k = bits(int_rows(rng, (b, hk, n, d), 127))
    v = bits(int_rows(rng, (b, hk, n, d), 127))
    q = bits(int_rows(rng, (b, hq, d), 127))
    top = np.full(hk, 99, np.int32)
    sm = 1.0 / 8192
    out = oracle.decode(k, v, q, top, top, B, ctx, sm)
    kf, vf, qf = (bf16_bits_to_float32(x).astype(np.float64) for x in (k, v, q))
    for bb in range(b):
        for h in range(hq):
            g = h // (hq // hk)
            ref = oracle.dense_attention(qf[bb, h][None], kf[bb, g, :ctx], vf[bb, g, :ctx],
                                         np.ones((1, ctx), np.uint8), sm)[0]
            assert np.abs(out[bb, h] - ref).max() < 1e-4


def test_decode_equals_augmented_dense_with_int4():
    b, hk, hq, n, d, B = 1, 2, 4, 900, 64, 64
    ctx = 897
    k = normal_bf16(16, 2, b * hk * n * d).reshape(b, hk, n, d)
    v = normal_bf16(16, 3, b * hk * n * d).reshape(b, hk, n, d)
    q = normal_bf16(16, 6, b * hq * d).reshape(b, hq, d)
    hi, keep = np.array([1, 0], np.int32), np.array([5, 9], np.int32)
    sm = 0.125
    out = oracle.decode(k, v, q, hi, keep, B, ctx, sm)
    q8, q4 = _dequant(q, 127), _dequant(q, 7)
    k8, k4, v8, v4 = _dequant(k, 127), _dequant(k, 7), _dequant(v, 127), _dequant(v, 7)
    c = (ctx - 1) // B
    for h in range(hq):
        g = h // 2
        act = np.array([oracle.tile_action(c, j // B, hi[g], keep[g]) for j in range(ctx)])
        qa = np.concatenate([q8[0, h], q4[0, h]])[None]
        ka = np.concatenate([np.concatenate([k8[0, g, :ctx], np.zeros((ctx, d))], 1),
                             np.concatenate([np.zeros((ctx, d)), k4[0, g, :ctx]], 1)], 0)
        va = np.concatenate([v8[0, g, :ctx], v4[0, g, :ctx]], 0)
        mask = np.concatenate([act == 8, act == 4])[None].astype(np.uint8)
        ref = oracle.dense_attention(qa, ka, va, mask, sm)[0]
        assert np.abs(out[0, h] - ref).max() < 1e-6


def test_decode_matches_prefill_last_row():
    # cross-path: decode at t and prefill row t agree when every head of the group
    # shares one policy, all kept blocks are int8, and inputs are integer-exact
    rng = np.random.default_rng(9)
    b, hk, hq, n, d, B = 1, 1, 2, 256, 64, 64
    k = bits(int_rows(rng, (b, hk, n, d), 127))
    v = bits(int_rows(rng, (b, hk, n, d), 127))  # decode quantises V; amax 127 keeps it exact
    qp = bits(int_rows(rng, (b, hq, n, d), 127))
    top = np.full(hq, 9, np.int32)
    sm = 1.0 / 8192
    pre = oracle.prefill(qp, k, v, top, top, B, sm, reference_mode=True)
    dec = oracle.decode(k, v, qp[:, :, n - 1], top[:hk], top[:hk], B, n, sm)
    assert np.abs(pre[:, :, n - 1] - dec).max() < 1e-5


# ------------------------------------------------------------------ calibration (cost model, allocator)
@pytest.mark.parametrize("n,block", [(512, 64), (1000, 128), (64, 64), (8192, 128)])
def test_policy_cost_closed_forms(n, block):
    """Whole-tile costs of the extreme policies: protected only = block 0 and the
    diagonal (2 nb - 1 tiles), everything int8 = all nb (nb + 1) / 2 causal tiles,
    everything else int4 beyond the protected tiles."""
    nb = -(-n // block)
    b2 = float(block * block)
    assert oracle.policy_cost(n, block, 0, 0, 1.0, 1.0) == (2 * nb - 1) * b2
    assert oracle.policy_cost(n, block, nb - 1, nb - 1, 1.0, 1.0) == nb * (nb + 1) // 2 * b2
    assert oracle.policy_cost(n, block, 0, nb - 1, 3.0, 0.5) == (3.0 * (2 * nb - 1) + 0.5 * (nb * (nb + 1) // 2 - (2 * nb - 1))) * b2
    # hi beyond the sequence saturates
    assert oracle.policy_cost(n, block, nb + 5, nb + 9, 1.0, 1.0) == nb * (nb + 1) // 2 * b2


def _tables(rng, H, K, decreasing=True):
    e = rng.uniform(0.1, 1.0, size=(H, K + 1, K + 1))
    if decreasing:  # error falls with more context and more precision
        e = np.sort(e, axis=2)[:, :, ::-1]
        e = np.sort(e, axis=1)[:, ::-1, :]
    return np.ascontiguousarray(e)


def test_allocator_budget_extremes():
    rng = np.random.default_rng(7)
    n, block, H, K = 1024, 128, 4, 5
    e = _tables(rng, H, K)
    base = H * oracle.policy_cost(n, block, 0, 0)
    hi, keep, tc, te = oracle.allocate_policy(n, block, e, base)
    assert (hi == 0).all() and (keep == 0).all() and tc == base
    hi, keep, tc, te = oracle.allocate_policy(n, block, e, 1e30)   # strictly decreasing tables, no limit
    assert (hi == K).all() and (keep == K).all()
    with pytest.raises(ValueError):
        oracle.allocate_policy(n, block, e, base * 0.999)


def test_allocator_against_brute_force():
    """Tiny instances: the greedy choice fits the budget, its summed cost is the sum of
    its heads' costs, and its summed error is never below the optimum over all
    per-head (hi, keep) combinations that fit (greedy is a heuristic, not exact)."""
    import itertools
    rng = np.random.default_rng(11)
    for trial in range(40):
        n, block = int(rng.integers(64, 700)), 64
        H, K = int(rng.integers(1, 4)), int(rng.integers(0, 4))
        e = _tables(rng, H, K, decreasing=bool(trial % 2))
        pairs = [(a, k) for a in range(K + 1) for k in range(a, K + 1)]
        cost = {pk: oracle.policy_cost(n, block, pk[0], pk[1]) for pk in pairs}
        base = H * cost[(0, 0)]
        budget = base + rng.uniform(0, 1) * (H * max(cost.values()) - base)
        hi, keep, tc, te = oracle.allocate_policy(n, block, e, budget)
        assert tc <= budget
        assert abs(tc - sum(cost[(int(hi[h]), int(keep[h]))] for h in range(H))) <= 1e-9 * max(tc, 1.0)
        best = min(sum(e[h, a, k] for h, (a, k) in enumerate(choice))
                   for choice in itertools.product(pairs, repeat=H)
                   if sum(cost[c] for c in choice) <= budget)
        assert te >= best - 1e-12



# ---------------------------------------------------------------- allocator: hand-worked greedy traces
# TriAttention summary page (rit.work), section on how calibration distributes
# compute between heads: one global allocator gives more context or more precision
# where the added work lowers the error most.  The instances below are small enough
# to run the greedy by hand.  Sequence of 4 blocks of 64 (n = 256, nb = 4); costs
# in units of one tile (64 * 64 pairs).  Kept tiles per (hi, keep), from the tile
# rule (10 causal tiles; block 0 and the diagonal always int8):
#   (0,0): 7 int8            (0,1): 7 int8 + 2 int4    (0,2): 7 int8 + 3 int4
#   (1,1): 9 int8            (1,2): 9 int8 + 1 int4    (2,2): 10 int8
# With an int8 tile at 2 and an int4 tile at 1 the costs are 14, 16, 17, 18, 19, 20;
# with both at 1 they are 7, 9, 10, 9, 10, 10.
# Moves from (a, k): keep -> (a, k + 1) if k < K; hi -> (a + 1, max(k, a + 1)) if a < K.
_N, _B = 256, 64
_U = float(_B * _B)


def _err_table(*heads, K=2):
    """Error tables in units of 1/64 (exact in binary, so equal ratios tie exactly)."""
    e = np.full((len(heads), K + 1, K + 1), 99.0)
    for h, vals in enumerate(heads):
        for (a, k), x in vals.items():
            e[h, a, k] = x / 64.0
    return e


def test_allocator_cost_table_by_hand():
    want = {(0, 0): (14, 7), (0, 1): (16, 9), (0, 2): (17, 10), (1, 1): (18, 9), (1, 2): (19, 10), (2, 2): (20, 10)}
    for (a, k), (c21, c11) in want.items():
        assert oracle.policy_cost(_N, _B, a, k, 2.0, 1.0) == c21 * _U
        assert oracle.policy_cost(_N, _B, a, k, 1.0, 1.0) == c11 * _U


# Instance A: two heads, int8 tile 2, int4 tile 1.  Errors (x 1/64):
#   head 0: (0,0) 64, (0,1) 56, (0,2) 52, (1,1) 48, (1,2) 44, (2,2) 40
#   head 1: (0,0) 64, (0,1) 56, (0,2) 40, (1,1) 60, (1,2) 50, (2,2) 49
# Greedy by hand (score = error drop / cost added, per tile), start cost 28:
#   1. h0 keep 8/2=4, h0 hi 16/4=4, h1 keep 8/2=4, h1 hi 4/4=1: a three-way tie;
#      the lower head wins, and within it the keep move -> h0 (0,1), cost 30
#   2. h0 keep 4/1=4, h0 hi 8/2=4, h1 keep 4, h1 hi 1 -> tie, h0 keep -> h0 (0,2), 31
#   3. h0 hi (1,2) 8/2=4, h1 keep 4 -> tie, lower head -> h0 (1,2), 33
#   4. h0 hi (2,2) 4/1=4, h1 keep 4 -> tie, lower head -> h0 (2,2), 34
#   5. h1 keep 4, h1 hi 1 -> h1 (0,1), 36
#   6. h1 keep (0,2) 16/1=16; h1 hi (1,1) raises the error (60 > 56) -> h1 (0,2), 37
#   7. h1 hi (1,2) raises the error (50 > 40): no move lowers any error; stop.
# Under a budget the trace stops where the next chosen move no longer fits and no
# other move fits either (every move here costs at least one tile).
_A = _err_table({(0, 0): 64, (0, 1): 56, (0, 2): 52, (1, 1): 48, (1, 2): 44, (2, 2): 40},
                {(0, 0): 64, (0, 1): 56, (0, 2): 40, (1, 1): 60, (1, 2): 50, (2, 2): 49})
_A_TRACE = [  # (budget in tiles, hi, keep, cost in tiles, error x 64)
    (28, [0, 0], [0, 0], 28, 128),
    (29, [0, 0], [0, 0], 28, 128),
    (30, [0, 0], [1, 0], 30, 120),
    (31, [0, 0], [2, 0], 31, 116),
    (32, [0, 0], [2, 0], 31, 116),   # step 3's moves (h0 hi, h1 keep) both add 2
    (33, [1, 0], [2, 0], 33, 108),
    (34, [2, 0], [2, 0], 34, 104),
    (35, [2, 0], [2, 0], 34, 104),   # h1 keep adds 2, h1 hi adds 4
    (36, [2, 0], [2, 1], 36, 96),
    (37, [2, 0], [2, 2], 37, 80),
    (1e9, [2, 0], [2, 2], 37, 80),   # stops on step 7: nothing lowers an error
]

# Instance B: one head, int8 tile 2, int4 tile 1, where the best move may not fit.
#   errors: (0,0) 64, (0,1) 60, (0,2) 58, (1,1) 32, (1,2) 30, (2,2) 16
#   no limit: from (0,0) keep 4/2=2, hi 32/4=8 -> (1,1) [18]; keep (1,2) 2/1=2, hi
#   (2,2) 16/2=8 -> (2,2) [20].  Budget 16: hi does not fit (18), keep does -> (0,1)
#   [16]; nothing more fits.  Budget 19: -> (1,1) [18]; hi (2,2) needs 20, keep
#   (1,2) fits -> (1,2) [19].
_B_INST = _err_table({(0, 0): 64, (0, 1): 60, (0, 2): 58, (1, 1): 32, (1, 2): 30, (2, 2): 16})
_B_TRACE = [(16, [0], [1], 16, 60), (19, [1], [2], 19, 30), (1e9, [2], [2], 20, 16)]

# Instance C: one head, both tiles cost 1, so raising hi inside the kept range is
# free.  errors: (0,0) 64, (0,1) 48, (0,2) 40, (1,1) 50, (1,2) 39, (2,2) 38
#   from (0,0): keep 16/2=8, hi 14/2=7 -> (0,1) [9]; keep (0,2) 8/1=8, hi (1,1) raises
#   the error -> (0,2) [10]; hi (1,2) drops 1 at no cost -> (1,2) [10]; hi (2,2) drops
#   1 at no cost -> (2,2) [10].  Budget 9: stops at (0,1).
_C_INST = _err_table({(0, 0): 64, (0, 1): 48, (0, 2): 40, (1, 1): 50, (1, 2): 39, (2, 2): 38})
_C_TRACE = [(9, [0], [1], 9, 48), (10, [2], [2], 10, 38), (1e9, [2], [2], 10, 38)]

# Instance D: free moves go first.  Five blocks (n = 320, K = 3), both tiles cost 1:
# the cost depends on keep only, 9, 12, 14, 15 for keep 0..3.  Errors (x 1/64):
#   head 0: (0,0) 64, (0,1) 43, (0,2) 33, (1,2) 32, (0,3) 31, (1,3) 8
#   head 1: (0,0) 64, (0,1) 28, (0,2) 12, (0,3) 8;  every other entry 99
# Start 18.  1. h0 keep 21/3=7, h1 keep 36/3=12 -> h1 (0,1) [21]; 2. h1 keep 16/2=8 ->
# h1 (0,2) [23]; 3. h0 keep 7, h1 keep 4/1=4 -> h0 (0,1) [26]; 4. h0 keep 10/2=5 ->
# h0 (0,2) [28]; 5. h0 hi (1,2) drops 1 at no cost, ahead of h1's 4 and h0's keep 2
# -> h0 (1,2) [28]; 6. h0 keep (1,3) 24/1=24 -> h0 (1,3) [29]; 7. h1 keep -> (0,3)
# [30]; nothing else lowers an error.  With 29 tiles the free move at step 5 is
# what lets head 0 take the last tile (ranked after h1's 4, it would go to head 1).
_D_INST = _err_table({(0, 0): 64, (0, 1): 43, (0, 2): 33, (1, 2): 32, (0, 3): 31, (1, 3): 8},
                     {(0, 0): 64, (0, 1): 28, (0, 2): 12, (0, 3): 8}, K=3)
_D_TRACE = [(18, [0, 0], [0, 0], 18, 128), (21, [0, 0], [0, 1], 21, 92), (23, [0, 0], [0, 2], 23, 76),
            (26, [0, 0], [1, 2], 26, 55), (28, [1, 0], [2, 2], 28, 44), (29, [1, 0], [3, 2], 29, 20),
            (30, [1, 0], [3, 3], 30, 16), (1e9, [1, 0], [3, 3], 30, 16)]

# Instance E: a move that lowers no error is not taken, even where a later move would
# lower it a lot.  One head, 4 blocks, int8 tile 2, int4 tile 1: (0,0), (0,1) and
# (1,1) all 64, (0,2) 10 -> stays at (0,0) [14].
_E_INST = _err_table({(0, 0): 64, (0, 1): 64, (1, 1): 64, (0, 2): 10})
_E_TRACE = [(1e9, [0], [0], 14, 64)]

ALLOC_CASES = [("A", _N, _A, 2.0, _A_TRACE), ("B", _N, _B_INST, 2.0, _B_TRACE), ("C", _N, _C_INST, 1.0, _C_TRACE),
               ("D", 320, _D_INST, 1.0, _D_TRACE), ("E", _N, _E_INST, 2.0, _E_TRACE)]


@pytest.mark.parametrize("name,n,err,c8,trace", ALLOC_CASES, ids=[c[0] for c in ALLOC_CASES])
def test_allocator_hand_worked_traces(name, n, err, c8, trace):
    for budget, hi, keep, cost, e64 in trace:
        b = 1e30 if budget >= 1e9 else budget * _U
        got_hi, got_keep, tc, te = oracle.allocate_policy(n, _B, err, b, c8, 1.0)
        assert got_hi.tolist() == hi and got_keep.tolist() == keep, (name, budget, got_hi, got_keep)
        assert tc == cost * _U and te * 64 == e64, (name, budget, tc / _U, te * 64)
