"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: codes, scales, schedules and packed cache bytes bit-exact; attention outputs
within max|diff| <= 2e-2 and mean relative error sum|diff| / sum|ref| <= 1e-3.
Small shapes are compared element by element over every output; the full-size
workloads (the launch configuration the benchmark times) on sampled query blocks
the oracle recomputes one by one.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
MEAN_REL = 1e-3
# The base-2 log-sum-exp M + log2(l) (an optional output with no stated tolerance):
# the kernel forms t in fp32 and the oracle in double, so a weight whose fp32 value
# lies within rounding of a bf16 rounding boundary can round one way on the GPU and
# the other in the oracle.  One such flip changes l by at most 2^-8 of that weight,
# hence the LSE by at most log2(1 + 2^-8) = 5.6e-3 when that weight dominates its
# row.  Bound: 1e-2 on every row (room for about two flips of a dominant weight),
# and 1e-5 on the mean over rows (flips are rare).
LSE_MAX = 1e-2
LSE_MEAN = 1e-5


def assert_lse_close(gpu: np.ndarray, ref: np.ndarray, what: str):
    diff = np.abs(gpu.astype(np.float64) - ref.astype(np.float64))
    print(f"[parity] {what} LSE: max|diff|={diff.max():.3e} mean={diff.mean():.3e}", flush=True)
    assert diff.max() <= LSE_MAX and diff.mean() <= LSE_MEAN, (what, diff.max(), diff.mean())


@pytest.fixture(scope="module")
def tria():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_sparse_mixed_head_amd as t
    return t


def dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str):
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    diff = np.abs(gpu.astype(np.float64) - ref.astype(np.float64))
    mx = diff.max()
    rel = diff.sum() / max(np.abs(ref).sum(), 1e-30)
    print(f"[parity] {what}: max|diff|={mx:.3e} mean_rel={rel:.3e}", flush=True)
    assert mx <= MAX_ABS and rel <= MEAN_REL, (what, mx, rel)


def inputs(cfg):
    q, k, v = synth.make_prefill_inputs(cfg)
    return q, k, v


def run_prefill(tria, cfg, q, k, v, hi, keep, with_lse=False):
    d = tria.make_dims(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.block, cfg.seq_len)
    sched = torch.from_numpy(tria.build_policy(d, hi, keep)).cuda()
    qd, kd, vd = dev(q), dev(k), dev(v)
    qz = tria.quantize_qk(d, qd, kd)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda") if with_lse else None
    out = tria.prefill(d, sched, qz, vd, 1.0 / math.sqrt(cfg.head_dim), lse=lse)
    torch.cuda.synchronize()
    return out, lse, qz


# ------------------------------------------------------------------ quantiser
@pytest.mark.parametrize("cid", ["tiny", "llama3_8b_layer"])
def test_quantizer_bit_exact(tria, cid):
    cfg = synth.CONFIGS[cid]
    print(f"[case] quantize config {cid}", flush=True)
    q, k, _ = inputs(cfg)
    d = tria.make_dims(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.block, cfg.seq_len)
    qz = tria.quantize_qk(d, dev(q), dev(k))
    torch.cuda.synchronize()
    for x, c8, c4, s8, s4 in ((q, qz.q8, qz.q4, qz.q8s, qz.q4s), (k, qz.k8, qz.k4, qz.k8s, qz.k4s)):
        r8, rs8 = oracle.quantize_rows(x, 127)
        r4, rs4 = oracle.quantize_rows(x, 7)
        assert np.array_equal(c8.cpu().numpy(), r8)
        assert np.array_equal(s8.cpu().numpy().view(np.uint32), rs8.view(np.uint32))
        assert np.array_equal(c4.cpu().numpy(), oracle.pack_nibbles(r4))
        assert np.array_equal(s4.cpu().numpy().view(np.uint32), rs4.view(np.uint32))


def test_quantizer_edge_rows(tria):
    # zero rows, constant rows, exact .5 ties, huge and tiny magnitudes
    b, h, n, d = 1, 1, 64, 128
    x = np.random.default_rng(0).standard_normal((b, h, n, d)).astype(np.float32)
    x[0, 0, 0] = 0
    x[0, 0, 1] = -3.5
    x[0, 0, 2] = 0
    x[0, 0, 2, 0] = 127.0
    x[0, 0, 2, 1:6] = [0.5, 1.5, 2.5, -0.5, -2.5]
    x[0, 0, 3] *= 1e30
    x[0, 0, 4] *= 1e-30
    bits = synth.float32_to_bf16_bits(x)
    dd = tria.make_dims(b, h, h, d, 64, n)
    qz = tria.quantize_qk(dd, dev(bits), dev(bits))
    torch.cuda.synchronize()
    r8, s8 = oracle.quantize_rows(bits, 127)
    r4, s4 = oracle.quantize_rows(bits, 7)
    assert np.array_equal(qz.q8.cpu().numpy(), r8) and np.array_equal(qz.k8.cpu().numpy(), r8)
    assert np.array_equal(qz.q4.cpu().numpy(), oracle.pack_nibbles(r4))
    assert np.array_equal(qz.q8s.cpu().numpy(), s8) and np.array_equal(qz.q4s.cpu().numpy(), s4)


# ------------------------------------------------------------------ prefill, small shapes (every output)
def small_cfg(b, hq, hk, d, n, blk, seed=21):
    return synth.Config("small", b, hq, hk, d, n, blk, seed=seed)


SMALL = [
    # (b, hq, hk, d, n, blk, hi, keep)
    (1, 2, 1, 64, 512, 64, [2, 2], [4, 4]),             # the tiny workload's shape and policy
    (1, 4, 2, 128, 700, 128, [0, 1, 2, 6], [6, 3, 2, 6]),   # ragged n, B=128
    (2, 3, 3, 64, 333, 64, [0, 1, 9], [0, 4, 9]),       # MHA, ragged, batch 2
    (1, 4, 1, 128, 640, 64, [1, 0, 3, 0], [1, 9, 5, 2]),    # MQA, B=64, d=128
    (1, 7, 1, 128, 1000, 128, [7, 0, 0, 1, 2, 3, 4], [7, 0, 7, 5, 4, 3, 6]),  # G=7 edge policies
    (1, 2, 1, 64, 40, 64, [0, 3], [0, 3]),              # n < block
    (1, 2, 2, 128, 129, 128, [0, 0], [0, 1]),            # one full block + one token
    (2, 4, 2, 128, 1, 128, [0, 1, 2, 3], [1, 2, 3, 4]),   # a single token (one unit per head, one row)
    (1, 4, 2, 64, 700, 128, [0, 1, 2, 3], [2, 4, 3, 5]),    # d=64 with B=128: sink, int4 ranges, ragged
]


@pytest.mark.parametrize("case", SMALL, ids=[f"b{c[0]}h{c[1]}k{c[2]}d{c[3]}n{c[4]}B{c[5]}" for c in SMALL])
def test_prefill_small_every_output(tria, case):
    b, hq, hk, d, n, blk, hi, keep = case
    print(f"[case] prefill small {case}", flush=True)
    cfg = small_cfg(b, hq, hk, d, n, blk)
    q, k, v = inputs(cfg)
    hi, keep = np.array(hi, np.int32), np.array(keep, np.int32)
    out, lse, _ = run_prefill(tria, cfg, q, k, v, hi, keep, with_lse=True)
    ref, rlse = oracle.prefill(q, k, v, hi, keep, blk, 1.0 / math.sqrt(d), with_lse=True)
    assert_close(out.cpu().numpy(), ref, f"prefill {case}")
    assert_lse_close(lse.cpu().numpy(), rlse, "prefill")


@pytest.mark.parametrize("case", SMALL, ids=[f"b{c[0]}h{c[1]}k{c[2]}d{c[3]}n{c[4]}B{c[5]}" for c in SMALL])
def test_prefill_bf16q_equals_two_step(tria, case):
    """prefill_bf16q (Q quantised inside the kernel) gives out and LSE bit for bit
    those of quantize_qk + prefill, and quantize_k writes quantize_qk's K outputs."""
    b, hq, hk, d, n, blk, hi, keep = case
    print(f"[case] prefill bf16q {case}", flush=True)
    cfg = small_cfg(b, hq, hk, d, n, blk, seed=71)
    q, k, v = inputs(cfg)
    dd = tria.make_dims(b, hq, hk, d, blk, n)
    sched = torch.from_numpy(tria.build_policy(dd, np.array(hi, np.int32), np.array(keep, np.int32))).cuda()
    qd, kd, vd = dev(q), dev(k), dev(v)
    sm = 1.0 / math.sqrt(d)
    qz = tria.quantize_qk(dd, qd, kd)
    kz = tria.quantize_k(dd, kd)
    for name in ("k8", "k4", "k8s", "k4s"):
        assert torch.equal(getattr(qz, name), getattr(kz, name)), name
    lse0 = torch.empty((b, hq, n), dtype=torch.float32, device="cuda")
    lse1 = torch.empty_like(lse0)
    out0 = tria.prefill(dd, sched, qz, vd, sm, lse=lse0)
    out1 = tria.prefill_bf16q(dd, sched, qd, kz, vd, sm, lse=lse1)
    torch.cuda.synchronize()
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1)


def test_prefill_bf16q_full_size_layer(tria):
    """The Llama-3-8B-shaped layer: the fused path equals the two-step path on every
    output (the two-step path is compared with the oracle on every output above)."""
    c = synth.CONFIGS["llama3_8b_layer"]
    print("[case] prefill bf16q full-size llama3_8b_layer", flush=True)
    q, k, v = (dev(x) for x in synth.make_prefill_inputs(c))
    hi, keep = c.policy()
    dd = tria.make_dims(c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim, c.block, c.seq_len)
    sched = torch.from_numpy(tria.build_policy(dd, hi, keep)).cuda()
    sm = 1.0 / math.sqrt(c.head_dim)
    qz = tria.quantize_qk(dd, q, k)
    out0 = tria.prefill(dd, sched, qz, v, sm)
    out1 = tria.prefill_bf16q(dd, sched, q, tria.quantize_k(dd, k), v, sm)
    torch.cuda.synchronize()
    assert torch.equal(out0, out1)


VARLEN = [
    # (hq, hk, d, blk, lengths, hi, keep)
    (4, 2, 64, 64, [1, 199, 63, 437, 64], [0, 1, 2, 9], [0, 4, 3, 9]),
    (4, 1, 128, 128, [300, 129, 7, 900], [1, 0, 3, 2], [5, 8, 3, 2]),
    (2, 2, 128, 64, [640], [1, 2], [3, 7]),       # one sequence: the fixed-length path's result
]


@pytest.mark.parametrize("case", VARLEN, ids=[f"h{c[0]}k{c[1]}d{c[2]}B{c[3]}s{len(c[4])}" for c in VARLEN])
def test_prefill_varlen_every_output(tria, case):
    """Sequences of different lengths packed along the rows of one batch element:
    every output row (and LSE) equals the oracle's prefill of its sequence alone."""
    hq, hk, d, blk, lens, hi, keep = case
    print(f"[case] prefill varlen {case}", flush=True)
    T = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    cfg = small_cfg(1, hq, hk, d, T, blk, seed=23)
    q, k, v = inputs(cfg)
    hi, keep = np.array(hi, np.int32), np.array(keep, np.int32)
    dd = tria.make_dims(1, hq, hk, d, blk, T)
    sched = torch.from_numpy(tria.build_policy_varlen(dd, hi, keep, cu)).cuda()
    qz = tria.quantize_qk(dd, dev(q), dev(k))
    lse = torch.empty((1, hq, T), dtype=torch.float32, device="cuda")
    out = tria.prefill_varlen(dd, cu, sched, qz, dev(v), 1.0 / math.sqrt(d), lse=lse)
    torch.cuda.synchronize()
    got, glse = out.cpu().numpy(), lse.cpu().numpy()
    for i in range(len(lens)):
        s0, s1 = int(cu[i]), int(cu[i + 1])
        ref, rlse = oracle.prefill(q[:, :, s0:s1], k[:, :, s0:s1], v[:, :, s0:s1], hi, keep, blk,
                                   1.0 / math.sqrt(d), with_lse=True)
        assert_close(got[:, :, s0:s1], ref, f"varlen {case} sequence {i}")
        assert_lse_close(glse[:, :, s0:s1], rlse, f"varlen sequence {i}")


def test_prefill_integer_inputs_and_determinism(tria):
    # all blocks kept and integer rows with amax 127 (codes = values, scales 1):
    # large exact integer scores; two runs must be bitwise equal
    rng = np.random.default_rng(3)
    b, hq, hk, d, n, blk = 1, 2, 1, 128, 300, 128
    x = rng.integers(-127, 128, size=(b, hq + 2 * hk, n, d)).astype(np.float32)
    x[..., 0] = 127.0
    x[:, hq + hk:] = rng.integers(-9, 10, size=(b, hk, n, d))
    bits = synth.float32_to_bf16_bits(x)
    q, k, v = bits[:, :hq].copy(), bits[:, hq:hq + hk].copy(), bits[:, hq + hk:].copy()
    top = np.full(hq, 99, np.int32)
    cfg = small_cfg(b, hq, hk, d, n, blk)
    out, _, _ = run_prefill(tria, cfg, q, k, v, top, top)
    out2, _, _ = run_prefill(tria, cfg, q, k, v, top, top)
    assert np.array_equal(out.cpu().numpy(), out2.cpu().numpy()), "not deterministic"
    ref = oracle.prefill(q, k, v, top, top, blk, 1.0 / math.sqrt(d))
    assert_close(out.cpu().numpy(), ref, "integer-exact all-kept")


def test_prefill_unit_order_does_not_matter(tria):
    """The schedule's record order is a dispatch order only: the same records in a
    random order give the same output and LSE bit for bit (every unit computes its
    own rows alone)."""
    b, hq, hk, d, n, blk = 2, 4, 2, 128, 1500, 128
    cfg = small_cfg(b, hq, hk, d, n, blk, seed=61)
    q, k, v = inputs(cfg)
    hi, keep = np.array([1, 0, 3, 2], np.int32), np.array([9, 4, 3, 11], np.int32)
    dd = tria.make_dims(b, hq, hk, d, blk, n)
    blob = tria.build_policy(dd, hi, keep)
    qz = tria.quantize_qk(dd, dev(q), dev(k))
    vd = dev(v)

    def run(words):
        out = torch.empty((b, hq, n, d), dtype=torch.float32, device="cuda")
        lse = torch.empty((b, hq, n), dtype=torch.float32, device="cuda")
        tria.prefill(dd, torch.from_numpy(words).cuda(), qz, vd, 1.0 / math.sqrt(d), out=out, lse=lse)
        torch.cuda.synchronize()
        return out.cpu().numpy(), lse.cpu().numpy()

    o0, l0 = run(blob)
    units = blob[16:].reshape(-1, 8)
    for seed in (1, 2):
        perm = np.random.default_rng(seed).permutation(len(units))
        shuffled = blob.copy()
        shuffled[16:] = units[perm].reshape(-1)
        o1, l1 = run(shuffled)
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1), seed
    ref = oracle.prefill(q, k, v, hi, keep, blk, 1.0 / math.sqrt(d))
    assert_close(o0, ref, "prefill under the dispatch order")


def test_prefill_skipped_blocks_never_read(tria):
    # NaN in key/value rows of blocks that every query block either skips or has
    # past the causal boundary must leave the output bit-identical
    b, hq, hk, d, n, blk = 1, 2, 1, 128, 1024, 128
    cfg = small_cfg(b, hq, hk, d, n, blk, seed=31)
    q, k, v = inputs(cfg)
    hi, keep = np.array([1, 0], np.int32), np.array([2, 2], np.int32)
    base, _, _ = run_prefill(tria, cfg, q, k, v, hi, keep)
    k2, v2 = k.copy(), v.copy()
    # block 2 is skipped for query blocks >= 5 (distance > 2); poison only rows those
    # blocks can see is impossible, so compare rows of query blocks >= 5 only
    k2[..., 2 * blk:3 * blk, :] = 0x7FC0
    v2[..., 2 * blk:3 * blk, :] = 0x7FC0
    pois, _, _ = run_prefill(tria, cfg, q, k2, v2, hi, keep)
    a = base.cpu().numpy()[:, :, 5 * blk:]
    p = pois.cpu().numpy()[:, :, 5 * blk:]
    assert np.array_equal(a, p)


def test_prefill_bad_schedule_gives_nan(tria):
    """A schedule whose header does not describe the call gives NaN in every output row
    and LSE; a malformed unit gives NaN in its own rows and leaves every other row as
    the intact schedule computes it; a unit that names no rows (a head out of range)
    writes nothing: the rows it replaced keep what the output held, every other row is
    as the intact schedule computes it.  The kernel exits normally in every case."""
    b, hq, hk, d, n, blk = 1, 4, 2, 128, 700, 128
    cfg = small_cfg(b, hq, hk, d, n, blk, seed=51)
    q, k, v = inputs(cfg)
    hi, keep = np.array([0, 1, 2, 6], np.int32), np.array([6, 3, 2, 6], np.int32)
    dd = tria.make_dims(b, hq, hk, d, blk, n)
    blob = tria.build_policy(dd, hi, keep)
    qz = tria.quantize_qk(dd, dev(q), dev(k))
    vd = dev(v)
    sm = 1.0 / math.sqrt(d)

    def run(words):
        out = torch.full((b, hq, n, d), 7.0, dtype=torch.float32, device="cuda")
        lse = torch.full((b, hq, n), 7.0, dtype=torch.float32, device="cuda")
        tria.prefill(dd, torch.from_numpy(words).cuda(), qz, vd, sm, out=out, lse=lse)
        torch.cuda.synchronize()
        return out.cpu().numpy(), lse.cpu().numpy()

    good, glse = run(blob)
    assert np.isfinite(good).all() and np.isfinite(glse).all()
    print("[case] bad schedule headers", flush=True)
    for word, val in ((0, 0x1234), (1, 2), (2, 2), (3, 8), (4, 1), (5, 64), (6, 64), (7, 5), (8, 23), (10, n + 1),
                      (11, 1)):
        bad = blob.copy()
        bad[word] = val
        o, l = run(bad)
        assert np.isnan(o).all() and np.isnan(l).all(), (word, val)
    units = blob[16:].reshape(-1, 8)
    i = int(np.nonzero((units[:, 0] == 0) & (units[:, 1] == 2) & (units[:, 2] == 3))[0][0])
    rows = np.zeros((b, hq, n), bool)
    rows[0, 2, 3 * blk:4 * blk] = True
    print("[case] malformed units", flush=True)
    for field, val in ((3, 4), (6, 2), (7, 99), (5, 0)):   # lo8 > qb, sink 2, ntiles, int4 range [0, 0] (block 0)
        bad = blob.copy()
        bad[16 + 8 * i + field] = val
        o, l = run(bad)
        assert np.isnan(o[rows]).all() and np.isnan(l[rows]).all(), (field, val)
        assert np.array_equal(o[~rows], good[~rows]) and np.array_equal(l[~rows], glse[~rows]), (field, val)
    print("[case] an int4 range that does not end where the int8 run begins", flush=True)
    j = int(np.nonzero((units[:, 0] == 0) & (units[:, 1] == 0) & (units[:, 2] == 5))[0][0])
    assert units[j, 5] - units[j, 4] >= 1 and units[j, 5] == units[j, 3] - 1
    bad = blob.copy()
    bad[16 + 8 * j + 5] -= 1   # hi4: one block short of lo8 - 1
    bad[16 + 8 * j + 7] -= 1   # ntiles that agrees with the shorter range
    o, l = run(bad)
    rows2 = np.zeros((b, hq, n), bool)
    rows2[0, 0, 5 * blk:] = True
    assert np.isnan(o[rows2]).all() and np.isnan(l[rows2]).all()
    assert np.array_equal(o[~rows2], good[~rows2]) and np.array_equal(l[~rows2], glse[~rows2])
    print("[case] a unit that names no rows", flush=True)
    bad = blob.copy()
    bad[16 + 8 * i + 1] = 99                               # head 99 of 4
    o, l = run(bad)
    assert (o[rows] == 7.0).all() and (l[rows] == 7.0).all()   # the replaced unit's rows: untouched
    assert np.array_equal(o[~rows], good[~rows]) and np.array_equal(l[~rows], glse[~rows])


def test_prefill_varlen_bad_schedule_gives_nan(tria):
    """Variable-length batch: a header with the wrong sequence count, or the fixed-length
    version, gives NaN everywhere."""
    hq, hk, d, blk = 2, 1, 64, 64
    lens = [100, 37, 200]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    cfg = small_cfg(1, hq, hk, d, T, blk, seed=52)
    q, k, v = inputs(cfg)
    hi, keep = np.array([0, 2], np.int32), np.array([1, 2], np.int32)
    dd = tria.make_dims(1, hq, hk, d, blk, T)
    blob = tria.build_policy_varlen(dd, hi, keep, cu)
    qz = tria.quantize_qk(dd, dev(q), dev(k))
    vd = dev(v)
    print("[case] varlen bad schedule headers", flush=True)
    for word, val in ((None, None), (1, 1), (2, 2), (7, 3)):
        bad = blob.copy()
        if word is not None:
            bad[word] = val
        out = tria.prefill_varlen(dd, cu, torch.from_numpy(bad).cuda(), qz, vd, 1.0 / math.sqrt(d))
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        assert np.isfinite(o).all() if word is None else np.isnan(o).all(), (word, val)


# ------------------------------------------------------------------ prefill, full-size workloads (sampled)
def sample_units(cfg, hi, keep, spread=29):
    """Query blocks sampled per (batch element, head): the first and the last, the
    blocks where the head's tile pattern changes shape (hi + 1: the last whose int8
    run reaches block 0; hi + 2: the first with block 0 kept apart; keep + 1 and
    keep + 2: the first whose int4 run ends at block 1 and the first with a skipped
    block), and `spread` blocks spaced evenly over the sequence."""
    nb = cfg.nb
    even = set(np.round(np.linspace(0, nb - 1, spread)).astype(int).tolist())
    units = []
    for bb in range(cfg.batch):
        for h in range(cfg.n_q_heads):
            edges = {int(hi[h]) + 1, int(hi[h]) + 2, int(keep[h]) + 1, int(keep[h]) + 2}
            qbs = ({0, nb - 1} | {e for e in edges if e < nb} | even)
            units += [(bb, h, int(x)) for x in sorted(qbs)]
    return units


def test_prefill_full_size_every_output(tria):
    """The Llama-3-8B-shaped layer (n = 8192) at full size, every output element and
    LSE entry against the oracle."""
    cfg = synth.CONFIGS["llama3_8b_layer"]
    print("[case] prefill full-size llama3_8b_layer, every output", flush=True)
    q, k, v = inputs(cfg)
    hi, keep = cfg.policy()
    out, lse, _ = run_prefill(tria, cfg, q, k, v, hi, keep, with_lse=True)
    ref, rlse = oracle.prefill(q, k, v, hi, keep, cfg.block, 1.0 / math.sqrt(cfg.head_dim), with_lse=True)
    assert_close(out.cpu().numpy(), ref, f"prefill {cfg.name} (every output)")
    assert_lse_close(lse.cpu().numpy(), rlse, "prefill")


@pytest.mark.parametrize("cid", ["long_prefill", "batched_mixed"])
def test_prefill_full_size_sampled(tria, cid):
    """The long-prefill and batched mixed-policy workloads at full size, every row of
    the sampled query blocks of every head and batch element against the oracle;
    every output finite; and the launch the benchmark times (query blocks quantised
    inside the kernel, K codes from tria_quantize_k) equal to it on every output."""
    cfg = synth.CONFIGS[cid]
    q, k, v = inputs(cfg)
    hi, keep = cfg.policy()
    units = sample_units(cfg, hi, keep)
    print(f"[case] prefill full-size {cid}: {len(units)} sampled units", flush=True)
    out, lse, _ = run_prefill(tria, cfg, q, k, v, hi, keep, with_lse=True)
    dd = tria.make_dims(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.block, cfg.seq_len)
    qd, kd = dev(q), dev(k)
    lse1 = torch.empty_like(lse)
    out1 = tria.prefill_bf16q(dd, torch.from_numpy(tria.build_policy(dd, hi, keep)).cuda(), qd,
                              tria.quantize_k(dd, kd), dev(v), 1.0 / math.sqrt(cfg.head_dim), lse=lse1)
    torch.cuda.synchronize()
    assert torch.equal(out, out1) and torch.equal(lse, lse1), "fused-Q prefill differs from the two-step path"
    del out1, lse1, qd, kd
    ref, rlse = oracle.prefill(q, k, v, hi, keep, cfg.block, 1.0 / math.sqrt(cfg.head_dim), units=units,
                               with_lse=True)
    got, want, gl, wl = [], [], [], []
    o_np, l_np = out.cpu().numpy(), lse.cpu().numpy()
    for (bb, h, qb) in units:
        r0, r1 = qb * cfg.block, min(cfg.seq_len, (qb + 1) * cfg.block)
        got.append(o_np[bb, h, r0:r1])
        want.append(ref[bb, h, r0:r1])
        gl.append(l_np[bb, h, r0:r1])
        wl.append(rlse[bb, h, r0:r1])
    assert_close(np.concatenate(got), np.concatenate(want), f"prefill {cfg.name} ({len(units)} sampled units)")
    assert_lse_close(np.concatenate(gl), np.concatenate(wl), f"prefill {cfg.name}")
    assert np.isfinite(o_np).all() and np.isfinite(l_np).all()


# ------------------------------------------------------------------ cache + decode
DEC_SMALL = [
    # (b, hq, hk, d, n, blk, ctx, hi, keep)  policies per KV head
    (2, 4, 2, 64, 900, 64, 897, [1, 0], [5, 9]),
    (1, 8, 2, 128, 1300, 128, 1300, [0, 2], [3, 10]),
    (3, 7, 1, 128, 700, 64, 650, [2], [4]),
    (1, 32, 1, 128, 512, 128, 500, [1], [2]),   # MQA with 32 query heads (two row groups)
    (1, 2, 2, 64, 64, 64, 1, [0, 0], [0, 0]),   # a single token
    (1, 4, 4, 128, 2000, 128, 2000, [99, 0, 0, 1], [99, 0, 99, 2]),
    (1, 8, 2, 64, 700, 128, 650, [1, 0], [3, 5]),  # d=64 with B=128
]


def _dec_case(tria, case, seed=41):
    b, hq, hk, d, n, blk, ctx, hi, keep = case
    cfg = synth.Config("dec", b, hq, hk, d, n, blk, seed=seed, decode=True)
    k, v, q = synth.make_decode_inputs(cfg)
    hi, keep = np.array(hi, np.int32), np.array(keep, np.int32)
    dd = tria.make_dims(b, hq, hk, d, blk, n)
    cache = tria.pack_kv_cache(dd, hi, keep, ctx, dev(k), dev(v))
    out = tria.decode(dd, cache, ctx, dev(q), 1.0 / math.sqrt(d))
    torch.cuda.synchronize()
    return cfg, k, v, q, hi, keep, dd, cache, out


@pytest.mark.parametrize("case", DEC_SMALL, ids=[f"b{c[0]}h{c[1]}k{c[2]}d{c[3]}ctx{c[6]}B{c[5]}" for c in DEC_SMALL])
def test_pack_and_decode_small(tria, case):
    print(f"[case] decode small {case}", flush=True)
    cfg, k, v, q, hi, keep, dd, cache, out = _dec_case(tria, case)
    b, hq, hk, d, n, blk, ctx = case[:7]
    ref_blob = oracle.pack_cache(k, v, hi, keep, hq, blk, ctx)
    assert cache.numel() == ref_blob.size
    assert np.array_equal(cache.cpu().numpy(), ref_blob), "packed cache differs from the oracle's bytes"
    tria.check_cache(dd, cache, ctx)
    ref = oracle.decode(k, v, q, hi, keep, blk, ctx, 1.0 / math.sqrt(d))
    assert_close(out.cpu().numpy(), ref, f"decode {case}")


def test_allocator_policy_through_prefill_and_decode(tria):
    """Calibration (TriAttention summary page, section on how calibration distributes
    compute between heads) feeding the hot path: the library's greedy allocator picks
    per-query-head (hi, keep) from seeded synthetic error tables under a budget of
    about half the dense cost; prefill over that policy, and the cache packed from it
    (merged per KV head by the group maximum) with one-token decode, match the
    oracle run on the same policy."""
    b, hq, hk, d, n, blk = 1, 8, 2, 128, 1500, 128
    nb = (n + blk - 1) // blk
    K = nb - 1
    rng = np.random.default_rng(77)
    e = rng.uniform(0.0, 1.0, size=(hq, K + 1, K + 1))
    e = np.ascontiguousarray(np.sort(np.sort(e, axis=2)[:, :, ::-1], axis=1)[:, ::-1, :])
    dd = tria.make_dims(b, hq, hk, d, blk, n)
    dense = hq * tria.policy_cost(dd, K, K, 2.0, 1.0)
    hi, keep, tc, _ = tria.allocate_policy(dd, e, 0.5 * dense, 2.0, 1.0)
    o_hi, o_keep, o_tc, _ = oracle.allocate_policy(n, blk, e, 0.5 * dense, 2.0, 1.0)
    assert np.array_equal(hi, o_hi) and np.array_equal(keep, o_keep) and tc == o_tc
    print(f"[case] allocator policy hi={hi.tolist()} keep={keep.tolist()}", flush=True)
    assert len(set(zip(hi.tolist(), keep.tolist()))) > 1, "expected the heads to differ"
    cfg = small_cfg(b, hq, hk, d, n, blk, seed=78)
    q, k, v = inputs(cfg)
    out, lse, _ = run_prefill(tria, cfg, q, k, v, hi, keep, with_lse=True)
    ref, rlse = oracle.prefill(q, k, v, hi, keep, blk, 1.0 / math.sqrt(d), with_lse=True)
    assert_close(out.cpu().numpy(), ref, "prefill under the allocator's policy")
    assert_lse_close(lse.cpu().numpy(), rlse, "prefill")
    ctx = n - 5
    cache = tria.pack_kv_cache(dd, hi, keep, ctx, dev(k), dev(v))
    assert np.array_equal(cache.cpu().numpy(), oracle.pack_cache(k, v, hi, keep, hq, blk, ctx))
    qd = np.ascontiguousarray(q[:, :, ctx - 1])
    o = tria.decode(dd, cache, ctx, dev(qd), 1.0 / math.sqrt(d))
    torch.cuda.synchronize()
    assert_close(o.cpu().numpy(), oracle.decode(k, v, qd, hi, keep, blk, ctx, 1.0 / math.sqrt(d)),
                 "decode under the allocator's policy")


VARLEN_DEC = [
    # (hq, hk, d, n, blk, ctx_lens, hi, keep)  policies per KV head
    (8, 2, 128, 1300, 128, [1300, 1, 640, 129], [1, 0], [5, 3]),
    (7, 1, 64, 900, 64, [65, 900, 333], [2], [6]),
    (4, 4, 128, 700, 64, [700, 700], [99, 0, 0, 1], [99, 0, 99, 3]),   # equal lengths, edge policies
]


def _varlen_cache_from_oracle(k, v, hi, keep, hq, blk, d, ctx_lens):
    """The expected version-3 bytes, spliced from the oracle's cache of each sequence
    alone: header fields for the batch, each directory entry with its offset moved
    and its sequence's ctx_len in words 10-11, then the sequences' records in order."""
    b, hk = len(ctx_lens), k.shape[1]
    data0 = (64 + 64 * b * hk + 255) // 256 * 256
    one0 = (64 + 64 * hk + 255) // 256 * 256
    blobs = [oracle.pack_cache(k[i:i + 1], v[i:i + 1], hi, keep, hq, blk, int(ctx_lens[i])) for i in range(b)]
    recs = [bl[one0:] for bl in blobs]
    total = data0 + sum(r.size for r in recs)
    out = np.zeros(total, np.uint8)
    hd = np.zeros(8, np.int32)
    hd[:8] = [0x43564B54, 3, b, hk, d, blk, (max(ctx_lens) - 1) // blk + 1, -1]
    out[0:32] = hd.view(np.uint8)
    out[32:64] = np.array([0, total, 64, data0], np.int64).view(np.uint8)
    pos = data0
    for i, bl in enumerate(blobs):
        for g in range(hk):
            e = bl[64 + 64 * g: 128 + 64 * g].copy()
            off = int(e[0:8].view(np.int64)[0])
            e[0:8] = np.array([off - one0 + pos], np.int64).view(np.uint8)
            e[40:48] = np.array([ctx_lens[i]], np.int64).view(np.uint8)
            p_ = 64 + 64 * (i * hk + g)
            out[p_:p_ + 64] = e
        out[pos:pos + recs[i].size] = recs[i]
        pos += recs[i].size
    return out


@pytest.mark.parametrize("case", VARLEN_DEC, ids=[f"h{c[0]}k{c[1]}d{c[2]}B{c[4]}b{len(c[5])}" for c in VARLEN_DEC])
def test_varlen_cache_and_decode(tria, case):
    """A batch whose sequences sit at different lengths: the packed bytes equal the
    oracle's per-sequence caches spliced into the version-3 layout, and each
    sequence's decode output equals the oracle's decode of that sequence alone."""
    hq, hk, d, n, blk, ctx_lens, hi, keep = case
    print(f"[case] varlen cache + decode {case}", flush=True)
    b = len(ctx_lens)
    cfg = synth.Config("vdec", b, hq, hk, d, n, blk, seed=47, decode=True)
    k, v, q = synth.make_decode_inputs(cfg)
    hi, keep = np.array(hi, np.int32), np.array(keep, np.int32)
    dd = tria.make_dims(b, hq, hk, d, blk, n)
    cache = tria.pack_kv_cache_varlen(dd, hi, keep, ctx_lens, dev(k), dev(v))
    out = tria.decode_varlen(dd, cache, dev(q), 1.0 / math.sqrt(d))
    torch.cuda.synchronize()
    want = _varlen_cache_from_oracle(k, v, hi, keep, hq, blk, d, ctx_lens)
    assert cache.numel() == want.size
    assert np.array_equal(cache.cpu().numpy(), want), "variable-length cache differs from the spliced oracle bytes"
    got = out.cpu().numpy()
    for i in range(b):
        ref = oracle.decode(k[i:i + 1], v[i:i + 1], q[i:i + 1], hi, keep, blk, int(ctx_lens[i]), 1.0 / math.sqrt(d))
        assert_close(got[i:i + 1], ref, f"varlen decode {case} sequence {i}")


UPD_CASES = [
    # (b, hq, hk, d, n, blk, ctx0, steps, hi, keep)  policies per KV head
    (2, 4, 2, 64, 400, 64, 120, 150, [1, 0], [3, 5]),     # crosses block starts 128, 192, 256
    (1, 8, 2, 128, 700, 128, 250, 140, [0, 2], [1, 4]),   # crosses 256, 384; hi = 0 demotes at once
    (1, 2, 1, 64, 300, 64, 1, 140, [0], [2]),             # from a single token
    (1, 4, 4, 128, 600, 128, 380, 20, [99, 0, 0, 1], [99, 0, 99, 2]),  # all-int8, protected-only, all-int4
]


@pytest.mark.parametrize("case", UPD_CASES, ids=[f"b{c[0]}k{c[2]}d{c[3]}B{c[5]}ctx{c[6]}+{c[7]}" for c in UPD_CASES])
def test_update_matches_pack(tria, case):
    """Appending tokens one at a time with tria_update_kv_cache gives, after every
    step, the bytes of a cache packed from scratch for that ctx_len: compared with
    the GPU packer at every step and with the oracle's packer at every block start
    and at the end."""
    print(f"[case] cache update {case}", flush=True)
    b, hq, hk, d, n, blk, ctx0, steps, hi, keep = case
    cfg = synth.Config("upd", b, hq, hk, d, n, blk, seed=43, decode=True)
    k, v, _ = synth.make_decode_inputs(cfg)
    hi, keep = np.array(hi, np.int32), np.array(keep, np.int32)
    dd = tria.make_dims(b, hq, hk, d, blk, n)
    kd, vd = dev(k), dev(v)
    cache = tria.pack_kv_cache(dd, hi, keep, ctx0, kd, vd)
    for ctx in range(ctx0 + 1, ctx0 + steps + 1):
        prev = cache
        cache = tria.update_kv_cache(dd, hi, keep, ctx, kd, vd, cache)
        assert (cache.data_ptr() == prev.data_ptr()) == ((ctx - 1) % blk != 0)
        ref = tria.pack_kv_cache(dd, hi, keep, ctx, kd, vd)
        assert cache.numel() == ref.numel()
        assert torch.equal(cache, ref), f"ctx {ctx}: updated cache differs from the packed one"
        if (ctx - 1) % blk == 0 or ctx == ctx0 + steps:
            blob = oracle.pack_cache(k, v, hi, keep, hq, blk, ctx)
            assert np.array_equal(cache.cpu().numpy(), blob), f"ctx {ctx}: differs from the oracle's bytes"
            tria.check_cache(dd, cache, ctx)


def test_pack_merges_query_head_policies(tria):
    b, hq, hk, d, n, blk, ctx = 1, 4, 2, 64, 600, 64, 600
    cfg = synth.Config("dec", b, hq, hk, d, n, blk, seed=5, decode=True)
    k, v, q = synth.make_decode_inputs(cfg)
    hi = np.array([0, 2, 1, 1], np.int32)
    keep = np.array([3, 2, 1, 6], np.int32)
    dd = tria.make_dims(b, hq, hk, d, blk, n)
    cache = tria.pack_kv_cache(dd, hi, keep, ctx, dev(k), dev(v))
    torch.cuda.synchronize()
    assert np.array_equal(cache.cpu().numpy(), oracle.pack_cache(k, v, hi, keep, hq, blk, ctx))


def test_decode_rejects_corrupt_cache(tria):
    case = (1, 4, 2, 64, 900, 64, 897, [1, 0], [5, 9])
    cfg, k, v, q, hi, keep, dd, cache, out = _dec_case(tria, case)
    bad = cache.clone()
    bad[0] = 0  # magic
    from block_sparse_mixed_head_amd import TriaError
    with pytest.raises(TriaError):
        tria.check_cache(dd, bad, 897)
    with pytest.raises(TriaError):
        tria.check_cache(dd, cache, 896)  # wrong context length
    o = tria.decode(dd, bad, 897, dev(q), 0.125)
    torch.cuda.synchronize()
    assert torch.isnan(o).all().item()
    bad = cache.clone()
    bad[64 + 8:64 + 12] = torch.tensor([255, 255, 0, 0], dtype=torch.uint8)  # n8 of pair 0
    o = tria.decode(dd, bad, 897, dev(q), 0.125)
    torch.cuda.synchronize()
    assert torch.isnan(o).all().item()


def test_decode_full_size_workload(tria):
    cfg = synth.CONFIGS["decode_b16"]
    print("[case] pack + decode full-size decode workload b16 ctx32768", flush=True)
    k, v, q = synth.make_decode_inputs(cfg)
    hi, keep = cfg.policy()
    dd = tria.make_dims(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.block, cfg.seq_len)
    kd, vd = dev(k), dev(v)
    cache = tria.pack_kv_cache(dd, hi, keep, cfg.seq_len, kd, vd)
    out = tria.decode(dd, cache, cfg.seq_len, dev(q), 1.0 / math.sqrt(cfg.head_dim))
    torch.cuda.synchronize()
    tria.check_cache(dd, cache, cfg.seq_len)
    # byte-exact cache on a sample of pairs (directory entries + their records)
    ref_blob = oracle.pack_cache(k, v, hi, keep, cfg.n_q_heads, cfg.block, cfg.seq_len)
    got = cache.cpu().numpy()
    assert got.size == ref_blob.size and np.array_equal(got, ref_blob)
    ref = oracle.decode(k, v, q, hi, keep, cfg.block, cfg.seq_len, 1.0 / math.sqrt(cfg.head_dim))
    assert_close(out.cpu().numpy(), ref, "decode workload b16 ctx32768")


@pytest.mark.gpu
def test_decode_reuses_one_workspace(tria):
    """Calls sharing one workspace: three decodes of different context lengths and
    policies, with a rejected cache in between, all match the oracle."""
    b, hq, hk, d, n, blk = 2, 8, 2, 128, 1400, 128
    cfg = synth.Config("dec", b, hq, hk, d, n, blk, seed=77, decode=True)
    k, v, q = synth.make_decode_inputs(cfg)
    dd = tria.make_dims(b, hq, hk, d, blk, n)
    kd, vd, qd = dev(k), dev(v), dev(q)
    ws = torch.empty(tria.decode_workspace_bytes(dd, n), dtype=torch.uint8, device="cuda")
    runs = [(1400, [1, 0], [6, 3]), (777, [0, 2], [2, 9]), (1400, [3, 3], [3, 3])]
    for i, (ctx, hi, keep) in enumerate(runs):
        print(f"[case] shared workspace run {i}: ctx {ctx}", flush=True)
        hi, keep = np.array(hi, np.int32), np.array(keep, np.int32)
        cache = tria.pack_kv_cache(dd, hi, keep, ctx, kd, vd)
        out = tria.decode(dd, cache, ctx, qd, 1.0 / math.sqrt(d), workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.decode(k, v, q, hi, keep, blk, ctx, 1.0 / math.sqrt(d))
        assert_close(out.cpu().numpy(), ref, f"decode with a shared workspace, run {i}")
        if i == 0:
            bad = cache.clone()
            bad[0] = 0
            o = tria.decode(dd, bad, ctx, qd, 0.125, workspace=ws)
            torch.cuda.synchronize()
            assert torch.isnan(o).all().item()


@pytest.mark.gpu
def test_measured_ceilings_are_plausible(tria):
    """The MFMA loops and the streaming read run and give rates inside what the part
    can do: at most its published peaks (int8 5.0 POPS, bf16 2.5 PFLOPS, HBM 8 TB/s),
    at least a fifth of them."""
    sink = torch.zeros(8192, dtype=torch.int32, device="cuda")
    src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")

    def rate(enqueue):
        work = enqueue()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        work = enqueue()
        e1.record()
        e1.synchronize()
        return work / (e0.elapsed_time(e1) * 1e-3)

    i8 = rate(lambda: tria.peak_mfma(0, 2000, sink))
    bf = rate(lambda: tria.peak_mfma(1, 2000, sink))
    rd = rate(lambda: tria.peak_read(src, sink))
    print(f"int8 {i8 / 1e12:.0f} TOPS, bf16 {bf / 1e12:.0f} TFLOPS, read {rd / 1e9:.0f} GB/s", flush=True)
    assert 1.0e15 <= i8 <= 5.0e15
    assert 0.5e15 <= bf <= 2.5e15
    assert 1.6e12 <= rd <= 8.0e12

