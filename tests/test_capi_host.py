"""Host-side checks of the C-ABI library (no GPU needed).

* the library loads and exports every function include/tria.h declares;
* tria_build_policy (host) holds the oracle's unit records bit for bit on the five
  workloads and on random shapes, including ragged sequence lengths, in a dispatch
  order whose XCD placement and chunking are checked separately;
* tria_kv_cache_bytes matches the oracle's cache size;
* validation returns the documented status codes and enqueues nothing.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def tria():
    import block_sparse_mixed_head_amd as t
    return t


def test_library_exports_every_declared_symbol(tria):
    from block_sparse_mixed_head_amd import _lib
    header = open(os.path.join(ROOT, "include", "tria.h")).read()
    declared = set(re.findall(r"\b(tria_[a-z_0-9]+)\s*\(", header))
    assert declared, "no declarations parsed"
    for name in sorted(declared):
        assert hasattr(_lib.lib, name), name
    assert declared == set(_lib.EXPORTED)
    assert _lib.lib.tria_version() >> 16 == 1


def _by_unit(blob, n_units):
    """Unit records sorted by (b, h, qb): the schedule's content without its order."""
    u = blob[16:16 + 8 * n_units].reshape(-1, 8)
    return u[np.lexsort((u[:, 2], u[:, 1], u[:, 0]))]


def _same_schedule(mine, ref):
    """Same header and the same unit records (the oracle lists them longest first;
    the library in its dispatch order)."""
    n = int(ref[8])
    return (mine.dtype == np.int32 and mine.shape == ref.shape and np.array_equal(mine[:16], ref[:16])
            and np.array_equal(_by_unit(mine, n), _by_unit(ref, n)))


@pytest.mark.parametrize("cid", ["tiny", "llama3_8b_layer", "long_prefill", "batched_mixed"])
def test_schedule_bit_exact_on_workloads(tria, cid):
    c = synth.CONFIGS[cid]
    hi, keep = c.policy()
    d = tria.make_dims(c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim, c.block, c.seq_len)
    mine = tria.build_policy(d, hi, keep)
    ref = oracle.build_schedule(c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim, c.block, c.seq_len, hi, keep)
    assert _same_schedule(mine, ref)


def _check_dispatch_order(units, xcds=8, chunk=32):
    """The library's dispatch order: position p runs on XCD p mod 8 while all eight
    XCDs still have records; each XCD's records are chunks of at most `chunk`
    consecutive q-blocks of one (b, h), taken from the lane's last block down (a
    chunk starts at nb - 1 - chunk * k), the chunks in non-increasing order of
    their tiles.  The full rotation is found from the records themselves: in it,
    the record at p either starts a chunk or continues the one at p - 8.  Returns
    the tiles per XCD over the full rounds and the fraction of positions in them."""
    n = len(units)
    nb = {}
    for b, h, qb in units[:, :3]:
        nb[(b, h)] = max(nb.get((b, h), 0), qb + 1)

    def starts(u):
        return (nb[(u[0], u[1])] - 1 - u[2]) % chunk == 0

    rounds = 0
    while (rounds + 1) * xcds <= n:
        ok = True
        for x in range(xcds):
            p = rounds * xcds + x
            u = units[p]
            if starts(u):
                continue
            prev = units[p - xcds] if p >= xcds else None
            if prev is None or tuple(prev[:2]) != tuple(u[:2]) or prev[2] != u[2] + 1:
                ok = False
        if not ok:
            break
        rounds += 1
    full = rounds * xcds
    tiles = []
    for x in range(xcds):
        seq = units[x:full:xcds]
        tiles.append(int(seq[:, 7].sum()))
        works, i = [], 0
        while i < len(seq):
            j = i + 1
            while j < len(seq) and not starts(seq[j]):
                j += 1
            assert j - i <= chunk
            works.append(int(seq[i:j, 7].sum()))
            i = j
        # the last chunk may be cut by the end of the full rounds
        assert all(a >= b for a, b in zip(works[:-2], works[1:-1])), works
    return tiles, full / n


@pytest.mark.parametrize("cid", ["llama3_8b_layer", "long_prefill", "batched_mixed"])
def test_dispatch_order_on_workloads(tria, cid):
    c = synth.CONFIGS[cid]
    hi, keep = c.policy()
    d = tria.make_dims(c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim, c.block, c.seq_len)
    units = tria.build_policy(d, hi, keep)[16:].reshape(-1, 8)
    tiles, frac = _check_dispatch_order(units)
    assert frac == 1.0
    # balanced to within one chunk of the largest size (32 units of at most nb tiles)
    nb = (c.seq_len + c.block - 1) // c.block
    assert max(tiles) - min(tiles) <= 32 * nb, tiles
    assert max(tiles) / np.mean(tiles) < 1.01, tiles


def test_dispatch_order_varlen_and_random_policies(tria):
    """Shapes with whole 32-block chunks on every XCD: two batch rows of 16 heads, 64
    query blocks each, random policies; and a variable-length batch of the same size
    (sequence lengths that are not multiples of the chunk)."""
    rng = np.random.default_rng(5)
    for blk in (64, 128):
        hi = rng.integers(0, 20, size=16).astype(np.int32)
        keep = (hi + rng.integers(0, 50, size=16)).astype(np.int32)
        d = tria.make_dims(2, 16, 4, 128, blk, 64 * blk)
        units = tria.build_policy(d, hi, keep)[16:].reshape(-1, 8)
        tiles, frac = _check_dispatch_order(units)
        assert frac == 1.0 and max(tiles) - min(tiles) <= 32 * 64, tiles
        lens = np.array([50 * blk + 7, 30 * blk, 48 * blk - 3], np.int64)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        d = tria.make_dims(1, 16, 4, 128, blk, int(cu[-1]))
        blob = tria.build_policy_varlen(d, hi, keep, cu)
        n_units = int(blob[8])
        tiles, frac = _check_dispatch_order(blob[16:16 + 8 * n_units].reshape(-1, 8))
        assert frac > 0.75, frac


def test_schedule_bit_exact_random_shapes(tria):
    rng = np.random.default_rng(0)
    for _ in range(40):
        blk = int(rng.choice([64, 128]))
        hd = int(rng.choice([64, 128]))
        hk = int(rng.integers(1, 4))
        hq = hk * int(rng.integers(1, 5))
        b = int(rng.integers(1, 3))
        n = int(rng.integers(1, 20 * blk))
        nb = (n + blk - 1) // blk
        hi = rng.integers(0, nb + 2, size=hq).astype(np.int32)
        keep = (hi + rng.integers(0, nb + 2, size=hq)).astype(np.int32)
        d = tria.make_dims(b, hq, hk, hd, blk, n)
        mine = tria.build_policy(d, hi, keep)
        assert _same_schedule(mine, oracle.build_schedule(b, hq, hk, hd, blk, n, hi, keep))


def test_tiny_workload_tile_counts(tria):
    c = synth.CONFIGS["tiny"]
    hi, keep = c.policy()
    d = tria.make_dims(c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim, c.block, c.seq_len)
    units = tria.build_policy(d, hi, keep)[16:].reshape(-1, 8)
    per_head = {}
    for b, h, qb, lo8, lo4, hi4, sink, nt in units:
        e = per_head.setdefault(h, [0, 0])
        e[0] += (qb - lo8 + 1) + sink
        e[1] += hi4 - lo4 + 1
    # 26 int8 and 7 int4 tiles per head, 3 skipped, of the 36 causal tiles
    assert per_head == {0: [26, 7], 1: [26, 7]}


@pytest.mark.parametrize("cid", ["llama3_8b_layer", "decode_b16", "batched_mixed"])
def test_cache_bytes_match_oracle(tria, cid):
    c = synth.CONFIGS[cid]
    hi, keep = c.policy()
    d = tria.make_dims(c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim, c.block, c.seq_len)
    for ctx in (1, c.block, c.seq_len - 77, c.seq_len):
        assert tria.kv_cache_bytes(d, hi, keep, ctx) == oracle.cache_bytes(
            c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim, c.block, ctx, hi, keep)


def test_cache_bytes_dense_policy_pins_page_formula(tria):
    # every block stored at int8: codes are the page's formula with p = 1 byte
    b, hk, hd, blk, n = 2, 8, 128, 128, 4096
    d = tria.make_dims(b, hk, hk, hd, blk, n)
    top = np.full(hk, n // blk, np.int32)
    header = (64 + 64 * b * hk + 255) // 256 * 256
    assert tria.kv_cache_bytes(d, top, top, n) == header + oracle.kv_formula_bytes(1, hk, hd, n, b, 1) + 2 * hk * n * b * 4


def test_decode_workspace_is_positive(tria):
    d = tria.make_dims(16, 32, 8, 128, 128, 32768)
    assert tria.decode_workspace_bytes(d, 32768) > 0


def _status(fn, *args):
    return fn(*args)


def test_validation_errors(tria):
    from block_sparse_mixed_head_amd import _lib
    L = _lib.lib
    hi = np.array([1, 2], np.int32)
    keep = np.array([3, 2], np.int32)
    need = C.c_size_t(0)

    def bp(d, h=hi, k=keep, n=2):
        return L.tria_build_policy(C.byref(d), h.ctypes.data, k.ctypes.data, n, None, 0, C.byref(need))

    good = tria.make_dims(1, 2, 1, 64, 64, 512)
    assert bp(good) == _lib.TRIA_OK and need.value == 64 + 32 * 16
    assert bp(tria.make_dims(1, 3, 2, 64, 64, 512), n=3) == _lib.TRIA_ERR_INVALID_ARG  # Hq % Hkv
    assert bp(tria.make_dims(1, 2, 1, 96, 64, 512)) == _lib.TRIA_ERR_UNSUPPORTED       # head_dim
    assert bp(tria.make_dims(1, 2, 1, 64, 32, 512)) == _lib.TRIA_ERR_UNSUPPORTED       # block
    assert bp(tria.make_dims(1, 2, 1, 64, 64, 0)) == _lib.TRIA_ERR_INVALID_ARG         # seq_len
    assert bp(good, h=np.array([4, 2], np.int32)) == _lib.TRIA_ERR_INVALID_ARG         # hi > keep
    assert bp(good, h=np.array([-1, 2], np.int32)) == _lib.TRIA_ERR_INVALID_ARG        # hi < 0
    assert bp(good, n=1) == _lib.TRIA_ERR_INVALID_ARG                                  # head count
    assert b"keep" in L.tria_last_error() or b"n_policy" in L.tria_last_error()
    small = np.zeros(10, np.int32)
    assert L.tria_build_policy(C.byref(good), hi.ctypes.data, keep.ctypes.data, 2, small.ctypes.data, 40,
                               C.byref(need)) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    assert need.value == 64 + 32 * 16
    bad = tria.make_dims(1, 2, 1, 64, 64, 512)
    bad.reserved = 1
    assert bp(bad) == _lib.TRIA_ERR_INVALID_ARG
    # device calls: validation happens before any HIP call, so these run without a GPU
    z = C.c_void_p(0)
    one = C.c_void_p(16)
    assert L.tria_quantize_qk(C.byref(good), z, one, *([one] * 8), None) == _lib.TRIA_ERR_INVALID_ARG
    assert L.tria_prefill(C.byref(good), one, 10, *([one] * 8), one, C.c_float(0.125), one, None,
                          None) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    assert L.tria_prefill(C.byref(good), one, 64 + 32 * 16, *([one] * 8), one, C.c_float(-1.0), one, None,
                          None) == _lib.TRIA_ERR_INVALID_ARG
    assert b"sm_scale" in L.tria_last_error()
    # a schedule larger than the dims imply is not the blob built for them
    assert L.tria_prefill(C.byref(good), one, 64 + 32 * 16 + 4, *([one] * 8), one, C.c_float(0.125), one, None,
                          None) == _lib.TRIA_ERR_INVALID_ARG
    assert b"schedule" in L.tria_last_error()
    cu = np.array([0, 200, 512], np.int64)
    vneed = 64 + 32 * 2 * (4 + 5) + 8 * 2   # 2 heads x (4 + 5) query blocks, 2 {start, length} records
    for nbytes, want in ((vneed - 1, _lib.TRIA_ERR_BUFFER_TOO_SMALL), (vneed + 8, _lib.TRIA_ERR_INVALID_ARG)):
        assert L.tria_prefill_varlen(C.byref(good), 2, cu.ctypes.data, one, nbytes, *([one] * 8), one,
                                     C.c_float(0.125), one, None, None) == want
    sz = C.c_size_t(0)
    assert L.tria_kv_cache_bytes(C.byref(good), hi.ctypes.data, keep.ctypes.data, 2, 0, C.byref(sz)) == _lib.TRIA_ERR_INVALID_ARG
    assert L.tria_kv_cache_bytes(C.byref(good), hi.ctypes.data, keep.ctypes.data, 2, 513, C.byref(sz)) == _lib.TRIA_ERR_INVALID_ARG
    assert L.tria_kv_cache_bytes(C.byref(good), hi.ctypes.data, keep.ctypes.data, 3, 100, C.byref(sz)) == _lib.TRIA_ERR_INVALID_ARG
    assert L.tria_pack_kv_cache(C.byref(good), hi.ctypes.data, keep.ctypes.data, 2, 512, one, one, one, 100,
                                None) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    assert L.tria_decode(C.byref(good), one, 1 << 20, 512, one, C.c_float(0.125), one, one, 16,
                         None) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    mqa = tria.make_dims(1, 64, 1, 64, 64, 512)
    assert L.tria_decode(C.byref(mqa), one, 1 << 20, 512, one, C.c_float(0.125), one, one, 1 << 30,
                         None) == _lib.TRIA_ERR_UNSUPPORTED
    # the fused-Q prefill and the K-only quantiser validate like their two-step forms
    need_good = 64 + 32 * 2 * 8   # 2 heads x 8 query blocks of the (1, 2, 1, 64, 64, 512) dims
    assert L.tria_prefill_bf16q(C.byref(good), one, need_good, None, *([one] * 4), one, C.c_float(0.125), one,
                                None, None) == _lib.TRIA_ERR_INVALID_ARG          # no Q
    assert L.tria_prefill_bf16q(C.byref(good), one, need_good - 1, one, *([one] * 4), one, C.c_float(0.125), one,
                                None, None) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    assert L.tria_prefill_bf16q(C.byref(good), one, need_good, one, *([one] * 4), one, C.c_float(0.0), one,
                                None, None) == _lib.TRIA_ERR_INVALID_ARG          # sm_scale 0
    assert L.tria_prefill_bf16q(C.byref(good), one, need_good, one, one, one, one, None, one, C.c_float(0.125), one,
                                None, None) == _lib.TRIA_ERR_INVALID_ARG          # no K scales
    assert L.tria_quantize_k(C.byref(good), one, one, one, one, None, None) == _lib.TRIA_ERR_INVALID_ARG
    assert L.tria_quantize_k(C.byref(tria.make_dims(1, 2, 1, 96, 64, 512)), one, one, one, one, one,
                             None) == _lib.TRIA_ERR_UNSUPPORTED
    # prefill byte offsets within a head's rows are 32-bit: (seq_len + 4 block) * 2 d < 2^31
    for d, blk in ((128, 128), (64, 64)):
        n = (1 << 31) // (2 * d) - 4 * blk + 1
        big = tria.make_dims(1, 1, 1, d, blk, n)
        need = 64 + 32 * ((n + blk - 1) // blk)
        assert L.tria_prefill(C.byref(big), one, need, *([one] * 8), one, C.c_float(0.125), one, None,
                              None) == _lib.TRIA_ERR_UNSUPPORTED
        assert b"2^31" in L.tria_last_error()


def test_decode_noalloc_validates(tria):
    """The decode entry point that allocates nothing rejects, before any HIP call, a
    call whose workspace exceeds its 64 MiB scratch, and the decode's bad arguments."""
    from block_sparse_mixed_head_amd import _lib
    L = _lib.lib
    one = C.c_void_p(16)
    big = tria.make_dims(2048, 32, 1, 128, 128, 4096)    # 32 query heads per KV head, 2048 pairs
    assert tria.decode_workspace_bytes(big, 4096) > 64 << 20
    assert L.tria_decode_noalloc(C.byref(big), one, 1 << 30, 4096, one, C.c_float(0.125), one,
                                 None) == _lib.TRIA_ERR_UNSUPPORTED
    assert b"64" in L.tria_last_error() or b"scratch" in L.tria_last_error()
    ok = tria.make_dims(1922, 32, 1, 128, 128, 4096)     # the largest that fits
    assert tria.decode_workspace_bytes(ok, 4096) <= 64 << 20
    good = tria.make_dims(1, 2, 1, 64, 64, 512)
    assert L.tria_decode_noalloc(C.byref(good), one, 10, 512, one, C.c_float(0.125), one,
                                 None) == _lib.TRIA_ERR_BUFFER_TOO_SMALL     # cache below its directory
    assert L.tria_decode_noalloc(C.byref(good), one, 1 << 20, 0, one, C.c_float(0.125), one,
                                 None) == _lib.TRIA_ERR_INVALID_ARG          # ctx_len
    assert L.tria_decode_noalloc(C.byref(good), one, 1 << 20, 512, one, C.c_float(0.125), None,
                                 None) == _lib.TRIA_ERR_INVALID_ARG          # out


def test_peak_helpers_validate_arguments(tria):
    """The measured-ceiling helpers check their arguments before any HIP call."""
    from block_sparse_mixed_head_amd import _lib
    L = _lib.lib
    work = C.c_double(0.0)
    sink = C.c_void_p(16)
    assert L.tria_peak_mfma(2, 10, sink, C.byref(work), None) == _lib.TRIA_ERR_INVALID_ARG   # kind
    assert L.tria_peak_mfma(0, 0, sink, C.byref(work), None) == _lib.TRIA_ERR_INVALID_ARG    # iters
    assert L.tria_peak_mfma(1, 10, None, C.byref(work), None) == _lib.TRIA_ERR_INVALID_ARG   # sink
    src = C.c_void_p(4096)
    assert L.tria_peak_read(src, _lib.PEAK_READ_ALIGN + 1, sink, C.byref(work), None) == _lib.TRIA_ERR_INVALID_ARG
    assert L.tria_peak_read(src, 0, sink, C.byref(work), None) == _lib.TRIA_ERR_INVALID_ARG
    assert L.tria_peak_read(None, _lib.PEAK_READ_ALIGN, sink, C.byref(work), None) == _lib.TRIA_ERR_INVALID_ARG


def test_update_validates_buffers(tria):
    """tria_update_kv_cache rejects, before any HIP call, an in-place call at a block
    start, partially overlapping buffers, too-small buffers and ctx_len < 2."""
    from block_sparse_mixed_head_amd import _lib
    L = _lib.lib
    d = tria.make_dims(1, 2, 1, 64, 64, 512)
    hi, keep = np.array([1], np.int32), np.array([3], np.int32)
    old = tria.kv_cache_bytes(d, hi, keep, 128)     # ctx 128: blocks 0, 1
    new = tria.kv_cache_bytes(d, hi, keep, 129)     # ctx 129: token 128 starts block 2
    kv = C.c_void_p(1 << 20)

    def upd(ctx, cin, nin, cout, nout):
        return L.tria_update_kv_cache(C.byref(d), hi.ctypes.data, keep.ctypes.data, 1, ctx, kv, kv,
                                      C.c_void_p(cin), nin, C.c_void_p(cout), nout, None)

    base = 1 << 30
    assert upd(129, base, old, base, new) == _lib.TRIA_ERR_INVALID_ARG                 # in place at a block start
    assert upd(129, base, old, base + 64, new) == _lib.TRIA_ERR_INVALID_ARG            # partial overlap
    assert upd(129, base, old - 1, base + (1 << 24), new) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    assert upd(129, base, old, base + (1 << 24), new - 1) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    assert upd(1, base, old, base + (1 << 24), new) == _lib.TRIA_ERR_INVALID_ARG       # ctx_len < 2
    assert upd(513, base, old, base + (1 << 24), new) == _lib.TRIA_ERR_INVALID_ARG     # past seq_len


def test_policy_cost_matches_oracle_and_schedule(tria):
    """The library's cost equals the oracle's tile-by-tile count, and with unit pair
    costs it is block^2 times the head's tiles in the prefill schedule."""
    import oracle
    rng = np.random.default_rng(3)
    for _ in range(30):
        blk = int(rng.choice([64, 128]))
        n = int(rng.integers(1, 3000))
        hi = int(rng.integers(0, 12))
        keep = int(rng.integers(hi, 30))
        c8, c4 = float(rng.uniform(0.2, 2.0)), float(rng.uniform(0.2, 2.0))
        d = tria.make_dims(1, 1, 1, 64, blk, n)
        assert tria.policy_cost(d, hi, keep, c8, c4) == oracle.policy_cost(n, blk, hi, keep, c8, c4)
        sched = tria.build_policy(d, np.array([hi], np.int32), np.array([keep], np.int32))
        units = sched[16:].reshape(-1, 8)
        assert tria.policy_cost(d, hi, keep) == float(units[:, 7].sum()) * blk * blk


def test_allocator_matches_oracle(tria):
    """Greedy allocation: the library's heap-driven run equals the oracle's scan, bit
    for bit (choices, summed cost and summed error), on random instances including
    equal pair costs (raising precision is then free) and flat tables."""
    import oracle
    rng = np.random.default_rng(5)
    for trial in range(60):
        blk = int(rng.choice([64, 128]))
        n = int(rng.integers(64, 5000))
        H, K = int(rng.integers(1, 9)), int(rng.integers(0, 12))
        e = rng.uniform(0.0, 1.0, size=(H, K + 1, K + 1))
        if trial % 3 == 0:
            e = np.sort(np.sort(e, axis=2)[:, :, ::-1], axis=1)[:, ::-1, :]
        if trial % 5 == 0:
            e = np.round(e, 1)  # ties
        e = np.ascontiguousarray(e)
        c8, c4 = (1.0, 1.0) if trial % 4 == 0 else (float(rng.uniform(0.5, 2)), float(rng.uniform(0.2, 1)))
        d = tria.make_dims(1, H, 1, 64, blk, n)
        base = H * oracle.policy_cost(n, blk, 0, 0, c8, c4)
        budget = base * float(rng.uniform(1.0, 6.0))
        got = tria.allocate_policy(d, e, budget, c8, c4)
        want = oracle.allocate_policy(n, blk, e, budget, c8, c4)
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1]), trial
        assert got[2] == want[2] and got[3] == want[3], trial


def test_allocator_follows_hand_worked_traces(tria):
    """The library's allocator on the hand-worked instances the oracle is pinned to
    (tests/test_oracle_pins.py): the same choices, cost and error at every budget."""
    from test_oracle_pins import ALLOC_CASES, _B, _U
    for name, n, err, c8, trace in ALLOC_CASES:
        d = tria.make_dims(1, err.shape[0], 1, 64, _B, n)
        for budget, hi, keep, cost, e64 in trace:
            b = 1e30 if budget >= 1e9 else budget * _U
            got_hi, got_keep, tc, te = tria.allocate_policy(d, err, b, c8, 1.0)
            assert got_hi.tolist() == hi and got_keep.tolist() == keep, (name, budget, got_hi, got_keep)
            assert tc == cost * _U and te * 64 == e64, (name, budget)


def test_allocator_validates(tria):
    from block_sparse_mixed_head_amd import _lib
    d = tria.make_dims(1, 2, 1, 64, 64, 512)
    e = np.ones((2, 3, 3))
    with pytest.raises(_lib.TriaError):
        tria.allocate_policy(d, e, 0.0)                     # below the protected-only cost
    with pytest.raises(_lib.TriaError):
        tria.allocate_policy(d, e, 1e12, cost_int8=0.0)     # pair cost must be > 0
    bad = e.copy()
    bad[1, 0, 2] = np.nan
    with pytest.raises(_lib.TriaError):
        tria.allocate_policy(d, bad, 1e12)
    with pytest.raises(_lib.TriaError):
        tria.policy_cost(d, 3, 2)                           # hi > keep


def test_varlen_schedule_matches_oracle(tria):
    """The variable-length schedule = each sequence's own schedule (the oracle's, for
    that length alone) with its batch index replaced by the sequence index, all
    units together (in the library's dispatch order), then the {start, length}
    table."""
    import oracle
    rng = np.random.default_rng(9)
    for _ in range(20):
        blk = int(rng.choice([64, 128]))
        hq = int(rng.integers(1, 6))
        lens = rng.integers(1, 700, size=int(rng.integers(1, 7)))
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        T = int(cu[-1])
        hi = rng.integers(0, 6, size=hq).astype(np.int32)
        keep = (hi + rng.integers(0, 8, size=hq)).astype(np.int32)
        d = tria.make_dims(1, hq, 1, 64, blk, T)
        blob = tria.build_policy_varlen(d, hi, keep, cu)
        parts = []
        for s_, L in enumerate(lens):
            u = oracle.build_schedule(1, hq, 1, 64, blk, int(L), hi, keep)[16:].reshape(-1, 8).copy()
            u[:, 0] = s_
            parts.append(u)
        want = np.concatenate(parts)
        want = want[np.lexsort((want[:, 2], want[:, 1], want[:, 0]))]
        n_units = len(want)
        assert blob[1] == 2 and blob[2] == len(lens) and blob[8] == n_units
        assert np.array_equal(_by_unit(blob, n_units), want)
        seqs = blob[16 + 8 * n_units:].reshape(-1, 2)
        assert np.array_equal(seqs[:, 0], cu[:-1]) and np.array_equal(seqs[:, 1], lens)


def test_varlen_validation(tria):
    from block_sparse_mixed_head_amd import _lib
    hi, keep = np.array([1], np.int32), np.array([2], np.int32)
    d = tria.make_dims(1, 1, 1, 64, 64, 100)
    for cu in ([0, 50, 99], [1, 50, 100], [0, 50, 50, 100]):
        with pytest.raises(_lib.TriaError):
            tria.build_policy_varlen(d, hi, keep, cu)
    with pytest.raises(_lib.TriaError):
        tria.build_policy_varlen(tria.make_dims(2, 1, 1, 64, 64, 100), hi, keep, [0, 100])



def test_skip_and_paged_calls_validate(tria):
    """The skipping-decode and paged-cache entry points reject, before any HIP call,
    NULL buffers, short buffers, bad scales and unsupported shapes (fake device
    addresses: nothing may be enqueued)."""
    from block_sparse_mixed_head_amd import _lib
    L = _lib.lib
    d = tria.make_dims(2, 8, 2, 128, 128, 4096)
    ctx = 1000
    dev = C.c_void_p(1 << 30)
    sz = C.c_size_t(0)
    assert L.tria_block_summaries_bytes(C.byref(d), ctx, C.byref(sz)) == _lib.TRIA_OK
    sums = sz.value
    assert sums == 64 + 4 * 8 * (2 * 128 + 16)
    assert L.tria_decode_skip_workspace_bytes(C.byref(d), ctx, C.byref(sz)) == _lib.TRIA_OK
    ws = sz.value
    assert ws > tria.decode_workspace_bytes(d, ctx)
    cache = 1 << 20

    def skip(cache_b=cache, sums_b=sums, q=dev, th=dev, sm=0.1, out=dev, w=dev, ws_b=ws, dims=d):
        return L.tria_decode_skip(C.byref(dims), dev, cache_b, ctx, dev, sums_b, q, th, sm, out, w, ws_b, None)

    assert skip(sums_b=sums - 1) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    assert skip(ws_b=ws - 1) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    assert skip(cache_b=64) == _lib.TRIA_ERR_BUFFER_TOO_SMALL           # smaller than the directory
    assert skip(th=None) == _lib.TRIA_ERR_INVALID_ARG
    assert skip(q=None) == _lib.TRIA_ERR_INVALID_ARG
    assert skip(sm=0.0) == _lib.TRIA_ERR_INVALID_ARG
    assert skip(sm=float("nan")) == _lib.TRIA_ERR_INVALID_ARG
    assert skip(dims=tria.make_dims(1, 66, 2, 128, 128, 4096)) == _lib.TRIA_ERR_UNSUPPORTED   # G = 33
    assert L.tria_build_block_summaries(C.byref(d), dev, cache, ctx, dev, sums - 1, None) == \
        _lib.TRIA_ERR_BUFFER_TOO_SMALL
    assert L.tria_skip_masks(C.byref(d), dev, cache, ctx, dev, sums, dev, dev, C.c_float(0.1), dev, 4 * 4 * 8 - 1,
                             None) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    # paged
    assert L.tria_paged_table_bytes(C.byref(d), ctx, C.byref(sz)) == _lib.TRIA_OK
    tb = sz.value
    assert tb == 64 + 64 * 4 + 4 * 4 * 8
    assert L.tria_paged_page_bytes(C.byref(d), C.byref(sz)) == _lib.TRIA_OK and sz.value == 2 * 128 * 128 + 8 * 128
    page = sz.value
    hi, keep = np.array([1, 2], np.int32), np.array([3, 5], np.int32)

    def ppack(table_b=tb, pool_b=page * 64, ctx_=ctx, table=dev):
        return L.tria_pack_kv_cache_paged(C.byref(d), hi.ctypes.data, keep.ctypes.data, 2, ctx_, dev, dev, table,
                                          table_b, None, 0, dev, pool_b, None)

    assert ppack(table_b=tb - 1) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    assert ppack(pool_b=page - 1) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    assert ppack(ctx_=4097) == _lib.TRIA_ERR_INVALID_ARG
    assert ppack(table=None) == _lib.TRIA_ERR_INVALID_ARG

    def pdec(table_b=tb, w_b=ws, pool=dev):
        return L.tria_decode_paged(C.byref(d), dev, table_b, pool, page * 64, ctx, dev, C.c_float(0.1), dev, dev,
                                   w_b, None)

    assert pdec(table_b=tb - 1) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    assert pdec(w_b=ws - 1) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    assert pdec(pool=None) == _lib.TRIA_ERR_INVALID_ARG


def test_varlen_and_paged_skip_calls_validate(tria):
    """The variable-length and paged variants reject bad buffers before any HIP call."""
    from block_sparse_mixed_head_amd import _lib
    L = _lib.lib
    d = tria.make_dims(2, 8, 2, 128, 128, 4096)
    dev = C.c_void_p(1 << 30)
    sz = C.c_size_t(0)
    assert L.tria_block_summaries_bytes(C.byref(d), 4096, C.byref(sz)) == _lib.TRIA_OK
    sums = sz.value
    assert L.tria_decode_skip_workspace_bytes(C.byref(d), 4096, C.byref(sz)) == _lib.TRIA_OK
    ws = sz.value
    cache = 1 << 20
    assert L.tria_build_block_summaries_varlen(C.byref(d), dev, cache, dev, sums - 1, None) == \
        _lib.TRIA_ERR_BUFFER_TOO_SMALL
    assert L.tria_build_block_summaries_varlen(C.byref(d), None, cache, dev, sums, None) == _lib.TRIA_ERR_INVALID_ARG

    def vskip(sums_b=sums, ws_b=ws, th=dev):
        return L.tria_decode_skip_varlen(C.byref(d), dev, cache, dev, sums_b, dev, th, C.c_float(0.1), dev, dev, ws_b,
                                         None)

    assert vskip(sums_b=sums - 1) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    assert vskip(ws_b=ws - 1) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    assert vskip(th=None) == _lib.TRIA_ERR_INVALID_ARG
    ctx = 1000
    assert L.tria_paged_table_bytes(C.byref(d), ctx, C.byref(sz)) == _lib.TRIA_OK
    tb = sz.value
    assert L.tria_block_summaries_bytes(C.byref(d), ctx, C.byref(sz)) == _lib.TRIA_OK
    psums = sz.value
    assert L.tria_build_block_summaries_paged(C.byref(d), dev, tb - 1, dev, 1 << 24, ctx, dev, psums, None) == \
        _lib.TRIA_ERR_BUFFER_TOO_SMALL
    assert L.tria_build_block_summaries_paged(C.byref(d), dev, tb, None, 1 << 24, ctx, dev, psums, None) == \
        _lib.TRIA_ERR_INVALID_ARG
    assert L.tria_decode_skip_paged(C.byref(d), dev, tb, dev, 1 << 24, ctx, dev, psums - 1, dev, dev, C.c_float(0.1),
                                    dev, dev, ws, None) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    hi, keep = np.array([1, 2], np.int32), np.array([3, 5], np.int32)
    lens = np.array([100, 5000], np.int64)      # past seq_len
    assert L.tria_pack_kv_cache_paged_varlen(C.byref(d), hi.ctypes.data, keep.ctypes.data, 2, lens.ctypes.data, dev,
                                             dev, dev, tb, None, 0, dev, 1 << 24, None) == _lib.TRIA_ERR_INVALID_ARG
    lens = np.array([100, 300], np.int64)
    assert L.tria_pack_kv_cache_paged_varlen(C.byref(d), hi.ctypes.data, keep.ctypes.data, 2, lens.ctypes.data, dev,
                                             dev, dev, 64, None, 0, dev, 1 << 24, None) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    assert L.tria_decode_paged_varlen(C.byref(d), dev, tb, dev, 1 << 24, dev, C.c_float(0.1), dev, dev, ws - 1,
                                      None) == _lib.TRIA_ERR_BUFFER_TOO_SMALL


def test_paged_varlen_skip_calls_validate(tria):
    """The variable-length paged skipping calls reject an index or workspace below their
    sizes for dims->seq_len, a table smaller than its directory (the rest of the table
    is checked on the device) and missing buffers before any HIP call."""
    from block_sparse_mixed_head_amd import _lib
    L = _lib.lib
    d = tria.make_dims(2, 8, 2, 128, 128, 4096)
    dev = C.c_void_p(1 << 30)
    sz = C.c_size_t(0)
    assert L.tria_paged_table_bytes(C.byref(d), 4096, C.byref(sz)) == _lib.TRIA_OK
    tb = sz.value
    assert L.tria_block_summaries_bytes(C.byref(d), 4096, C.byref(sz)) == _lib.TRIA_OK
    sums = sz.value
    assert L.tria_decode_skip_workspace_bytes(C.byref(d), 4096, C.byref(sz)) == _lib.TRIA_OK
    ws = sz.value
    pool = 1 << 24

    def build(table_b=tb, pool_p=dev, sums_p=dev, sums_b=sums):
        return L.tria_build_block_summaries_paged_varlen(C.byref(d), dev, table_b, pool_p, pool, sums_p, sums_b, None)

    assert build(sums_b=sums - 1) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    dir_end = 64 + 64 * 2 * 2
    assert tb > dir_end
    assert build(table_b=dir_end - 1) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    assert build(pool_p=None) == _lib.TRIA_ERR_INVALID_ARG
    assert build(sums_p=None) == _lib.TRIA_ERR_INVALID_ARG

    def skip(table_b=tb, sums_b=sums, ws_b=ws, th=dev, q=dev, scale=0.1):
        return L.tria_decode_skip_paged_varlen(C.byref(d), dev, table_b, dev, pool, dev, sums_b, q, th,
                                               C.c_float(scale), dev, dev, ws_b, None)

    assert skip(sums_b=sums - 1) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    assert skip(ws_b=ws - 1) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    assert skip(table_b=dir_end - 1) == _lib.TRIA_ERR_BUFFER_TOO_SMALL
    assert skip(th=None) == _lib.TRIA_ERR_INVALID_ARG
    assert skip(q=None) == _lib.TRIA_ERR_INVALID_ARG
    assert skip(scale=0.0) == _lib.TRIA_ERR_INVALID_ARG


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: asked for more, it prints one JSON line saying so and
    exits with status 2 before touching a device."""
    import json
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]
