"""The decode entry point that allocates nothing (tria_decode_noalloc), called through
the C ABI, against tria_decode with a caller workspace: two calls in a row on one GPU,
the second with a smaller input (the library's scratch still holds the first call's
partials), each equal to tria_decode bit for bit (the same kernels over the same
split) and within tolerance of the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from test_gpu_parity import assert_close, dev

pytestmark = pytest.mark.gpu

CASES = [
    # (b, hq, hk, d, n, blk, ctx, hi, keep)  policies per KV head; the larger call first
    (8, 32, 8, 128, 4096, 128, 4000, [2, 5, 1, 0, 3, 9, 2, 4], [9, 20, 1, 0, 30, 31, 2, 8]),
    (2, 8, 2, 64, 900, 64, 700, [1, 0], [4, 9]),
]


def test_decode_noalloc_matches_decode():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_sparse_mixed_head_amd as tria
    for case in CASES:
        b, hq, hk, d, n, blk, ctx, hi, keep = case
        print(f"[case] decode without allocation {case[:7]}", flush=True)
        cfg = synth.Config("noalloc", b, hq, hk, d, n, blk, seed=91, decode=True)
        k, v, q = synth.make_decode_inputs(cfg)
        hi, keep = np.array(hi, np.int32), np.array(keep, np.int32)
        dd = tria.make_dims(b, hq, hk, d, blk, n)
        cache = tria.pack_kv_cache(dd, hi, keep, ctx, dev(k), dev(v))
        qd = dev(q)
        sm = 1.0 / math.sqrt(d)
        ref = tria.decode(dd, cache, ctx, qd, sm)
        out = torch.full_like(ref, float("nan"))
        tria.decode_noalloc(dd, cache, ctx, qd, sm, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), case[:7]
        assert_close(out.cpu().numpy(), oracle.decode(k, v, q, hi, keep, blk, ctx, sm), f"decode_noalloc {case[:7]}")
