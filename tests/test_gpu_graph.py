"""The hot path under HIP graph capture: quantise, prefill, pack and decode captured
once and replayed several times, with eager work (and synchronisations) between
the replays; every replay equals the eager result bit for bit."""
import math

import numpy as np
import pytest
import torch

import synth
from test_gpu_parity import dev

pytestmark = pytest.mark.gpu


def test_graph_replays_equal_eager():
    import block_sparse_mixed_head_amd as tria
    cfg = synth.Config("graph", 1, 8, 2, 128, 1100, 128, seed=81, hi_range=(1, 3), keep_max=6)
    qh, kh, vh = synth.make_prefill_inputs(cfg)
    hi, keep = cfg.policy()
    q, k, v = dev(qh), dev(kh), dev(vh)
    d = tria.make_dims(1, 8, 2, 128, 128, 1100)
    sm = 1.0 / math.sqrt(128)
    sched = torch.from_numpy(tria.build_policy(d, hi, keep).view(np.uint8)).cuda()
    qz = tria.quantize_qk(d, q, k)
    out = torch.empty((1, 8, 1100, 128), dtype=torch.float32, device="cuda")
    cache = torch.empty(tria.kv_cache_bytes(d, hi, keep, 1100), dtype=torch.uint8, device="cuda")
    ws = torch.empty(tria.decode_workspace_bytes(d, 1100), dtype=torch.uint8, device="cuda")
    qdec = q[:, :, 1099].contiguous()
    dout = torch.empty((1, 8, 128), dtype=torch.float32, device="cuda")

    def work():
        tria.quantize_qk(d, q, k, out=qz)
        tria.prefill(d, sched, qz, v, sm, out=out)
        tria.pack_kv_cache(d, hi, keep, 1100, k, v, cache=cache)
        tria.decode(d, cache, 1100, qdec, sm, out=dout, workspace=ws)

    work()
    torch.cuda.synchronize()
    ref = (out.clone(), dout.clone(), cache.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for r in range(4):
        print(f"[case] graph replay {r}", flush=True)
        out.zero_()
        dout.zero_()
        cache.zero_()
        work()                 # eager work between the replays
        torch.cuda.synchronize()
        out.zero_()
        dout.zero_()
        cache.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(dout, ref[1]) and torch.equal(cache, ref[2]), r
