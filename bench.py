"""Benchmark of the block-sparse mixed-precision attention path on one MI355X.

A step is one pass of the whole path over one batch of the long-prefill workload
(the largest of the path's workloads: b=1, 32 query / 8 KV heads, d=128,
n=65536, block 128, seeded policies hi ~ U[2,16], keep ~ U[hi,128], K with four
x8 outlier channels):
  policy expansion (host) + schedule upload, K quantisation, fused prefill (which
  quantises each query block itself: tria_prefill_bf16q), compressed-cache packing
  for the last position, one-token decode.
`value` is whole-step prompt tokens per second with inputs already in HBM.

The JSON line also carries
  * roofline: the prefill kernel (the dominant one) on the step's workload against
    the MFMA roofline, from its average launch time measured with HIP events on
    its stream (launches back to back, as the step loop runs them);
  * prefill_workloads: the same prefill measurement on the Llama-3-8B-shaped layer
    (n=8192) and the batched mixed-policy workload (b=4, 28/4 heads, n=16384);
  * decode: the decode kernels on the decode workload (b=16, ctx 32768) against
    8 TB/s, with the last-level cache flushed between launches;
  * cpu_baseline: the CPU oracle timed on a bounded sample of the step's workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       [--workload long_prefill|llama3_8b_layer|batched_mixed]
       [--only prefill|decode|skip|paged|copy|step]  (--only is for profiler runs)
"""
import argparse
import ctypes as C
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 MFMA, published
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E, published

# HBM traffic of the prefill kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE passes,
# per workload, kept with the source hash of the kernel it was measured on
PREFILL_TRAFFIC = {
    "long_prefill": os.path.join(ROOT, "profiles", "prefill_kernel.long_prefill_n65536.hbm_traffic.txt"),
    "llama3_8b_layer": os.path.join(ROOT, "profiles", "prefill_kernel.llama3_8b_n8192.hbm_traffic.txt"),
    "batched_mixed": os.path.join(ROOT, "profiles", "prefill_kernel.batched_mixed_b4_n16384.hbm_traffic.txt"),
}
# the kernel and the host code that orders its work units (the order sets the L2 reuse)
PREFILL_SOURCES = [os.path.join(ROOT, "block_sparse_mixed_head_amd", "csrc", f)
                   for f in ("prefill.hip", "device_common.h", "kernels.h", "capi.cpp")]


def source_hash(paths) -> str:
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """Bytes per prefill launch from the committed counter summary of the workload
    (FETCH_SIZE x fetch factor + WRITE_SIZE x write factor, factors from a plain
    1 GiB copy), or None when the summary is missing or the kernel source changed
    since."""
    try:
        kv = {}
        with open(PREFILL_TRAFFIC[workload]) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("source_sha256") != source_hash(PREFILL_SOURCES):
            return None
        return (float(kv["fetch_kib_per_dispatch"]) * 1024 * float(kv["copy_fetch_factor"]) +
                float(kv["write_kib_per_dispatch"]) * 1024 * float(kv["copy_write_factor"]))
    except (OSError, KeyError, ValueError):
        return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", choices=["prefill", "decode", "skip", "paged", "copy", "step"], default=None)
    p.add_argument("--workload", choices=["long_prefill", "llama3_8b_layer", "batched_mixed"],
                   default="long_prefill", help="the step's prefill workload")
    p.add_argument("--reps", type=int, default=20)
    return p.parse_args()


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def kept_pairs(units: np.ndarray, block: int, n: int) -> int:
    """Exact kept causal (query, key) pairs of a schedule: full off-diagonal tiles
    plus the causal part of the diagonal tile, per query row."""
    qb = units[:, 2].astype(np.int64)
    nt = units[:, 7].astype(np.int64)
    rows = np.minimum(n - qb * block, block)
    return int(np.sum(rows * (nt - 1) * block + rows * (rows + 1) // 2))


def decode_bytes(cache_bytes_total: int, batch: int, hq: int, d: int, header: int) -> int:
    """Algorithmic decode bytes: every stored record once, q in (bf16), out (fp32)."""
    return (cache_bytes_total - header) + batch * hq * d * 2 + batch * hq * d * 4


def skip_at_batch(b, tria, c4, h4, kp4, reps, flush_caches, event_avg, log):
    """Plain vs skipping decode on the decode workload's shapes at batch b: keys
    N(0,1) times one magnitude per (b, KV head, block) ~ U[0.1, 1], values and
    queries N(0,1), thresholds 0.6-0.9 x ||q|| (torch generator, seed b)."""
    import torch
    hq, hk, d, n, blk = c4.n_q_heads, c4.n_kv_heads, c4.head_dim, c4.seq_len, c4.block
    gen = torch.Generator(device="cuda")
    gen.manual_seed(b)
    k = torch.empty((b, hk, n, d), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    nb = n // blk
    for i in range(b):   # one batch element at a time (fp32 temporaries)
        mag = 0.1 + 0.9 * torch.rand((hk, nb, 1, 1), generator=gen, device="cuda")
        kf = torch.randn((hk, nb, blk, d), generator=gen, device="cuda") * mag
        k[i] = kf.reshape(hk, n, d).to(torch.bfloat16)
        v[i] = torch.randn((hk, n, d), generator=gen, device="cuda").to(torch.bfloat16)
    q = torch.randn((b, hq, d), generator=gen, device="cuda").to(torch.bfloat16)
    gamma = 0.6 + 0.3 * torch.rand((b, hq), generator=gen, device="cuda")
    th = (gamma * q.float().norm(dim=-1)).contiguous()
    dims = tria.make_dims(b, hq, hk, d, blk, n)
    sm = 1.0 / math.sqrt(d)
    cache = tria.pack_kv_cache(dims, h4, kp4, n, k, v)
    del k, v
    sums = tria.build_block_summaries(dims, cache, n)
    out = torch.empty((b, hq, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(tria.decode_workspace_bytes(dims, n), dtype=torch.uint8, device="cuda")
    wss = torch.empty(tria.decode_skip_workspace_bytes(dims, n), dtype=torch.uint8, device="cuda")
    run_p = lambda: tria.decode(dims, cache, n, q, sm, out=out, workspace=ws)
    run_s = lambda: tria.decode_skip(dims, cache, n, sums, q, th, sm, out=out, workspace=wss)
    for _ in range(3):
        run_p()
        run_s()
    tp = event_avg(run_p, reps, before=flush_caches)[0]
    ts = event_avg(run_s, reps, before=flush_caches)[0]
    masks = tria.skip_masks(dims, cache, n, sums, q, th, sm).cpu().numpy().view(np.uint32)
    hdr = (64 + 64 * b * hk + 255) // 256 * 256
    dirs = cache[:hdr].cpu().numpy()
    rec8, rec4 = 2 * blk * d + 8 * blk, blk * d + 8 * blk
    kept = 0
    for pi in range(b * hk):
        n8, n4 = (int(x) for x in dirs[64 + 64 * pi + 8:64 + 64 * pi + 16].view(np.int32))
        m = masks[pi, :n8 + n4]
        kept += int((m[:n8] != 0).sum()) * rec8 + int((m[n8:] != 0).sum()) * rec4
    stored = cache.numel() - hdr
    res = {"workload": f"decode b{b} h{hq}/{hk} d{d} ctx{n} B{blk}", "cache_bytes": cache.numel(),
           "plain_us": tp * 1e6, "skip_us": ts * 1e6, "speedup": tp / ts, "bytes_read_fraction": kept / stored,
           "plain_GB_per_s": stored / tp / 1e9, "skip_GB_per_s_kept": kept / ts / 1e9}
    log(f"[bench] batch {b}: plain decode {tp * 1e6:.1f} us, skipping {ts * 1e6:.1f} us "
        f"({kept / stored:.3f} of the records read, x{tp / ts:.2f})")
    del cache, sums, ws, wss
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the path has no "
                                   "multi-GPU mode (each GPU would take whole (batch, KV head) groups; nothing here runs on more than one)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import block_sparse_mixed_head_amd as tria
    import synth

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    # ------------------------------------------------------------ step workload
    cfg = synth.CONFIGS[args.workload]
    b, hq, hk, d, n, blk = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.seq_len, cfg.block
    sm = 1.0 / math.sqrt(d)
    qh = kh = vh = None
    if args.only in (None, "step", "prefill"):
        log(f"[bench] generating {cfg.name}")
        qh, kh, vh = synth.make_prefill_inputs(cfg)
        hi, keep = cfg.policy()
        q, k, v = dev(qh), dev(kh), dev(vh)
        dims = tria.make_dims(b, hq, hk, d, blk, n)
        sched_np = tria.build_policy(dims, hi, keep)
        units = sched_np[16:].reshape(-1, 8)
        W = kept_pairs(units, blk, n)
        sched_bytes = sched_np.nbytes
        pinned = [torch.empty(sched_bytes, dtype=torch.uint8).pin_memory() for _ in range(2)]
        pinned_ev = [torch.cuda.Event() for _ in range(2)]
        sched_dev = torch.empty(sched_bytes, dtype=torch.uint8, device="cuda")
        kz = tria.quantize_k(dims, k)
        out = torch.empty((b, hq, n, d), dtype=torch.float32, device="cuda")
        ctx = n
        cache_n = tria.kv_cache_bytes(dims, hi, keep, ctx)
        cache = torch.empty(cache_n, dtype=torch.uint8, device="cuda")
        ws = torch.empty(tria.decode_workspace_bytes(dims, ctx), dtype=torch.uint8, device="cuda")
        qdec = q[:, :, ctx - 1].contiguous()
        dout = torch.empty((b, hq, d), dtype=torch.float32, device="cuda")
        hi_c = np.ascontiguousarray(hi, np.int32)
        keep_c = np.ascontiguousarray(keep, np.int32)
        need = C.c_size_t(0)
        sched_dev.copy_(torch.from_numpy(sched_np.view(np.uint8)))

    def step(i: int):
        buf = pinned[i % 2]
        pinned_ev[i % 2].synchronize()  # the copy that last read this buffer is done
        tria.check(tria._lib.lib.tria_build_policy(C.byref(dims), hi_c.ctypes.data, keep_c.ctypes.data, hq,
                                                   C.c_void_p(buf.data_ptr()), sched_bytes, C.byref(need)))
        sched_dev.copy_(buf, non_blocking=True)
        pinned_ev[i % 2].record(stream)
        tria.quantize_k(dims, k, out=kz)                        # K codes; Q is quantised
        tria.prefill_bf16q(dims, sched_dev, q, kz, v, sm, out=out)  # inside the prefill
        tria.pack_kv_cache(dims, hi, keep, ctx, k, v, cache=cache)
        tria.decode(dims, cache, ctx, qdec, sm, out=dout, workspace=ws)

    def timed_loop(fn, warm, reps):
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(reps):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / reps

    def event_avg(fn, reps, before=None):
        """Average device time of fn() measured with HIP events on the stream."""
        ts = []
        for i in range(reps):
            if before is not None:
                before()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        ts = np.array(ts)
        return float(np.mean(ts)), float(np.median(ts)), float(np.percentile(ts, 10)), float(np.percentile(ts, 90))

    def back_to_back(fn, reps):
        """Per-launch device times of fn() launched back to back (an event between
        consecutive launches on the stream, one synchronisation at the end), the way a
        serving loop keeps the part busy; untimed launches first, about 300 ms of them,
        so that the clock has settled (after the idle gap of the host's input
        generation, the first ~100 ms of a short kernel run measurably slower)."""
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        one = time.perf_counter() - t0
        for _ in range(max(1, min(5000, int(0.3 / max(one, 1e-5))))):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for i in range(reps):
            fn()
            ev[i + 1].record(stream)
        ev[-1].synchronize()
        ts = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e-3 for i in range(reps)])
        return float(ts.mean()), float(np.median(ts)), float(np.percentile(ts, 10)), float(np.percentile(ts, 90))

    def prefill_stats(name, dims_, sched_, q_, kz_, qz_, v_, out_, W_, b_, hq_, d_, n_, reps):
        """Prefill alone on one workload, launched back to back: HIP-event times and
        the MFMA roofline, for the step's kernel (each query block quantised inside
        it) and for the attention alone (qz_: codes from tria_quantize_qk)."""
        mean, med, p10, p90 = back_to_back(
            lambda: tria.prefill_bf16q(dims_, sched_, q_, kz_, v_, 1.0 / math.sqrt(d_), out=out_), reps)
        ops = 4.0 * d_ * W_                                # 2dW int8 ops + 2dW bf16 flops
        t_roof = 2.0 * d_ * W_ / (PEAK_INT8_TOPS * 1e12) + 2.0 * d_ * W_ / (PEAK_BF16_TFLOPS * 1e12)
        achieved = ops / mean / 1e12
        res = {"workload": synth.CONFIGS[name].name, "ms": mean * 1e3, "ms_median": med * 1e3, "ms_p10": p10 * 1e3,
               "ms_p90": p90 * 1e3, "tokens_per_s": b_ * n_ / mean,
               "dense_equiv_tflops": 4.0 * b_ * hq_ * d_ * n_ * n_ / 2 / mean / 1e12,
               "effective_tflops": achieved, "frac_of_roofline": t_roof / mean,
               "frac_of_int8_peak": achieved / PEAK_INT8_TOPS, "kept_pairs": W_,
               "kept_density": W_ / (b_ * hq_ * n_ * (n_ + 1) / 2), "t_roof_ms": t_roof * 1e3,
               "traffic_bytes": measured_traffic(name)}
        # the attention alone: the same prefill over Q codes quantised beforehand
        # (tria_quantize_qk + tria_prefill), timed the same way
        a_mean = back_to_back(lambda: tria.prefill(dims_, sched_, qz_, v_, 1.0 / math.sqrt(d_), out=out_), reps)[0]
        res["attention_only"] = {"kernel": "tria_prefill over tria_quantize_qk codes", "ms": a_mean * 1e3,
                                 "frac_of_roofline": t_roof / a_mean}
        log(f"[bench] prefill {name}: {mean * 1e3:.3f} ms, {achieved:.1f} T mixed ops/s, "
            f"frac {t_roof / mean:.3f} (roofline {t_roof * 1e3:.3f} ms); over codes quantised beforehand "
            f"{a_mean * 1e3:.3f} ms, frac {t_roof / a_mean:.3f}")
        return res

    if args.only == "prefill":   # profiler run: prefill launches only, back to back
        # after the same ~300 ms of untimed launches as the measurement below
        back_to_back(lambda: tria.prefill_bf16q(dims, sched_dev, q, kz, v, sm, out=out), args.steps)
        print("done", flush=True)
        return
    if args.only == "copy":      # profiler calibration: a plain 1 GiB device copy
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("done", flush=True)
        return

    prefill_main = None
    prefill_others = {}
    if args.only in (None, "step"):
        log(f"[bench] step on {cfg.name}: warmup {args.warmup}, timed {args.steps}")
        sec_eager = timed_loop(step, args.warmup, args.steps)
        log(f"[bench] step (eager launches) {sec_eager * 1e3:.3f} ms")
        # The same step with its device work (schedule upload, quantise, prefill, pack,
        # decode) launched as one HIP graph per pinned schedule buffer: the host still
        # expands the policy into the buffer every step.  Replays are checked against
        # the eager step (bit for bit, eager work in between) before timing.
        ref = (out.clone(), dout.clone(), cache.clone())
        graphs = []
        for slot in range(2):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                sched_dev.copy_(pinned[slot], non_blocking=True)
                tria.quantize_k(dims, k, out=kz)
                tria.prefill_bf16q(dims, sched_dev, q, kz, v, sm, out=out)
                tria.pack_kv_cache(dims, hi, keep, ctx, k, v, cache=cache)
                tria.decode(dims, cache, ctx, qdec, sm, out=dout, workspace=ws)
            graphs.append(g)

        def gstep(i: int):
            buf = pinned[i % 2]
            pinned_ev[i % 2].synchronize()
            tria.check(tria._lib.lib.tria_build_policy(C.byref(dims), hi_c.ctypes.data, keep_c.ctypes.data, hq,
                                                       C.c_void_p(buf.data_ptr()), sched_bytes, C.byref(need)))
            graphs[i % 2].replay()
            pinned_ev[i % 2].record(stream)

        for i in range(4):
            out.zero_()
            dout.zero_()
            step(i)            # eager work between the replays
            torch.cuda.synchronize()
            out.zero_()
            dout.zero_()
            gstep(i)
            torch.cuda.synchronize()
            if not (torch.equal(out, ref[0]) and torch.equal(dout, ref[1]) and torch.equal(cache, ref[2])):
                raise SystemExit("graph replay differs from the eager step")
        del ref
        sec_graph = timed_loop(gstep, args.warmup, args.steps)
        sec = sec_graph
        value = b * n / sec
        log(f"[bench] step (graph launches) {sec * 1e3:.3f} ms -> {value:.4g} tokens/s")

        # per-kernel device times (events on the launch stream, launches back to back as
        # in the step)
        qz = tria.quantize_qk(dims, q, k)
        prefill_main = prefill_stats(args.workload, dims, sched_dev, q, kz, qz, v, out, W, b, hq, d, n, args.reps)
        del qz
        q_mean = back_to_back(lambda: tria.quantize_k(dims, k, out=kz), args.reps)[0]
        k_mean = back_to_back(lambda: tria.pack_kv_cache(dims, hi, keep, ctx, k, v, cache=cache), args.reps)[0]
        d_mean = back_to_back(lambda: tria.decode(dims, cache, ctx, qdec, sm, out=dout, workspace=ws), args.reps)[0]
        del graphs, q, k, v, kz, out, cache, ws, sched_dev
        torch.cuda.empty_cache()

        # the other prefill workloads, prefill alone (their inputs drawn from the same recipe)
        for name in ("llama3_8b_layer", "long_prefill", "batched_mixed"):
            if name == args.workload:
                continue
            c = synth.CONFIGS[name]
            log(f"[bench] generating {c.name}")
            qo, ko, vo = (dev(x) for x in synth.make_prefill_inputs(c))
            ho, kpo = c.policy()
            do = tria.make_dims(c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim, c.block, c.seq_len)
            so = tria.build_policy(do, ho, kpo)
            Wo = kept_pairs(so[16:].reshape(-1, 8), c.block, c.seq_len)
            sdo = torch.from_numpy(so).cuda()
            kzo = tria.quantize_k(do, ko)
            qzo = tria.quantize_qk(do, qo, ko)
            oo = torch.empty((c.batch, c.n_q_heads, c.seq_len, c.head_dim), dtype=torch.float32, device="cuda")
            for _ in range(2):
                tria.prefill_bf16q(do, sdo, qo, kzo, vo, 1.0 / math.sqrt(c.head_dim), out=oo)
            prefill_others[name] = prefill_stats(name, do, sdo, qo, kzo, qzo, vo, oo, Wo, c.batch, c.n_q_heads,
                                                 c.head_dim, c.seq_len, args.reps)
            del qo, ko, vo, kzo, qzo, oo, sdo
            torch.cuda.empty_cache()

    # ------------------------------------------------------------ decode workload (b16, ctx 32768)
    dec = None
    if args.only in (None, "decode", "skip", "paged"):
        c4 = synth.CONFIGS["decode_b16"]
        log(f"[bench] generating {c4.name}")
        k4h, v4h, q4h = synth.make_decode_inputs(c4)
        # the same inputs with block structure in K and per-head thresholds (skipping)
        k4s, th4 = synth.apply_block_structure(c4, k4h, q4h)
        h4, kp4 = c4.policy()
        dims4 = tria.make_dims(c4.batch, c4.n_q_heads, c4.n_kv_heads, c4.head_dim, c4.block, c4.seq_len)
        k4d, v4d = dev(k4h), dev(v4h)
        del k4h, v4h
        cache4 = tria.pack_kv_cache(dims4, h4, kp4, c4.seq_len, k4d, v4d)
        q4 = dev(q4h)
        ws4 = torch.empty(tria.decode_workspace_bytes(dims4, c4.seq_len), dtype=torch.uint8, device="cuda")
        o4 = torch.empty((c4.batch, c4.n_q_heads, c4.head_dim), dtype=torch.float32, device="cuda")
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

        def flush_caches():
            flush.add_(1)  # 1 GiB read + write: evicts the 256 MB last-level cache and L2

        def run_dec():
            tria.decode(dims4, cache4, c4.seq_len, q4, 1.0 / math.sqrt(c4.head_dim), out=o4, workspace=ws4)

        for _ in range(3):
            run_dec()
        if args.only == "skip":      # profiler run: index build, then skipping decodes
            k4s_d = dev(k4s)
            cs = tria.pack_kv_cache(dims4, h4, kp4, c4.seq_len, k4s_d, v4d)
            sm_ = tria.build_block_summaries(dims4, cs, c4.seq_len)
            th_ = torch.from_numpy(th4).cuda()
            for _ in range(args.steps):
                flush_caches()
                tria.decode_skip(dims4, cs, c4.seq_len, sm_, q4, th_, 1.0 / math.sqrt(c4.head_dim), out=o4)
            torch.cuda.synchronize()
            print("done", flush=True)
            return
        if args.only == "paged":     # profiler run: the cache in pages, paged decodes
            n_pg = c4.batch * c4.n_kv_heads * ((c4.seq_len - 1) // c4.block + 1)
            tb_, _, _ = tria.build_paged_table(dims4, h4, kp4, c4.seq_len, n_pg, np.arange(n_pg, dtype=np.int32))
            tb_d_ = torch.from_numpy(tb_).cuda()
            pool_ = torch.empty(n_pg * tria.paged_page_bytes(dims4), dtype=torch.uint8, device="cuda")
            tria.pack_kv_cache_paged(dims4, h4, kp4, c4.seq_len, k4d, v4d, tb_d_, pool_)
            for _ in range(args.steps):
                flush_caches()
                tria.decode_paged(dims4, tb_d_, pool_, c4.seq_len, q4, 1.0 / math.sqrt(c4.head_dim), out=o4)
            torch.cuda.synchronize()
            print("done", flush=True)
            return
        if args.only == "decode":
            for _ in range(args.steps):
                flush_caches()
                run_dec()
            torch.cuda.synchronize()
            print("done", flush=True)
            return
        dm, dmed, d10, d90 = event_avg(run_dec, args.reps, before=flush_caches)
        warm = event_avg(run_dec, args.reps)[0]
        # per-token cache maintenance on this workload: in place inside a block (token
        # 32767), and at a block start (token 32640 opens block 255: records move to
        # another buffer)
        c_prev = tria.pack_kv_cache(dims4, h4, kp4, c4.seq_len - 1, k4d, v4d)
        upd_in = event_avg(lambda: tria.update_kv_cache(dims4, h4, kp4, c4.seq_len, k4d, v4d, c_prev), args.reps)
        s0 = (c4.seq_len // c4.block - 1) * c4.block
        c_blk = tria.pack_kv_cache(dims4, h4, kp4, s0, k4d, v4d)
        c_out = torch.empty(tria.kv_cache_bytes(dims4, h4, kp4, s0 + 1), dtype=torch.uint8, device="cuda")
        upd_bs = event_avg(lambda: tria.update_kv_cache(dims4, h4, kp4, s0 + 1, k4d, v4d, c_blk, out=c_out),
                           args.reps)
        del c_prev, c_blk, c_out
        hdr = (64 + 64 * c4.batch * c4.n_kv_heads + 255) // 256 * 256
        # the same cache in pages (page table built on the host, pool of int8-record
        # pages): decode over it, and one more token per step as a paged update (the
        # current block rewritten in place; at a block start only the new records)
        pg_bytes = tria.paged_page_bytes(dims4)
        rmax4 = (c4.seq_len - 1) // c4.block + 1
        n_pages = c4.batch * c4.n_kv_heads * rmax4
        free0 = np.arange(n_pages, dtype=np.int32)
        tb, used0, _ = tria.build_paged_table(dims4, h4, kp4, c4.seq_len, n_pages, free0)
        pool = torch.empty(n_pages * pg_bytes, dtype=torch.uint8, device="cuda")
        tb_d = torch.from_numpy(tb).cuda()
        tria.pack_kv_cache_paged(dims4, h4, kp4, c4.seq_len, k4d, v4d, tb_d, pool)
        wsp = torch.empty(tria.decode_skip_workspace_bytes(dims4, c4.seq_len), dtype=torch.uint8, device="cuda")
        run_pg = lambda: tria.decode_paged(dims4, tb_d, pool, c4.seq_len, q4, 1.0 / math.sqrt(c4.head_dim), out=o4,
                                           workspace=wsp)
        for _ in range(3):
            run_pg()
        pgd = event_avg(run_pg, args.reps, before=flush_caches)
        # updates: token 32767 -> 32768 in place, and 32640 -> 32641 (block start)
        t_prev, u_prev, _ = tria.build_paged_table(dims4, h4, kp4, c4.seq_len - 1, n_pages, free0)
        tp_d = torch.from_numpy(t_prev).cuda()
        upd_pin = event_avg(lambda: tria.pack_kv_cache_paged(dims4, h4, kp4, c4.seq_len, k4d, v4d, tb_d, pool,
                                                             old_table=tp_d), args.reps)
        t_s0, u_s0, _ = tria.build_paged_table(dims4, h4, kp4, s0, n_pages, free0)
        t_s1, u_s1, rel_s1 = tria.build_paged_table(dims4, h4, kp4, s0 + 1, n_pages, free0[u_s0:], t_s0)
        ts0_d, ts1_d = torch.from_numpy(t_s0).cuda(), torch.from_numpy(t_s1).cuda()
        tria.pack_kv_cache_paged(dims4, h4, kp4, s0, k4d, v4d, ts0_d, pool)
        upd_pbs = event_avg(lambda: tria.pack_kv_cache_paged(dims4, h4, kp4, s0 + 1, k4d, v4d, ts1_d, pool,
                                                             old_table=ts0_d), args.reps)
        paged = {"decode_us": pgd[0] * 1e6, "decode_us_p10": pgd[2] * 1e6, "page_bytes": pg_bytes,
                 "pool_bytes": pool.numel(), "update_in_block_us": upd_pin[1] * 1e6,
                 "update_block_start_us": upd_pbs[1] * 1e6, "new_pages_at_block_start": u_s1,
                 "released_at_block_start": int(rel_s1.size),
                 "note": "update = tria_pack_kv_cache_paged with the previous table (median)"}
        log(f"[bench] paged cache: decode {pgd[0] * 1e6:.1f} us; update {upd_pin[1] * 1e6:.1f} us in a block, "
            f"{upd_pbs[1] * 1e6:.1f} us at a block start ({u_s1} new pages)")
        # continuous batching: the 16 sequences at their own lengths (16K-32K tokens) in
        # one pool; a step = every sequence one token longer: host table from the previous
        # one, upload, paged update (only what changed), decode
        rngv = np.random.default_rng(4)
        lens = rngv.integers(c4.seq_len // 2, c4.seq_len - 200, c4.batch).astype(np.int64)
        free_v = np.arange(n_pages, dtype=np.int32)
        tv, usedv, _ = tria.build_paged_table(dims4, h4, kp4, lens, n_pages, free_v)
        free_v = free_v[usedv:]
        tv_d = torch.from_numpy(tv).cuda()
        tria.pack_kv_cache_paged(dims4, h4, kp4, lens, k4d, v4d, tv_d, pool)
        wsv = torch.empty(tria.decode_skip_workspace_bytes(dims4, c4.seq_len), dtype=torch.uint8, device="cuda")
        host_us, dev_us = [], []
        for it in range(args.reps + 3):
            lens = lens + 1
            h0 = time.perf_counter()
            tv2, usedv, relv = tria.build_paged_table(dims4, h4, kp4, lens, n_pages, free_v, tv)
            free_v = np.concatenate([free_v[usedv:], relv])
            host_us.append((time.perf_counter() - h0) * 1e6)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            tv2_d = torch.from_numpy(tv2).cuda(non_blocking=False)
            tria.pack_kv_cache_paged(dims4, h4, kp4, lens, k4d, v4d, tv2_d, pool, old_table=tv_d)
            tria.decode_paged_varlen(dims4, tv2_d, pool, q4, 1.0 / math.sqrt(c4.head_dim), out=o4, workspace=wsv)
            e1.record(stream)
            e1.synchronize()
            dev_us.append(e0.elapsed_time(e1) * 1e3)
            tv, tv_d = tv2, tv2_d
        paged["continuous_batching"] = {
            "sequences": c4.batch, "lengths": "16K-32K, each one token longer per step",
            "step_device_us": float(np.median(dev_us[3:])), "table_build_host_us": float(np.median(host_us[3:])),
            "note": "device: table upload + paged update + variable-length paged decode (median)"}
        log(f"[bench] continuous batching (16 sequences, paged): {np.median(dev_us[3:]):.1f} us per step on the "
            f"device (upload + update + decode), table build {np.median(host_us[3:]):.0f} us on the host")
        del wsv
        del pool, wsp, tb_d, tp_d, ts0_d, ts1_d, k4d
        # dynamic block skipping (ETA-style) on the same workload, keys with block
        # structure: the index (built once per cache block), then the skipping decode
        # (keep bits + compaction + split-KV over kept records + merge) against the
        # plain decode of the same cache
        ctx4, sm4 = c4.seq_len, 1.0 / math.sqrt(c4.head_dim)
        ks_d = dev(k4s)
        del k4s
        cache_s = tria.pack_kv_cache(dims4, h4, kp4, ctx4, ks_d, v4d)
        del ks_d, v4d
        sums = tria.build_block_summaries(dims4, cache_s, ctx4)
        sum_t = event_avg(lambda: tria.build_block_summaries(dims4, cache_s, ctx4, out=sums), args.reps,
                          before=flush_caches)
        thd = torch.from_numpy(th4).cuda()
        wss = torch.empty(tria.decode_skip_workspace_bytes(dims4, ctx4), dtype=torch.uint8, device="cuda")

        def run_skip():
            tria.decode_skip(dims4, cache_s, ctx4, sums, q4, thd, sm4, out=o4, workspace=wss)

        for _ in range(3):
            run_skip()
        sk = event_avg(run_skip, args.reps, before=flush_caches)
        plain_s = event_avg(lambda: tria.decode(dims4, cache_s, ctx4, q4, sm4, out=o4, workspace=ws4), args.reps,
                            before=flush_caches)
        masks = tria.skip_masks(dims4, cache_s, ctx4, sums, q4, thd, sm4).cpu().numpy().view(np.uint32)
        dirs = cache_s[:hdr].cpu().numpy()
        rec8 = 2 * c4.block * c4.head_dim + 8 * c4.block
        rec4 = c4.block * c4.head_dim + 8 * c4.block
        G4 = c4.n_q_heads // c4.n_kv_heads
        kept_b = stored_rec = head_keep = 0
        for pi in range(c4.batch * c4.n_kv_heads):
            n8, n4 = (int(x) for x in dirs[64 + 64 * pi + 8:64 + 64 * pi + 16].view(np.int32))
            m = masks[pi, :n8 + n4]
            kept_b += int((m[:n8] != 0).sum()) * rec8 + int((m[n8:] != 0).sum()) * rec4
            stored_rec += n8 + n4
            head_keep += sum(bin(int(x)).count("1") for x in m)
        stored_b = cache_s.numel() - hdr
        sum_read = stored_rec * (2 * c4.head_dim + 16)
        io_b = c4.batch * c4.n_q_heads * c4.head_dim * (2 + 4)
        skip = {
            "us_per_call": sk[0] * 1e6, "us_p10": sk[2] * 1e6, "us_p90": sk[3] * 1e6,
            "plain_decode_same_cache_us": plain_s[0] * 1e6,
            "speedup_vs_plain": plain_s[0] / sk[0],
            "kept_record_bytes": kept_b, "stored_record_bytes": stored_b,
            "bytes_read_fraction": kept_b / stored_b,
            "head_density": head_keep / (stored_rec * G4),
            "algorithmic_bytes": kept_b + sum_read + io_b,
            "GB_per_s": (kept_b + sum_read + io_b) / sk[0] / 1e9,
            "index_bytes": sums.numel(), "index_fraction_of_cache": sums.numel() / cache_s.numel(),
            "index_build_us": sum_t[1] * 1e6,
            "inputs": "decode workload keys x one magnitude per (b, KV head, block) ~ U[0.1, 1]; "
                      "threshold per (b, head) = gamma * ||q||, gamma ~ U[0.6, 0.9]",
        }
        log(f"[bench] skip decode {sk[0] * 1e6:.1f} us vs {plain_s[0] * 1e6:.1f} us plain on the same cache; "
            f"reads {kept_b / stored_b:.3f} of the records, head density {skip['head_density']:.3f}, "
            f"{skip['GB_per_s']:.0f} GB/s; index {sums.numel() / 1e6:.2f} MB built in {sum_t[1] * 1e6:.1f} us")
        del cache_s, sums, wss
        # the same shapes at batch 32 and 64 (2x and 4x the cache), where the skipped
        # bytes start to pay for the plan: inputs drawn on the GPU from a seeded torch
        # generator (timing only; parity at these batches is not checked)
        for bb in (32, 64):
            skip[f"batch{bb}"] = skip_at_batch(bb, tria, c4, h4, kp4, args.reps, flush_caches, event_avg, log)
        dbytes = decode_bytes(cache4.numel(), c4.batch, c4.n_q_heads, c4.head_dim, hdr)
        dense_bytes = 2 * c4.batch * c4.n_kv_heads * c4.seq_len * c4.head_dim * 2
        dec = {
            "workload": c4.name,
            "us_per_call": dm * 1e6, "us_p10": d10 * 1e6, "us_p90": d90 * 1e6,
            "algorithmic_bytes": dbytes,
            "GB_per_s": dbytes / dm / 1e9,
            "frac_of_hbm_peak": dbytes / dm / 1e9 / PEAK_HBM_GBPS,
            "cache_flushed": True,
            "us_per_call_warm_cache": warm * 1e6,
            "dense_bf16_cache_bytes": dense_bytes,
            "cache_update_us": {"in_place_within_block": upd_in[1] * 1e6, "at_block_start": upd_bs[1] * 1e6,
                                "note": "median; tria_update_kv_cache for one more token (all 128 pairs)"},
            "skip": skip,
            "paged": paged,
        }
        log(f"[bench] decode {dm * 1e6:.1f} us, {dec['GB_per_s']:.0f} GB/s (warm {warm * 1e6:.1f} us); "
            f"cache update {upd_in[1] * 1e6:.1f} us in place, {upd_bs[1] * 1e6:.1f} us at a block start")
        del cache4, flush

    if args.only is not None:
        print(json.dumps({"decode": dec}))
        return

    # ------------------------------------------------------------ measured ceilings
    # What the part sustains for the instructions and access pattern the kernels use
    # (MFMA issue loops, a non-temporal streaming read of 1 GiB), so the fractions can
    # also be read against measured ceilings; the roofline object keeps the published
    # peaks.
    sink = torch.zeros(tria._lib.PEAK_SINK_INTS, dtype=torch.int32, device="cuda")
    rd_src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    iters = 20000
    w_i8, w_bf, w_rd = tria.peak_mfma(0, iters, sink), tria.peak_mfma(1, iters, sink), tria.peak_read(rd_src, sink)
    t_i8 = event_avg(lambda: tria.peak_mfma(0, iters, sink), 5)[1]
    t_bf = event_avg(lambda: tria.peak_mfma(1, iters, sink), 5)[1]
    t_rd = event_avg(lambda: tria.peak_read(rd_src, sink), 10)[1]
    del rd_src
    i8, bf, rd = w_i8 / t_i8 / 1e12, w_bf / t_bf / 1e12, w_rd / t_rd / 1e9
    blend = 2.0 / (1.0 / i8 + 1.0 / bf)  # equal int8 ops and bf16 flops, in series
    achieved = prefill_main["effective_tflops"]
    ceilings = {
        "mfma_i8_tops": i8, "mfma_bf16_tflops": bf, "mfma_series_blend_tflops": blend, "hbm_read_gbps": rd,
        "prefill_frac": achieved / blend,
        "decode_frac": dec["GB_per_s"] / rd if dec else None,
        "method": "median of 5 launches of 512 work groups x 4 wavefronts, each wavefront issuing "
                  f"{iters} rounds of 8 independent v_mfma_i32_16x16x64_i8 / v_mfma_f32_16x16x32_bf16; "
                  "median of 10 non-temporal streaming reads of 1 GiB (8192 wavefronts, one contiguous "
                  "range each, 1 KB loads, 8 in flight)",
    }
    log(f"[bench] measured ceilings: int8 {i8:.0f} TOPS, bf16 {bf:.0f} TFLOPS, read {rd:.0f} GB/s; "
        f"prefill {achieved / blend:.3f}, decode {ceilings['decode_frac'] or 0:.3f} of them")

    # ------------------------------------------------------------ CPU baseline (the oracle, sampled)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        # whole query heads of the step's workload, one after another, until about 10 s
        # of work is done (at most all heads); scaled by kept pairs to the whole step
        G = hq // hk
        t_sample, w_sample, heads = 0.0, 0, 0
        for h0 in range(hq):
            sel = units[(units[:, 1] == h0) & (units[:, 0] == 0)]
            g0 = h0 // G
            t0 = time.perf_counter()
            oracle.prefill(qh[:1, h0:h0 + 1], kh[:1, g0:g0 + 1], vh[:1, g0:g0 + 1], hi[h0:h0 + 1],
                           keep[h0:h0 + 1], blk, sm)
            t_sample += time.perf_counter() - t0
            w_sample += kept_pairs(sel, blk, n)
            heads += 1
            if t_sample >= 10.0:
                break
        est_total = t_sample * W / w_sample
        cpu = {"value": b * n / est_total, "unit": "tokens/s", "cores": oracle.nthreads(), "kind": "oracle",
               "cpu_model": cpu_model(),
               "sample": f"oracle prefill (quantisation + attention) of {heads} of the workload's {hq} query heads "
                         f"(batch element 0), all query blocks ({w_sample:.3g} of {W:.3g} kept pairs), took "
                         f"{t_sample:.2f} s on {oracle.nthreads()} threads; the whole step's time is extrapolated "
                         f"by kept pairs (est. {est_total:.1f} s); pack/decode are <1% of its work and not timed"}
        log(f"[bench] cpu oracle sample {heads} heads {t_sample:.2f} s on {oracle.nthreads()} threads "
            f"-> est. {est_total:.1f} s for the step's prefill")

    line = {
        "metric": "prefill tokens/s + decode HBM GB/s, block-sparse int8/int4 attn; % roofline",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec * 1e3,
        "ms_per_step_eager_launches": sec_eager * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8/int4 QK^T (int32 acc), bf16 P.V (fp32 acc), fp32 softmax",
        "data": "synthetic (seeded N(0,1) bf16, K outlier channels x8, seeded per-head policies)",
        "config": {"workload": cfg.name, "batch": b, "seq_len": n, "n_q_heads": hq, "n_kv_heads": hk,
                   "head_dim": d, "block": blk, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "prefill_kernel", "achieved": achieved,
                     "peak": 4.0 * d * W / (prefill_main["t_roof_ms"] * 1e-3) / 1e12,
                     "unit": "TFLOP/s", "frac": prefill_main["frac_of_roofline"],
                     "traffic": prefill_main["traffic_bytes"],
                     "work": f"4*d*W mixed ops per launch: 2dW int8 ops (QK^T) + 2dW bf16 flops (P.V), "
                             f"W = {W} kept causal pairs; peak = int8 {PEAK_INT8_TOPS:.0f} and bf16 "
                             f"{PEAK_BF16_TFLOPS:.0f} T/s combined in series"},
        "prefill": prefill_main,
        "prefill_workloads": prefill_others,
        "kernels_ms": {"quantize_k": q_mean * 1e3, "prefill_bf16q": prefill_main["ms"], "pack": k_mean * 1e3,
                       "decode_step_workload": d_mean * 1e3},
        # prompt tokens/s of the K quantiser and the prefill kernel (which quantises Q)
        # together (their device times)
        "quantise_plus_prefill_tokens_per_s": b * n / (q_mean + prefill_main["ms"] * 1e-3),
        "decode": dec,
        "measured_ceilings": ceilings,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
