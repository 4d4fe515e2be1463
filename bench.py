"""Benchmark of the NVFP4 KV-cache hot path on one MI355X.

A step is one decode iteration of the paged large-batch workload (batch 128,
32 query / 8 KV heads, head_dim 128, context lengths U[1024, 8192], 16-token
pages placed by a seeded permutation): quantize-and-append one new K/V token
per sequence (nvfp4_kv_append), then decode attention over the whole NVFP4
cache (nvfp4_decode_attn).  The cache, queries and new tokens are resident in
HBM before timing starts.  Each step appends at the same position, so every
step does identical work.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints one JSON line.  `value` is the step's algorithmic bytes (cache bytes
read by decode at 0.5625 B/element, plus the append's bf16 input and NVFP4
output, plus queries and outputs) per second.  `roofline` is for the decode
kernels, timed with HIP events on their stream around each decode call of a
second pass of K steps (the same work as the timed steps).  `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload.  `extra` holds the other
measured paths (bulk append, prefill, the other decode workloads).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4-KV decode attention HBM GB/s (% of peak) + append quantize GB/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA
F16_PEAK_TFLOPS = 2500.0       # MI355X dense FP16 MFMA
BYTES_PER_TOKEN_HEAD = 2 * 128 * 0.5625   # K and V, codes + scales


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gen_decode(w, threads=16):
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(w.kv, range(w.B)))


def build_cache(api, torch, w, data, s_tk, s_tv, chunk=16, fmt=None):
    """The workload's cache in NVFP4 (fmt None; s_t the NVFP4 tensor scales)
    or in a comparison format (api.CMP_FP8 with FP8 tensor scales s_t, or
    api.CMP_BF16), built through the library's append."""
    if fmt is None:
        cache = api.KVCache(w.num_pages, w.Hkv, s_tk, s_tv, fill=0)
        put = api.append
    else:
        cache = api.CmpCache(fmt, w.num_pages, w.Hkv, s_tk, s_tv, fill=0)
        put = api.cmp_append
    pt = torch.from_numpy(w.page_table).cuda()
    for b0 in range(0, w.B, chunk):
        idx = range(b0, min(w.B, b0 + chunk))
        k = np.concatenate([data[b][0] for b in idx])
        v = np.concatenate([data[b][1] for b in idx])
        seq = np.concatenate([np.full(len(data[b][0]), b, np.int32) for b in idx])
        pos = np.concatenate([np.arange(len(data[b][0]), dtype=np.int32) for b in idx])
        put(cache, torch.from_numpy(k).to(torch.bfloat16).cuda(), torch.from_numpy(v).to(torch.bfloat16).cuda(),
            torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), pt)
    torch.cuda.synchronize()
    return cache, pt


# bytes per (token, KV head) of K and V in each cache format
FORMAT_BYTES = {"nvfp4": 144, "fp8": 256, "bf16": 512}


def format_caches(api, torch, w, data, nv_scales, amax):
    """(name, cache, page table, decode fn) for NVFP4, FP8 and BF16 caches of
    the same data; amax = (K amax, V amax) for the FP8 tensor scales."""
    out = []
    for name, fmt in (("nvfp4", None), ("fp8", api.CMP_FP8), ("bf16", api.CMP_BF16)):
        if fmt is None:
            s_k, s_v = nv_scales
        elif fmt == api.CMP_FP8:
            s_k, s_v = api.cmp_fp8_scale_from_amax(amax[0]), api.cmp_fp8_scale_from_amax(amax[1])
        else:
            s_k = s_v = 1.0
        c, pt = build_cache(api, torch, w, data, s_k, s_v, fmt=fmt)
        out.append((name, c, pt, api.decode if fmt is None else api.cmp_decode))
    return out


def device_scale(api, torch, arrays):
    """Calibrate s_t on the device: exact amax of every chunk, then the max."""
    amax = 0.0
    for a in arrays:
        t = torch.from_numpy(a).to(torch.bfloat16).cuda()
        amax = max(amax, api.abs_max(t).item())
    return api.tensor_scale_from_amax(amax), amax


def time_region(torch, fn, iters, stream):
    """Average milliseconds of fn() over iters launches, HIP events on stream."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(iters):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / iters


def call_times(torch, fn, iters, stream):
    """Milliseconds of each of iters calls of fn(), HIP events on stream."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for s, e in ev:
        s.record(stream)
        fn()
        e.record(stream)
    ev[-1][1].synchronize()
    return [s.elapsed_time(e) for s, e in ev]


def host_threads():
    """(threads used, CPUs this process may run on, CPUs the host shows).  A
    GPU machine's share for one GPU is 16 cores, whatever the host shows."""
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = os.cpu_count() or 1
    return max(1, min(16, affinity)), affinity, os.cpu_count() or 1


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_decode_cfg(cfg, threads_all):
    """Oracle decode of a whole decode workload (configurations 1-3): the
    codes come from the oracle's own quantizer (timed on all threads, as the
    append), the attention is timed on all threads and on one."""
    import oracle
    from decode_attention_nvfp4_amd import workloads as W
    w = W.decode_workload(cfg)
    data = [w.kv(b) for b in range(w.B)]
    k_all = np.concatenate([d[0] for d in data])
    v_all = np.concatenate([d[1] for d in data])
    s_tk, s_tv = oracle.tensor_scale(k_all), oracle.tensor_scale(v_all)
    def quant(x, st):
        # rows split over the threads (the C calls release the GIL)
        bounds = np.linspace(0, len(x), threads_all + 1).astype(int)
        with ThreadPoolExecutor(max_workers=threads_all) as ex:
            parts = list(ex.map(lambda i: oracle.quantize_rows(x[bounds[i]:bounds[i + 1]], st), range(threads_all)))
        return np.concatenate([a for a, _ in parts]), np.concatenate([b for _, b in parts])

    t0 = time.perf_counter()
    codes = [(*quant(k, s_tk), *quant(v, s_tv)) for k, v in data]
    t_quant = time.perf_counter() - t0
    q = w.q(0)
    nbytes = int(w.lens.sum()) * w.Hkv * BYTES_PER_TOKEN_HEAD
    out = {"cache_mb": round(nbytes / 1e6, 2)}
    for name, th in (("all", threads_all), ("one", 1)):
        t0 = time.perf_counter()
        oracle.decode_batch(q, codes, w.Hkv, s_tk, s_tv, threads=th)
        dt = time.perf_counter() - t0
        out[f"decode_s_{name}"] = round(dt, 4)
        out[f"decode_gbs_{name}"] = round(nbytes / dt / 1e9, 4)
    n_el = 2 * k_all.size
    out["quantize_s_all"] = round(t_quant, 3)
    out["quantize_gbs_all"] = round(n_el * (2 + 0.5625) / t_quant / 1e9, 4)
    return out


def cpu_baseline(w, data, s_tk, s_tv, q, threads):
    """The oracle, untuned, on the same decode step (all 128 sequences; the
    codes come from the oracle's own quantizer, untimed), on the machine's host
    threads and on one thread; then the other workloads (configurations 1-3
    whole, the prefill on a sample of query rows)."""
    import oracle
    sample = list(range(w.B))
    with ThreadPoolExecutor(max_workers=threads) as ex:
        codes = list(ex.map(lambda b: (*oracle.quantize_rows(data[b][0], s_tk),
                                       *oracle.quantize_rows(data[b][1], s_tv)), sample))
    nbytes = sum(int(w.lens[b]) for b in sample) * w.Hkv * BYTES_PER_TOKEN_HEAD
    t0 = time.perf_counter()
    oracle.decode_batch(q[sample], codes, w.Hkv, s_tk, s_tv, threads=threads)
    dt = time.perf_counter() - t0
    one = list(range(0, w.B, 8))                      # every eighth sequence on one thread
    nb1 = sum(int(w.lens[b]) for b in one) * w.Hkv * BYTES_PER_TOKEN_HEAD
    t0 = time.perf_counter()
    oracle.decode_batch(q[one], [codes[b] for b in one], w.Hkv, s_tk, s_tv, threads=1)
    dt1 = time.perf_counter() - t0
    used, affinity, visible = host_threads()
    res = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "seconds": round(dt, 3),
           "sample": f"decode attention of the whole step (128 sequences, all heads, full length; "
                     f"{nbytes / 1e6:.1f} MB of NVFP4 cache), without the append",
           "one_thread_gbs": round(nb1 / dt1 / 1e9, 4),
           "one_thread_sample": f"16 of the 128 sequences ({nb1 / 1e6:.1f} MB), one thread",
           "cpu_model": cpu_model(), "host_cpus_allowed": affinity, "host_cpus_visible": visible,
           "threads_note": "a GPU box's share for one GPU is 16 cores"}
    per = {}
    for cfg in (1, 2, 3):
        per[f"config{cfg}"] = _oracle_decode_cfg(cfg, threads)
        log(f"oracle config {cfg}: {per[f'config{cfg}']}")
    per["config5"] = _oracle_prefill_sample(threads)
    log(f"oracle config 5: {per['config5']}")
    res["per_config"] = per
    return res


def _oracle_prefill_sample(threads):
    """Oracle prefill of configuration 5 on a sample of query rows (all 64
    heads, every visible key): 16 rows on the box's threads, 2 on one."""
    import oracle
    from decode_attention_nvfp4_amd import workloads as W
    pw = W.PrefillWorkload()
    kp, vp = pw.prefix_kv()
    kc, vc = pw.chunk_kv()
    k = np.concatenate([kp, kc])
    v = np.concatenate([vp, vc])
    s_tk, s_tv = oracle.tensor_scale(k), oracle.tensor_scale(v)
    bounds = np.linspace(0, len(k), threads + 1).astype(int)
    with ThreadPoolExecutor(max_workers=threads) as ex:
        kq = list(ex.map(lambda i: oracle.quantize_rows(k[bounds[i]:bounds[i + 1]], s_tk), range(threads)))
        vq = list(ex.map(lambda i: oracle.quantize_rows(v[bounds[i]:bounds[i + 1]], s_tv), range(threads)))
    kcodes, kscales = np.concatenate([a for a, _ in kq]), np.concatenate([b for _, b in kq])
    vcodes, vscales = np.concatenate([a for a, _ in vq]), np.concatenate([b for _, b in vq])
    q = pw.q()
    out = {}
    for name, th, rows in (("all", threads, np.linspace(0, pw.T - 1, 16).astype(np.int32)),
                           ("one", 1, np.array([0, pw.T - 1], np.int32))):
        flops = 4.0 * 128 * pw.Hq * float(sum(pw.prefix + int(i) + 1 for i in rows))
        t0 = time.perf_counter()
        oracle.prefill_rows(q[rows], rows, pw.Hkv, kcodes, kscales, s_tk, vcodes, vscales, s_tv, pw.prefix,
                            causal=True, threads=th)
        dt = time.perf_counter() - t0
        out[f"rows_{name}"] = len(rows)
        out[f"seconds_{name}"] = round(dt, 3)
        out[f"gflops_{name}"] = round(flops / dt / 1e9, 3)
    out["sample"] = "query rows of the 2048-row chunk, all 64 heads, every visible key (of 2.268 TFLOP in all)"
    return out


def bench_prefill(api, torch, stream, iters=3, modes=None, mx=True):
    """Chunked prefill at its full size: the chunk's bulk append and the
    attention, once per operand mode (FP8 as in the pages' flow, then exact
    16-bit operands), then over an MXFP4 cache of the same data."""
    from decode_attention_nvfp4_amd import workloads as W
    modes = [api.PREFILL_FP8, api.PREFILL_F16] if modes is None else modes
    pw = W.PrefillWorkload()
    kp, vp = pw.prefix_kv()
    kc, vc = pw.chunk_kv()
    s_tk, _ = device_scale(api, torch, [kp, kc])
    s_tv, _ = device_scale(api, torch, [vp, vc])
    cache = api.KVCache(pw.num_pages, pw.Hkv, s_tk, s_tv, fill=0)
    pt = torch.from_numpy(pw.page_table()).cuda()
    dev = lambda a: torch.from_numpy(a).to(torch.bfloat16).cuda()  # noqa: E731
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()  # noqa: E731
    api.append(cache, dev(kp), dev(vp), i32(np.zeros(pw.prefix)), i32(np.arange(pw.prefix)), pt)
    kcd, vcd = dev(kc), dev(vc)
    seq, pos = i32(np.zeros(pw.T)), i32(pw.prefix + np.arange(pw.T))
    q = dev(pw.q())
    out = torch.empty((pw.T, pw.Hq, 128), dtype=torch.float32, device="cuda")

    def chunk_append():
        api.append(cache, kcd, vcd, seq, pos, pt)

    chunk_append()
    torch.cuda.synchronize()
    t_app = time_region(torch, chunk_append, iters, stream)
    app_bytes = pw.T * pw.Hkv * 128 * 2 * (2 + 0.5625)
    flops = 4.0 * 128 * pw.Hq * sum(pw.prefix + i + 1 for i in range(pw.T))
    res = {
        "workload": "chunked prefill: 2048 causal queries after a 32768-token NVFP4 prefix, 64 q / 8 kv heads",
        "chunk_append_ms": round(t_app, 4), "chunk_append_gbs": round(app_bytes / t_app / 1e6, 1),
    }
    for mode in modes:
        ws = torch.empty(api.prefill_workspace_bytes(pw.T, pw.Hq, pw.Hkv, pw.prefix, mode), dtype=torch.uint8,
                         device="cuda")

        def attend():
            api.prefill(cache, q, pt[0], pw.prefix, causal=True, workspace=ws, out=out, mode=mode)

        attend()
        torch.cuda.synchronize()
        t_att = time_region(torch, attend, iters, stream)
        tf = flops / t_att / 1e9
        if mode == api.PREFILL_FP8:
            res.update({"attention_ms": round(t_att, 4), "tflops": round(tf, 2),
                        "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4)})
        else:
            res["f16_operands"] = {"attention_ms": round(t_att, 4), "tflops": round(tf, 2),
                                   "frac_f16_peak": round(tf / F16_PEAK_TFLOPS, 4)}
        del ws
    if mx:
        # the same chunk over an MXFP4 cache: FP4 K with its block scales in
        # the score products, FP8 Q, P and V (V expanded, K read in place)
        amax = lambda a: float(np.abs(a).max())  # noqa: E731
        mcache = api.MxCache(pw.num_pages, pw.Hkv, api.mx_exp_offset_from_amax(max(amax(kp), amax(kc))),
                             api.mx_exp_offset_from_amax(max(amax(vp), amax(vc))), fill=0)
        api.mx_append(mcache, dev(kp), dev(vp), i32(np.zeros(pw.prefix)), i32(np.arange(pw.prefix)), pt)
        api.mx_append(mcache, kcd, vcd, seq, pos, pt)
        ws = torch.empty(api.mx_prefill_workspace_bytes(pw.T, pw.Hq, pw.Hkv, pw.prefix), dtype=torch.uint8,
                         device="cuda")

        def attend_mx():
            api.mx_prefill(mcache, q, pt[0], pw.prefix, causal=True, workspace=ws, out=out)

        attend_mx()
        torch.cuda.synchronize()
        t_att = time_region(torch, attend_mx, iters, stream)
        tf = flops / t_att / 1e9
        res["mxfp4_cache"] = {"attention_ms": round(t_att, 4), "tflops": round(tf, 2),
                              "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4)}
        del ws, mcache
    return res


def stream_read_probe(api, torch, stream, gib=1, iters=10):
    """Streaming-read reference: nvfp4_abs_max over `gib` GiB of bf16 (one
    16-byte load per lane per step, each byte read once; larger than the
    256 MB LLC)."""
    x = torch.ones((gib << 30) // 2, dtype=torch.bfloat16, device="cuda")
    api.abs_max(x)
    torch.cuda.synchronize()
    t = time_region(torch, lambda: api.abs_max(x, stream=stream), iters, stream)
    del x
    return {"what": f"nvfp4_abs_max over {gib} GiB of bf16", "ms": round(t, 4),
            "gbs": round((gib << 30) / (t * 1e-3) / 1e9, 1)}


def llc_flush(api, torch):
    """A read of 1 GiB (four times the 256 MB last-level cache) by the
    library's streaming kernel, so that the next kernel finds the cache full
    of other, clean lines.  (Filling a buffer instead would leave dirty lines
    that the next kernel's reads must first write back.)"""
    buf = torch.ones((1 << 30) // 2, dtype=torch.bfloat16, device="cuda")
    return lambda: api.abs_max(buf)


def time_calls(torch, stream, fn, iters, before=None):
    """Per-call microseconds of fn() (HIP events on stream), with `before`
    enqueued ahead of each call outside the timed region."""
    ts = []
    for _ in range(iters):
        if before is not None:
            before()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record(stream)
        fn()
        e.record(stream)
        e.synchronize()
        ts.append(s.elapsed_time(e) * 1e3)
    return np.array(ts)


def gpu_busy(torch, us=60.0):
    """A GPU-side spin of about `us` microseconds, enqueued ahead of a timed
    call so that the call's kernels are queued before the GPU reaches them:
    the events then time the GPU, not the host's launch latency."""
    return lambda: torch.cuda._sleep(int(us * 2400))


def pct(a):
    return {"us_median": round(float(np.median(a)), 2), "us_p10": round(float(np.percentile(a, 10)), 2),
            "us_p90": round(float(np.percentile(a, 90)), 2)}


def bench_small_decode(api, torch, stream, cfg, iters=20):
    """Decode of configurations 2 (GQA batch 8, L 4096) and 3 (L 65536), in
    NVFP4 and in the FP8 and BF16 comparison formats built from the same
    data.  The caches fit in the 256 MB last-level cache; the cold timing
    rotates over 4 replicas and reads 1 GiB between launches (llc_flush)."""
    from decode_attention_nvfp4_amd import workloads as W
    w = W.decode_workload(cfg)
    data = gen_decode(w)
    s_tk, amax_k = device_scale(api, torch, [d[0] for d in data])
    s_tv, amax_v = device_scale(api, torch, [d[1] for d in data])
    q = torch.from_numpy(w.q(0)).to(torch.bfloat16).cuda()
    lens = torch.from_numpy(w.lens).cuda()
    L = int(w.lens.max())
    out = torch.empty((w.B, w.Hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, 2 * api.decode_workspace_bytes(w.B, w.Hq, w.Hkv, L)), dtype=torch.uint8,
                     device="cuda")
    flush = llc_flush(api, torch)
    res = {"workload": f"decode config {cfg}: batch {w.B}, {w.Hq}/{w.Hkv} heads, L {L}",
           "splits": api.decode_num_splits(w.B, w.Hkv, L)}
    reps = [format_caches(api, torch, w, data, (s_tk, s_tv), (amax_k, amax_v)) for _ in range(4)]
    for f, name in enumerate(FORMAT_BYTES):
        state = {"i": 0}

        def one():
            _, c, pt, fn = reps[state["i"] % 4][f]
            state["i"] += 1
            fn(c, q, pt, lens, L, workspace=ws, out=out)

        one(); torch.cuda.synchronize()
        cold = time_calls(torch, stream, one, iters, before=flush)
        t_cold = float(np.median(cold)) * 1e-3
        _, c0, pt0, fn0 = reps[0][f]
        warm = time_calls(torch, stream, lambda: fn0(c0, q, pt0, lens, L, workspace=ws, out=out), iters,
                          before=gpu_busy(torch))
        t_warm = float(np.median(warm)) * 1e-3
        nbytes = int(w.lens.sum()) * w.Hkv * FORMAT_BYTES[name]
        entry = {"cache_mb": round(nbytes / 1e6, 2), "cold_us": round(t_cold * 1e3, 2),
                 "cold_gbs": round(nbytes / t_cold / 1e6, 1), "warm_us": round(t_warm * 1e3, 2),
                 "warm_gbs": round(nbytes / t_warm / 1e6, 1),
                 "cold_us_p10": round(float(np.percentile(cold, 10)), 2),
                 "cold_us_p90": round(float(np.percentile(cold, 90)), 2)}
        if name == "nvfp4":
            res.update(entry)
        else:
            res[name] = entry
    for name in ("fp8", "bf16"):
        res[f"nvfp4_speedup_vs_{name}_cold"] = round(res[name]["cold_us"] / res["cold_us"], 3)
    if cfg == 2:
        res["steps"] = _cfg2_steps(api, torch, stream, w, reps[0][0][1], reps[0][0][2], flush)
    del reps
    torch.cuda.empty_cache()
    return res


def _cfg2_steps(api, torch, stream, w, cache, pt, flush):
    """Configuration 2's decode loop: 16 steps, each appending one token per
    sequence (nvfp4_kv_append, 8 rows x 8 KV heads) and then attending over
    L + step + 1 tokens; per-step microseconds of the append and the decode
    (HIP events), once warm (a GPU spin ahead of each step, the cache in the
    LLC) and once with the LLC flushed before each step."""
    out = torch.empty((w.B, w.Hq, 128), dtype=torch.float32, device="cuda")
    bidx = torch.arange(w.B, dtype=torch.int32, device="cuda")
    new = [tuple(torch.from_numpy(x).to(torch.bfloat16).cuda() for x in w.append_kv(s)) for s in range(w.steps)]
    qs = [torch.from_numpy(w.q(s)).to(torch.bfloat16).cuda() for s in range(w.steps)]
    ws = torch.empty(max(1, api.decode_workspace_bytes(w.B, w.Hq, w.Hkv, int(w.lens.max()) + w.steps)),
                     dtype=torch.uint8, device="cuda")
    res = {}
    poss = [torch.from_numpy((w.lens + s).astype(np.int32)).cuda() for s in range(w.steps)]
    lenss = [torch.from_numpy((w.lens + s + 1).astype(np.int32)).cuda() for s in range(w.steps)]
    busy = gpu_busy(torch)
    for mode in ("warm", "cold"):
        ta, td = [], []
        for s in range(w.steps):
            pos, lens = poss[s], lenss[s]
            L = int(w.lens.max()) + s + 1
            (flush if mode == "cold" else busy)()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            ev[0].record(stream)
            api.append(cache, new[s][0], new[s][1], bidx, pos, pt)
            ev[1].record(stream)
            api.decode(cache, qs[s], pt, lens, L, workspace=ws, out=out)
            ev[2].record(stream)
            ev[2].synchronize()
            ta.append(ev[0].elapsed_time(ev[1]) * 1e3)
            td.append(ev[1].elapsed_time(ev[2]) * 1e3)
        res[mode] = {"append_us_mean": round(float(np.mean(ta)), 2), "decode_us_mean": round(float(np.mean(td)), 2),
                     "step_us_mean": round(float(np.mean(np.array(ta) + np.array(td))), 2),
                     "append_us_per_step": [round(x, 2) for x in ta], "decode_us_per_step": [round(x, 2) for x in td]}
    return res


def bench_cfg1(api, torch, stream, iters=50):
    """Configuration 1 (one sequence, one head, L 1024, FP32 K/V/Q): the
    decode call's latency in microseconds, warm and after an LLC flush (its
    147 KB are a latency, not a bandwidth, problem)."""
    from decode_attention_nvfp4_amd import workloads as W
    w = W.decode_workload(1)
    k, v = w.kv(0)
    s_tk = api.tensor_scale_from_amax(float(np.abs(k).max()))
    s_tv = api.tensor_scale_from_amax(float(np.abs(v).max()))
    cache = api.KVCache(w.num_pages, w.Hkv, s_tk, s_tv, fill=0)
    pt = torch.from_numpy(w.page_table).cuda()
    api.append(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
               torch.zeros(len(k), dtype=torch.int32, device="cuda"),
               torch.arange(len(k), dtype=torch.int32, device="cuda"), pt)
    q = torch.from_numpy(w.q(0)).cuda()
    lens = torch.from_numpy(w.lens).cuda()
    out = torch.empty((1, 1, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, api.decode_workspace_bytes(1, 1, 1, 1024)), dtype=torch.uint8, device="cuda")

    def call():
        api.decode(cache, q, pt, lens, 1024, workspace=ws, out=out)

    call(); torch.cuda.synchronize()
    warm = time_calls(torch, stream, call, iters, before=gpu_busy(torch))
    cold = time_calls(torch, stream, call, iters, before=llc_flush(api, torch))
    return {"workload": "decode config 1: 1 sequence, 1/1 heads, L 1024, FP32 K/V/Q",
            "splits": api.decode_num_splits(1, 1, 1024), "warm": pct(warm), "cold": pct(cold)}


def bench_gather_probe(api, torch, stream, cache, pt, lens, L, decode_us, iters=10):
    """The page-gather ceiling: the decode kernel's own wave ranges, page walk
    and page loads over the same cache, without the math or the merge
    (nvfp4_decode_gather_probe)."""
    sink = api.decode_gather_probe(cache, pt, lens, L)
    torch.cuda.synchronize()
    t = time_calls(torch, stream, lambda: api.decode_gather_probe(cache, pt, lens, L, sink=sink), iters,
                   before=gpu_busy(torch, 200.0))
    nbytes = int((lens.cpu().numpy()).sum()) * cache.num_kv_heads * BYTES_PER_TOKEN_HEAD
    med = float(np.median(t))
    return {"what": "nvfp4_decode_gather_probe on the headline cache", **pct(t),
            "gbs": round(nbytes / med / 1e3, 1), "frac_hbm_peak": round(nbytes / med / 1e3 / HBM_PEAK_GBS, 4),
            "decode_frac_of_ceiling": round(med / decode_us, 4)}


def bench_formats_cfg4(api, torch, stream, w, data, nv_scales, amax, q_np, iters=10):
    """Configuration 4's decode (batch 128, L_b ~ U[1024, 8192], permuted
    pages) over NVFP4, FP8 and BF16 caches of the same data: the speed ratio
    of the formats on one GPU.  Every cache exceeds the 256 MB last-level
    cache, so each call streams it from HBM."""
    q = torch.from_numpy(q_np).to(torch.bfloat16).cuda()
    lens = torch.from_numpy(w.lens.astype(np.int32)).cuda()
    L = int(w.lens.max())
    out = torch.empty((w.B, w.Hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, 2 * api.decode_workspace_bytes(w.B, w.Hq, w.Hkv, L)), dtype=torch.uint8,
                     device="cuda")
    res = {"workload": "decode config 4: batch 128, 32/8 heads, context U[1024,8192], same data per format"}
    for name, c, pt, fn in format_caches(api, torch, w, data, nv_scales, amax):
        fn(c, q, pt, lens, L, workspace=ws, out=out)
        torch.cuda.synchronize()
        t = time_region(torch, lambda: fn(c, q, pt, lens, L, workspace=ws, out=out), iters, stream)
        nbytes = int(w.lens.sum()) * w.Hkv * FORMAT_BYTES[name]
        res[name] = {"cache_mb": round(nbytes / 1e6, 1), "us": round(t * 1e3, 2),
                     "gbs": round(nbytes / t / 1e6, 1), "frac_hbm_peak": round(nbytes / t / 1e6 / HBM_PEAK_GBS, 4)}
        del c
        torch.cuda.empty_cache()
    for name in ("fp8", "bf16"):
        res[f"nvfp4_speedup_vs_{name}"] = round(res[name]["us"] / res["nvfp4"]["us"], 3)
    return res


def _mx_dequant_seq(torch, c, pt_row, L, plane):
    """MXFP4 values [L][Hkv][128] of one sequence's K (plane 0) or V (plane 1),
    read from the device planes by the layout the header states."""
    H = c.num_kv_heads
    pos = torch.arange(L, device="cuda")
    pages = pt_row.long()[pos // 16]
    slots = pos % 16
    if plane == 0:
        b = c.k_codes.view(c.num_pages, H, 16, 64)[pages, :, slots]              # [L][H][64]
        codes = torch.stack([b & 15, b >> 4], dim=-1).reshape(L, H, 128)
        sc = c.k_scales.view(c.num_pages, H, 16, 4)[pages, :, slots]             # [L][H][4]
    else:
        vb = c.v_codes.view(c.num_pages, H, 4, 16, 2, 8)
        nib = torch.stack([vb & 15, vb >> 4], dim=-1).permute(0, 1, 2, 4, 6, 3, 5)
        codes = nib.reshape(c.num_pages, H, 16, 128)[pages, :, slots]
        sc = c.v_scales.view(c.num_pages, H, 4, 16).permute(0, 1, 3, 2)[pages, :, slots]
    grid = torch.tensor([0, .5, 1, 1.5, 2, 3, 4, 6], dtype=torch.float64, device="cuda")
    mag = grid[(codes & 7).long()]
    val = torch.where((codes & 8) != 0, -mag, mag)
    return val * torch.exp2(sc.double() - 127).repeat_interleave(32, dim=-1)


def bench_block_scales(api, torch, stream, w, data, scales, amax, q_np, sample=8, iters=3, dec_iters=10):
    """Configuration 4's data under three block-scale rules: NVFP4 with the
    amax/6 scale, NVFP4 with the MSE-searched scale, and MXFP4 (E8M0 per 32):
    bulk-append time of the whole cache, decode time, the quantization error
    of K and V, and the decode output's error against attention over the
    unquantized bf16 K/V (FP32, on the device), on a sample of sequences."""
    s_tk, s_tv = scales
    pt = torch.from_numpy(w.page_table).cuda()
    kd = torch.from_numpy(np.concatenate([d[0] for d in data])).to(torch.bfloat16).cuda()
    vd = torch.from_numpy(np.concatenate([d[1] for d in data])).to(torch.bfloat16).cuda()
    seq = torch.from_numpy(np.concatenate([np.full(int(L), b, np.int32) for b, L in enumerate(w.lens)])).cuda()
    pos = torch.from_numpy(np.concatenate([np.arange(int(L), dtype=np.int32) for L in w.lens])).cuda()
    ntok = kd.shape[0]
    res = {"workload": f"decode config 4 data ({ntok} tokens x {w.Hkv} heads); errors over sequences "
                       f"0..{sample - 1}"}
    caches = {}
    for name, put in (("amax6", api.append), ("mse", api.append_mse), ("mxfp4", api.mx_append)):
        if name == "mxfp4":
            c = api.MxCache(w.num_pages, w.Hkv, api.mx_exp_offset_from_amax(amax[0]),
                            api.mx_exp_offset_from_amax(amax[1]), fill=0)
            per_elem = 0.53125
        else:
            c = api.KVCache(w.num_pages, w.Hkv, s_tk, s_tv, fill=0)
            per_elem = 0.5625
        put(c, kd, vd, seq, pos, pt)
        torch.cuda.synchronize()
        t = time_region(torch, lambda: put(c, kd, vd, seq, pos, pt), iters, stream)
        caches[name] = c
        nbytes = ntok * w.Hkv * 128 * 2 * (2 + per_elem)
        res[name] = {"bulk_append_ms": round(t, 3), "bulk_append_gbs": round(nbytes / t / 1e6, 1)}
    del kd, vd, seq, pos
    torch.cuda.empty_cache()
    G = w.Hq // w.Hkv
    scale = 1.0 / np.sqrt(128.0)
    q = torch.from_numpy(q_np).to(torch.bfloat16).cuda()
    qf = q.float()
    refs = []
    for b in range(sample):
        k = torch.from_numpy(data[b][0]).cuda()
        v = torch.from_numpy(data[b][1]).cuda()
        o = torch.empty((w.Hq, 128), dtype=torch.float32, device="cuda")
        for h in range(w.Hkv):
            kh = k[:, h, :].contiguous()
            sc = torch.matmul(qf[b, h * G:(h + 1) * G], kh.t().contiguous()) * scale
            o[h * G:(h + 1) * G] = torch.matmul(torch.softmax(sc, dim=-1), v[:, h, :].contiguous())
        refs.append(o)
    ref = torch.stack(refs)
    lens = torch.from_numpy(w.lens.astype(np.int32)).cuda()
    L = int(w.lens.max())
    out = torch.empty((w.B, w.Hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, api.decode_workspace_bytes(w.B, w.Hq, w.Hkv, L)), dtype=torch.uint8, device="cuda")
    for name, c in caches.items():
        se = {"k": 0.0, "v": 0.0}
        sq = {"k": 0.0, "v": 0.0}
        for b in range(sample):
            Lb = int(w.lens[b])
            if name == "mxfp4":
                kh, vh = _mx_dequant_seq(torch, c, pt[b], Lb, 0), _mx_dequant_seq(torch, c, pt[b], Lb, 1)
            else:
                kh, vh = api.dequant(c, pt[b], 0, Lb)
            for nm, xh, x in (("k", kh, data[b][0]), ("v", vh, data[b][1])):
                xd = torch.from_numpy(x).cuda().double()
                se[nm] += float(((xh.double() - xd) ** 2).sum())
                sq[nm] += float((xd ** 2).sum())
        dec = api.mx_decode if name == "mxfp4" else api.decode
        dec(c, q, pt, lens, L, workspace=ws, out=out)
        torch.cuda.synchronize()
        d = out[:sample].double() - ref.double()
        t = time_region(torch, lambda: dec(c, q, pt, lens, L, workspace=ws, out=out), dec_iters, stream)
        nbytes = int(w.lens.sum()) * w.Hkv * 256 * (0.53125 if name == "mxfp4" else 0.5625)
        res[name].update({
            "rel_mse_k": se["k"] / sq["k"], "rel_mse_v": se["v"] / sq["v"],
            "decode_rel_l2_err": float(d.norm() / ref.double().norm()),
            "decode_us": round(t * 1e3, 2), "decode_gbs": round(nbytes / t / 1e6, 1),
        })
    for other in ("mse", "mxfp4"):
        for key in ("rel_mse_k", "rel_mse_v", "decode_rel_l2_err", "decode_us"):
            res[f"{other}_over_amax6_{key}"] = round(res[other][key] / res["amax6"][key], 4)
    res["mse_append_slowdown"] = round(res["mse"]["bulk_append_ms"] / res["amax6"]["bulk_append_ms"], 3)
    del caches
    torch.cuda.empty_cache()
    return res


def bench_to_fp8(api, torch, stream, rows=16384, cols=16384, iters=10):
    """NVFP4 -> FP8 conversion of a weight-sized [rows][cols] tensor of random
    NVFP4 bytes (block scales 0..126): HBM bytes 0.5 + 1/16 in and 1 out per
    element."""
    n = rows * cols
    gen = torch.Generator(device="cuda").manual_seed(7)
    codes = torch.randint(0, 256, (n // 2,), dtype=torch.uint8, device="cuda", generator=gen)
    scales = torch.randint(0, 127, (n // 16,), dtype=torch.uint8, device="cuda", generator=gen)
    out = torch.empty(n, dtype=torch.uint8, device="cuda")
    g = 2688.0 / 3.0
    s8 = 6.0 / g
    api.to_fp8(codes, scales, g, s8, out=out)
    torch.cuda.synchronize()
    t = time_region(torch, lambda: api.to_fp8(codes, scales, g, s8, out=out), iters, stream)
    nbytes = n * (0.5 + 1.0 / 16 + 1.0)
    res = {"workload": f"NVFP4 -> FP8 of a [{rows}][{cols}] tensor", "us": round(t * 1e3, 2),
           "gbs": round(nbytes / t / 1e6, 1), "frac_hbm_peak": round(nbytes / t / 1e6 / HBM_PEAK_GBS, 4)}
    del codes, scales, out
    torch.cuda.empty_cache()
    return res


def prefill_sweep(api, torch, stream, iters=5):
    """Cost of re-expanding the prefix at every chunk: the prefill call of a
    2048-token chunk (and of a 512-token one) after prefixes of 0 to 131072
    tokens, 64/8 heads, both operand modes, on caches of random bytes (E4M3
    block scales drawn from codes 1..126).  Each call runs expand_kernel over
    all prefix + chunk tokens, then fa_kernel; a kernel trace of this run
    splits the two (the configurations run in the printed order, `iters`
    calls each after one untimed call)."""
    Hq, Hkv = 64, 8
    gen = torch.Generator(device="cuda").manual_seed(11)
    rows = []
    for mode in (api.PREFILL_FP8, api.PREFILL_F16):
        for prefix, T in ((0, 2048), (4096, 2048), (16384, 2048), (32768, 2048), (65536, 2048), (131072, 2048),
                          (32768, 512)):
            total = prefix + T
            npages = -(-total // 16)
            cache = api.KVCache(npages, Hkv, 1.0 / 2688, 1.0 / 2688, fill=None)
            for t in (cache.k_codes, cache.v_codes):
                t.copy_(torch.randint(0, 256, t.shape, dtype=torch.uint8, device="cuda", generator=gen))
            for t in (cache.k_scales, cache.v_scales):
                t.copy_(torch.randint(1, 127, t.shape, dtype=torch.uint8, device="cuda", generator=gen))
            pt = torch.arange(npages, dtype=torch.int32, device="cuda")
            q = torch.randn((T, Hq, 128), device="cuda", generator=gen).to(torch.bfloat16)
            out = torch.empty((T, Hq, 128), dtype=torch.float32, device="cuda")
            ws = torch.empty(api.prefill_workspace_bytes(T, Hq, Hkv, prefix, mode), dtype=torch.uint8, device="cuda")

            def call():
                api.prefill(cache, q, pt, prefix, causal=True, workspace=ws, out=out, mode=mode, stream=stream)

            call()
            torch.cuda.synchronize()
            t = time_region(torch, call, iters, stream)
            flops = 4.0 * 128 * Hq * (T * prefix + T * (T + 1) / 2)
            exp_bytes = total * Hkv * 128 * 2 * (0.5625 + (1 if mode == api.PREFILL_FP8 else 2))
            rows.append({"mode": "fp8" if mode == api.PREFILL_FP8 else "f16", "prefix": prefix, "chunk": T,
                         "call_ms": round(t, 4), "tflops": round(flops / t / 1e9, 1),
                         "expand_bytes": int(exp_bytes)})
            del cache, ws, out, q
            torch.cuda.empty_cache()
    return {"workload": "chunk prefill after prefixes 0..131072 (64/8 heads), random cache bytes",
            "calls_per_config": iters + 1, "configs": rows}


def append_only(api, torch, stream, steps, warmup):
    """Configuration 4's bulk append alone: every token of the workload
    (594,571 x 8 KV heads, positions 0 .. L_b - 1 of each sequence) quantized
    into an NVFP4 cache and into an MXFP4 cache, from random bf16 K/V drawn on
    the device, so that profilers see the append kernels after a few seconds.
    Per-call HIP events on the launch stream: median, p10 and p90."""
    from decode_attention_nvfp4_amd import workloads as W
    w = W.decode_workload(4)
    ntok = int(w.lens.sum())
    gen = torch.Generator(device="cuda").manual_seed(7)
    kd = torch.randn((ntok, w.Hkv, 128), device="cuda", generator=gen).to(torch.bfloat16)
    vd = torch.randn((ntok, w.Hkv, 128), device="cuda", generator=gen).to(torch.bfloat16)
    seq = torch.from_numpy(np.concatenate([np.full(int(L), b, np.int32) for b, L in enumerate(w.lens)])).cuda()
    pos = torch.from_numpy(np.concatenate([np.arange(int(L), dtype=np.int32) for L in w.lens])).cuda()
    pt = torch.from_numpy(w.page_table).cuda()
    res = {"workload": f"bulk append of configuration 4's tokens ({ntok} x {w.Hkv} heads, bf16 in), random data",
           "calls": steps}
    for name in ("nvfp4", "mxfp4"):
        if name == "mxfp4":
            c, put, per_elem = api.MxCache(w.num_pages, w.Hkv, 0, 0, fill=0), api.mx_append, 0.53125
        else:
            c, put, per_elem = api.KVCache(w.num_pages, w.Hkv, 1.0 / 400, 1.0 / 400, fill=0), api.append, 0.5625
        for _ in range(max(1, warmup)):
            put(c, kd, vd, seq, pos, pt, stream=stream)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for s, e in ev:
            s.record(stream)
            put(c, kd, vd, seq, pos, pt, stream=stream)
            e.record(stream)
        torch.cuda.synchronize()
        t = np.array([s.elapsed_time(e) for s, e in ev]) * 1e3
        nbytes = ntok * w.Hkv * 128 * 2 * (2 + per_elem)
        res[name] = {"bytes": int(nbytes), "us_median": round(float(np.median(t)), 1),
                     "us_p10": round(float(np.percentile(t, 10)), 1), "us_p90": round(float(np.percentile(t, 90)), 1),
                     "tbs_median": round(nbytes / float(np.median(t)) / 1e6, 3)}
        del c
    return res


def decode_only(api, torch, stream, steps, warmup):
    """Configuration 4's decode call alone, on a cache of random bytes (block
    scales drawn from the finite E4M3 codes 0..126) filled on the device: the
    shape, page table and lengths of the workload without its data generation
    and appends, so that profilers see the decode kernels after a few seconds.
    Per-call HIP events on the launch stream; median, p10, p90 and mean."""
    from decode_attention_nvfp4_amd import workloads as W
    w = W.decode_workload(4)
    gen = torch.Generator(device="cuda").manual_seed(4)
    cache = api.KVCache(w.num_pages, w.Hkv, 1.0 / 2688, 1.0 / 2688, fill=None)
    for t in (cache.k_codes, cache.v_codes):
        t.copy_(torch.randint(0, 256, t.shape, dtype=torch.uint8, device="cuda", generator=gen))
    for t in (cache.k_scales, cache.v_scales):
        t.copy_(torch.randint(0, 127, t.shape, dtype=torch.uint8, device="cuda", generator=gen))
    pt = torch.from_numpy(w.page_table).cuda()
    lens = torch.from_numpy(w.lens.astype(np.int32)).cuda()
    L = int(w.lens.max())
    q = torch.randn((w.B, w.Hq, 128), device="cuda", generator=gen).to(torch.bfloat16)
    out = torch.empty((w.B, w.Hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, api.decode_workspace_bytes(w.B, w.Hq, w.Hkv, L)), dtype=torch.uint8, device="cuda")

    def call():
        api.decode(cache, q, pt, lens, L, workspace=ws, out=out, stream=stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for s, e in ev:
        s.record(stream)
        call()
        e.record(stream)
    torch.cuda.synchronize()
    t = np.array([s.elapsed_time(e) for s, e in ev]) * 1e3
    nbytes = int(w.lens.sum()) * w.Hkv * BYTES_PER_TOKEN_HEAD
    return {"workload": "decode config 4 shape (batch 128, 32/8 heads, U[1024,8192], permuted pages), "
                        "random cache bytes", "calls": steps, "cache_mb": round(nbytes / 1e6, 1),
            "us_mean": round(float(t.mean()), 2), "us_median": round(float(np.median(t)), 2),
            "us_p10": round(float(np.percentile(t, 10)), 2), "us_p90": round(float(np.percentile(t, 90)), 2),
            "tbs_median": round(nbytes / float(np.median(t)) / 1e6, 3),
            "splits": api.decode_num_splits(w.B, w.Hkv, L)}


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "decode_paged_b128_traffic.json")
DECODE_SOURCES = [os.path.join(ROOT, "decode_attention_nvfp4_amd", "csrc", f)
                  for f in ("decode.hip", "common.h", "internal.h", "api.cpp")]


def calibration_copy(torch, mib: int):
    """The device-to-device copy of `mib` MiB whose FETCH_SIZE and WRITE_SIZE
    scale a counter run's readings to bytes (ideal: mib MiB each way)."""
    src = torch.ones(mib << 18, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def sources_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def decode_traffic():
    """HBM bytes per decode call (decode_kernel + merge_kernel) from the
    committed counter record, or None when the kernels changed since."""
    try:
        with open(TRAFFIC_RECORD) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_digest():
        return None
    return rec.get("bytes_per_call")


def _pmc_per_kernel(d: str, counter: str):
    """{kernel name: [value per dispatch]} of one rocprofv3 --pmc csv run."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = {}
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            if r.get("Counter_Name") != counter:
                continue
            key = (r["Kernel_Name"], r.get("Dispatch_Id") or r.get("Correlation_Id"))
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return out


def write_traffic_record(fetch_dir: str, write_dir: str):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of decode_kernel and
    merge_kernel, each scaled by what the same counter reads for the plain
    device copy of --copy-mib MiB (ideal: that many MiB read and written)."""
    fetch = _pmc_per_kernel(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_kernel(write_dir, "WRITE_SIZE")

    def pick(table, part):
        vals = [v for k, vs in table.items() if part in k for v in vs]
        if not vals:
            raise SystemExit(f"no dispatch of {part} in the counter output")
        return float(np.median(vals))

    # the calibration copy is the largest device-to-device copy dispatch
    def largest(table, part):
        vals = [v for k, vs in table.items() if part in k for v in vs]
        if not vals:
            raise SystemExit(f"no dispatch of {part} in the counter output")
        return max(vals)

    copy_f, copy_w = largest(fetch, "copyBuffer"), largest(write, "copyBuffer")
    mib = int(os.environ.get("COPY_MIB", "512"))
    ideal_kib = mib * 1024.0
    fk, wk = ideal_kib / copy_f, ideal_kib / copy_w
    dec_f, dec_w = pick(fetch, "decode_kernel"), pick(write, "decode_kernel")
    mer_f, mer_w = pick(fetch, "merge_kernel"), pick(write, "merge_kernel")
    rec = {
        "workload": "paged decode, batch 128, 32/8 heads, context U[1024, 8192] (bench.py --decode-only)",
        "copy_mib": mib, "copy_fetch_kib": copy_f, "copy_write_kib": copy_w,
        "fetch_factor": fk, "write_factor": wk,
        "decode_kernel_kib": {"fetch": dec_f, "write": dec_w},
        "merge_kernel_kib": {"fetch": mer_f, "write": mer_w},
        "bytes_per_call": round(((dec_f + mer_f) * fk + (dec_w + mer_w) * wk) * 1024.0),
        "sources_sha256": sources_digest(),
    }
    with open(TRAFFIC_RECORD, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true", help="skip the secondary measurements")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed steps, copy this many MiB device to device three times "
                         "(the calibration kernel of the HBM traffic counters)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the chunked prefill (both operand modes) and print its record; "
                         "a profiling entry, not the benchmark line")
    ap.add_argument("--small-decode", action="store_true",
                    help="time only the decode of configurations 1-3 and print their record; a profiling "
                         "entry, not the benchmark line")
    ap.add_argument("--prefill-sweep", action="store_true",
                    help="time the prefill call over prefix lengths 0..131072 (expansion against attention; "
                         "split the two kernels with a kernel trace of this run)")
    ap.add_argument("--append-only", action="store_true",
                    help="time only configuration 4's bulk append (NVFP4 and MXFP4) on random data and print "
                         "its record; a profiling entry, not the benchmark line")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only configuration 4's decode call on a random-byte cache and print its "
                         "record; a profiling entry, not the benchmark line")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the decode traffic record from two rocprofv3 --pmc outputs "
                         "(FETCH_SIZE, then WRITE_SIZE) of a run with --copy-mib, then exit")
    args = ap.parse_args()
    if args.traffic_from:
        write_traffic_record(*args.traffic_from)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the NVFP4 KV hot path here is a "
              "single-GPU build and no multi-GPU run is defined.", file=sys.stderr)
        sys.exit(2)

    import torch
    from decode_attention_nvfp4_amd import api
    from decode_attention_nvfp4_amd import workloads as W

    api.lib()
    torch.cuda.init()
    stream = torch.cuda.current_stream()
    threads = host_threads()[0]
    if args.prefill_only:
        print(json.dumps({"prefill_cfg5": bench_prefill(api, torch, stream, iters=max(1, args.steps))}),
              flush=True)
        return
    if args.small_decode:
        rec = {"decode_cfg1": bench_cfg1(api, torch, stream)}
        for cfg in (2, 3):
            rec[f"decode_cfg{cfg}"] = bench_small_decode(api, torch, stream, cfg, iters=max(1, args.steps))
        print(json.dumps(rec), flush=True)
        return
    if args.prefill_sweep:
        print(json.dumps({"prefill_sweep": prefill_sweep(api, torch, stream, iters=max(1, args.steps))}), flush=True)
        return
    if args.append_only:
        rec = {"append_cfg4": append_only(api, torch, stream, max(1, args.steps), args.warmup)}
        if args.copy_mib:
            calibration_copy(torch, args.copy_mib)
            rec["copy_mib"] = args.copy_mib
        print(json.dumps(rec), flush=True)
        return
    if args.decode_only:
        rec = {"decode_cfg4": decode_only(api, torch, stream, max(1, args.steps), args.warmup)}
        if args.copy_mib:
            calibration_copy(torch, args.copy_mib)
            rec["copy_mib"] = args.copy_mib
        print(json.dumps(rec), flush=True)
        return

    # ---- workload: paged large-batch decode
    t0 = time.time()
    w = W.decode_workload(4)
    data = gen_decode(w, threads)
    log(f"generated {int(w.lens.sum())} tokens x {w.Hkv} heads in {time.time() - t0:.1f}s")
    s_tk, amax_k = device_scale(api, torch, [d[0] for d in data])
    s_tv, amax_v = device_scale(api, torch, [d[1] for d in data])

    # bulk append of the whole cache: timed (HIP events) as the append GB/s
    cache = api.KVCache(w.num_pages, w.Hkv, s_tk, s_tv, fill=0)
    pt = torch.from_numpy(w.page_table).cuda()
    kd = torch.from_numpy(np.concatenate([d[0] for d in data])).to(torch.bfloat16).cuda()
    vd = torch.from_numpy(np.concatenate([d[1] for d in data])).to(torch.bfloat16).cuda()
    seq = torch.from_numpy(np.concatenate([np.full(int(L), b, np.int32) for b, L in enumerate(w.lens)])).cuda()
    pos = torch.from_numpy(np.concatenate([np.arange(int(L), dtype=np.int32) for L in w.lens])).cuda()
    ntok = kd.shape[0]

    def bulk():
        api.append(cache, kd, vd, seq, pos, pt)

    # two warm-up calls, then the median of 7 calls timed one by one
    bulk(); bulk(); torch.cuda.synchronize()
    t_bulk = float(np.median(call_times(torch, bulk, 7, stream)))
    bulk_bytes = ntok * w.Hkv * 128 * 2 * (2 + 0.5625) + ntok * 8
    del kd, vd
    q_np = w.q(0)
    q = torch.from_numpy(q_np).to(torch.bfloat16).cuda()
    knew, vnew = w.append_kv(0)
    knew = torch.from_numpy(knew).to(torch.bfloat16).cuda()
    vnew = torch.from_numpy(vnew).to(torch.bfloat16).cuda()
    bidx = torch.arange(w.B, dtype=torch.int32, device="cuda")
    newpos = torch.from_numpy(w.lens.astype(np.int32)).cuda()          # append at position L_b
    lens1 = torch.from_numpy((w.lens + 1).astype(np.int32)).cuda()     # then attend L_b + 1 tokens
    Lmax = int(w.lens.max()) + 1
    out = torch.empty((w.B, w.Hq, 128), dtype=torch.float32, device="cuda")
    ws_bytes = api.decode_workspace_bytes(w.B, w.Hq, w.Hkv, Lmax)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def append_step():
        api.append(cache, knew, vnew, bidx, newpos, pt)

    def decode_step():
        api.decode(cache, q, pt, lens1, Lmax, workspace=ws, out=out)

    def step():
        append_step()
        decode_step()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps, synchronized on both sides
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    # per-call timing with HIP events on the launch stream: a second pass of
    # K steps, events around each append and each decode call, so every call
    # runs in the same context as in the timed steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for e in ev:
        e[0].record(stream)
        append_step()
        e[1].record(stream)
        e[2].record(stream)
        decode_step()
        e[3].record(stream)
    torch.cuda.synchronize()
    t_app = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    dec_calls = np.array([e[2].elapsed_time(e[3]) for e in ev]) * 1e3
    t_dec = float(np.mean(dec_calls)) * 1e-3
    # decode calls back to back (no append between them) run slower on the
    # boxes measured; reported for reference
    t_dec_b2b = None if args.no_extra else time_region(torch, decode_step, args.steps, stream)

    if args.copy_mib:
        calibration_copy(torch, args.copy_mib)

    cache_bytes = int((w.lens + 1).sum()) * w.Hkv * BYTES_PER_TOKEN_HEAD
    q_out_bytes = w.B * w.Hq * 128 * (2 + 4)
    app_bytes = w.B * w.Hkv * 128 * 2 * (2 + 0.5625)
    step_bytes = cache_bytes + q_out_bytes + app_bytes
    value = step_bytes / (ms_step * 1e-3) / 1e9
    achieved = cache_bytes / (t_dec * 1e-3) / 1e9

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded N(0,1) bf16 K/V/Q; no model weights)",
        "config": {
            "workload": "paged decode step: append 1 token/seq + decode attention; batch 128, 32 q / 8 kv "
                        "heads, head_dim 128, context U[1024,8192] (seeded), 16-token pages by seeded "
                        "permutation, NVFP4 cache",
            "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": 128,
            "total_context_tokens": int((w.lens + 1).sum()), "splits": api.decode_num_splits(w.B, w.Hkv, Lmax),
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": decode_traffic(),
            "kernel": "nvfp4 decode_kernel + merge_kernel (one nvfp4_decode_attn call)",
            "bytes_per_launch": cache_bytes, "avg_ms": round(t_dec, 5),
        },
        "extra": {
            "decode_ms": round(t_dec, 5), "decode_calls": pct(dec_calls), "append_step_us": round(t_app * 1e3, 2),
            "decode_back_to_back_ms": None if t_dec_b2b is None else round(t_dec_b2b, 5),
            "bulk_append": {"tokens": ntok, "ms": round(t_bulk, 3),
                            "gbs": round(bulk_bytes / (t_bulk * 1e-3) / 1e9, 1),
                            "frac_hbm_peak": round(bulk_bytes / (t_bulk * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "tensor_amax": {"k": amax_k, "v": amax_v},
        },
    }
    if not args.no_extra:
        try:
            res["extra"]["gather_ceiling"] = bench_gather_probe(api, torch, stream, cache, pt, lens1, Lmax,
                                                                float(np.median(dec_calls)))
        except Exception as e:  # noqa: BLE001
            res["extra"]["gather_ceiling"] = {"error": repr(e)}
        log(f"gather ceiling: {res['extra']['gather_ceiling']}")
        del cache
        torch.cuda.empty_cache()
        try:
            res["extra"]["decode_cfg1"] = bench_cfg1(api, torch, stream)
        except Exception as e:  # noqa: BLE001
            res["extra"]["decode_cfg1"] = {"error": repr(e)}
        log(f"decode config 1: {res['extra']['decode_cfg1']}")
        try:
            probe = stream_read_probe(api, torch, stream)
            probe["decode_frac"] = round(achieved / probe["gbs"], 4)
            res["extra"]["stream_read"] = probe
        except Exception as e:  # noqa: BLE001
            res["extra"]["stream_read"] = {"error": repr(e)}
        log(f"stream read: {res['extra']['stream_read']}")
        for cfg in (2, 3):
            try:
                res["extra"][f"decode_cfg{cfg}"] = bench_small_decode(api, torch, stream, cfg)
            except Exception as e:  # noqa: BLE001
                res["extra"][f"decode_cfg{cfg}"] = {"error": repr(e)}
            log(f"decode config {cfg}: {res['extra'][f'decode_cfg{cfg}']}")
        try:
            res["extra"]["kv_formats_cfg4"] = bench_formats_cfg4(api, torch, stream, w, data, (s_tk, s_tv),
                                                                 (amax_k, amax_v), q_np)
        except Exception as e:  # noqa: BLE001
            res["extra"]["kv_formats_cfg4"] = {"error": repr(e)}
        log(f"kv formats: {res['extra']['kv_formats_cfg4']}")
        try:
            res["extra"]["block_scales_cfg4"] = bench_block_scales(api, torch, stream, w, data, (s_tk, s_tv),
                                                                   (amax_k, amax_v), q_np)
        except Exception as e:  # noqa: BLE001
            res["extra"]["block_scales_cfg4"] = {"error": repr(e)}
        log(f"block scales: {res['extra']['block_scales_cfg4']}")
        try:
            res["extra"]["nvfp4_to_fp8"] = bench_to_fp8(api, torch, stream)
        except Exception as e:  # noqa: BLE001
            res["extra"]["nvfp4_to_fp8"] = {"error": repr(e)}
        log(f"nvfp4 -> fp8: {res['extra']['nvfp4_to_fp8']}")
        try:
            res["extra"]["prefill_cfg5"] = bench_prefill(api, torch, stream)
        except Exception as e:  # noqa: BLE001
            res["extra"]["prefill_cfg5"] = {"error": repr(e)}
        log(f"prefill: {res['extra']['prefill_cfg5']}")
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(w, data, s_tk, s_tv, q_np, threads)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
