"""Benchmark: latent-cache decode attention on one MI355X.

One step = one decode step of a looped model at the high-capacity point
(Ouro-1.4B shapes: T=4 loops x D=24 layers, H=16, d_head=128, r_k=16, r_v=32,
batch 768, context 4096, shuffled 16-token pages): append the new token's
latents for every layer (lla_encode_append), then run lla_decode_attn for every
(loop, layer) pair -- T*D = 96 calls, loop-major as the looped model issues
them, so consecutive calls read different layers' pools and the working set
(116 GB) never stays in the 256 MB last-level cache.

value = cached-token reads / s over the timed steps (one read = one token's
latents for one layer during one call: all 16 heads' c_k and c_v).  Inputs are
resident in HBM before timing starts.  The roofline object describes the decode
kernel, timed with HIP events on the stream it is launched on.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
DECODE_SOURCES = ("lla_decode_g.hip", "lla_device.h", "lla_internal.h", "lla_api.hip")
PREFILL_SOURCES = ("lla_prefill.hip", "lla_device.h", "lla_internal.h", "lla_api.hip")
ABSORBED_SOURCES = ("lla_absorbed.hip", "lla_merge.hip", "lla_device.h", "lla_internal.h", "lla_api.hip")
FULL_SOURCES = ("lla_full.hip", "lla_merge.hip", "lla_device.h", "lla_internal.h", "lla_api.hip")
D2D_SOURCES = ("lla_decode2d.hip", "lla_device.h", "lla_internal.h", "lla_api.hip")
HBM_BYTES = 288e9


def kernel_source_digest(names=DECODE_SOURCES) -> str:
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "looped_transformer_latent_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled_traffic(workload: str, kernel: str = "decode_g_kernel", sources=DECODE_SOURCES):
    """HBM bytes per decode launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary of this workload, or None when the kernel sources have
    changed since those counters were taken (or no summary exists)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.split(":", 1)[0] in ("kernel_source_sha256", "traffic_bytes_per_launch"):
                k, v = line.split(":", 1)
                fields[k] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_digest(sources):
        return None
    v = fields.get("traffic_bytes_per_launch")
    return int(v) if v else None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", default="ouro1.4b-21x-b768-paged",
                   help="decode workload: ouro1.4b-21x-b768-paged (default), ouro1.4b-21x-b32, "
                        "ouro1.4b-21x-b768-contig, lla2d-t8-h32-b128")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-full-cache", action="store_true", help="skip the full K/V cache baseline")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle sample time")
    p.add_argument("--calibrate-copy", type=float, default=0.0, metavar="GIB",
                   help="only run a plain device copy of GIB gibibytes, three times (a known "
                        "byte count for scaling the HBM traffic counters)")
    return p.parse_args()


def calibrate_copy(gib: float) -> None:
    import torch
    n = int(gib * 2 ** 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_launch": 4 * n,
                      "bytes_written_per_launch": 4 * n, "launches": 3}), flush=True)


def spread(ms) -> dict:
    """Median, p10 and p90 of per-launch times (ms) and how many there were."""
    a = np.asarray(ms, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "n": int(a.size)}


def cpu_baseline(w, codec_h, pt_h, layer, loop, target_s):
    """Time the fp64 oracle on a bounded sample of the same call: whole
    sequences (all heads, full context) of one (layer, loop), with every host
    thread it may use (OpenMP over (sequence, head)) and with one thread."""
    import oracle
    from looped_transformer_latent_amd import workloads as wl

    # the oracle sees one layer: that layer's codec slice and pool pages
    one = dict(w.dims, D=1)
    codec1 = {k: np.ascontiguousarray(v[layer:layer + 1]) for k, v in codec_h.items()}

    # latent pages of the first (up to) 4 sequences, regenerated on the host; longer
    # samples cycle through them (the oracle's cost does not depend on the values)
    n_data = min(4, w.batch)
    pages = pt_h[:n_data].reshape(-1)
    kp = wl.pool_pages_host(w, "k", layer, pages)[None]
    vp = wl.pool_pages_host(w, "v", layer, pages)[None]
    kr = wl.pool_pages_host(w, "kr", layer, pages)[None] if w.d_rope else None
    local = np.arange(len(pages), dtype=np.int32).reshape(n_data, -1)

    def run(n_seq, threads):
        pt_local = np.ascontiguousarray(local[np.arange(n_seq) % n_data])
        q = wl.q_host(w, n_seq)
        ctx = np.full(n_seq, w.ctx, np.int32)
        t0 = time.perf_counter()
        if w.d_rope:
            _, rc = oracle.decoupled_decode(one, codec1, kp, vp, kr, pt_local, 0, loop, q, ctx - 1, ctx, w.d_rope,
                                            threads=threads)
        else:
            _, rc = oracle.decode(one, codec1, kp, vp, pt_local, 0, loop, q, ctx - 1, ctx, threads=threads)
        dt = time.perf_counter() - t0
        assert rc == 0
        return dt

    threads = oracle.max_threads(0)       # the OpenMP default of this host (before any override)
    t1 = run(1, threads)
    n = int(max(1, min(w.batch, round(target_s / max(t1, 1e-3)))))
    dt = run(n, threads) if n > 1 else t1
    # one thread: whole sequences again, about a quarter of the time budget
    s1 = run(1, 1)
    n1 = int(max(1, min(w.batch, round(target_s / 4 / max(s1, 1e-3)))))
    dt1 = run(n1, 1) if n1 > 1 else s1
    oracle.max_threads(threads)           # restore the default for later oracle calls
    return {"value": n * w.ctx / dt, "unit": "cached-token reads/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {w.batch} sequences x full context {w.ctx} x all {w.H} heads, "
                      f"one (layer, loop) call (latent data of {n_data} sequences, reused); "
                      f"fp64 C oracle, OpenMP over (sequence, head), {threads} threads; {dt:.1f} s",
            "single_thread": {"value": n1 * w.ctx / dt1, "cores": 1,
                              "sample": f"{n1} sequences of the same call, 1 thread; {dt1:.1f} s"},
            "host_cpu": host_cpu()}


def host_cpu() -> str:
    """CPU model of this host and the logical CPUs it reports."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model}; {os.cpu_count()} logical CPUs visible"


def cpu_prefill_baseline(w, codec_h, pt_h, layer, loop, n_new, target_s):
    """Time the fp64 oracle's causal prefill on a bounded sample: the first
    queries of one sequence's chunk (all heads), each over its full causal
    context p0 + i + 1."""
    import oracle
    from looped_transformer_latent_amd import gen
    from looped_transformer_latent_amd import workloads as wl

    one = dict(w.dims, D=1)
    codec1 = {k: np.ascontiguousarray(v[layer:layer + 1]) for k, v in codec_h.items()}
    pages = pt_h[0]
    kp = wl.pool_pages_host(w, "k", layer, pages)[None]
    vp = wl.pool_pages_host(w, "v", layer, pages)[None]
    local = np.arange(len(pages), dtype=np.int32)[None]
    p0 = np.array([w.ctx - n_new], np.int32)

    def run(n_q):
        q = gen.normal(w.seed, wl.STREAMS["q"], (1, n_q, w.H, w.d_head),
                       dtype="bf16" if w.dtype == wl.BF16 else "f32")
        t0 = time.perf_counter()
        _, rc = oracle.prefill(one, codec1, kp, vp, local, 0, loop, n_q, q, p0)
        dt = time.perf_counter() - t0
        assert rc == 0
        return dt

    threads = oracle.max_threads(0)
    t1 = run(1)
    n = int(max(1, min(n_new, round(target_s / max(t1, 1e-3)))))
    dt = run(n) if n > 1 else t1
    return {"value": n / dt, "unit": "prefill query tokens/s (all heads)", "cores": threads, "kind": "oracle",
            "sample": f"queries 0..{n - 1} of one sequence's {n_new}-token chunk at positions "
                      f"{w.ctx - n_new}.., all {w.H} heads, one (layer, loop); fp64 C oracle, "
                      f"OpenMP over (query, head); {dt:.1f} s"}


def bench_window(w, D, codec, cache, rope, calls, q, q_pos, ctx, codec_h, pt_h, stream, n_sink=4, window=256,
                 cpu_s=0.0):
    """Token eviction composed with LLA: every (loop, layer) call of the step
    attends over a 4-token sink plus the last 256 tokens (lla_decode_window_attn),
    timed with HIP events; roofline on the retained tokens' latent bytes."""
    import torch
    from looped_transformer_latent_amd import lla

    out = torch.empty((len(calls), w.batch, w.H, w.d_head), dtype=q.dtype, device="cuda")
    ws = lla.workspace(D, lla.OP_WINDOW_DECODE, w.batch, w.ctx, n_sink + window)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]

    def one_pass(record):
        for i, (t, l) in enumerate(calls):
            if record:
                ev[i][0].record(stream)
            lla.decode_window_attn(D, codec, cache, rope, l, t, q[i], q_pos, ctx, n_sink, window, w.ctx, out[i], ws)
            if record:
                ev[i][1].record(stream)

    one_pass(False)
    torch.cuda.synchronize()
    ms = []
    for _ in range(2):
        one_pass(True)
        torch.cuda.synchronize()
        ms += [a.elapsed_time(b) for a, b in ev]
    assert lla.device_error_word(ws) == 0
    assert torch.isfinite(out.float()).all().item()
    avg = float(np.mean(ms))
    kept = min(w.ctx, n_sink + window)
    nbytes = w.batch * kept * w.read_bytes()
    gbs = nbytes / (avg / 1e3) / 1e9
    res = {"kernel": "decode_g_kernel (eviction)", "n_sink": n_sink, "window": window, "calls": len(calls),
           "avg_ms": avg, "call_ms": spread(ms), "value": w.batch * kept / (avg / 1e3), "unit": "retained-token reads/s",
           "retained_latent_bytes_per_sequence_all_layers": kept * w.read_bytes() * w.D,
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS,
                        "traffic": profiled_traffic(w.name + "-window", "decode_g_kernel"),
                        "traffic_unit": "HBM bytes per launch (rocprofv3)", "algorithmic_bytes_per_launch": nbytes}}
    if cpu_s > 0:
        import oracle
        from looped_transformer_latent_amd import workloads as wl
        layer, loop = calls[-1][1], calls[-1][0]
        one = dict(w.dims, D=1)
        codec1 = {k: np.ascontiguousarray(v[layer:layer + 1]) for k, v in codec_h.items()}
        n_data = min(4, w.batch)
        pages = pt_h[:n_data].reshape(-1)
        kp = wl.pool_pages_host(w, "k", layer, pages)[None]
        vp = wl.pool_pages_host(w, "v", layer, pages)[None]
        local = np.arange(len(pages), dtype=np.int32).reshape(n_data, -1)

        def run(n_seq):
            pt_local = np.ascontiguousarray(local[np.arange(n_seq) % n_data])
            qh = wl.q_host(w, n_seq)
            c = np.full(n_seq, w.ctx, np.int32)
            t0 = time.perf_counter()
            _, rc = oracle.decode_window(one, codec1, kp, vp, pt_local, 0, loop, qh, c - 1, c, n_sink, window)
            assert rc == 0
            return time.perf_counter() - t0

        t1 = run(1)
        n = int(max(1, min(w.batch, round(cpu_s / max(t1, 1e-3)))))
        dt = run(n) if n > 1 else t1
        res["cpu_baseline"] = {"value": n * kept / dt, "unit": "retained-token reads/s",
                               "cores": oracle.max_threads(0), "kind": "oracle",
                               "sample": f"{n} of {w.batch} sequences x {kept} retained tokens x all {w.H} heads, "
                                         f"one (layer, loop) call; fp64 C oracle; {dt:.1f} s"}
    return res


def cpu_encode_baseline(w, codec_h, layer, target_s):
    """Time the fp64 oracle's encode + append on a bounded sample: tokens of one
    layer (all heads), drawn from the same generator streams as the GPU's x."""
    import oracle
    from looped_transformer_latent_amd import gen
    from looped_transformer_latent_amd import workloads as wl

    one = dict(w.dims, D=1)
    codec1 = {k: np.ascontiguousarray(v[layer:layer + 1]) for k, v in codec_h.items()}
    inner = (w.H, w.T, w.d_head) if w.variant == wl.PER_HEAD else (w.T, w.H, w.d_head)

    def run(n_tok):
        pages = (n_tok + 15) // 16
        shp = (1, 1, n_tok) + inner
        xk = gen.normal(w.seed, wl.STREAMS["x_k"], shp)
        xv = gen.normal(w.seed, wl.STREAMS["x_v"], shp)
        kp = np.zeros((1, pages) + w.pool_shape("k")[2:], np.uint16)
        vp = np.zeros((1, pages) + w.pool_shape("v")[2:], np.uint16)
        pt = np.arange(pages, dtype=np.int32)[None]
        t0 = time.perf_counter()
        rc = oracle.encode(one, codec1, kp, vp, pt, xk, xv, np.zeros(1, np.int32), n_tok, 0, 1)
        dt = time.perf_counter() - t0
        assert rc == 0
        return dt

    t1 = run(16)
    n = int(max(16, min(1 << 16, round(16 * target_s / max(t1, 1e-4)))))
    dt = run(n)
    return {"value": n / dt, "unit": "appended token-layers/s (all heads)", "cores": 1, "kind": "oracle",
            "sample": f"{n} tokens of one layer, all {w.H} heads; fp64 C oracle, whose encode is a serial "
                      f"loop (1 thread is all it uses); {dt:.1f} s"}


def bench_prefill(w, D, codec, cache, rope, calls, n_new, dt_t, p0, stream):
    """lla_prefill_attn over every (loop, layer) of the step, timed with HIP
    events on the launch stream; roofline against the bf16 matrix-core peak."""
    import torch
    from looped_transformer_latent_amd import lla
    from looped_transformer_latent_amd import workloads as wl

    q = torch.empty((w.batch, n_new, w.H, w.d_head), dtype=dt_t, device="cuda")
    lla.gen_normal_(q, w.seed, wl.STREAMS["q"], offset=1 << 40)
    out = torch.empty_like(q)
    ws = lla.workspace(D, lla.OP_PREFILL, w.batch, w.ctx, n_new)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]

    def one_pass(record):
        for i, (t, l) in enumerate(calls):
            if record:
                ev[i][0].record(stream)
            lla.prefill_attn(D, codec, cache, rope, l, t, n_new, q, p0, w.ctx, out, ws)
            if record:
                ev[i][1].record(stream)

    one_pass(False)
    torch.cuda.synchronize()
    ms = []
    for _ in range(2):
        one_pass(True)
        torch.cuda.synchronize()
        ms += [a.elapsed_time(b) for a, b in ev]
    assert lla.device_error_word(ws) == 0
    assert torch.isfinite(out.float()).all().item()
    avg = float(np.mean(ms))
    # algorithmic work per call: K rebuilt once per cached token and head
    # (2 d r_k), scores and latent-space value sums per (query, key) pair
    # (2 d + 2 r_v), one up-projection per query and head (2 r_v d)
    keys = float(np.sum(np.arange(w.ctx - n_new, w.ctx) + 1))
    flops = w.batch * w.H * (w.ctx * 2.0 * w.d_head * w.r_k + keys * 2.0 * (w.d_head + w.r_v)
                             + n_new * 2.0 * w.r_v * w.d_head)
    tflops = flops / (avg / 1e3) / 1e12
    return {"kernel": "prefill_kernel", "calls": len(calls), "queries_per_call": w.batch * n_new,
            "positions": [w.ctx - n_new, w.ctx - 1], "avg_ms": avg, "call_ms": spread(ms),
            "value": w.batch * n_new / (avg / 1e3), "unit": "prefill query tokens/s (all heads, one (loop, layer))",
            "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                         "traffic": profiled_traffic(w.name, "prefill_kernel", PREFILL_SOURCES),
                         "traffic_unit": "HBM bytes per launch (rocprofv3)",
                         "algorithmic_flops_per_launch": flops}}


def bench_full_cache(w, D, codec, cache, rope, calls, q, q_pos, ctx, out_lat, lat_ms, stream):
    """The full-memory baseline on the same step: each (loop, layer) call's K/V
    rebuilt as a full bf16 cache (lla_reconstruct_kv) and attended by a plain
    decode over it (lla_full_decode_attn), against the latent decode's time.
    One (loop, layer) slice of the full cache is resident at a time; the whole
    model's full cache is reported with whether it would fit in HBM."""
    import torch
    from looped_transformer_latent_amd import lla
    from looped_transformer_latent_amd import workloads as wl

    sub = list(range(len(calls)))[-4:]            # the last four (loop, layer) calls of the step
    shape = (w.num_pages, w.H, wl.PAGE, w.d_head)
    kf = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    vf = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    ws_r = lla.workspace(D, lla.OP_RECONSTRUCT, w.batch, w.ctx)
    ws_f = lla.workspace(D, lla.OP_FULL_DECODE, w.batch, w.ctx)
    out = torch.empty_like(out_lat[0])
    mk = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    ev = [(mk(), mk()) for _ in sub]
    rel = 0.0

    def one_pass(record):
        nonlocal rel
        for j, i in enumerate(sub):
            t, l = calls[i]
            if record:
                ev[j][0][0].record(stream)
            lla.reconstruct_kv(D, codec, cache, rope, l, t, ctx, w.ctx, kf, vf, ws_r)
            if record:
                ev[j][0][1].record(stream)
                ev[j][1][0].record(stream)
            lla.full_decode_attn(D, cache, kf, vf, rope, q[i], q_pos, ctx, w.ctx, out, ws_f)
            if record:
                ev[j][1][1].record(stream)
            # same query, same latents: the two paths agree to bf16 rounding
            a, b = out.float(), out_lat[i].float()
            rel = max(rel, ((a - b).abs().amax(-1) / b.abs().amax(-1)).max().item())

    one_pass(False)
    torch.cuda.synchronize()
    rec_ms, full_ms = [], []
    for _ in range(2):
        one_pass(True)
        torch.cuda.synchronize()
        rec_ms += [r[0].elapsed_time(r[1]) for r, _ in ev]
        full_ms += [f[0].elapsed_time(f[1]) for _, f in ev]
    assert lla.device_error_word(ws_r) == 0 and lla.device_error_word(ws_f) == 0
    assert rel < 2e-2, rel
    rec, full = float(np.mean(rec_ms)), float(np.mean(full_ms))
    tokens = w.batch * w.ctx
    full_bytes = tokens * w.H * w.d_head * 2 * 2          # K and V, bf16, one (loop, layer)
    lat_bytes = tokens * w.groups * (w.r_k + w.r_v) * w.esize   # the rebuild reads c_k, c_v
    gbs = full_bytes / (full / 1e3) / 1e9
    whole = tokens * w.D * w.T * w.H * w.d_head * 2 * 2    # every layer's per-loop K/V
    return {"kernels": ["reconstruct_kernel", "full_decode_kernel"], "calls": len(sub),
            "latent_decode_ms": lat_ms, "full_decode_ms": full, "reconstruct_ms": rec,
            "reconstruct_then_attend_ms": rec + full,
            "latent_speedup_vs_full_decode": full / lat_ms,
            "latent_speedup_vs_reconstruct_then_attend": (rec + full) / lat_ms,
            "reconstruct_gbs": (full_bytes + lat_bytes) / (rec / 1e3) / 1e9,
            "bytes_per_token_per_call": {"full": w.H * w.d_head * 4, "latent": w.groups * (w.r_k + w.r_v) * w.esize},
            "full_cache_bytes_whole_model": whole, "full_cache_fits_hbm": whole <= HBM_BYTES,
            "max_row_rel_diff_vs_latent_decode": rel,
            "roofline": {"kernel": "full_decode_kernel", "bound": "hbm", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "traffic": profiled_traffic(w.name, "full_decode_kernel", FULL_SOURCES),
                         "traffic_unit": "HBM bytes per launch (rocprofv3)",
                         "algorithmic_bytes_per_launch": full_bytes},
            "cpu_baseline": "the oracle's decode is this same reconstruct-then-attend: see cpu_baseline"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU only; run with --gpus 1"}))
        sys.exit(2)
    if args.calibrate_copy > 0:
        calibrate_copy(args.calibrate_copy)
        return
    import torch

    from looped_transformer_latent_amd import lla
    from looped_transformer_latent_amd import workloads as wl

    w = wl.WORKLOADS[args.workload]
    dev = "cuda"
    torch.cuda.set_device(0)
    D = lla.dims_from_dict(w.dims)
    dt_t = torch.bfloat16 if w.dtype == wl.BF16 else torch.float32

    codec_h = wl.codec_host(w)
    codec_d = {k: wl.to_device(v, dev) for k, v in codec_h.items()}
    codec = lla.make_codec(codec_d["mu_k"], codec_d["mu_v"], codec_d["w_down_k"],
                           codec_d["w_down_v"], codec_d["w_up_k"], codec_d["w_up_v"])
    pt_h = wl.page_table_host(w)
    pt = wl.to_device(pt_h, dev)
    k_pool = wl.device_pool(w, "k", dev)
    v_pool = wl.device_pool(w, "v", dev)
    cache = lla.make_cache(k_pool, v_pool, pt, w.num_pages)
    rope = lla.rope_table(D, w.ctx)

    decoupled = w.d_rope > 0
    calls = [(t, l) for t in range(w.T) for l in range(w.D)]
    q = torch.empty((len(calls), w.batch, w.H, w.q_width), dtype=dt_t, device=dev)
    lla.gen_normal_(q, w.seed, wl.STREAMS["q"])
    out = torch.empty((len(calls), w.batch, w.H, w.d_head), dtype=dt_t, device=dev)
    if decoupled:
        # rotary keys of every cached token (stored rotated), the RoPE table of the
        # d_rope-wide branch, and the step's new rotary keys
        kr_pool = wl.device_pool(w, "kr", dev)
        rope_r = lla.rope_table(lla.dims_from_dict(dict(w.dims, d_head=w.d_rope)), w.ctx)
        x_r = torch.empty((w.D, w.batch, max(1, w.n_new), w.d_rope), dtype=dt_t, device=dev)
        lla.gen_normal_(x_r, w.seed, wl.STREAMS["x_r"])
        ws_app = lla.workspace(D, lla.OP_ROPE_KEY_APPEND, w.batch, 0)
        ws_dec = lla.workspace(D, lla.OP_DECOUPLED_DECODE, w.batch, w.ctx, w.d_rope)
    ctx = torch.full((w.batch,), w.ctx, dtype=torch.int32, device=dev)
    q_pos = ctx - 1
    if not decoupled:
        ws_dec = lla.workspace(D, lla.OP_DECODE, w.batch, w.ctx)
    # the step's new token: its per-loop K/V for every layer, appended at ctx - 1
    # the step's new tokens: one per sequence for a decode step; workloads that
    # name an append chunk (the 4x point: 512 tokens per sequence) append it
    n_new = max(1, w.n_new)
    xs = (w.D, w.batch, n_new) + ((w.H, w.T, w.d_head) if w.variant == wl.PER_HEAD else (w.T, w.H, w.d_head))
    x_k = torch.empty(xs, dtype=dt_t, device=dev)
    x_v = torch.empty(xs, dtype=dt_t, device=dev)
    lla.gen_normal_(x_k, w.seed, wl.STREAMS["x_k"])
    lla.gen_normal_(x_v, w.seed, wl.STREAMS["x_v"])
    pos0 = ctx - n_new
    ws_enc = lla.workspace(D, lla.OP_ENCODE, w.batch, 0, w.D)
    stream = torch.cuda.current_stream()
    # one set of events per timed step: the steps run back to back (as in a
    # serving loop) and are synchronised only at the ends of the timed region
    def mk_events():
        return ([(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls],
                (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
    step_events = [mk_events() for _ in range(args.steps)]
    ev, ev_enc = step_events[0]

    def step(record):
        if record:
            ev_enc[0].record(stream)
        lla.encode_append(D, codec, cache, x_k, x_v, pos0, n_new, 0, w.D, ws_enc)
        if decoupled:
            lla.rope_key_append(D, cache, kr_pool, rope_r, x_r, pos0, n_new, 0, w.D, ws_app)
        if record:
            ev_enc[1].record(stream)
        for i, (t, l) in enumerate(calls):
            if record:
                ev[i][0].record(stream)
            if decoupled:
                lla.decoupled_decode_attn(D, codec, cache, kr_pool, rope_r, l, t, q[i], q_pos, ctx, w.ctx,
                                          out[i], ws_dec)
            else:
                lla.decode_attn(D, codec, cache, rope, l, t, q[i], q_pos, ctx, w.ctx, out[i], ws_dec)
            if record:
                ev[i][1].record(stream)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    kern_ms, enc_ms = [], []
    t0 = time.perf_counter()
    for k in range(args.steps):
        ev, ev_enc = step_events[k]
        step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    for evs, enc in step_events:
        kern_ms += [a.elapsed_time(b) for a, b in evs]
        enc_ms.append(enc[0].elapsed_time(enc[1]))
    assert lla.device_error_word(ws_dec) == 0 and lla.device_error_word(ws_enc) == 0
    assert not decoupled or lla.device_error_word(ws_app) == 0
    assert torch.isfinite(out.float()).all().item()

    ms_step = 1e3 * elapsed / args.steps
    reads_per_step = len(calls) * w.batch * w.ctx
    value = reads_per_step / (ms_step / 1e3)
    kern_avg_ms = float(np.mean(kern_ms))
    bytes_per_launch = w.batch * w.ctx * w.read_bytes()
    if w.variant == wl.PER_HEAD:
        achieved = bytes_per_launch / (kern_avg_ms / 1e3) / 1e9
        kname = "decode_g_kernel" if w.dtype == wl.BF16 else "decode_ph_kernel"
        if decoupled:
            kname = "absorbed_kernel"
        roof = {"kernel": kname, "bound": "hbm", "achieved": achieved,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                "traffic": profiled_traffic(w.name, kname, ABSORBED_SOURCES if decoupled else DECODE_SOURCES), "traffic_unit": "HBM bytes per launch (rocprofv3)",
                "algorithmic_bytes_per_launch": bytes_per_launch, "avg_launch_ms": kern_avg_ms,
                "launch_ms": spread(kern_ms)}
    else:
        # LLA-2D is bound by the matrix cores: per token and head, rebuilding K is
        # 2 d r_k FLOP and the latent-space value sum 2 r_v FLOP
        flops = w.batch * w.ctx * w.H * (2 * w.d_head * w.r_k + 2 * w.r_v)
        achieved = flops / (kern_avg_ms / 1e3) / 1e12
        roof = {"kernel": "decode_2d_kernel", "bound": "mfma", "achieved": achieved,
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                "traffic": profiled_traffic(w.name, "decode_2d_kernel", D2D_SOURCES),
                "traffic_unit": "HBM bytes per launch (rocprofv3)", "algorithmic_flops_per_launch": flops,
                "algorithmic_bytes_per_launch": bytes_per_launch,
                "hbm_gbs": bytes_per_launch / (kern_avg_ms / 1e3) / 1e9, "avg_launch_ms": kern_avg_ms,
                "launch_ms": spread(kern_ms)}
    result = {
        "metric": "latent-cache decode attention: cached-token reads/s and achieved HBM GB/s",
        "value": value,
        "unit": "cached-token reads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == wl.BF16 else "f32",
        "data": "synthetic (seeded generator; random codec parameters, N(0,1) latents)",
        "config": {"workload": w.name, "batch": w.batch, "ctx": w.ctx, "T": w.T, "D": w.D,
                   "H": w.H, "d_head": w.d_head, "r_k": w.r_k, "r_v": w.r_v, "page_size": 16,
                   "page_table": "shuffled" if w.shuffled else "identity",
                   "step": (f"encode_append({n_new} token(s) per sequence x {w.D} layers) + " +
                            (f"rope_key_append (d_rope {w.d_rope}) + {len(calls)} lla_decoupled_decode_attn calls"
                             if decoupled else f"{len(calls)} lla_decode_attn calls"))},
        "roofline": roof,
    }
    # encode + append of the step's tokens into every layer (HBM-bound GEMM):
    # reads x_k, x_v and W_down, writes the latents
    enc_avg = float(np.mean(enc_ms))
    tok = w.batch * n_new * w.D
    width = w.T * w.d_head * (w.H if w.variant == wl.TWO_D else 1)
    enc_bytes = (tok * w.groups * width * 2 * w.esize + tok * w.groups * (w.r_k + w.r_v) * w.esize
                 + w.D * w.groups * width * (w.r_k + w.r_v) * w.esize)
    enc_flops = 2 * tok * w.groups * width * (w.r_k + w.r_v)
    result["encode"] = {"kernel": "encode_mfma_kernel", "tokens_per_layer": w.batch * n_new,
                        "layers": w.D, "avg_ms": enc_avg, "call_ms": spread(enc_ms),
                        "value": tok / (enc_avg / 1e3), "unit": "appended token-layers/s (all heads)",
                        "algorithmic_bytes": enc_bytes,
                        "achieved_gbs": enc_bytes / (enc_avg / 1e3) / 1e9,
                        "frac_hbm": enc_bytes / (enc_avg / 1e3) / 1e9 / HBM_PEAK_GBS,
                        "tflops": enc_flops / (enc_avg / 1e3) / 1e12}
    # causal prefill of the appended chunk: its n_new queries at positions
    # ctx - n_new .. ctx - 1 attend over the cache, one call per (loop, layer)
    if n_new > 1 and lla.supported(D, lla.OP_PREFILL):
        result["prefill"] = bench_prefill(w, D, codec, cache, rope, calls, n_new, dt_t, pos0, stream)
    # token eviction on top of the latent cache: sink 4 + window 256 per call
    if not decoupled and w.ctx > 260 and lla.supported(D, lla.OP_WINDOW_DECODE):
        result["window"] = bench_window(w, D, codec, cache, rope, calls, q, q_pos, ctx, codec_h, pt_h, stream,
                                        cpu_s=0.0 if args.no_cpu_baseline else args.cpu_seconds / 4)
    # the full-memory baseline of the same calls (per-head bf16 shapes it covers)
    full_ok = lla.supported(D, lla.OP_RECONSTRUCT) and lla.supported(D, lla.OP_FULL_DECODE)
    if decoupled:
        # the pages' comparison set for the absorbed kernel: the full-RoPE latent
        # decode, the full-cache ("teacher") decode and reconstruct-then-attend,
        # all with the content part of the same queries
        qc = q[..., :w.d_head].contiguous()
        out_fr = torch.empty_like(out)
        ws_fr = lla.workspace(D, lla.OP_DECODE, w.batch, w.ctx)
        evf = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
        for rep_ in range(2):
            for i, (t, l) in enumerate(calls):
                evf[i][0].record(stream)
                lla.decode_attn(D, codec, cache, rope, l, t, qc[i], q_pos, ctx, w.ctx, out_fr[i], ws_fr)
                evf[i][1].record(stream)
            torch.cuda.synchronize()
        assert lla.device_error_word(ws_fr) == 0
        fr_ms = float(np.mean([a_.elapsed_time(b_) for a_, b_ in evf]))
        result["full_rope_latent_decode"] = {
            "kernel": "decode_g_kernel", "avg_ms": fr_ms, "bytes_per_launch": w.batch * w.ctx * w.groups * (w.r_k + w.r_v) * w.esize,
            "absorbed_speedup": fr_ms / kern_avg_ms}
        if not args.no_full_cache and full_ok:
            fc = bench_full_cache(w, D, codec, cache, rope, calls, qc, q_pos, ctx, out_fr, fr_ms, stream)
            fc["absorbed_ms"] = kern_avg_ms
            fc["absorbed_speedup_vs_full_decode"] = fc["full_decode_ms"] / kern_avg_ms
            fc["absorbed_speedup_vs_reconstruct_then_attend"] = fc["reconstruct_then_attend_ms"] / kern_avg_ms
            result["full_cache"] = fc
    elif not args.no_full_cache and full_ok:
        result["full_cache"] = bench_full_cache(w, D, codec, cache, rope, calls, q, q_pos, ctx, out,
                                                kern_avg_ms, stream)
    if not args.no_cpu_baseline:
        if "prefill" in result:
            result["prefill"]["cpu_baseline"] = cpu_prefill_baseline(
                w, codec_h, pt_h, w.D - 1, w.T - 1, n_new, target_s=args.cpu_seconds / 3)
        result["cpu_baseline"] = cpu_baseline(w, codec_h, pt_h, layer=w.D - 1, loop=w.T - 1,
                                              target_s=args.cpu_seconds)
        if n_new > 1:
            result["encode"]["cpu_baseline"] = cpu_encode_baseline(w, codec_h, w.D - 1,
                                                                   target_s=args.cpu_seconds / 3)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
