"""Paged decode attention benchmark on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
the copy-on-write block copies (if the workload has any), the cache writes of
the step's new tokens, then paged decode (partition kernel + log-sum-exp
merge). Inputs are resident in HBM before the timed region starts.

Prints ONE JSON line. `value` is K+V GB/s: the algorithmic bytes one decode
must read (2 * ctx * Hkv * D * element size, summed over the batch) divided
by the measured time per step (the timed steps carry no events between their
kernels). `roofline` reports the partition kernel alone -- its average
duration over the same number of back-to-back launches, between two HIP
events on the launch stream -- against the 8 TB/s MI355X HBM peak. `cpu_baseline` is the
float64 CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

METRIC = "paged decode attention: KV GB/s read (% of HBM peak), seqs/sec"
HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCE = os.path.join(ROOT, "paged_kv_cache_165_amd", "csrc", "pa_decode.hip")
PREFILL_SOURCE = os.path.join(ROOT, "paged_kv_cache_165_amd", "csrc", "pa_prefill.hip")
PREFILL_KERNELS = ("pa_prefill_mfma", "pa_prefill_f32")
PARTITION_KERNELS = ("pa_decode_stream", "pa_decode_mfma", "pa_decode_valu")
PLAN_KERNELS = {"valu": "pa_decode_valu", "mfma": "pa_decode_mfma", "mfma_wave": "pa_decode_mfma_wave",
                "mfma_stream": "pa_decode_stream"}
CALIBRATION_KERNEL = "neg_kernel"  # torch's elementwise negate: reads N bytes, writes N bytes


def kernel_source_hash(path: str = KERNEL_SOURCE) -> str:
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


WARMUP_MIN_S = 0.25  # warm-up runs at least this long, whatever --warmup says


def warm_up(step, count: int) -> int:
    """Run `step` `count` times, then on until WARMUP_MIN_S has passed (the
    GPU's clocks settle under sustained load: right after set-up the same
    launches run up to 15 % slower). Returns the steps run."""
    import torch
    n = 0
    t0 = time.perf_counter()
    while n < count or time.perf_counter() - t0 < WARMUP_MIN_S:
        step()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def progress(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="gqa8b",
                    choices=["tiny", "layout", "mha7b", "gqa8b", "prefix", "long"])
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--tp", type=int, default=1,
                    help="time one GPU's shard of the workload split by KV head over this many GPUs: the same "
                         "sequences, contexts and block tables with num_heads / N query and num_kv_heads / N "
                         "KV heads")
    ap.add_argument("--block-size", type=int, default=None,
                    help="page the gqa8b sequences with this block size instead of 16 (block-size sweep)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--engine-steps", type=int, default=0,
                    help="instead of the headline line, drive the workload's sequences through the "
                         "multi-step decoder (native block manager + the three device calls) for this "
                         "many steps and report host and device time per step")
    ap.add_argument("--engine-layers", type=int, default=1,
                    help="with --engine-steps: caches of this many layers sharing one block table per "
                         "sequence; each step runs the block manager, tables and copies once and each "
                         "layer's write + decode")
    ap.add_argument("--prefill", choices=["prompts", "chunked"], default=None,
                    help="instead of the headline line, time paged prefill attention (cache write of the "
                         "new tokens + pa_prefill) on this workload and print its own line")
    ap.add_argument("--cache-layers", type=int, default=0,
                    help="instead of the headline line, time the decode step's cache write (256 scattered "
                         "tokens) and 192 copy-on-write block copies for this many layers: one layered launch "
                         "against one launch per layer")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target duration of the all-core CPU oracle sample (the one-thread samples take half "
                         "and a quarter of it)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="counter-derived HBM bytes per partition-kernel launch, if measured")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="after timing, run a plain N-MB elementwise copy (torch negate) so that "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE can be scaled to bytes")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of a run with "
                         "--copy-calibration-mb into --traffic-json, then exit")
    return ap.parse_args()


def _counter_rows(path, counter):
    """(kernel name, value in KiB) per dispatch from a rocprofv3 counter CSV."""
    import csv
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") != counter:
                continue
            key = r.get("Dispatch_Id") or r.get("Correlation_Id")
            name = r.get("Kernel_Name", "")
            per.setdefault(key, [name, 0.0])[1] += float(r["Counter_Value"])
    return list(per.values())


def resolved_partition(w) -> int:
    """Tokens per partition the decode of workload ``w`` runs with."""
    import torch
    import paged_kv_cache_165_amd as pa
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    return w.partition_size or pa.default_partition_size(w.num_seqs, w.num_heads, w.num_kv_heads,
                                                         w.max_context_len, w.block_size, dt)


def summarize_counters(fetch_csv, write_csv, out_json, workload, calib_mb, partition_size=0, prefill=None):
    """Scale per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the partition
    kernel (with ``prefill``: of the prefill kernel, recorded under the
    prefill workload's name) by what the same counters read for a copy of
    known size. The record keeps the kernel source hash and (decode) the
    partition size the counters were taken with; the bench reports them only
    while both still hold."""
    import workloads as W
    kernels, source = PARTITION_KERNELS, KERNEL_SOURCE
    if prefill:
        from workloads import prefill as P
        w = P.BUILDERS[prefill]()
        workload, kernels, source = w.name, PREFILL_KERNELS, PREFILL_SOURCE
    else:
        w = W.build(workload)
        if partition_size:
            w.partition_size = partition_size
    calib_bytes = calib_mb * (1 << 20)
    res = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path, counter)
        cal = [v for n, v in rows if CALIBRATION_KERNEL in n]
        part = [v for n, v in rows if any(k in n for k in kernels)]
        if not cal or not part:
            raise SystemExit(f"{path}: no {counter} rows for the calibration copy or the partition kernel")
        scale = calib_bytes / (sum(cal) / len(cal) * 1024.0)
        res[counter] = {"calibration_kib": sum(cal) / len(cal), "scale": scale,
                        "partition_kib_mean": sum(part) / len(part), "dispatches": len(part),
                        "partition_bytes": sum(part) / len(part) * 1024.0 * scale}
    data = {}
    if os.path.exists(out_json):
        with open(out_json) as f:
            data = json.load(f)
    data[workload] = {
        "bytes_per_launch": round(res["FETCH_SIZE"]["partition_bytes"] + res["WRITE_SIZE"]["partition_bytes"]),
        "read_bytes": round(res["FETCH_SIZE"]["partition_bytes"]),
        "write_bytes": round(res["WRITE_SIZE"]["partition_bytes"]),
        "fetch_scale": res["FETCH_SIZE"]["scale"], "write_scale": res["WRITE_SIZE"]["scale"],
        "calibration_mb": calib_mb, "kernel_source_sha256_16": kernel_source_hash(source),
        "partition_size": None if prefill else resolved_partition(w), "counters": res,
    }
    with open(out_json, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print(json.dumps(data[workload], indent=1))


def host_cores() -> int:
    """CPU cores this process may run on (its share of the host)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - Linux has sched_getaffinity
        return os.cpu_count() or 1


def time_oracle(w, q_h, kc_h, vc_h, seconds: float, threads: int) -> dict:
    """Time the oracle, unmodified, on the batch's sequences in order and
    cycling, until about `seconds` of CPU work has been done, with `threads`
    BLAS threads."""
    import oracle
    from threadpoolctl import threadpool_limits
    dt = {"f32": oracle.F32, "bf16": oracle.BF16}[w.dtype]
    done, t_used, kv = 0, 0.0, 0
    e = 4 if w.dtype == "f32" else 2
    t0 = time.perf_counter()
    with threadpool_limits(limits=threads):
        while t_used < seconds:
            i = done % w.num_seqs
            ts = time.perf_counter()
            oracle.paged_decode(q_h[i:i + 1], kc_h, vc_h, w.block_tables[i:i + 1], w.context_lens[i:i + 1],
                                w.scale, w.block_size, dt)
            t_used += time.perf_counter() - ts
            kv += 2 * int(w.context_lens[i]) * w.num_kv_heads * w.head_dim * e
            done += 1
    wall = time.perf_counter() - t0
    return {"gbs": round(kv / t_used / 1e9, 4), "seqs_per_s": round(done / t_used, 3), "threads": threads,
            "decodes": done, "kv_mb": round(kv / 1e6, 1), "seconds": round(wall, 1)}


def cpu_baseline(w, q_h, kc_h, vc_h, seconds: float) -> dict:
    """The float64 oracle on the host's cores: BLAS threads = the cores this
    process may use (the reported value), then one thread on the same batch
    and on the 4-sequence fp32 batch (``tiny``)."""
    import workloads as W
    cores = host_cores()
    allc = time_oracle(w, q_h, kc_h, vc_h, seconds, cores)
    one = time_oracle(w, q_h, kc_h, vc_h, seconds / 2, 1)
    t = W.build("tiny")
    tv = W.make_values(t, device="cpu", poison=False)
    tiny = time_oracle(t, tv["q"].numpy(), tv["k_cache"].numpy(), tv["v_cache"].numpy(), seconds / 4, 1)
    return {
        "value": allc["gbs"], "unit": "GB/s", "cores": cores, "kind": "oracle",
        "seqs_per_s": allc["seqs_per_s"],
        "sample": f"{allc['decodes']} sequence decodes cycling over the {w.num_seqs} sequences of {w.name} "
                  f"({allc['kv_mb']} MB of K+V), float64 numpy oracle, {cores} BLAS threads "
                  f"(= the host cores this process may use), {allc['seconds']} s",
        "single_thread": {w.name: one, "tiny": tiny},
    }


def run_env() -> dict:
    """GPU, compiler target and software versions of the run."""
    import platform
    import torch
    props = torch.cuda.get_device_properties(0)
    return {"gpu": torch.cuda.get_device_name(0), "gfx": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "hbm_gib": round(props.total_memory / 2 ** 30, 1),
            "hip": torch.version.hip, "torch": torch.__version__, "python": platform.python_version(),
            "host_cores": host_cores()}


def percentiles(xs) -> dict:
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "n": int(a.size)}


def per_call_us(fn, calls: int, warmup: int = 10) -> dict:
    """Time `calls` calls of `fn` one by one, each between two HIP events on
    the launch stream, after `warmup` untimed calls: median, p10, p90 (us)."""
    import torch
    for _ in range(warmup):
        fn()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return percentiles([1e3 * a.elapsed_time(b) for a, b in evs])


def pattern_ceiling(w, kc, vc, dev) -> dict:
    """The decode's access pattern without its arithmetic: the K and V tiles
    of every block of every sequence's table (per KV head), read by the
    bandwidth probe (pa_probe_read_tiles). The best rate over its launch
    shapes bounds what the decode can reach on this device."""
    import numpy as np
    import torch
    import paged_kv_cache_165_amd as pa
    hkv, b = w.num_kv_heads, w.block_size
    parts = []
    for s in range(w.num_seqs):
        nb = -(-int(w.context_lens[s]) // b)
        blocks = w.block_tables[s, :nb].astype(np.int64)
        parts.append((blocks[None, :] * hkv + np.arange(hkv)[:, None]).ravel())
    tiles_h = np.concatenate(parts)
    # (block, head) slices over 8 KB go to the probe as 8 KB tiles
    slice_bytes = b * w.head_dim * kc.element_size()
    tile_bytes = min(slice_bytes, 8192)
    sub = slice_bytes // tile_bytes
    tiles_h = (tiles_h[:, None] * sub + np.arange(sub)[None, :]).ravel().astype(np.int32)
    tiles = torch.from_numpy(tiles_h).to(dev)
    nbytes = 2 * len(tiles_h) * tile_bytes
    sink = torch.empty(16 * 256 * 1024, dtype=torch.uint8, device=dev)
    best, runs = None, []
    for u in (1, 2, 4):
        for wg in (256, 512, 1024):
            fn = lambda: pa.probe_read_tiles(kc, vc, tiles, u, wg, sink, tile_bytes)
            for _ in range(3):
                fn()
            a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(10):
                fn()
            e.record()
            torch.cuda.synchronize()
            us = 1e3 * a.elapsed_time(e) / 10
            gbs = nbytes / (us * 1e-6) / 1e9
            runs.append({"tiles_in_flight": u, "workgroups": wg, "us": round(us, 2), "gbs": round(gbs, 1)})
            if best is None or gbs > best["gbs"]:
                best = runs[-1]
    return {"gbs": best["gbs"], "us": best["us"], "bytes": nbytes, "tiles": int(len(tiles_h)),
            "tile_bytes": tile_bytes, "best": {"tiles_in_flight": best["tiles_in_flight"],
                                               "workgroups": best["workgroups"]},
            "runs": runs,
            "what": "K and V tiles of every block in every table row (per KV head), read with the decode's "
                    "nontemporal 16-byte loads and no arithmetic (pa_probe_read_tiles), best of 9 launch shapes, "
                    "10 back-to-back launches each; whole tiles, so the last block's empty slots are read too"}


def engine_bench(args, dev):
    """Multi-step decode of the workload's sequences through PagedDecoder:
    every step appends one token to every sequence (block manager, copies,
    cache write) and decodes. Reports wall time per step (host bookkeeping,
    uploads and launches overlapped with the device) and the device time of
    the same steps."""
    import numpy as np
    import torch
    import workloads as W
    from paged_kv_cache_165_amd.engine import PagedDecoder
    w = W.build(args.workload)
    n, bs = w.num_seqs, w.block_size
    total = args.warmup + args.engine_steps
    lens0 = w.context_lens.astype(np.int64) - 1  # prompts; every step appends one token
    need = int(sum(-(-(int(L) + total) // bs) for L in lens0))
    maxb = int(max(-(-(int(L) + total) // bs) for L in lens0))
    dtype = torch.float32 if w.dtype == "f32" else torch.bfloat16
    rng = np.random.default_rng(w.seed)
    nl = max(1, args.engine_layers)
    eng = PagedDecoder(need + 8, bs, w.num_heads, w.num_kv_heads, w.head_dim, max_blocks_per_seq=maxb,
                       dtype=dtype, device=dev, partition_size=w.partition_size,
                       free_order=rng.permutation(need + 8), num_layers=nl)
    lead = (nl,) if nl > 1 else ()
    g = torch.Generator(device=dev).manual_seed(w.seed)
    progress(f"engine: prefilling {n} sequences ({int(lens0.sum())} tokens)")
    for s, L in enumerate(lens0):
        k = torch.randn(*lead, int(L), w.num_kv_heads, w.head_dim, generator=g, device=dev).to(dtype)
        v = torch.randn(*lead, int(L), w.num_kv_heads, w.head_dim, generator=g, device=dev).to(dtype)
        eng.prefill(s, k, v)
    seqs = list(range(n))
    q = torch.randn(n, w.num_heads, w.head_dim, generator=g, device=dev).to(dtype)
    kn = torch.randn(n, w.num_kv_heads, w.head_dim, generator=g, device=dev).to(dtype)
    vn = torch.randn(n, w.num_kv_heads, w.head_dim, generator=g, device=dev).to(dtype)
    out = torch.empty_like(q)

    def one_step():
        if nl == 1:
            eng.step(seqs, q, kn, vn, w.scale, out=out)
            return
        st = eng.begin_step(seqs)
        for layer in range(nl):
            eng.decode_layer(st, layer, q, kn, vn, w.scale, out=out)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    host = []
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.engine_steps):
        th = time.perf_counter()
        one_step()
        host.append(time.perf_counter() - th)
    end.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.engine_steps
    dev_ms = start.elapsed_time(end) / args.engine_steps
    eng.blocks.check()
    kv = nl * int(2 * (int(lens0.sum()) + n * (total + 1) // 2) * w.num_kv_heads * w.head_dim *
                  (4 if w.dtype == "f32" else 2))
    print(json.dumps({
        "metric": "multi-step paged decode through the block manager: wall time per step",
        "value": round(wall * 1e6, 1), "unit": "us", "n_gpus": 1, "steps": args.engine_steps,
        "warmup": args.warmup, "higher_is_better": False, "data": "synthetic", "dtype": w.dtype,
        "config": {"workload": w.name, "num_seqs": n, "block_size": bs, "prompt_tokens": int(lens0.sum()),
                   "num_layers": nl},
        "host_us_per_step": round(1e6 * float(np.mean(host)), 1),
        "gpu_stream_us_per_step": round(1e3 * dev_ms, 1),
        "wall_us_per_layer": round(wall * 1e6 / nl, 1),
        "kv_gb_per_s_wall": round(kv / wall / 1e9, 1),
    }), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 matrix peak


def cache_layers_bench(args, dev):
    """Cache maintenance for a model of `args.cache_layers` layers (GQA 8 KV
    heads, head_dim 128, bf16, block 16): the decode step's write of 256 new
    tokens at scattered slots, and 192 copy-on-write block copies, each as one
    layered launch and as one launch per layer. Bytes are moved bytes (read +
    written) of K and V."""
    import numpy as np
    import torch
    import paged_kv_cache_165_amd as pa
    nl, nb, hkv, bs, d, dt = args.cache_layers, 4096, 8, 16, 128, torch.bfloat16
    rng = np.random.default_rng(1670)
    g = torch.Generator(device=dev).manual_seed(1670)
    kc, vc = pa.alloc_cache_layers(nl, nb, hkv, bs, d, dt, device=dev)
    kc.zero_()
    vc.zero_()
    blocks = rng.permutation(nb)
    slots = torch.from_numpy((blocks[:256] * bs + rng.integers(0, bs, 256)).astype(np.int32)).to(dev)
    pairs = torch.from_numpy(np.stack([blocks[256:448], blocks[448:640]], 1).astype(np.int32)).to(dev)
    k = torch.randn(nl, 256, hkv, d, generator=g, device=dev).to(dt)
    v = torch.randn(nl, 256, hkv, d, generator=g, device=dev).to(dt)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(args.steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return 1e3 * a.elapsed_time(b) / args.steps

    def write_per_layer():
        for layer in range(nl):
            pa.write_cache(k[layer], v[layer], kc[layer], vc[layer], slots)

    def copy_per_layer():
        for layer in range(nl):
            pa.copy_blocks(kc[layer], vc[layer], pairs)

    w1 = timed(lambda: pa.write_cache_layers(k, v, kc, vc, slots))
    wn = timed(write_per_layer)
    c1 = timed(lambda: pa.copy_blocks_layers(kc, vc, pairs))
    cn = timed(copy_per_layer)
    wbytes = 2 * 2 * nl * 256 * hkv * d * 2       # K and V rows, read once and written once
    cbytes = 2 * 2 * nl * 192 * hkv * bs * d * 2  # K and V blocks, read once and written once
    print(json.dumps({
        "metric": "multi-layer cache write and block copy: one layered launch against one launch per layer",
        "value": round(wn / w1, 3), "unit": "x (write speedup)", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "cache_layers", "layers": nl, "num_kv_heads": hkv, "head_dim": d, "block_size": bs,
                   "write_tokens": 256, "copy_pairs": 192},
        "write_us": {"layered": round(w1, 2), "per_layer": round(wn, 2)},
        "write_gb_per_s": {"layered": round(wbytes / w1 / 1e3, 1), "per_layer": round(wbytes / wn / 1e3, 1)},
        "copy_us": {"layered": round(c1, 2), "per_layer": round(cn, 2)},
        "copy_gb_per_s": {"layered": round(cbytes / c1 / 1e3, 1), "per_layer": round(cbytes / cn / 1e3, 1)},
        "copy_speedup": round(cn / c1, 3),
    }), flush=True)


def prefill_cpu_baseline(w, q_h, kc_h, vc_h, seconds: float):
    """Time the oracle's paged prefill on the last rows of the workload's
    sequences, cycling, until about `seconds` of CPU work has been done; BLAS
    threads = the host cores this process may use."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits
    cores = host_cores()
    limiter = threadpool_limits(limits=cores)
    qs = w.query_start
    rows_per_call = 8
    done, t_used, flops = 0, 0.0, 0
    t0 = time.perf_counter()
    while t_used < seconds:
        s = done % w.num_seqs
        L, m = int(w.context_lens[s]), min(rows_per_call, int(w.query_lens[s]))
        rows = np.arange(qs[s + 1] - m, qs[s + 1])
        ts = time.perf_counter()
        oracle.paged_prefill(q_h[rows], kc_h, vc_h, w.block_tables[s:s + 1], [L], [0, m], w.scale,
                             w.block_size, oracle.BF16)
        t_used += time.perf_counter() - ts
        flops += 4 * w.head_dim * w.num_heads * sum(L - m + i + 1 for i in range(m))
        done += 1
    wall = time.perf_counter() - t0
    limiter.restore_original_limits()
    return {
        "value": round(flops / t_used / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
        "sample": f"{done} calls of the last {rows_per_call} new rows of one sequence, cycling over the "
                  f"{w.num_seqs} sequences of {w.name}, float64 numpy oracle, {cores} BLAS threads, {wall:.1f} s",
    }


def prefill_bench(args, dev):
    """Paged prefill: each step writes the K/V rows of every sequence's new
    tokens into their slots (pa_write_cache) and runs pa_prefill over the
    batch. `value` is causal attention TFLOP/s of the whole step (4 * D * Hq
    multiply-add flops per visible (row, key) pair); `roofline` reports the
    prefill kernel alone against the dense bf16 MFMA peak."""
    import numpy as np
    import torch
    import paged_kv_cache_165_amd as pa
    from workloads import prefill as P
    w = P.BUILDERS[args.prefill]()
    progress(f"prefill workload {w.name}: {w.summary()}")
    vals = P.make_values(w, device=dev, poison=True)
    q, kc, vc = vals["q"], vals["k_cache"], vals["v_cache"]
    g = torch.Generator(device=dev).manual_seed(w.seed + 1)
    kn = torch.randn(w.num_tokens, w.num_kv_heads, w.head_dim, generator=g, device=dev).to(q.dtype)
    vn = torch.randn(w.num_tokens, w.num_kv_heads, w.head_dim, generator=g, device=dev).to(q.dtype)
    pos = w.positions()
    seq_of = np.repeat(np.arange(w.num_seqs), w.query_lens)
    slots_h = (w.block_tables[seq_of, pos // w.block_size].astype(np.int64) * w.block_size
               + pos % w.block_size).astype(np.int32)
    slots = torch.from_numpy(slots_h).to(dev)
    tables = torch.from_numpy(w.block_tables).to(dev)
    lens = torch.from_numpy(w.context_lens).to(dev)
    qs = torch.from_numpy(w.query_start).to(dev)
    out = torch.empty_like(q)
    pargs = (out, q, kc, vc, tables, lens, qs, w.scale, w.max_query_len, w.max_context_len)

    def step():
        pa.write_cache(kn, vn, kc, vc, slots)
        pa.prefill(*pargs)

    warmed = warm_up(step, args.warmup)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    ka, kb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ka.record()
    for _ in range(args.steps):
        pa.prefill(*pargs)
    kb.record()
    torch.cuda.synchronize()
    k_us = 1e3 * ka.elapsed_time(kb) / args.steps
    if args.copy_calibration_mb:
        # the copy of known size the counter summary scales by
        n = args.copy_calibration_mb * (1 << 20) // 2
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    traffic = None  # counter bytes, valid only for the kernel source they were taken on
    if os.path.exists(args.traffic_json):
        try:
            with open(args.traffic_json) as f:
                tj = json.load(f).get(w.name)
            if tj and tj.get("kernel_source_sha256_16") == kernel_source_hash(PREFILL_SOURCE):
                traffic = tj.get("bytes_per_launch")
        except Exception:
            traffic = None
    flops = w.flops()
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (k_us * 1e-6) / 1e12
    progress(f"step {ms_step * 1e3:.1f} us, prefill kernel {k_us:.1f} us per launch")
    cpu = None
    if not args.no_cpu_baseline:
        def host(t):
            t = t.detach().cpu().contiguous()
            return t.view(torch.uint16).numpy() if t.dtype == torch.bfloat16 else t.numpy()
        cpu = prefill_cpu_baseline(w, host(q), host(kc), host(vc), args.cpu_seconds)
        progress(f"cpu baseline: {cpu}")
    print(json.dumps({
        "metric": "paged prefill attention: causal TFLOP/s",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "warmup_run": {"steps": warmed, "min_seconds": WARMUP_MIN_S},
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {**w.summary(), "new_tokens": w.num_tokens, "attended_pairs": w.attended_pairs(),
                   "flops": flops, "parallelism": "none (1 GPU)"},
        "tokens_per_s": round(w.num_tokens / (ms_step * 1e-3), 1),
        "roofline": {"bound": "mfma", "kernel": "pa_prefill (pa_prefill_mfma)", "achieved": round(achieved, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                     "traffic_gbs": round(traffic / (k_us * 1e-6) / 1e9, 2) if traffic else None,
                     "kernel_us_mean": round(k_us, 2),
                     "kernel_timing": f"{args.steps} back-to-back launches between two HIP events on the launch stream"},
        "cpu_baseline": cpu,
    }), flush=True)


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1], args.traffic_json,
                           args.workload, args.copy_calibration_mb, args.partition_size or 0, args.prefill)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    progress("importing torch")
    import numpy as np
    import torch

    import paged_kv_cache_165_amd as pa
    import workloads as W

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    lib = pa.library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.engine_steps:
        engine_bench(args, dev)
        return
    if args.prefill:
        prefill_bench(args, dev)
        return
    if args.cache_layers:
        cache_layers_bench(args, dev)
        return
    progress(f"device {torch.cuda.get_device_name(dev)}; building workload {args.workload}")
    if args.block_size and args.workload != "gqa8b":
        print("--block-size applies to the gqa8b workload only", file=sys.stderr)
        sys.exit(2)
    w = W.build(args.workload, **({"block_size": args.block_size} if args.block_size else {}))
    if args.tp > 1:
        if w.num_kv_heads % args.tp or w.num_heads % args.tp:
            raise SystemExit(f"{w.name}: {w.num_kv_heads} KV heads do not split over {args.tp} GPUs")
        w = dataclasses.replace(w, name=f"{w.name}_tp{args.tp}", num_heads=w.num_heads // args.tp,
                                num_kv_heads=w.num_kv_heads // args.tp)
    if args.partition_size:
        w.partition_size = args.partition_size
    vals = W.make_values(w, device=dev, poison=True)
    q, kc, vc = vals["q"], vals["k_cache"], vals["v_cache"]
    tables = torch.from_numpy(w.block_tables).to(dev)
    lens = torch.from_numpy(w.context_lens).to(dev)
    pairs = torch.from_numpy(w.cow_pairs.astype(np.int32)).to(dev)
    slots = [torch.from_numpy(op.slots.astype(np.int32)).to(dev) for op in w.writes]
    out = torch.empty_like(q)
    ws = pa.alloc_workspace(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.max_context_len,
                            w.block_size, w.partition_size, q.dtype, device=dev)
    dargs = (out, q, kc, vc, tables, lens, w.scale, w.max_context_len, w.partition_size, ws)
    # a batch whose tables share blocks tells the library so (pa_decode_ex,
    # PA_DECODE_SHARED_BLOCKS): the same results, tiles kept in the L2
    hint = {"shared_blocks": True} if w.refcount_max > 1 else {}

    def step():
        if len(w.cow_pairs):
            pa.copy_blocks(kc, vc, pairs)
        for sl, (k, v) in zip(slots, vals["writes"]):
            pa.write_cache(k, v, kc, vc, sl)
        pa.decode_partitions(*dargs, **hint)
        pa.decode_merge(*dargs)

    progress(f"warmup {args.warmup} steps, at least {WARMUP_MIN_S} s")
    warmed = warm_up(step, args.warmup)
    progress(f"timing {args.steps} steps (after {warmed} warm-up steps)")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(end) / args.steps
    # The partition kernel alone: the same number of launches back to back
    # between two events on the launch stream (an event between two kernels
    # adds a launch gap of about 5 us that is not the kernel's).
    ka, kb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ka.record()
    for _ in range(args.steps):
        pa.decode_partitions(*dargs, **hint)
    kb.record()
    torch.cuda.synchronize()
    part_us = 1e3 * ka.elapsed_time(kb) / args.steps

    # The cache maintenance calls of the step, each timed the same way
    # (writing the same rows, or copying the same blocks, again changes
    # nothing): moved bytes are read + written.
    def back_to_back(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return 1e3 * a.elapsed_time(b) / args.steps

    row_bytes = w.num_kv_heads * w.head_dim * q.element_size()
    cache_ops = {"timing": f"{args.steps} back-to-back launches between two HIP events on the launch stream",
                 "write": [], "copy": None}
    for sl, (k, v) in zip(slots, vals["writes"]):
        us = back_to_back(lambda: pa.write_cache(k, v, kc, vc, sl))
        moved = 4 * sl.shape[0] * row_bytes
        cache_ops["write"].append({"tokens": int(sl.shape[0]), "us": round(us, 2),
                                   "moved_gbs": round(moved / (us * 1e-6) / 1e9, 1)})
    if len(w.cow_pairs):
        us = back_to_back(lambda: pa.copy_blocks(kc, vc, pairs))
        moved = 4 * len(w.cow_pairs) * w.block_size * row_bytes
        cache_ops["copy"] = {"pairs": int(len(w.cow_pairs)), "us": round(us, 2),
                             "moved_gbs": round(moved / (us * 1e-6) / 1e9, 1)}
    kv = w.kv_bytes()
    unique = w.unique_kv_bytes()
    props = torch.cuda.get_device_properties(dev)
    lds = getattr(props, "shared_memory_per_multiprocessor", 0) or 163840
    plan = pa.decode_plan(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.max_context_len, w.block_size,
                          w.partition_size, torch.float32 if w.dtype == "f32" else torch.bfloat16,
                          lds_per_cu=lds, lds_per_workgroup=lds)
    value = kv / (ms_step * 1e-3) / 1e9
    achieved = kv / (part_us * 1e-6) / 1e9
    progress(f"step {ms_step * 1e3:.1f} us, partition kernel {part_us:.1f} us per launch")

    # Per-call timings (median, p10, p90 of single calls between two events):
    # pa_decode (partition kernel + merge) and the partition kernel alone.
    calls = max(50, args.steps)
    per_call = {"calls": calls, "warmup": 10,
                "decode_us": per_call_us(lambda: pa.decode(*dargs, **hint), calls),
                "partition_us": per_call_us(lambda: pa.decode_partitions(*dargs, **hint), calls),
                "timing": "each call between two HIP events on the launch stream (an event pair adds a few us "
                          "of queue time around the kernel)"}
    progress(f"per call: decode {per_call['decode_us']}, partition kernel {per_call['partition_us']}")
    progress("pattern ceiling (bandwidth probe over the same tiles)")
    ceiling = pattern_ceiling(w, kc, vc, dev)
    ceiling["decode_kernel_pct_of_ceiling"] = round(100.0 * (kv / (part_us * 1e-6) / 1e9) / ceiling["gbs"], 2)
    ceiling["decode_kernel_pct_of_ceiling_same_bytes"] = round(
        100.0 * (ceiling["bytes"] / (part_us * 1e-6) / 1e9) / ceiling["gbs"], 2)
    progress(f"pattern ceiling {ceiling['gbs']} GB/s ({ceiling['best']}); the partition kernel reaches "
             f"{ceiling['decode_kernel_pct_of_ceiling']} % of it")

    # A measured ceiling next to the peak: a plain device copy of 1 GiB (bytes
    # read plus written, per time), after the timed region.
    cbuf = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev)
    cdst = torch.empty_like(cbuf)
    for _ in range(3):
        cdst.copy_(cbuf)
    ca, cb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ca.record()
    for _ in range(10):
        cdst.copy_(cbuf)
    cb.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 30) / (ca.elapsed_time(cb) / 10 * 1e-3) / 1e9
    del cbuf, cdst

    if args.copy_calibration_mb:
        n = args.copy_calibration_mb * (1 << 20) // 2
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    traffic = None  # counter bytes, valid only for the kernel source they were taken on
    if os.path.exists(args.traffic_json):
        try:
            with open(args.traffic_json) as f:
                tj = json.load(f).get(w.name)
            if (tj and tj.get("kernel_source_sha256_16") == kernel_source_hash()
                    and tj.get("partition_size") == resolved_partition(w)):
                traffic = tj.get("bytes_per_launch")
        except Exception:
            traffic = None

    cpu = None
    if not args.no_cpu_baseline:
        progress("cpu baseline (oracle) on a bounded sample")

        def host(t):
            t = t.detach().cpu().contiguous()
            return t.view(torch.uint16).numpy() if t.dtype == torch.bfloat16 else t.numpy()

        cpu = cpu_baseline(w, host(q), host(kc), host(vc), args.cpu_seconds)
        progress(f"cpu baseline: {cpu}")
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_run": {"steps": warmed, "min_seconds": WARMUP_MIN_S},
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "num_heads": w.num_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
                   "partition_size": resolved_partition(w), "ctx": w.ctx_recipe, "tokens": int(w.context_lens.sum()), "tail_waste": round(W.tail_waste(w), 5),
                   "kv_bytes": kv, "seed": w.seed, "decode_flags": "shared_blocks" if hint else "none",
                   "parallelism": "none (1 GPU)" if args.tp == 1 else
                   f"one GPU's shard of a {args.tp}-way split by KV head (no exchange needed)"},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "copy_ceiling": {"gbs": round(copy_gbs, 1), "pct_of_ceiling": round(100.0 * value / copy_gbs, 2),
                         "what": "device copy of 1 GiB (bytes read + written per time), 10 launches, same run"},
        "unique_kv_gbs": round(unique / (ms_step * 1e-3) / 1e9, 2),
        "unique_kv_bytes": unique,
        "seqs_per_s": round(w.num_seqs / (ms_step * 1e-3), 1),
        "wall_ms_per_step": round(1e3 * t_wall / args.steps, 5),
        "cache_ops": cache_ops,
        "roofline": {"bound": "hbm", "kernel": f"pa_decode_partitions ({PLAN_KERNELS[plan['kernel']]})",
                     "plan": plan,
                     "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel_us_mean": round(part_us, 2),
                     "traffic_gbs": round(traffic / (part_us * 1e-6) / 1e9, 2) if traffic else None,
                     "kernel_timing": f"{args.steps} back-to-back launches between two HIP events on the launch stream",
                     "bytes_per_launch": kv},
        "cpu_baseline": cpu,
        "pattern_ceiling": ceiling,
        "per_call": per_call,
        "env": run_env(),
    }
    if w.refcount_max > 1:
        result["prefix_sharing"] = w.sharing_savings()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
