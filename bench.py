"""Benchmark: one Hybrid Block decode step (full attention + token selection + 3 sparse
layers) on one MI355X, at the million-token configuration by default.

A step is hs2_full_attn_select followed by three hs2_sparse_attn calls over the
same KV cache and index set, with every input already resident in HBM.  Prints
one JSON line (rank 0) with ctx-tokens/s, the scan kernel's roofline position
(HIP events around the scan launch, on the launch stream) and the CPU oracle's
throughput on a bounded sample.

  python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload million]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Hybrid-Block decode ctx-tokens/s & KV GB/s (%HBM peak) at 1M context"
CHUNK_METRIC = "Hybrid-Block 64-token chunk query-tokens/s & scan MFMA TFLOP/s (%bf16 dense peak)"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
SCAN_SOURCES = [os.path.join(ROOT, "long_context_decode_full_amd", "csrc", f)
                for f in ("hs2_scan_mfma.hip", "hs2_rowops.h", "hs2_device.h", "hs2_internal.h")]
BRIDGE_SOURCES = [os.path.join(ROOT, "long_context_decode_full_amd", "csrc", f)
                  for f in ("hs2_bridge.hip", "hs2_device.h", "hs2_internal.h")]
CHUNK_SOURCES = [os.path.join(ROOT, "long_context_decode_full_amd", "csrc", f)
                 for f in ("hs2_chunk_mfma.hip", "hs2_rowops.h", "hs2_device.h", "hs2_internal.h")]
BRIDGE_METRIC = "KV Bridging projection tokens/s & MFMA TFLOP/s (%bf16 dense peak)"
DECODE_METRIC = "Cross-Decoder decode tokens/s (KV Bridging append + 6 Hybrid Blocks per token)"
DECODE_LOOPS = {
    # name: (decode workload whose caches every block starts from, blocks, hidden)
    "decode_loop_million": ("million", 6, 2048),
    "decode_loop_batched": ("batched", 6, 2048),
    "decode_loop_tiny": ("tiny", 6, 2048),
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def scan_source_hash(files=None):
    h = hashlib.sha256()
    for p in files or SCAN_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def kv_bytes(inp):
    """Algorithmic bytes one full-attention scan must read: every visible K and V row of
    every KV head once (plus the per-token fp32 scales of an fp8 cache)."""
    ctx = int(np.sum(inp["ctx_len"]))
    Hkv, D = inp["k"].shape[1], inp["k"].shape[3]
    if inp["k"].dtype == np.uint8:
        return ctx * Hkv * 2 * (D * 1 + 4)
    return ctx * Hkv * 2 * D * 2


def measured_traffic(workload, files=None, key="scan_source_sha256"):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3 counter
    runs, if they were taken on the current source of that kernel; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    e = rec.get(workload)
    if not e or e.get(key) != scan_source_hash(files):
        return None
    return e.get("hbm_bytes_per_launch")


def scan_flops(inp):
    """Algorithmic FLOPs of one full-attention scan: q.k and p.v (2 x 128 multiply-adds)
    for every query head and every position visible to its token."""
    B, Lq, Hq = inp["q_full"].shape[:3]
    D = inp["q_full"].shape[3]
    total = 0
    for b in range(B):
        for j in range(Lq):
            total += max(0, int(inp["ctx_len"][b]) - Lq + j + 1)
    return total * Hq * 4 * D


def host_description():
    """The host the CPU oracle is timed on: processor model and the threads this process
    may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_threads": usable}


def measured_copy_peak(torch, nbytes=1 << 30, reps=10):
    """A second bandwidth denominator measured on this device: a plain 1 GiB
    device-to-device copy (read + write bytes over its event-timed duration)."""
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbps = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbps


def cpu_baseline(inp, groups, min_s=10.0, max_reps=100000, mode="token", threads=None):
    """The float64 oracle, as it is, on KV groups `groups` of sequence 0 / token 0,
    repeated until about `min_s` seconds of CPU work; returns seconds per repetition.
    `threads` limits the BLAS/OpenMP pools (None: as configured)."""
    import contextlib
    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limit = threadpool_limits(threads) if threads else contextlib.nullcontext()
    except Exception:  # pragma: no cover
        threadpool_info = None
        limit = contextlib.nullcontext()
    with limit:
        if threadpool_info is not None:
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        else:  # pragma: no cover
            cores = threads or os.cpu_count()
        reps = 0
        ref = None
        t0 = time.perf_counter()
        while reps < max_reps:
            ref = oracle.hybrid_block_token(inp, 0, 0, groups=groups, mode=mode)
            reps += 1
            if time.perf_counter() - t0 >= min_s:
                break
        dt = time.perf_counter() - t0
    return dt / reps, cores, reps, ref


def check_sample(got, ref, mode, topk=1024, window=128, block=64, n_blocks=18):
    """The timed outputs of sequence 0 / token 0 against the oracle's, with the test
    suite's rules (tests/parity.py): index sets equal except swaps inside the 1e-6 tie
    band in kernel precision (ties in position order), outputs within 2e-3 of each row's
    max |reference|."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import parity
    band = 0
    try:
        for g, s in enumerate(ref["s"]):
            if mode == "token":
                band += parity.check_idx_row(got["idx"][0, 0, g], ref["idx"][g], s, ref["n"], window, topk)
            else:
                band += parity.check_block_row(got["idx"][0, 0, g], ref["idx"][g], s, ref["n"], block, n_blocks)
    except AssertionError as e:
        return {"pass": False, "idx": f"KV head {g}: {e}"}
    e_full = float(parity.out_row_errors(got["out_full"][0, 0], ref["out_full"]).max())
    e_sp = max(float(parity.out_row_errors(o[0, 0], r).max())
               for o, r in zip(got["out_sparse"], ref["out_sparse"]))
    return {"pass": bool(e_full <= parity.OUT_TOL and e_sp <= parity.OUT_TOL),
            "idx": "identical" if band == 0 else f"{band} swap(s) within the 1e-6 tie band",
            "max_rel_err_full": e_full, "max_rel_err_sparse": e_sp}


def step_distribution(dev, reps, flush=None):
    """Per-step GPU times (ms) from events on the launch stream; with `flush`, a 512 MiB
    write before each step evicts the L2 and the 256 MB last-level cache."""
    import torch
    times = []
    for _ in range(reps):
        if flush is not None:
            flush.fill_(1)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        dev.step()
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()
    return [times[len(times) // 2], times[min(len(times) - 1, int(0.9 * len(times)))]]


def bridge_flops(w):
    """Algorithmic FLOPs of one bridging call: one multiply-add per (token, hidden dim,
    output feature), output features = layers x {K, V} x KV heads x 128."""
    return 2 * w.n_tokens * w.hidden * (w.n_layers * 2 * w.n_kv_heads * w.head_dim)


def bridge_bytes(w):
    """Algorithmic HBM bytes of one call: X and W read once, the K/V rows (and fp8
    scales) written once."""
    n_feat = w.n_layers * 2 * w.n_kv_heads * w.head_dim
    out = w.n_tokens * n_feat * (1 if w.kv_dtype == "fp8" else 2)
    if w.kv_dtype == "fp8":
        out += w.n_tokens * w.n_layers * 2 * w.n_kv_heads * 4
    return 2 * w.n_tokens * w.hidden + 2 * n_feat * w.hidden + out


def bench_bridge(args):
    """KV Bridging projection (HySparse2 article, section 02 "KV Bridging"; section 04):
    one hs2_kv_bridge call per step on the prefill chunk of a 1M-token context."""
    import torch
    import oracle
    from long_context_decode_full_amd import workloads as wl
    from long_context_decode_full_amd.runner import BridgeDevice

    w = wl.bridge_workloads()[args.workload]
    log(f"generating inputs: {w.name}")
    inp = wl.make_bridge_inputs(w)
    dev = BridgeDevice(inp, device="cuda:0")
    torch.cuda.synchronize()
    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        dev.run()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        dev.run(stream)          # one kernel launch per call, on this stream
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern_s = ev0.elapsed_time(ev1) * 1e-3 / args.steps
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    flops = bridge_flops(w)
    nbytes = bridge_bytes(w)
    tflops = flops / kern_s / 1e12
    n_feat = w.n_layers * 2 * w.n_kv_heads * w.head_dim
    result = {
        "metric": BRIDGE_METRIC,
        "value": w.n_tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"KV Bridging, {w.name}: T={w.n_tokens} tokens, hidden {w.hidden}, "
                        f"{w.n_layers} target layers x (K, V) x {w.n_kv_heads} KV heads x {w.head_dim} "
                        f"= {n_feat} features, {w.kv_dtype} caches of {w.capacity} rows",
            "n_tokens": w.n_tokens, "hidden": w.hidden, "n_layers": w.n_layers,
            "n_kv_heads": w.n_kv_heads, "kv_dtype": w.kv_dtype,
        },
        "kernel_us": kern_s * 1e6,
        "hbm_gbps_algorithmic": nbytes / kern_s / 1e9,
        "roofline": {
            "bound": "mfma",
            "achieved": tflops,
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
            "traffic": measured_traffic(args.workload, BRIDGE_SOURCES, "bridge_source_sha256"),
            "kernel": "bridge_kernel (projection GEMM on the matrix cores + quantise + cache scatter)",
            "algorithmic_flops_per_launch": flops,
            "algorithmic_bytes_per_launch": nbytes,
        },
        "cpu_baseline": None,
    }
    # parity sample: the oracle's decisions for a few tokens against the cache rows
    rng = np.random.default_rng(5)
    sample = np.sort(rng.choice(w.n_tokens, size=min(64, w.n_tokens), replace=False))
    got = dev.rows(sample)
    from oracle import bridge as ob
    Y = ob.project(inp["x"][sample], inp["weight"].reshape(n_feat, w.hidden))
    Y32 = Y.astype(np.float32).reshape(len(sample), w.n_layers, 2, w.n_kv_heads, w.head_dim)
    if w.kv_dtype == "fp8":
        codes, scales = ob.quantize_rows(Y32)
        tab = oracle.e4m3fn_table()
        eq = float(np.mean(tab[codes] == tab[got["codes"]]))
        rel = float(np.max(np.abs(got["scales"] / scales - 1.0)))
        result["parity_sample"] = {"tokens": int(len(sample)), "codes_equal_frac": eq,
                                   "scale_max_rel_diff": rel}
    else:
        eq = float(np.mean(ob.bf16_rne(Y32) == got["codes"]))
        result["parity_sample"] = {"tokens": int(len(sample)), "codes_equal_frac": eq}

    if not args.no_cpu_baseline:
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:  # pragma: no cover
            cores = os.cpu_count()
        n = min(1024, w.n_tokens)
        xs = inp["x"][:n]
        seq = np.zeros(n, dtype=np.int32)
        pos = np.arange(n, dtype=np.int32)
        shape = (w.n_layers, 1, w.n_kv_heads, n, w.head_dim)
        if w.kv_dtype == "fp8":
            caches = dict(k=np.zeros(shape, np.uint8), v=np.zeros(shape, np.uint8),
                          k_scale=np.zeros(shape[:4], np.float32), v_scale=np.zeros(shape[:4], np.float32))
        else:
            caches = dict(k=np.zeros(shape, np.uint16), v=np.zeros(shape, np.uint16))
        log(f"cpu oracle on {n} tokens")
        reps = 0
        c0 = time.perf_counter()
        while reps < 20:
            oracle.kv_bridge(xs, inp["weight"], seq, pos, caches)
            reps += 1
            if time.perf_counter() - c0 >= 10.0:
                break
        dt = (time.perf_counter() - c0) / reps
        result["cpu_baseline"] = {
            "value": n / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "host": host_description(),
            "sample": f"float64 numpy oracle (projection, rounding, scatter) on the first {n} tokens "
                      f"of the chunk into a {n}-row cache, {reps} repetition(s) of {dt:.2f}s",
        }
    print(json.dumps(result), flush=True)


def event_pairs(torch, n):
    """n (begin, end) pairs of timing events, each recorded once so that its HIP event
    exists before its handle is passed to the library."""
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n)]
    for a, b in pairs:
        a.record()
        b.record()
    torch.cuda.synchronize()
    return pairs


def events_ms(pairs):
    """Per-pair elapsed milliseconds (the events must have completed)."""
    return [a.elapsed_time(b) for a, b in pairs]


def bench_decode_loop(args):
    """Multi-step decode (HySparse2 article, section 02): each step appends every
    sequence's new token to the caches of all Hybrid Blocks through KV Bridging and
    runs every block's full and sparse layers -- one hs2_decode_step, captured once
    into a HIP graph and replayed per token."""
    import dataclasses
    import torch
    import oracle
    from long_context_decode_full_amd import workloads as wl
    from long_context_decode_full_amd.runner import DecodeLoopDevice

    base, n_blocks, hidden = DECODE_LOOPS[args.workload]
    w0 = wl.standard_workloads()[base]
    grow = args.warmup + 2 * args.steps + 64          # graph + eager passes each append
    w = dataclasses.replace(w0, capacity=max(w0.ctx_lens) + grow)
    log(f"generating inputs: {w.name}, {n_blocks} blocks, capacity {w.capacity}")
    inp = wl.make_inputs(w, threads=16)
    dec = wl.make_decode_steps(w, n_blocks=n_blocks, steps=1, hidden=hidden, seed=4001)
    dev = DecodeLoopDevice(inp, n_blocks, dec["w_bits"])
    dev.set_inputs(dec["x"][0], dec["q_full"][0], dec["q_sparse"][0])
    g = dev.capture()
    log(f"warmup {args.warmup} replays")
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"timing {args.steps} replays")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    graph_ms = (t1 - t0) * 1e3 / args.steps
    # the same steps issued eagerly
    torch.cuda.synchronize()
    e0 = time.perf_counter()
    for _ in range(args.steps):
        dev.step()
    torch.cuda.synchronize()
    e1 = time.perf_counter()
    eager_ms = (e1 - e0) * 1e3 / args.steps
    # each block's full layer once more, events around its context scan (the scan of a
    # step reads the same caches and lengths)
    pairs = event_pairs(torch, n_blocks)
    for l in range(n_blocks):
        dev.full_layer(l, events=pairs[l])
    torch.cuda.synchronize()
    scan_ms, scan_n = sum(events_ms(pairs)), n_blocks
    ctx = dev.ctx_len.cpu().numpy()
    Hkv, D = w.n_kv_heads, w.head_dim
    row_bytes = 2 * D * (1 if w.kv_dtype == "fp8" else 2) + (8 if w.kv_dtype == "fp8" else 0)
    scan_bytes = int(ctx.sum()) * Hkv * row_bytes
    scan_s = scan_ms * 1e-3 / scan_n
    achieved = scan_bytes / scan_s / 1e9
    result = {
        "metric": DECODE_METRIC,
        "value": w.batch / (graph_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": graph_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3fn" if w.kv_dtype == "fp8" else "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"decode loop over {n_blocks} Hybrid Blocks ({w.name} caches: B={w.batch}, "
                        f"ctx {w0.ctx_lens[0]}+, Hq={w.n_q_heads}/Hkv={Hkv}), KV Bridging from hidden "
                        f"{hidden}, 1 full + {w.n_sparse_layers} sparse layers per block, one HIP graph per step",
            "batch": w.batch, "n_blocks": n_blocks, "hidden": hidden, "ctx_end": ctx.tolist(),
        },
        "eager_ms_per_step": eager_ms,
        "graph_speedup": eager_ms / graph_ms,
        "scan_us": scan_s * 1e6,
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS, "traffic": measured_traffic(args.workload),
            "kernel": "scan_mfma_kernel (each block's full-attention scan; eager pass, library events)",
            "algorithmic_bytes_per_launch": scan_bytes,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:  # pragma: no cover
            cores = os.cpu_count()
        # the oracle for one block of one sequence, and the bridge oracle for its token
        one = dict(inp, q_full=dec["q_full"][0][0], q_sparse=dec["q_sparse"][0][:w.n_sparse_layers])
        one["ctx_len"] = inp["ctx_len"].copy()

        def repeated(fn, min_s=8.0, min_reps=3, max_reps=1000):
            """Seconds per call of fn, repeated to about min_s of CPU work."""
            reps, total = 0, 0.0
            while reps < max_reps and (total < min_s or reps < min_reps):
                c0 = time.perf_counter()
                fn()
                total += time.perf_counter() - c0
                reps += 1
            return total / reps, reps

        t_block, r_block = repeated(lambda: oracle.hybrid_block_token(one, 0, 0))
        shape = (n_blocks, 1, Hkv, 1, D)
        caches = dict(k=np.zeros(shape, np.uint16), v=np.zeros(shape, np.uint16))
        t_bridge, r_bridge = repeated(lambda: oracle.kv_bridge(dec["x"][0][:1], dec["w_bits"], np.zeros(1, np.int32),
                                                               np.zeros(1, np.int32), caches), min_s=2.0)
        per_seq = t_bridge + n_blocks * t_block
        result["cpu_baseline"] = {
            "value": 1.0 / per_seq, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "host": host_description(),
            "sample": f"float64 oracle: one Hybrid Block for sequence 0 ({t_block:.3f}s, mean of {r_block} "
                      f"repetitions) x {n_blocks} blocks + the bridge for its token ({t_bridge:.4f}s, mean of "
                      f"{r_bridge}), per sequence",
        }
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps first: the GPU reaches its sustained clocks after a few tens of ms")
    ap.add_argument("--workload", default="million",
                    help="tiny | batched | fp8_256k | million | chunk | mqa_million | mqa_chunk | fp8_chunk; KV Bridging: "
                         "bridge_prefill | bridge_prefill_bf16 | bridge_mqa | bridge_decode; decode loop: "
                         "decode_loop_million | decode_loop_batched | decode_loop_tiny")
    ap.add_argument("--select", default="token", choices=["token", "block", "gen1"],
                    help="token selection (window 128 + top-k 1024), the first-generation block "
                         "comparator (18 blocks of 64, no forced window), or the full first-generation "
                         "comparator (block selection + a separate 128-token sliding-window branch "
                         "over each sparse layer's own local ring)")
    ap.add_argument("--deterministic", action="store_true",
                    help="fixed step shares in the context scan (bitwise reproducible, slower)")
    ap.add_argument("--chunk-per-token", action="store_true",
                    help="query chunks: the decode scan once per token (HS2_FLAG_CHUNK_PER_TOKEN) "
                         "instead of the chunk kernel, for comparison")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is a design note, not an implemented mode.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        # A plain device-to-device copy of known size: its FETCH_SIZE / WRITE_SIZE
        # counters give the factor between counter readings and bytes moved.
        nbytes = 1 << 30
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": nbytes, "launches": 5}), flush=True)
        return
    if args.workload.startswith("bridge"):
        bench_bridge(args)
        return
    if args.workload in DECODE_LOOPS:
        bench_decode_loop(args)
        return
    from long_context_decode_full_amd import HS2_FLAG_CHUNK_PER_TOKEN, HS2_FLAG_DETERMINISTIC
    from long_context_decode_full_amd import workloads as wl
    from long_context_decode_full_amd.runner import HybridBlockDevice

    w = wl.standard_workloads()[args.workload]
    log(f"generating inputs: {w.name}")
    t0 = time.perf_counter()
    inp = wl.make_inputs(w, threads=16)
    log(f"inputs ready in {time.perf_counter() - t0:.1f}s; uploading")
    rings = None
    if args.select == "gen1":
        # each sparse layer's own local ring: the 128-token window of every query token
        rings = wl.make_local_rings(w, 128 + w.q_len - 1, seed=w.seed + 100)
    flags = (HS2_FLAG_DETERMINISTIC if args.deterministic else 0) | \
            (HS2_FLAG_CHUNK_PER_TOKEN if args.chunk_per_token else 0)
    dev = HybridBlockDevice(inp, device="cuda:0", mode=args.select, local_rings=rings, flags=flags)
    torch.cuda.synchronize()

    # Auxiliary measurements first (they are reported, not part of the timed steps):
    # the copy-kernel denominator, per-step distributions warm and cold, and the
    # per-launch distribution of the scan and of one sparse layer's gather.
    copy_gbps = measured_copy_peak(torch)
    nrep = max(20, min(args.steps, 100))
    warm_dist = step_distribution(dev, nrep)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    cold_dist = step_distribution(dev, nrep, flush)
    del flush
    nd = min(max(args.steps, 20), 30)
    scan_pairs, gather_pairs = event_pairs(torch, nd), event_pairs(torch, nd)
    for i in range(nd):
        dev.step(scan_events=scan_pairs[i], gather_events=gather_pairs[i])
    torch.cuda.synchronize()
    per_scan = sorted(t * 1e3 for t in events_ms(scan_pairs))
    gather_us = sorted(t * 1e3 for t in events_ms(gather_pairs))

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        dev.step()
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    pairs = event_pairs(torch, args.steps)   # around each step's context scan
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        dev.step(scan_events=pairs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    scan_ms, scan_n = sum(events_ms(pairs)), args.steps

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    ctx = int(np.sum(inp["ctx_len"]))
    chunk = w.q_len > 1
    # decode: context tokens per second; chunk: query tokens per second
    value = (w.batch * w.q_len if chunk else ctx) / (ms_per_step * 1e-3)
    scan_avg_s = scan_ms * 1e-3 / scan_n
    algo = kv_bytes(inp)
    achieved = algo / scan_avg_s / 1e9
    flops = scan_flops(inp)
    idx = dev.idx.cpu().numpy()
    assert np.all((idx >= -1)), "invalid index output"

    result = {
        "metric": CHUNK_METRIC if chunk else METRIC,
        "value": value,
        "unit": "query-tokens/s" if chunk else "ctx-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3fn" if w.kv_dtype == "fp8" else "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: B={w.batch}, ctx_len={w.ctx_lens}, q_len={w.q_len}, "
                        f"Hq={w.n_q_heads}/Hkv={w.n_kv_heads}, head_dim={w.head_dim}, "
                        f"{w.kv_dtype} KV, "
                        + {"token": "window 128 + top-k 1024",
                           "block": "block comparator: 18 blocks of 64",
                           "gen1": "first-generation comparator: 18 blocks of 64 + a separate "
                                   "128-token sliding-window branch per sparse layer"}[args.select]
                        + f", 1 full + {w.n_sparse_layers} sparse layers",
            "batch": w.batch, "ctx_tokens": ctx, "q_len": w.q_len,
            "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads, "kv_dtype": w.kv_dtype,
            "deterministic": bool(args.deterministic),
            "chunk_per_token": bool(args.chunk_per_token),
        },
        "kv_gbps": achieved,
        "scan_us": scan_avg_s * 1e6,
        "scan_us_min_med_max": [per_scan[0], per_scan[len(per_scan) // 2], per_scan[-1]],
        "sparse_gather_us_median": gather_us[len(gather_us) // 2],
        "step_ms_median_p90": {"warm": warm_dist, "cold": cold_dist, "reps": nrep},
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            # counters were taken for token selection (the record path's scan)
            "traffic": measured_traffic(args.workload) if args.select == "token" else None,
            "kernel": "scan_mfma_kernel (split-K full-attention scan on the matrix cores)",
            "algorithmic_bytes_per_launch": algo,
            "measured_copy_gbps": copy_gbps,
            "frac_of_measured_copy": achieved / copy_gbps,
        },
        "cpu_baseline": None,
    }
    if chunk:
        tflops = flops / scan_avg_s / 1e12
        result["roofline"] = {
            "bound": "mfma",
            "achieved": tflops,
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
            "traffic": (measured_traffic(args.workload, CHUNK_SOURCES, "chunk_source_sha256")
                        if args.select == "token" else None),
            "kernel": "chunk_mfma_kernel (64-token chunk full-attention scan on the matrix cores)",
            "algorithmic_flops_per_launch": flops,
            "kv_gbps": achieved,
        }
        result["config"]["ctx_lens"] = [int(c) for c in inp["ctx_len"]]

    if args.select == "gen1":
        # the oracle's comparator path is checked by tests/test_gpu_gen1.py; its timing
        # sample would be the block path's plus a 128-row attention per layer
        args.no_cpu_baseline = True
        result["sparse_layer_us_note"] = "per branch: each gen-1 sparse layer runs two gathers"
    if not args.no_cpu_baseline:
        Hkv = inp["k"].shape[1]
        groups = list(range(Hkv))
        log(f"cpu oracle on KV groups {groups} of {Hkv}")
        dt, cores, reps, ref = cpu_baseline(inp, groups, mode=args.select)
        result["parity_sample"] = dict(check_sample(dev.results(), ref, args.select),
                                       sample="sequence 0, query token 0, every KV head")
        # the oracle's cost per (sequence, query token) row grows with its visible length
        n00 = max(1, int(inp["ctx_len"][0]) - w.q_len + 1)
        rows_scale = sum(max(0, int(inp["ctx_len"][b]) - w.q_len + j + 1)
                         for b in range(w.batch) for j in range(w.q_len)) / n00
        full_est = dt * Hkv / len(groups) * rows_scale
        result["cpu_baseline"] = {
            "value": (w.batch * w.q_len if chunk else ctx) / full_est,
            "unit": "query-tokens/s" if chunk else "ctx-tokens/s",
            "cores": cores,
            "kind": "oracle",
            "sample": (f"float64 numpy oracle, full layer + selection + {w.n_sparse_layers} sparse "
                       f"layers for {len(groups)} of {Hkv} KV groups of sequence 0 / token 0, "
                       f"{reps} repetition(s) of {dt:.2f}s, scaled by {rows_scale:.1f} (the step's "
                       f"visible positions over all (sequence, query token) rows / this row's)"),
            "host": host_description(),
        }
        if args.workload in ("tiny", "batched"):
            # the short-context configurations also report the oracle on one thread
            dt1, cores1, reps1, _ = cpu_baseline(inp, groups, min_s=5.0, mode=args.select, threads=1)
            result["cpu_baseline"]["one_thread"] = {
                "value": (w.batch * w.q_len if chunk else ctx) / (dt1 * Hkv / len(groups) * rows_scale),
                "cores": cores1, "sample": f"{reps1} repetition(s) of {dt1:.3f}s, same scaling"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
