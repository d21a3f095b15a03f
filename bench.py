#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

A step is one paged decode-attention call for the whole batch (split kernel +
LSE merge) on inputs already resident in HBM. The default workload is the
hybrid-model long-context decode: batch 1, q_len 1, 24 query / 4 KV heads,
head_dim 256, page 784, context 32768, bf16 K/V with 5% of key rows x4.

To measure HBM and not the 256 MB Infinity Cache, steps rotate through
``--pools`` independent copies of the KV pool (16 by default, about 2.7 GB, as
16 full-attention layers of one decode step would). Timing uses HIP events on
the stream the library launches on. One JSON line goes to stdout; with
``--ladder``, one line per context / page-size row and a summary line with the
fit t(L) = a + b * L and the page-size check.

Every run checks the timed output against the fp64 oracle (every element, or
sampled rows for prefill) with max abs error <= 2e-3 and max relative error
<= 1e-2 (relative to max(|oracle|, 1e-3)); the result is in the line's
``parity`` field, and a failed or skipped check makes the run exit with
status 3. The ``identity`` field carries the sha256 of the loaded libpkv.so,
of the kernel sources and of the input bytes.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn µs/step and KV-read GB/s (% of HBM peak) at 32K ctx, batch 1"
METRIC_PREFILL = "chunked-prefill attention TFLOP/s (4 * head_dim flops per row, head and visible token)"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA, MI355X


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=1000,
                    help="untimed steps first; fewer than about 500 leave the first timed region "
                         "about 5%% slow while the GPU settles (about 30 ms of work at the default size)")
    ap.add_argument("--workload", default="hybrid",
                    choices=["hybrid", "single", "dense", "mixed", "verify", "varlen", "prefill"],
                    help="hybrid: one 24/4/256 sequence (page --block-size, --context tokens); single: batch 1, "
                         "page 16, 512 tokens, 32 of 64 pages; dense: 32/8/128, page 16; mixed: 16 sequences; "
                         "verify: --q-len causal rows; varlen: batched verify; prefill: one chunk of --chunk rows")
    ap.add_argument("--context", type=int, default=None,
                    help="tokens in the cache (default 32768; 8192 for prefill)")
    ap.add_argument("--chunk", type=int, default=4096, help="prefill: new query rows of the chunk")
    ap.add_argument("--q-len", type=int, default=16, help="verify: query rows per sequence (1..16)")
    ap.add_argument("--block-size", type=int, default=784)
    ap.add_argument("--pools", type=int, default=16)
    ap.add_argument("--splits", type=int, default=0, help="force a split count (0 = planner)")
    ap.add_argument("--kv-dtype", default="bf16", choices=["bf16", "fp8"],
                    help="K/V cache type: bf16, or OCP FP8 E4M3 codes with per-tensor scales")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window: each query row sees its last W positions (0 = whole context)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--repeats", type=int, default=5, help="extra timed regions for spread statistics")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay measurement")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before timing, copy this many MiB once (a kernel of known traffic, used to "
                         "scale rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--ladder", action="store_true",
                    help="the context ladder (1K, 4K, 16K, 32K at page 784; 32K at pages 832 and 16) of the "
                         "hybrid decode: one JSON line per row, then the fit t(L) = a + b * L and the page-size check")
    args = ap.parse_args()
    if args.workload == "single":
        args.context = 512
    elif args.context is None:
        args.context = 8192 if args.workload == "prefill" else 32768
    return args


class Hip:
    """HIP events through the runtime torch loaded (one runtime per process)."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so.7")
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]

    def event(self):
        ev = ctypes.c_void_p()
        rc = self.h.hipEventCreate(ctypes.byref(ev))
        assert rc == 0, f"hipEventCreate failed: {rc}"
        return ev

    def record(self, ev, stream):
        rc = self.h.hipEventRecord(ev, ctypes.c_void_p(stream))
        assert rc == 0, f"hipEventRecord failed: {rc}"

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.h.hipEventElapsedTime(ctypes.byref(ms), a, b)
        assert rc == 0, f"hipEventElapsedTime failed: {rc}"
        return ms.value

    def destroy(self, ev):
        self.h.hipEventDestroy(ev)


def make_workload(args):
    from paged_kv_cache_08_amd import workloads as W
    kv = dict(kv_dtype="fp8_e4m3") if args.kv_dtype == "fp8" else {}
    if args.workload == "single":
        case = W.single_seq_b16(poison=False, **kv)
        name = "single sequence: batch 1, q_len 1, 24 q / 4 KV heads, head_dim 256, page 16, 512 tokens, 32 of 64 pages"
    elif args.workload == "hybrid":
        case = W.hybrid_long_context(args.context, block_size=args.block_size, poison=False, **kv)
        name = (f"hybrid decode: batch 1, q_len 1, 24 q / 4 KV heads, head_dim 256, page {args.block_size}, "
                f"context {args.context}, 5% of keys x4")
    elif args.workload == "dense":
        case = W.dense_control(args.context, poison=False, **kv)
        name = f"dense control: batch 1, q_len 1, 32 q / 8 KV heads, head_dim 128, page 16, context {args.context}"
    elif args.workload == "mixed":
        case = W.mixed_batch(poison=False, **kv)
        name = "mixed batch: 16 sequences, q_len 1, 24 q / 4 KV heads, head_dim 256, page 784, log-uniform 500-32000"
    elif args.workload == "prefill":
        case, qp, cu = W.chunked_prefill(args.chunk, args.context, block_size=args.block_size, poison=False, **kv)
        name = (f"chunked prefill: one chunk of {args.chunk} new rows on a {args.context}-token cache, "
                f"24 q / 4 KV heads, head_dim 256, page {args.block_size}")
        return case, name, (qp, cu)
    elif args.workload == "varlen":
        case, qp, cu = W.batched_verify(poison=False, **kv)
        name = ("batched speculative verify (varlen): 32 requests, 1..5 rows each, 24 q / 4 KV heads, "
                "head_dim 256, page 784, contexts log-uniform 512..2048")
        return case, name, (qp, cu)
    else:
        case = W.spec_verify(args.context, q_len=args.q_len, poison=False, **kv)
        name = (f"speculative verify: batch 1, q_len {args.q_len} causal rows, 24 q / 4 KV heads, head_dim 256, "
                f"page 784, context {args.context}")
    return case, name, None


def traffic_from_profiles(kernel_src_hash: str, workload_key: str):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path)).get(workload_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_src_sha256") != kernel_src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


def oracle_call(case, varlen, window):
    """The oracle's result for the benchmark input (pool 0)."""
    import oracle.paged_attention as O
    if varlen is not None:
        qp, cu = varlen
        return O.paged_attention_varlen_ref(qp, cu, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                                            case.block_size, case.scale, window, case.kv_dtype, case.k_scale,
                                            case.v_scale)
    return O.paged_attention_ref(case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                                 case.block_size, case.scale, window, case.kv_dtype, case.k_scale, case.v_scale)


def oracle_rows(case, varlen, rows, window):
    """The oracle's result for rows of sequence 0 of a packed call, one by one:
    row i of n new rows sees the first L - n + i + 1 tokens, a one-row call on
    that prefix. Returns [len(rows), Hq, D]."""
    import numpy as np
    import oracle.paged_attention as O
    qp, cu = varlen
    n, L = int(cu[1] - cu[0]), int(case.seq_lens[0])
    out = []
    for i in rows:
        out.append(O.paged_attention_ref(qp[None, i:i + 1], case.k_cache, case.v_cache, case.block_table[:1],
                                         np.array([L - n + i + 1]), case.block_size, case.scale, window,
                                         case.kv_dtype, case.k_scale, case.v_scale)[0, 0])
    return np.stack(out)


def cpu_baseline_rows(case, varlen, window, seconds):
    """Prefill: the oracle over a seeded sample of the chunk's rows (a whole
    call is minutes of CPU work), reported as attention TFLOP/s."""
    import numpy as np
    from paged_kv_cache_08_amd import workloads as W
    threads = _blas_threads()
    n = int(varlen[1][1])
    order = np.random.default_rng(3).permutation(n)
    flops, done, t0 = 0, 0, time.perf_counter()
    L = int(case.seq_lens[0])
    while done < n:
        i = int(order[done])
        oracle_rows(case, varlen, [i], window)
        vis = L - n + i + 1 if window <= 0 else min(L - n + i + 1, window)
        flops += 4 * case.q.shape[3] * case.q.shape[2] * vis
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {
        "value": round(flops / el / 1e12, 6),
        "unit": "TFLOP/s",
        "us_per_row": round(el / done * 1e6, 1),
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} random rows of the {n}-row chunk (all {case.q.shape[2]} heads), one-row oracle calls "
                  f"on their causal prefixes (fp64 NumPy, BLAS threads={threads}), {el:.1f} s",
        "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
    }


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return int(os.environ.get("OMP_NUM_THREADS", "1"))


def _oracle_calls(case, varlen, window, seconds):
    """Whole oracle calls until about `seconds` have run: (calls, seconds)."""
    n, t0 = 0, time.perf_counter()
    while True:
        oracle_call(case, varlen, window)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= 1000:
            return n, el


def cpu_baseline(case, varlen, window, kv_bytes_per_call, seconds):
    """The oracle as it stands, on the host cores, over whole calls of the same
    workload until about `seconds` of CPU work has run; then the same with
    BLAS limited to one thread for a third of that time."""
    threads = _blas_threads()
    n, el = _oracle_calls(case, varlen, window, seconds)
    single = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            n1, el1 = _oracle_calls(case, varlen, window, seconds / 3)
        single = {"value": round(kv_bytes_per_call * n1 / el1 / 1e9, 3), "unit": "GB/s",
                  "us_per_call": round(el1 / n1 * 1e6, 1), "cores": 1,
                  "sample": f"{n1} full oracle calls, BLAS limited to 1 thread, {el1:.1f} s"}
    except ImportError:
        pass
    return {
        "value": round(kv_bytes_per_call * n / el / 1e9, 3),
        "unit": "GB/s",
        "us_per_call": round(el / n * 1e6, 1),
        "cores": threads,
        "kind": "oracle",
        "sample": f"{n} full oracle calls on the benchmark input (fp64 NumPy, BLAS threads={threads}), {el:.1f} s",
        "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "single_thread": single,
    }


PARITY_ATOL = 2e-3       # max |gpu - oracle|
PARITY_RTOL = 1e-2       # max |gpu - oracle| / max(|oracle|, 1e-3)
PARITY_REL_FLOOR = 1e-3


def _sha256(*arrays) -> str:
    import hashlib
    import numpy as np
    h = hashlib.sha256()
    for a in arrays:
        a = np.ascontiguousarray(a)
        h.update(str(a.dtype).encode() + str(a.shape).encode())
        h.update(a.view(np.uint8).reshape(-1).data)
    return h.hexdigest()


def _file_sha256(path: str) -> str:
    import hashlib
    h = hashlib.sha256()
    with open(path, "rb") as fh:
        for chunk in iter(lambda: fh.read(1 << 20), b""):
            h.update(chunk)
    return h.hexdigest()


def trace_from_profiles(kernel_src_hash: str, workload_key: str):
    """The split kernel's average duration in the committed rocprofv3 kernel
    trace of this workload, if that trace was taken on the current kernel
    source; else None."""
    path = os.path.join(ROOT, "profiles", "kernel_trace.json")
    try:
        rec = json.load(open(path)).get(workload_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_src_sha256") != kernel_src_hash:
        return None
    return rec


def measure(args, dev, hip, emit_cpu=True):
    """One workload: set up, warm up, time, check parity. Returns (record, parity_ok)."""
    import numpy as np
    import torch

    import paged_kv_cache_08_amd as P
    from paged_kv_cache_08_amd import workloads as W

    case, wl_name, varlen = make_workload(args)
    prefill = args.workload == "prefill"
    print(f"[bench] workload: {wl_name}", file=sys.stderr, flush=True)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    if varlen is None:
        q, cu_t, max_q = bf16(case.q), None, None
    else:
        q = bf16(varlen[0])
        cu_t = torch.from_numpy(varlen[1]).to(dev)
        max_q = int(np.diff(varlen[1]).max())
    if case.kv_dtype == "fp8_e4m3":
        k0 = torch.from_numpy(np.ascontiguousarray(case.k_cache)).to(dev)
        v0 = torch.from_numpy(np.ascontiguousarray(case.v_cache)).to(dev)
        scales = dict(k_scale=case.k_scale, v_scale=case.v_scale)
    else:
        k0, v0 = bf16(case.k_cache), bf16(case.v_cache)
        scales = {}
    table = torch.from_numpy(case.block_table).to(dev)
    lens = torch.from_numpy(case.seq_lens).to(dev)
    input_sha = _sha256(case.q if varlen is None else varlen[0], case.k_cache, case.v_cache, case.block_table,
                        case.seq_lens, *(() if varlen is None else (varlen[1],)))
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(max(args.pools, 1) - 1)]
    total_tokens = int(case.seq_lens.sum())
    rows = [case.q_len] * case.num_seqs if varlen is None else np.diff(varlen[1])
    kv_bytes = W.kv_read_bytes(case.seq_lens, case.k_cache.shape[2], case.k_cache.shape[3],
                               elem_bytes=case.k_cache.dtype.itemsize, window=args.window, rows=rows)
    flops = W.attention_flops(case.seq_lens, rows, case.q.shape[2], case.q.shape[3], window=args.window)
    stream = torch.cuda.current_stream(dev).cuda_stream
    call = P.PreparedDecode(q, k0, v0, table, lens, case.block_size, case.scale, max_seq_len=case.max_seq_len,
                            total_tokens=total_tokens, num_splits=args.splits, stream=stream,
                            cu_seqlens_q=cu_t, max_q_len=max_q, window=args.window, prefill=prefill, **scales)
    out = call.out

    ptrs = [(k.data_ptr(), v.data_ptr()) for k, v in pools]

    def step(i, c=call):
        kp, vp = ptrs[i % len(ptrs)]
        c.run_ptrs(kp, vp)

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        flush.fill_(3)                      # evict src from the caches before the measured copy
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy: {n} bytes read, {n} bytes written", file=sys.stderr, flush=True)
        del src, dst, flush

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    variant = P.last_variant()
    print(f"[bench] variant: {variant}", file=sys.stderr, flush=True)

    # The contract's timed region: exactly `steps` calls between two events.
    ev0, ev1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.record(ev0, stream)
    for i in range(args.steps):
        step(i)
    hip.record(ev1, stream)
    torch.cuda.synchronize()
    total_ms = hip.elapsed_ms(ev0, ev1)
    ms_per_step = total_ms / args.steps

    # Spread: more timed regions of the same length.
    region_us = [ms_per_step * 1e3]
    for _ in range(args.repeats):
        torch.cuda.synchronize()
        hip.record(ev0, stream)
        for i in range(args.steps):
            step(i)
        hip.record(ev1, stream)
        torch.cuda.synchronize()
        region_us.append(hip.elapsed_ms(ev0, ev1) / args.steps * 1e3)

    # Split-kernel duration: events recorded by the library right around it.
    pairs = [(hip.event(), hip.event()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        P.set_timing_events(pairs[i][0], pairs[i][1])
        step(i)
    P.set_timing_events(None, None)
    torch.cuda.synchronize()
    kern_us = [hip.elapsed_ms(a, b) * 1e3 for a, b in pairs]
    for a, b in pairs:
        hip.destroy(a)
        hip.destroy(b)
    kern_avg_us = sum(kern_us) / len(kern_us)

    # The same K steps captured once in a HIP graph and replayed (launch overhead removed).
    graph_us = None
    if not args.no_graph:
        gstream = torch.cuda.Stream(dev)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gstream):
            gcall = P.PreparedDecode(q, k0, v0, table, lens, case.block_size, case.scale,
                                     max_seq_len=case.max_seq_len, total_tokens=total_tokens,
                                     num_splits=args.splits, out=out, workspace=call.workspace,
                                     stream=gstream.cuda_stream, cu_seqlens_q=cu_t, max_q_len=max_q,
                                     window=args.window, prefill=prefill, **scales)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=gstream):
            for i in range(args.steps):
                step(i, gcall)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        rs = torch.cuda.current_stream(dev).cuda_stream
        graph_regions = []
        for _ in range(max(1, args.repeats)):
            hip.record(ev0, rs)
            graph.replay()
            hip.record(ev1, rs)
            torch.cuda.synchronize()
            graph_regions.append(hip.elapsed_ms(ev0, ev1) / args.steps * 1e3)
        graph_us = statistics.median(graph_regions)
        del graph

    # Parity on the timed output (pool 0 holds the seeded input): every element
    # against the oracle, or sampled rows one by one for prefill (a whole
    # prefill oracle call is minutes of CPU work). A failed or skipped check
    # fails the run.
    step(0)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    parity = {"atol": PARITY_ATOL, "rtol": PARITY_RTOL, "rel_floor": PARITY_REL_FLOOR, "ok": False}
    try:
        if prefill:
            n_rows = int(varlen[1][1])
            sample = sorted({0, 1, n_rows // 2 - 1, n_rows - 1} & set(range(n_rows)))
            g, ref = got[sample], oracle_rows(case, varlen, sample, args.window)
            parity["checked"] = f"rows {sample} of the chunk, every head and column"
        else:
            g, ref = got, oracle_call(case, varlen, args.window)
            parity["checked"] = "every output element"
        err = np.abs(g - ref)
        parity["max_abs_err"] = float(err.max())
        parity["max_rel_err"] = float((err / np.maximum(np.abs(ref), PARITY_REL_FLOOR)).max())
        parity["ok"] = bool(np.all(np.isfinite(g)) and parity["max_abs_err"] <= PARITY_ATOL
                            and parity["max_rel_err"] <= PARITY_RTOL)
    except Exception as e:
        parity["error"] = f"{type(e).__name__}: {e}"
        print(f"[bench] parity check failed to run: {e}", file=sys.stderr)

    gbs = kv_bytes / (ms_per_step * 1e-3) / 1e9
    kern_gbs = kv_bytes / (kern_avg_us * 1e-6) / 1e9
    from paged_kv_cache_08_amd.profiling import kernel_source_hash
    src_hash = kernel_source_hash()
    wl_key = (f"{args.workload}:{args.context}:{case.block_size}" + (f":q{args.chunk}" if prefill else "")
              + (f":q{args.q_len}" if args.workload == "verify" and args.q_len != 16 else "")
              + (f":w{args.window}" if args.window else "")
              + (":fp8" if args.kv_dtype == "fp8" else ""))
    traffic = traffic_from_profiles(src_hash, wl_key)
    trace = trace_from_profiles(src_hash, wl_key)

    cpu = None
    if emit_cpu and not args.no_cpu_baseline:
        if prefill:
            cpu = cpu_baseline_rows(case, varlen, args.window, args.cpu_seconds)
        else:
            cpu = cpu_baseline(case, varlen, args.window, kv_bytes, args.cpu_seconds)

    # The split kernel of the variant that ran (the library's run-time marker).
    kernel = ("verify_split_kernel (prefill blocks)" if variant.startswith("prefill_mfma") else
              "verify_split_kernel" if variant.startswith(("verify_mfma", "varlen_mfma")) else
              "decode_mfma_kernel" if variant.startswith(("decode_mfma", "verify_rows", "varlen_rows")) else
              "decode_split_kernel")
    timing_src = ("HIP events that the library records on its stream right around the split kernel "
                  "(hipExtLaunchKernel), averaged over the K launches after the timed regions")
    if prefill:   # a dense contraction: priced against the bf16 MFMA peak
        tflops = flops / (ms_per_step * 1e-3) / 1e12
        kern_tflops = flops / (kern_avg_us * 1e-6) / 1e12
        value, unit = round(tflops, 2), "TFLOP/s"
        roof = {"bound": "mfma", "kernel": kernel, "achieved": round(kern_tflops, 2),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(kern_tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
        per_us = lambda us: flops / (us * 1e-6) / 1e12  # noqa: E731
        peak = MFMA_BF16_PEAK_TFLOPS
    else:
        value, unit = round(gbs, 1), "GB/s"
        roof = {"bound": "hbm", "kernel": kernel, "achieved": round(kern_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(kern_gbs / HBM_PEAK_GBS, 4)}
        per_us = lambda us: kv_bytes / (us * 1e-6) / 1e9  # noqa: E731
        peak = HBM_PEAK_GBS
    roof.update({"traffic": traffic, "kernel_us_avg": round(kern_avg_us, 2), "kernel_us_min": round(min(kern_us), 2),
                 "timing": timing_src})
    if trace:
        us = trace["kernel_us_avg"]
        roof["trace"] = {"kernel_us_avg": us, "achieved": round(per_us(us), 1), "frac": round(per_us(us) / peak, 4),
                         "source": f"profiles/kernel_trace.json [{wl_key}] (rocprofv3 --kernel-trace, "
                                   f"{trace.get('calls', '?')} launches)"}

    med = statistics.median(region_us)
    rec = {
        "metric": METRIC_PREFILL if prefill else METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if case.kv_dtype == "bf16" else "fp8",
        "data": "synthetic",
        "config": {
            "workload": wl_name,
            "batch": int(case.num_seqs),
            "query_rows": int(case.num_seqs * case.q_len if varlen is None else varlen[1][-1]),
            "context": int(case.max_seq_len),
            "window": args.window,
            "kv_dtype": case.kv_dtype,
            "block_size": int(case.block_size),
            "kv_pools_rotated": len(pools),
            "kv_bytes_per_step": kv_bytes,
            "flops_per_step": flops,
            "variant": variant,
        },
        "us_per_step": round(ms_per_step * 1e3, 2),
        # 16 full-attention layers make one decode step of the hybrid model;
        # the pages quote per-step attention time for 16 such calls.
        "us_per_hybrid_step_16_layers": round(16 * ms_per_step * 1e3, 1),
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 1),
        "us_per_step_regions": {"median": round(med, 2), "min": round(min(region_us), 2),
                                "max": round(max(region_us), 2),
                                "range_pct": round(100.0 * (max(region_us) - min(region_us)) / med, 2)},
        "roofline": roof,
        "graph_us_per_step": None if graph_us is None else round(graph_us, 2),
        "graph_gbs": None if graph_us is None else round(kv_bytes / (graph_us * 1e-6) / 1e9, 1),
        "cpu_baseline": cpu,
        "parity": parity,
        "identity": {
            "libpkv_sha256": _file_sha256(P.binding.LIB_PATH),
            "kernel_src_sha256": src_hash,
            "input_sha256": input_sha,
            "library": P.version(),
        },
    }
    del pools, call
    torch.cuda.empty_cache()
    return rec, parity["ok"]


LADDER = [(1024, 784), (4096, 784), (16384, 784), (32768, 784), (32768, 832), (32768, 16)]


def ladder(args, dev, hip):
    """The hybrid decode over the context ladder and the page sizes: one JSON
    line per row, then a summary line with the least-squares fit
    t(L) = a + b * L over the page-784 contexts and the spread of the 32K
    times across page sizes (the no-cliff check, within 5%)."""
    import numpy as np
    rows, ok_all = [], True
    for ctx, bs in LADDER:
        a = argparse.Namespace(**vars(args))
        a.workload, a.context, a.block_size = "hybrid", ctx, bs
        rec, ok = measure(a, dev, hip, emit_cpu=False)
        ok_all &= ok
        row = {"ladder_row": True, "context": ctx, "block_size": bs, "us_per_step": rec["us_per_step"],
               "graph_us_per_step": rec["graph_us_per_step"], "gbs": rec["value"], "pct_hbm_peak": rec["pct_hbm_peak"],
               "kernel_us_avg": rec["roofline"]["kernel_us_avg"], "variant": rec["config"]["variant"],
               "parity_ok": ok, "max_abs_err": rec["parity"].get("max_abs_err"),
               "input_sha256": rec["identity"]["input_sha256"]}
        print(json.dumps(row), flush=True)
        rows.append(row)
    fit = [(r["context"], r["us_per_step"]) for r in rows if r["block_size"] == 784]
    L = np.array([f[0] for f in fit], dtype=np.float64)
    t = np.array([f[1] for f in fit], dtype=np.float64)
    b, a0 = np.polyfit(L, t, 1)
    # The same fit over HIP-graph replays of the same steps (no host launch
    # cost per call), when the rows measured them.
    fit_graph = None
    tg = [r["graph_us_per_step"] for r in rows if r["block_size"] == 784]
    if all(x is not None for x in tg):
        bg, ag = np.polyfit(L, np.array(tg, dtype=np.float64), 1)
        fit_graph = {"a_us": round(float(ag), 3), "b_ns_per_token": round(float(bg) * 1e3, 4),
                     "points": [[int(x), float(y)] for x, y in zip(L, tg)]}
    t32 = {r["block_size"]: r["us_per_step"] for r in rows if r["context"] == 32768}
    spread = (max(t32.values()) - min(t32.values())) / min(t32.values())
    summary = {
        "ladder_summary": True,
        "fit": {"a_us": round(float(a0), 3), "b_ns_per_token": round(float(b) * 1e3, 4),
                "points": [[int(x), float(y)] for x, y in fit],
                "b_16_layers_us_per_token": round(16 * float(b), 6),
                "pages_context_us_per_token": {"hybrid_dual_radeon": 4.840, "dense_8b_dual_radeon": 0.118}},
        "fit_graph_replay": fit_graph,
        "page_sizes_at_32k_us": {str(k): v for k, v in t32.items()},
        "page_size_spread_pct": round(100.0 * spread, 2),
        "no_cliff": bool(spread <= 0.05),
        "parity_ok": bool(ok_all),
        "steps": args.steps, "warmup": args.warmup,
    }
    print(json.dumps(summary), flush=True)
    return ok_all


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by sequence, KV head or context range; this harness measures one GPU's share)", file=sys.stderr)
        sys.exit(2)

    import torch

    assert torch.cuda.is_available(), "no GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hip = Hip()
    if args.ladder:
        ok = ladder(args, dev, hip)
    else:
        rec, ok = measure(args, dev, hip)
        print(json.dumps(rec), flush=True)
    if not ok:
        print("[bench] parity against the oracle failed or did not run: see the parity field", file=sys.stderr)
        sys.exit(3)


if __name__ == "__main__":
    main()
