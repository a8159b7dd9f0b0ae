"""Benchmark of the paged sliding-window + clamped image-range hot path on one GPU.

One step = the whole path over one synthetic batch of the Gemma-style
multimodal prefill (16,550 tokens, 60 images of 256 tokens, W 1024, 16 query /
8 KV heads, head dim 256, paged in blocks of 16):
  slot mapping of the new tokens -> KV-cache write -> paged prefill attention.
The decode half of the path (MLA-shaped split-KV decode: 64 requests, 128 heads,
576/512 latent, history partial + the current key's partial from one call,
LSE combine, V-up projection) is timed in the same run and reported under
"decode"; the other prefill workloads (tiny, batched chunked, non-causal chunk
lookback) under "prefill_configs".

Reported value: algorithmic TFLOP/s = 4 * head_dim FLOP per allowed
(query, key, head) triple over the measured step time (steps with no event
recorded between their launches).  The "roofline" object is for the dominant
kernel (prefill attention), timed over as many steps again with HIP events
around each of its launches on the stream it runs on.  Every timed section
follows a time-based warm-up that brings the clocks to their steady state.
"""
from __future__ import annotations

import os

# BLAS / OpenMP threads of the CPU-baseline leg: the cores this process may
# run on, fixed before numpy is first imported (an explicit setting wins)
_CORES = len(os.sched_getaffinity(0))
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_v, str(_CORES))

import argparse  # noqa: E402
import json  # noqa: E402
import subprocess  # noqa: E402
import sys  # noqa: E402
import time  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
METRIC = "SWA+MM-prefix prefill attn TFLOP/s (% MFMA peak); paged decode HBM GB/s"


def warm(torch, fn, min_ms=100.0, min_calls=3):
    """Untimed calls of fn until at least min_ms of wall time has passed, so a
    timing taken after a host-side pause starts at steady clocks."""
    torch.cuda.synchronize()
    t0, n = time.perf_counter(), 0
    while n < min_calls or (time.perf_counter() - t0) * 1e3 < min_ms:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warm-ms", type=float, default=200.0,
                    help="time-based warm-up before each timed section, on top of --warmup "
                         "steps: the clocks ramp up over the first ~25 ms of sustained load "
                         "and drop again after a pause")
    ap.add_argument("--skip-cpu", action="store_true", help="omit the CPU oracle baseline")
    ap.add_argument("--skip-decode", action="store_true", help="omit the decode half")
    ap.add_argument("--skip-extra", action="store_true",
                    help="omit everything but the headline step and the decode step")
    ap.add_argument("--decode-splits", type=int, default=1)
    ap.add_argument("--decode-partials", choices=["f32", "bf16", "f16"], default="bf16",
                    help="dtype of the history/current partial outputs")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="first run one plain device copy of this many bytes (a known-size "
                         "kernel to calibrate HBM byte counters against)")
    return ap.parse_args()


# ---- algorithmic work ---------------------------------------------------------

def allowed_pairs(w, r, rows=None):
    """Allowed (query, key) pairs of request r for one head, from the mask's
    definition: each row's allowed keys form one interval containing the query
    position (base window, optionally cut by the chunk-lookback edge, united
    with every image range that holds the query, clamped on the left by the
    window), so the count is the interval length, clamped to [0, seq_len)."""
    import numpy as np
    ctx, L, W = int(w.context_lens[r]), int(w.seq_lens[r]), w.window
    i = np.arange(int(w.query_lens[r]), dtype=np.int64) if rows is None else np.asarray(rows)
    q = ctx + i
    if w.causal:
        lo = q - W + 1 if W > 0 else np.zeros_like(q)
        hi = q.copy()
    else:
        lo = q - W + 1 if W > 0 else np.zeros_like(q)
        hi = q + W - 1 if W > 0 else np.full_like(q, L - 1)
    if w.chunk_lookback >= 0:
        lo = np.maximum(lo, (q // w.chunk_size - w.chunk_lookback) * w.chunk_size)
    for s, e in w.ranges_of(r):
        if s < e:
            inside = (q >= s) & (q <= e)
            img_lo = np.maximum(s, q - W + 1) if W > 0 else np.full_like(q, s)
            lo = np.where(inside, np.minimum(lo, img_lo), lo)
            hi = np.where(inside, np.maximum(hi, e), hi)
    lo, hi = np.maximum(lo, 0), np.minimum(hi, L - 1)
    return int(np.maximum(hi - lo + 1, 0).sum())


def prefill_flop(w):
    pairs = sum(allowed_pairs(w, r) for r in range(w.num_seqs))
    return pairs * w.num_q_heads * 4 * w.head_dim_qk, pairs


def timed_events(torch, fn, reps, rounds=5):
    """Median over `rounds` of the mean event time of `reps` back-to-back calls (ms)."""
    import numpy as np
    out = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / reps)
    return float(np.median(out))


# ---- CPU baseline (the oracle as written, on this host's cores) --------------

def cpu_model():
    try:
        txt = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in txt.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    return "unknown"


def cpu_baseline(budget_s=45.0):
    """The oracle legs per workload: dense masked attention (O4), the tile-pruned
    attention (O5, the method on the CPU), scalar slot mapping (O1) and the LSE
    merge (O7); best of up to 3 passes while the leg's single pass is short,
    within an overall time budget."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention_pruned_ref, attention_ref, lse_merge_ref, slot_mapping_ref
    from workloads import make_config

    t_start = time.perf_counter()

    def best(fn, max_passes=3):
        times = []
        while len(times) < max_passes:
            t0 = time.perf_counter()
            fn()
            times.append(time.perf_counter() - t0)
            if times[-1] > 2.0 or time.perf_counter() - t_start > budget_s:
                break
        return min(times), len(times)

    def attn_leg(w, fn_name, rows_limit=None, seqs_limit=None):
        fn = attention_ref if fn_name == "O4" else attention_pruned_ref
        q_all = w.q_f32()
        flop = 0
        calls = []
        for r in range(w.num_seqs if seqs_limit is None else seqs_limit):
            s0, s1 = int(w.query_start_loc[r]), int(w.query_start_loc[r + 1])
            n = s1 - s0 if rows_limit is None else min(rows_limit, s1 - s0)
            flop += allowed_pairs(w, r, rows=np.arange(n)) * w.num_q_heads * 4 * w.head_dim_qk
            kw = dict(context_len=int(w.context_lens[r]), seq_len=int(w.seq_lens[r]),
                      scale=w.scale, window=w.window, causal=w.causal, chunk_size=w.chunk_size,
                      chunk_lookback=w.chunk_lookback, ranges=w.ranges_of(r))
            calls.append((q_all[s0:s0 + n], w.k_f32(r), w.v_f32(r), kw))

        def run():
            for q, k, v, kw in calls:
                fn(q, k, v, **kw)
        t, n_pass = best(run)
        return {"TFLOPs": round(flop / t / 1e12, 6), "s": round(t, 4), "passes": n_pass,
                "flop": flop}

    def slot_leg(w):
        byts = w.num_tokens * 12 + (w.max_num_tokens - w.num_tokens) * 4
        t, n_pass = best(lambda: slot_mapping_ref(w.query_start_loc, w.positions, w.block_table,
                                                  w.block_size, w.max_num_tokens))
        return {"GBps": round(byts / t / 1e9, 6), "s": round(t, 5), "passes": n_pass}

    legs = {}
    threads = None
    for cfg in (2, 1, 5, 3, 4):
        if time.perf_counter() - t_start > budget_s:
            legs[f"config{cfg}"] = "skipped: time budget"
            continue
        w = make_config(cfg)
        d = {"workload": w.name}
        if cfg == 5:
            # the decode's dense oracle over every key of each request, and the
            # merge of its two partials' shape (64 x 128 rows of 512)
            d["O4_dense_decode_first_16_requests"] = attn_leg(w, "O4", seqs_limit=16)
            rng = np.random.default_rng(5)
            rows = w.num_tokens * w.num_q_heads
            outs = [rng.standard_normal((rows, w.head_dim_v)).astype(np.float32) for _ in range(2)]
            lses = [rng.standard_normal(rows).astype(np.float32) for _ in range(2)]
            t, n_pass = best(lambda: lse_merge_ref(outs, lses))
            byts = sum(o.nbytes for o in outs) + sum(x.nbytes for x in lses) + rows * w.head_dim_v * 2
            d["O7_lse_merge"] = {"GBps": round(byts / t / 1e9, 6), "s": round(t, 5), "passes": n_pass,
                                 "partials": 2}
        else:
            d["O4_dense"] = attn_leg(w, "O4")
            if cfg in (2, 4):
                # the pruned pass (a Python loop over query blocks) over the first
                # 2,048 rows of each request: one eighth / one half of the work
                d["O5_pruned_first_2048_rows"] = attn_leg(w, "O5", rows_limit=2048)
            else:
                d["O5_pruned"] = attn_leg(w, "O5")
            d["O1_slot_mapping"] = slot_leg(w)
        legs[f"config{cfg}"] = d
        if threads is None:
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    head = legs.get("config2", {})
    value = head["O4_dense"]["TFLOPs"] if isinstance(head, dict) and "O4_dense" in head else None
    return {"value": value, "unit": "TFLOP/s", "cores": _CORES, "kind": "oracle",
            "sample": "float64 numpy oracle (dense masked attention) over the whole 16,550-token "
                      "multimodal prefill, all 16 heads, one pass; per-workload legs below "
                      "(O4 dense, O5 pruned, O1 slot mapping, O7 LSE merge; best of up to 3 "
                      "passes)",
            "blas_threads": threads, "cpu_model": cpu_model(),
            "affinity_cores": _CORES, "legs": legs,
            "total_s": round(time.perf_counter() - t_start, 1)}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_attention_kv_write_gemma16550_traffic.json")
PREFILL_SOURCES = ["attention_prefill.hip", "asm_ops.h", "device_common.h", "mask_bounds.h",
                   "psw_internal.h"]


def measured_traffic():
    """HBM bytes per launch of the prefill kernel with the fused KV-cache write,
    from the committed counter runs, or None when the kernel sources differ from
    the ones the counters were taken on."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    h = hashlib.sha1()
    for f in PREFILL_SOURCES:
        h.update(open(os.path.join(ROOT, "paged_sliding_window_amd", "csrc", f), "rb").read())
    if h.hexdigest() != rec.get("sources_sha1"):
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path's multi-GPU sharding is a design note, not built)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import paged_sliding_window_amd as psw
    from tests.gpu_setup import GpuWorkload, bits_to_bf16
    from workloads import make_config

    torch.cuda.set_device(0)
    psw.load()
    t_setup = time.perf_counter()
    if args.copy_bytes > 0:
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---------------- prefill (headline) ----------------
    log("generating the prefill workload")
    w = make_config(2)
    flop, pairs = prefill_flop(w)
    gw = GpuWorkload(w, fill_cache=False)
    # the context part is empty (context_len 0): the step writes every new K/V row
    k_new = bits_to_bf16(np.concatenate(w.k_bits))
    v_new = bits_to_bf16(np.concatenate(w.v_bits))
    slots = torch.empty(w.max_num_tokens, dtype=torch.int32, device="cuda")
    out = torch.empty((w.num_tokens, w.num_q_heads, w.head_dim_v), dtype=torch.bfloat16,
                      device="cuda")
    lse = torch.empty((w.num_tokens, w.num_q_heads), dtype=torch.float32, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    ev_kv = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]

    def prefill_step(i=None):
        # slot mapping, then one launch that writes the new K/V rows into the
        # cache and computes the attention (reading the new keys from k_new /
        # v_new): the same work as the unfused step below, one launch fewer
        psw.slot_mapping(gw.qsl, gw.positions, gw.block_table, w.block_size, w.max_num_tokens,
                         out=slots)
        if i is not None:
            ev[i][0].record()
        psw.swa_mm_attention_kv_write(gw.q, k_new, v_new, slots, gw.k_cache, gw.v_cache,
                                      gw.block_table, gw.qsl, gw.seq_lens, scale=w.scale,
                                      window=w.window, causal=w.causal, mm_ranges=gw.mm_ranges,
                                      out=out, lse=lse)
        if i is not None:
            ev[i][1].record()

    def unfused_step(i=None):
        psw.slot_mapping(gw.qsl, gw.positions, gw.block_table, w.block_size, w.max_num_tokens,
                         out=slots)
        if i is not None:
            ev_kv[i].record()
        psw.kv_cache_write(k_new, v_new, slots, gw.k_cache, gw.v_cache)
        if i is not None:
            ev[i][0].record()
        psw.swa_mm_attention(gw.q, gw.k_cache, gw.v_cache, gw.block_table, gw.qsl, gw.seq_lens,
                             scale=w.scale, window=w.window, causal=w.causal,
                             mm_ranges=gw.mm_ranges, out=out, lse=lse)
        if i is not None:
            ev[i][1].record()

    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)

    def time_steps(step):
        """(ms per step, mean ms of the timed kernel): args.steps steps with no
        event recorded between their launches (each record costs a few
        microseconds of the stream's time), then args.steps more with events
        around the kernel."""
        t0.record()
        for _ in range(args.steps):
            step()
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        return ms, sum(a.elapsed_time(b) for a, b in ev) / args.steps

    log("timing prefill")
    for _ in range(args.warmup):
        prefill_step()
    warm_ms = warm(torch, prefill_step, min_ms=args.warm_ms)
    ms_per_step, attn_ms = time_steps(prefill_step)
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (attn_ms * 1e-3) / 1e12
    log(f"prefill {ms_per_step:.4f} ms/step, fused kernel {attn_ms:.4f} ms")

    log("timing the unfused prefill step")
    warm(torch, unfused_step, min_ms=args.warm_ms)
    u_ms, u_attn = time_steps(unfused_step)
    kv_ms = sum(a.elapsed_time(b[0]) for a, b in zip(ev_kv, ev)) / args.steps
    # each new row read once and written once, K and V
    kv_bytes = 2 * 2 * k_new.numel() * k_new.element_size() + w.num_tokens * 4
    log(f"unfused {u_ms:.4f} ms/step, attention kernel {u_attn:.4f} ms")

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "gemma_mm_prefill_16550",
            "tokens": w.num_tokens, "window": w.window, "causal": True, "images": 60,
            "image_tokens": 256, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim_qk, "block_size": w.block_size,
            "allowed_pairs_per_head": pairs, "flop_per_step": flop,
            "step": "slot_mapping + swa_mm_attention_kv_write (KV-cache write fused into the "
                    "attention launch)",
        },
        "roofline": {
            "kernel": "prefill attention with the fused KV-cache write, head dim 256 (workload 2)",
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(),
            "avg_launch_ms": round(attn_ms, 5),
            "clock_state": f"steady: {args.warmup} warm-up steps, then {warm_ms:.0f} ms of "
                           "back-to-back steps before the timed ones",
        },
        "unfused": {
            "step": "slot_mapping + kv_cache_write + swa_mm_attention",
            "ms_per_step": round(u_ms, 5),
            "TFLOPs": round(flop / (u_ms * 1e-3) / 1e12, 3),
            "attention_kernel_ms": round(u_attn, 5),
            "attention_kernel_TFLOPs": round(flop / (u_attn * 1e-3) / 1e12, 3),
            "attention_kernel_frac": round(flop / (u_attn * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "kv_cache_write": {"ms": round(kv_ms, 5), "bytes": kv_bytes,
                               "GBps": round(kv_bytes / (kv_ms * 1e-3) / 1e9, 1),
                               "what": "new K and V rows read and written to their slots, "
                                       "slots read"},
            "clock_state": f"steady: {args.warm_ms:.0f} ms of back-to-back steps before the timed ones",
        },
    }
    del gw, k_new, v_new, out, lse
    torch.cuda.empty_cache()

    # ---------------- decode (second half of the path) ----------------
    if not args.skip_decode:
        log("decode half")
        result["decode"] = bench_decode(args, torch, psw, np)
    if not args.skip_extra:
        log("other prefill workloads")
        result["prefill_configs"] = bench_prefill_configs(args, torch, psw)
        log("segmented splits, non-causal workload")
        result["prefill_segmented"] = bench_segmented(args, torch, psw)
        log("slot mapping, scaled batch")
        result["slot_mapping_scaled"] = bench_slot_mapping(args, torch, psw, np)
        log("library GEMM ceiling")
        result["library_gemm_ceiling"] = bench_gemm_ceiling(args, torch, achieved)
    if not args.skip_cpu:
        log("CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline()
    result["setup_s"] = round(time.perf_counter() - t_setup, 1)
    print(json.dumps(result), flush=True)


def bench_prefill_configs(args, torch, psw):
    """Attention alone on the tiny (latency), batched chunked and non-causal
    chunk-lookback workloads: event-timed median of 5 rounds after a warm-up."""
    from tests.gpu_setup import GpuWorkload
    from workloads import make_config
    res = {}
    for cfg in (1, 3, 4):
        w = make_config(cfg)
        flop, pairs = prefill_flop(w)
        gw = GpuWorkload(w)
        out = torch.empty((w.num_tokens, w.num_q_heads, w.head_dim_v), dtype=torch.bfloat16,
                          device="cuda")
        lse = torch.empty((w.num_tokens, w.num_q_heads), dtype=torch.float32, device="cuda")

        def fn():
            psw.swa_mm_attention(gw.q, gw.k_cache, gw.v_cache, gw.block_table, gw.qsl,
                                 gw.seq_lens, scale=w.scale, window=w.window, causal=w.causal,
                                 chunk_size=w.chunk_size, chunk_lookback=w.chunk_lookback,
                                 mm_ranges=gw.mm_ranges, out=out, lse=lse)
        warm(torch, fn, min_ms=args.warm_ms / 2)
        ms = timed_events(torch, fn, reps=50 if cfg == 1 else 20)
        tf = flop / (ms * 1e-3) / 1e12
        res[w.name] = {"head_dim": w.head_dim_qk, "tokens": w.num_tokens,
                       "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                       "allowed_pairs_per_head": pairs, "flop": flop,
                       "attention_ms": round(ms, 5), "TFLOPs": round(tf, 3),
                       "frac_of_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
        if cfg == 1:
            res[w.name]["latency_us"] = round(ms * 1e3, 2)
            res[w.name]["note"] = "launch-latency bound: the fraction of peak is not meaningful"
        del gw, out, lse
        torch.cuda.empty_cache()
    return res


def bench_gemm_ceiling(args, torch, attn_tflops, reps=10):
    """What a plain library bf16 GEMM (torch.matmul on hipBLASLt, then on
    rocBLAS) reaches on this GPU at steady clocks: the practical matrix-core
    rate that an attention kernel's fraction of the published peak can be read
    against.  Context only; no step of the path uses it."""
    best = None
    backends = []
    for lib in ("cublaslt", "cublas"):  # hipBLASLt and rocBLAS under ROCm
        try:
            torch.backends.cuda.preferred_blas_library(lib)
            backends.append(lib)
        except Exception:  # noqa: BLE001  (a backend this build lacks is skipped)
            continue
        for m, n, k in ((8192, 8192, 8192), (16384, 8192, 8192), (16384, 16384, 8192)):
            a = torch.randn(m, k, device="cuda", dtype=torch.bfloat16)
            b = torch.randn(k, n, device="cuda", dtype=torch.bfloat16)
            c = torch.empty(m, n, device="cuda", dtype=torch.bfloat16)
            fn = lambda: torch.matmul(a, b, out=c)  # noqa: E731
            warm(torch, fn, min_ms=args.warm_ms)
            ms = timed_events(torch, fn, reps, rounds=3)
            tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
            if best is None or tf > best["TFLOPs"]:
                best = {"shape_mnk": [m, n, k], "ms": round(ms, 4), "TFLOPs": round(tf, 1),
                        "library": {"cublaslt": "hipBLASLt", "cublas": "rocBLAS"}[lib]}
            del a, b, c
    torch.backends.cuda.preferred_blas_library("default")
    torch.cuda.empty_cache()
    if best is None:
        return None
    best["what"] = ("torch.matmul bf16 in, fp32 accumulate, bf16 out; best of three shapes "
                    "on each BLAS backend tried: " + ", ".join(backends))
    best["frac_of_mfma_peak"] = round(best["TFLOPs"] / MFMA_BF16_PEAK_TFLOPS, 4)
    best["prefill_kernel_frac_of_gemm"] = round(attn_tflops / best["TFLOPs"], 4)
    return best


def bench_segmented(args, torch, psw, splits=4, reps=20):
    """The non-causal chunk-lookback workload (2 x 4,096 tokens, 8 heads, d 128)
    unsplit and with each query block's tile loop cut into `splits` segmented
    pieces merged by the LSE combine.  Reports both times; not part of the step."""
    from tests.gpu_setup import GpuWorkload
    from workloads import make_config
    w = make_config(4)
    gw = GpuWorkload(w)
    N, Hq, D = w.num_tokens, w.num_q_heads, w.head_dim_v
    kw = dict(scale=w.scale, window=w.window, causal=w.causal, chunk_size=w.chunk_size,
              chunk_lookback=w.chunk_lookback, mm_ranges=gw.mm_ranges)
    out = torch.empty((N, Hq, D), dtype=torch.bfloat16, device="cuda")
    parts = torch.empty((splits, N, Hq, D), dtype=torch.bfloat16, device="cuda")
    lses = torch.empty((splits, N, Hq), dtype=torch.float32, device="cuda")
    pl = [parts[j].view(N * Hq, D) for j in range(splits)]
    ll = [lses[j].view(N * Hq) for j in range(splits)]

    def unsplit():
        psw.swa_mm_attention(gw.q, gw.k_cache, gw.v_cache, gw.block_table, gw.qsl, gw.seq_lens,
                             out=out, **kw)

    def segmented():
        psw.swa_mm_attention(gw.q, gw.k_cache, gw.v_cache, gw.block_table, gw.qsl, gw.seq_lens,
                             out=parts, lse=lses, num_splits=splits, **kw)
        psw.lse_combine(pl, ll, out=out.view(N * Hq, D))

    res = {"workload": "noncausal_chunk_lookback_2x4096", "splits": splits}
    for name, fn in (("unsplit_ms", unsplit), ("segmented_with_combine_ms", segmented)):
        warm(torch, fn, min_ms=args.warm_ms / 4)
        res[name] = round(timed_events(torch, fn, reps), 5)
    del gw
    torch.cuda.empty_cache()
    return res


def bench_slot_mapping(args, torch, psw, np, num_reqs=20000, seed=7):
    """Slot mapping over a 41 M-token batch (not one of the workloads: at their
    sizes the kernel moves under 0.3 MB and only latency shows).  Algorithmic
    bytes: 8 B position read + 4 B slot written per token, the block-table
    entries of the blocks touched, and 4 B per pad slot.  For scale, the same
    run times torch's int64 -> int32 copy of the positions (the same 8 B read
    and 4 B written per token): the plateau a streaming kernel of this shape
    reaches on this GPU."""
    from tests.gpu_setup import i32, i64
    from workloads.synth import make_slot_batch
    B = 16
    qsl, pos, bt = make_slot_batch(num_reqs, 1024, 3072, B, seed)
    n = int(qsl[-1])
    m = n + 65536
    need = int((bt >= 0).sum())
    d_qsl, d_pos, d_bt = i32(qsl), i64(pos), i32(bt)
    out = torch.empty(m, dtype=torch.int32, device="cuda")
    run = lambda: psw.slot_mapping(d_qsl, d_pos, d_bt, B, m, out=out)  # noqa: E731
    warm(torch, run, min_ms=args.warm_ms / 4)
    ms = timed_events(torch, run, reps=20)
    alg = n * 12 + need * 4 + (m - n) * 4
    gbs = alg / (ms * 1e-3) / 1e9
    cast = torch.empty(n, dtype=torch.int32, device="cuda")
    cp = lambda: cast.copy_(d_pos)  # noqa: E731
    warm(torch, cp, min_ms=args.warm_ms / 4)
    ms_copy = timed_events(torch, cp, reps=20)
    gbs_copy = n * 12 / (ms_copy * 1e-3) / 1e9
    res = {"tokens": n, "max_num_tokens": m, "requests": num_reqs, "block_size": B,
           "ms": round(ms, 5), "algorithmic_bytes": alg, "GBps": round(gbs, 1),
           "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
           "int64_to_int32_copy": {"ms": round(ms_copy, 5), "bytes": n * 12,
                                   "GBps": round(gbs_copy, 1),
                                   "frac_of_hbm_peak": round(gbs_copy / HBM_PEAK_GBS, 4)},
           "frac_of_copy": round(gbs / gbs_copy, 4)}

    # the same batch on rank 3 of an 8-rank context-parallel group (interleave 16,
    # 64-token KV blocks): each rank's table holds only its own logical blocks
    world, rank, inter, kvb = 8, 3, 16, 64
    lens = np.diff(qsl)
    need_cp = -(-lens // (kvb * world)) * (kvb // B)
    rng = np.random.default_rng(seed + 1)
    bt_cp = np.full((num_reqs, int(need_cp.max())), -1, dtype=np.int32)
    perm = rng.permutation(int(need_cp.sum())).astype(np.int32)
    starts = np.concatenate([[0], np.cumsum(need_cp)])
    for r in range(num_reqs):
        bt_cp[r, :need_cp[r]] = perm[starts[r]:starts[r + 1]]
    d_bt_cp = i32(bt_cp)

    def run_cp():
        psw.slot_mapping_cp(d_qsl, d_pos, d_bt_cp, B, m, kv_cache_block_size=kvb,
                            cp_world_size=world, cp_rank=rank, cp_interleave=inter, out=out)
    warm(torch, run_cp, min_ms=args.warm_ms / 4)
    ms_cp = timed_events(torch, run_cp, reps=20)
    alg_cp = n * 12 + int(need_cp.sum()) * 4 + (m - n) * 4
    gbs_cp = alg_cp / (ms_cp * 1e-3) / 1e9
    res["context_parallel_rank"] = {
        "cp_world_size": world, "cp_rank": rank, "cp_interleave": inter,
        "kv_cache_block_size": kvb, "ms": round(ms_cp, 5), "algorithmic_bytes": alg_cp,
        "GBps": round(gbs_cp, 1), "frac_of_hbm_peak": round(gbs_cp / HBM_PEAK_GBS, 4)}
    del d_pos, out, cast
    torch.cuda.empty_cache()
    return res


def bench_decode(args, torch, psw, np):
    from tests.gpu_setup import DecodeStep
    from workloads import make_config

    w = make_config(5, decode_splits=args.decode_splits)
    log("decode workload generated")
    pdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[args.decode_partials]
    ds = DecodeStep(w, partial_dtype=pdt)
    R, H, DV = w.num_seqs, w.num_q_heads, w.head_dim_v
    steps = max(args.steps, 10)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]

    def one_call():
        ds.attention()
        ds.combine()

    # first, so that the decode kernel's last launches are the timed steps below;
    # one step writes the current keys into the cache
    ds.run()
    two = None
    if not args.skip_extra:
        log("timing decode on two streams")
        two = bench_two_streams(args, torch, psw, np, ds, one_call)
    log("timing decode")
    for _ in range(args.warmup):
        ds.run()
    warm_ms = warm(torch, ds.run, min_ms=args.warm_ms)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    # the step time with no event recorded between launches (four records per
    # step add about 10 us of stream time), then the same steps with events
    # around the attention call and the tail
    t0.record()
    for _ in range(steps):
        ds.run()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    for i in range(steps):
        ds.run(ev[i])
    torch.cuda.synchronize()
    attn_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    tail_ms = sum(e[1].elapsed_time(e[3]) for e in ev) / steps
    kv_bytes = int(w.seq_lens.sum()) * w.head_dim_qk * 2
    part_bytes = ds.part_o.numel() * ds.part_o.element_size() + ds.part_l.numel() * 4
    # the tail reads the partials and W_UV and writes the projected output, the
    # merged rows and their LSEs
    tail_bytes = (part_bytes + ds.w_uv.numel() * 2 + ds.vup_out.numel() * 2 + ds.out.numel() * 2
                  + ds.out_lse.numel() * 4)
    # KV rows once + Q + block table + W_UV + the projected output (the merged
    # latent output is an intermediate)
    alg_bytes = (kv_bytes + ds.q.numel() * 2 + w.block_table.size * 4 + ds.w_uv.numel() * 2
                 + ds.vup_out.numel() * 2)
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    attn_gbs = (kv_bytes + ds.q.numel() * 2) / (attn_ms * 1e-3) / 1e9
    # the same tail as two launches (combine, then projection), timed apart
    comb_bytes = part_bytes + ds.out.numel() * 2 + ds.out_lse.numel() * 4
    vup_bytes = ds.out.numel() * 2 + ds.w_uv.numel() * 2 + ds.vup_out.numel() * 2
    warm(torch, ds.combine, min_ms=args.warm_ms / 4)
    comb_ms = timed_events(torch, ds.combine, 20)
    vup = lambda: psw.vup_projection(ds.out, ds.w_uv, out=ds.vup_out)  # noqa: E731
    warm(torch, vup, min_ms=args.warm_ms / 4)
    vup_ms = timed_events(torch, vup, 20)

    def two_tail():
        ds.combine()
        vup()
    warm(torch, two_tail, min_ms=args.warm_ms / 4)
    two_tail_ms = timed_events(torch, two_tail, 20)
    step_two = lambda: ds.run(fused_tail=False)  # noqa: E731
    warm(torch, step_two, min_ms=args.warm_ms / 2)
    step_two_ms = timed_events(torch, step_two, steps, rounds=3)
    res = {
        "workload": "mla_splitkv_decode_b64",
        "unit": "GB/s",
        "value": round(gbs, 1),
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "ms_per_step": round(ms, 5),
        "algorithmic_bytes_per_step": alg_bytes,
        "attention_ms": round(attn_ms, 5),
        "attention_GBps": round(attn_gbs, 1),
        "attention_frac_of_hbm_peak": round(attn_gbs / HBM_PEAK_GBS, 4),
        "combine_vup": {"ms": round(tail_ms, 5), "bytes": tail_bytes,
                        "GBps": round(tail_bytes / (tail_ms * 1e-3) / 1e9, 1),
                        "what": f"lse_combine_vup: {ds.P} partials ({args.decode_partials}) "
                                "merged and projected in one launch (merged rows and LSEs "
                                "written too)"},
        "tail_as_two_launches": {
            "ms": round(two_tail_ms, 5),
            "step_ms": round(step_two_ms, 5),
            "combine": {"ms": round(comb_ms, 5), "bytes": comb_bytes,
                        "GBps": round(comb_bytes / (comb_ms * 1e-3) / 1e9, 1)},
            "vup_projection": {"ms": round(vup_ms, 5), "bytes": vup_bytes,
                               "GBps": round(vup_bytes / (vup_ms * 1e-3) / 1e9, 1),
                               "shape": f"[{R}, {H}, {DV}] x [{H}, {DV}, {ds.dv_up}]"}},
        "history_splits": ds.S,
        "partials": ds.P,
        "partial_dtype": args.decode_partials,
        "clock_state": f"steady: {warm_ms:.0f} ms of back-to-back steps before the timed ones",
        "step": "slot_mapping + kv_cache_write + history and current partials (one call) "
                "+ lse_combine_vup (LSE combine and V-up projection in one launch)",
    }
    if two is not None:
        res["two_streams"] = two
    return res


def bench_two_streams(args, torch, psw, np, ds, one_call, reps=20, rounds=5):
    """Attention + combine of the decode step four ways: the history splits and
    the current key as ranges of one call; history then current as two calls on
    one stream; history on the main stream and current on a side stream with
    separate workspaces (they may overlap) or one shared workspace (current
    after history), joined before the combine."""
    w = ds.w
    DV, S = w.head_dim_v, ds.S
    hist, cur = ds.kr_all[:S].contiguous(), ds.kr_all[S:].contiguous()
    side = torch.cuda.Stream()
    kw = dict(scale=w.scale, window=0, causal=True, head_dim_v=DV)
    q, cache, bt, qsl, seq_lens, pdt, out = (ds.q, ds.cache, ds.bt, ds.qsl, ds.seq_lens, ds.pdt,
                                             ds.out)

    def two_calls():
        ho, hl = psw.swa_mm_attention(q, cache, None, bt, qsl, seq_lens, key_ranges=hist,
                                      out_dtype=pdt, return_lse=True, **kw)
        co, cl = psw.swa_mm_attention(q, cache, None, bt, qsl, seq_lens, key_ranges=cur,
                                      out_dtype=pdt, return_lse=True, **kw)
        rows = q.shape[0] * q.shape[1]
        psw.lse_combine([ho[j].view(rows, DV) for j in range(S)] + [co[0].view(rows, DV)],
                        [hl[j].view(rows) for j in range(S)] + [cl[0].view(rows)], out=out)

    def streams(shared):
        return lambda: psw.decode_two_streams(q, cache, None, bt, qsl, seq_lens,
                                              history_ranges=hist, current_ranges=cur,
                                              side_stream=side, partial_dtype=pdt,
                                              shared_workspace=shared, out=out, **kw)

    # round-robin rounds, median per variant: the first timings of a run are
    # slower while the clocks settle, which would favour whatever runs last
    variants = {"one_call_ms": one_call, "two_calls_one_stream_ms": two_calls,
                "two_streams_separate_workspaces_ms": streams(False),
                "two_streams_shared_workspace_ms": streams(True)}
    times = {k: [] for k in variants}
    for fn in variants.values():
        warm(torch, fn, min_ms=30.0)
    for _ in range(rounds):
        for k, fn in variants.items():
            times[k].append(timed_events(torch, fn, reps, rounds=1))
    res = {k: round(float(np.median(v)), 5) for k, v in times.items()}
    res["what"] = (f"attention + lse_combine of the decode step, median of {rounds} "
                   f"round-robin rounds of {reps} calls")
    return res


if __name__ == "__main__":
    main()
