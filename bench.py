"""Benchmark of the paged sliding-window + clamped image-range hot path on one GPU.

One step = the whole path over one synthetic batch of the Gemma-style
multimodal prefill (16,550 tokens, 60 images of 256 tokens, W 1024, 16 query /
8 KV heads, head dim 256, paged in blocks of 16):
  slot mapping of the new tokens -> KV-cache write -> paged prefill attention.
The decode half of the path (MLA-shaped split-KV decode: 64 requests, 128 heads,
576/512 latent, history partial(s) + the current key's partial from one call,
LSE combine) is timed in the same run and reported under "decode".

Reported value: algorithmic TFLOP/s = 4 * head_dim FLOP per allowed
(query, key, head) triple, 3.0115e11 per step, over the measured step time.
The "roofline" object is for the dominant kernel (prefill attention), timed
with HIP events around each of its launches on the stream it runs on.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E


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


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the GPU's clocks ramp up over the first ~25 ms of sustained load (a
    # 16,550-token prefill launch drops from 0.48 to 0.37 ms over its first ~60
    # launches, and climbs back after 2 s idle): 200 steps are ~100 ms
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--skip-cpu", action="store_true", help="omit the CPU oracle baseline")
    ap.add_argument("--skip-decode", action="store_true", help="omit the decode half")
    ap.add_argument("--decode-splits", type=int, default=1)
    ap.add_argument("--decode-partials", choices=["f32", "bf16"], default="bf16",
                    help="dtype of the history/current partial outputs")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="first run one plain device copy of this many bytes (a known-size "
                         "kernel to calibrate HBM byte counters against)")
    return ap.parse_args()


def allowed_pairs_per_head(w, r):
    """Allowed (query, key) pairs of request r for one head: each causal row's
    allowed keys form one interval (window part and image part both contain the
    query position), so the count is the interval length."""
    total = 0
    ctx = int(w.context_lens[r])
    L = int(w.seq_lens[r])
    ranges = [(s, e) for s, e in w.ranges_of(r) if s < e]
    W = w.window
    for i in range(int(w.query_lens[r])):
        q = ctx + i
        lo = max(0, q - W + 1) if W > 0 else 0
        hi = q
        for s, e in ranges:
            if s <= q <= e:
                lo = min(lo, max(s, q - W + 1) if W > 0 else s)
                hi = max(hi, e)
        total += min(hi, L - 1) - lo + 1
    return total


def prefill_flop(w):
    pairs = sum(allowed_pairs_per_head(w, r) for r in range(w.num_seqs))
    return pairs * w.num_q_heads * 4 * w.head_dim_qk, pairs


def cpu_baseline(w):
    """The oracle (as written) on the whole prefill workload, repeated until at
    least 10 s of CPU time have been spent (at most 5 passes)."""
    from threadpoolctl import threadpool_info

    from oracle import attention_ref
    q = w.q_f32()
    k, v = w.k_f32(0), w.v_f32(0)
    flop, _ = prefill_flop(w)
    passes, t0 = 0, time.perf_counter()
    while True:
        attention_ref(q, k, v, context_len=0, seq_len=int(w.seq_lens[0]), scale=w.scale,
                      window=w.window, causal=w.causal, ranges=w.ranges_of(0))
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or passes >= 5:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(flop * passes / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"float64 numpy oracle over the whole 16,550-token prefill (all 16 heads), "
                      f"{passes} pass(es) in {dt:.2f} s"}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_attention_gemma16550_traffic.json")
PREFILL_SOURCES = ["attention_prefill.hip", "asm_ops.h", "device_common.h", "mask_bounds.h",
                   "psw_internal.h"]


def measured_traffic():
    """HBM bytes per prefill launch from the committed counter runs, or None when
    the kernel sources differ from the ones the counters were taken on."""
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
    from tests.gpu_setup import GpuWorkload, bits_to_bf16, i32, i64
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

    def prefill_step(i=None):
        psw.slot_mapping(gw.qsl, gw.positions, gw.block_table, w.block_size, w.max_num_tokens,
                         out=slots)
        psw.kv_cache_write(k_new, v_new, slots, gw.k_cache, gw.v_cache)
        if i is not None:
            ev[i][0].record()
        psw.swa_mm_attention(gw.q, gw.k_cache, gw.v_cache, gw.block_table, gw.qsl, gw.seq_lens,
                             scale=w.scale, window=w.window, causal=w.causal,
                             mm_ranges=gw.mm_ranges, out=out, lse=lse)
        if i is not None:
            ev[i][1].record()

    log("timing prefill")
    for _ in range(args.warmup):
        prefill_step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        prefill_step(i)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / args.steps
    attn_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (attn_ms * 1e-3) / 1e12

    result = {
        "metric": "SWA+MM-prefix prefill attn TFLOP/s (% MFMA peak); paged decode HBM GB/s",
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
            "step": "slot_mapping + kv_cache_write + swa_mm_attention",
        },
        "roofline": {
            "kernel": "prefill_attention_kernel<PrefillShape<256, 4, 2>>",
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(),
            "avg_launch_ms": round(attn_ms, 5),
        },
    }
    del gw, k_new, v_new, out, lse
    torch.cuda.empty_cache()

    # ---------------- decode (second half of the path) ----------------
    log(f"prefill {ms_per_step:.4f} ms/step, attention {attn_ms:.4f} ms")
    if not args.skip_decode:
        log("decode half")
        result["decode"] = bench_decode(args, torch, psw, np)

    log("segmented splits, non-causal workload")
    result["prefill_segmented"] = bench_segmented(torch, psw)
    log("slot mapping, scaled batch")
    result["slot_mapping_scaled"] = bench_slot_mapping(torch, psw, np)
    if not args.skip_cpu:
        log("CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(w)
    result["setup_s"] = round(time.perf_counter() - t_setup, 1)
    print(json.dumps(result), flush=True)


def bench_segmented(torch, psw, splits=4, reps=20):
    """The non-causal chunk-lookback workload (2 x 4,096 tokens, 8 heads, d 128):
    with 128-row query blocks it has 528 workgroups, one round of the GPU's
    512 slots plus a few; segmented splits (each block's tile loop cut into
    `splits` pieces, merged by the LSE combine) spread the same tiles over
    more, shorter workgroups.  Reports both times; not part of the step."""
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
        warm(torch, fn)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(e0.elapsed_time(e1) / reps, 5)
    del gw
    torch.cuda.empty_cache()
    return res


def bench_slot_mapping(torch, psw, np, num_reqs=4096, seed=7):
    """Slot mapping over a large synthetic batch (not one of the workloads: at
    their sizes the kernel moves under 0.3 MB and only latency shows).
    Algorithmic bytes: 8 B position read + 4 B slot written per token, the
    block-table entries of the blocks touched, and 4 B per pad slot."""
    from tests.gpu_setup import i32, i64
    rng = np.random.default_rng(seed)
    B = 16
    lens = rng.integers(512, 2049, size=num_reqs)
    need = -(-lens // B)
    stride = int(need.max())
    bt = np.full((num_reqs, stride), -1, dtype=np.int32)
    perm = rng.permutation(int(need.sum())).astype(np.int32)
    off = 0
    for r in range(num_reqs):
        bt[r, :need[r]] = perm[off:off + need[r]]
        off += need[r]
    qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pos = np.concatenate([np.arange(L) for L in lens]).astype(np.int64)
    n = int(qsl[-1])
    m = n + 65536
    d_qsl, d_pos, d_bt = i32(qsl), i64(pos), i32(bt)
    out = torch.empty(m, dtype=torch.int32, device="cuda")
    warm(torch, lambda: psw.slot_mapping(d_qsl, d_pos, d_bt, B, m, out=out))
    reps = 50
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        psw.slot_mapping(d_qsl, d_pos, d_bt, B, m, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    alg = n * 12 + int(need.sum()) * 4 + (m - n) * 4
    gbs = alg / (ms * 1e-3) / 1e9
    res = {"tokens": n, "max_num_tokens": m, "requests": num_reqs, "block_size": B,
           "ms": round(ms, 5), "algorithmic_bytes": alg, "GBps": round(gbs, 1),
           "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}

    # the same batch on rank 3 of an 8-rank context-parallel group (interleave 16,
    # 64-token KV blocks): each rank's table holds only its own logical blocks
    world, rank, inter, kvb = 8, 3, 16, 64
    need_cp = -(-lens // (kvb * world)) * (kvb // B)
    bt_cp = np.full((num_reqs, int(need_cp.max())), -1, dtype=np.int32)
    perm = rng.permutation(int(need_cp.sum())).astype(np.int32)
    off = 0
    for r in range(num_reqs):
        bt_cp[r, :need_cp[r]] = perm[off:off + need_cp[r]]
        off += need_cp[r]
    d_bt_cp = i32(bt_cp)

    def run_cp():
        psw.slot_mapping_cp(d_qsl, d_pos, d_bt_cp, B, m, kv_cache_block_size=kvb,
                            cp_world_size=world, cp_rank=rank, cp_interleave=inter, out=out)
    warm(torch, run_cp)
    e0.record()
    for _ in range(reps):
        run_cp()
    e1.record()
    torch.cuda.synchronize()
    ms_cp = e0.elapsed_time(e1) / reps
    alg_cp = n * 12 + int(need_cp.sum()) * 4 + (m - n) * 4
    gbs_cp = alg_cp / (ms_cp * 1e-3) / 1e9
    res["context_parallel_rank"] = {
        "cp_world_size": world, "cp_rank": rank, "cp_interleave": inter,
        "kv_cache_block_size": kvb, "ms": round(ms_cp, 5), "algorithmic_bytes": alg_cp,
        "GBps": round(gbs_cp, 1), "frac_of_hbm_peak": round(gbs_cp / HBM_PEAK_GBS, 4)}
    return res


def bench_decode(args, torch, psw, np):
    from tests.gpu_setup import bits_to_bf16, i32, i64
    from workloads import make_config
    from workloads.synth import decode_split_ranges

    w = make_config(5, decode_splits=args.decode_splits)
    log("decode workload generated")
    B = w.block_size
    R, H, DV = w.num_seqs, w.num_q_heads, w.head_dim_v
    q = bits_to_bf16(w.q_bits)
    bt = i32(w.block_table)
    qsl = i32(w.query_start_loc)
    seq_lens = i32(w.seq_lens)
    positions = i64(w.positions)
    cache = torch.empty((w.num_blocks, B, 1, w.head_dim_qk), dtype=torch.bfloat16, device="cuda")
    # context rows [0, L-1) go in before timing, through the library itself
    qsl_ctx = np.concatenate([[0], np.cumsum(w.seq_lens - 1)]).astype(np.int32)
    pos_ctx = np.concatenate([np.arange(int(L) - 1) for L in w.seq_lens]).astype(np.int64)
    slots_ctx = psw.slot_mapping(i32(qsl_ctx), i64(pos_ctx), bt, B, int(qsl_ctx[-1]))
    psw.kv_cache_write(bits_to_bf16(np.concatenate([k[:-1] for k in w.k_bits])), None, slots_ctx,
                       cache, None)
    new_rows = bits_to_bf16(np.stack([k[-1] for k in w.k_bits]))
    del slots_ctx
    # the history splits and the current key are the key ranges of ONE call: it
    # emits S + 1 partials (each with its LSE), S history pieces and the current
    # key's partial last, which lse_combine then merges
    S = w.key_ranges.shape[0]
    kr_all = i32(np.concatenate([w.key_ranges, w.current_ranges], axis=0))
    P = S + 1
    pdt = torch.float32 if args.decode_partials == "f32" else torch.bfloat16
    part_o = torch.empty((P, R, H, DV), dtype=pdt, device="cuda")
    part_l = torch.empty((P, R, H), dtype=torch.float32, device="cuda")
    out = torch.empty((R * H, DV), dtype=torch.bfloat16, device="cuda")
    slots = torch.empty(R, dtype=torch.int32, device="cuda")
    outs = [part_o[j].view(R * H, DV) for j in range(P)]
    lses = [part_l[j].view(R * H) for j in range(P)]
    ws_args = psw.ops._attn_args(q, cache, None, bt, qsl, seq_lens, scale=w.scale, window=0,
                                 causal=True, chunk_size=0, chunk_lookback=-1, mm_ranges=None,
                                 key_ranges=kr_all, out=part_o, lse=part_l, head_dim_v=DV,
                                 out_dtype=0, num_splits=P)
    ws = torch.empty(max(1, psw.ops.attention_workspace_size(ws_args)), dtype=torch.uint8,
                     device="cuda")
    # V-up projection of the merged output (128 heads x 512 -> 128 per head)
    dv_up = 128
    from workloads.synth import f32_to_bf16_bits
    w_uv = bits_to_bf16(f32_to_bf16_bits(
        np.random.default_rng(55).standard_normal((H, DV, dv_up)).astype(np.float32) / DV ** 0.5))
    vup_out = torch.empty((R, H * dv_up), dtype=torch.bfloat16, device="cuda")
    steps = max(args.steps, 10)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]

    def step(i=None):
        psw.slot_mapping(qsl, positions, bt, B, R, out=slots)
        psw.kv_cache_write(new_rows, None, slots, cache, None)
        if i is not None:
            ev[i][0].record()
        psw.swa_mm_attention(q, cache, None, bt, qsl, seq_lens, scale=w.scale, window=0,
                             causal=True, key_ranges=kr_all, head_dim_v=DV, out=part_o,
                             lse=part_l, out_dtype=pdt, workspace=ws)
        if i is not None:
            ev[i][1].record()
        psw.lse_combine(outs, lses, out=out)
        if i is not None:
            ev[i][2].record()
        psw.vup_projection(out, w_uv, out=vup_out)
        if i is not None:
            ev[i][3].record()

    def one_call():
        psw.swa_mm_attention(q, cache, None, bt, qsl, seq_lens, scale=w.scale, window=0,
                             causal=True, key_ranges=kr_all, head_dim_v=DV, out=part_o,
                             lse=part_l, out_dtype=pdt, workspace=ws)
        psw.lse_combine(outs, lses, out=out)

    # first, so that the decode kernel's last launches are the timed steps below;
    # one step writes the current keys into the cache
    step()
    log("timing decode on two streams")
    two = bench_two_streams(torch, psw, np, w, q, cache, bt, qsl, seq_lens, kr_all, S, pdt, out,
                            one_call)
    log("timing decode")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    attn_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    comb_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    vup_ms = sum(e[2].elapsed_time(e[3]) for e in ev) / steps
    vup_bytes = out.numel() * 2 + w_uv.numel() * 2 + vup_out.numel() * 2
    kv_bytes = int(w.seq_lens.sum()) * w.head_dim_qk * 2
    # KV rows once + Q + block table + W_UV + the projected output (the merged
    # latent output is an intermediate)
    alg_bytes = (kv_bytes + q.numel() * 2 + w.block_table.size * 4 + w_uv.numel() * 2
                 + vup_out.numel() * 2)
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    attn_gbs = (kv_bytes + q.numel() * 2) / (attn_ms * 1e-3) / 1e9
    return {
        "workload": "mla_splitkv_decode_b64",
        "unit": "GB/s",
        "value": round(gbs, 1),
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "ms_per_step": round(ms, 5),
        "algorithmic_bytes_per_step": alg_bytes,
        "attention_ms": round(attn_ms, 5),
        "attention_GBps": round(attn_gbs, 1),
        "combine_ms": round(comb_ms, 5),
        "vup_projection": {"ms": round(vup_ms, 5), "algorithmic_bytes": vup_bytes,
                           "GBps": round(vup_bytes / (vup_ms * 1e-3) / 1e9, 1),
                           "shape": f"[{R}, {H}, {DV}] x [{H}, {DV}, {dv_up}]"},
        "history_splits": S,
        "partials": P,
        "partial_dtype": args.decode_partials,
        "step": "slot_mapping + kv_cache_write + history and current partials (one call) "
                "+ lse_combine + vup_projection",
        "two_streams": two,
    }


def bench_two_streams(torch, psw, np, w, q, cache, bt, qsl, seq_lens, kr_all, S, pdt, out,
                      one_call, reps=20, rounds=5):
    """Attention + combine of the decode step four ways: the history splits and
    the current key as ranges of one call; history then current as two calls on
    one stream; history on the main stream and current on a side stream with
    separate workspaces (they may overlap) or one shared workspace (current
    after history), joined before the combine."""
    DV = w.head_dim_v
    hist, cur = kr_all[:S].contiguous(), kr_all[S:].contiguous()
    side = torch.cuda.Stream()
    kw = dict(scale=w.scale, window=0, causal=True, head_dim_v=DV)

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

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps

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
            times[k].append(timed(fn))
    res = {k: round(float(np.median(v)), 5) for k, v in times.items()}
    res["what"] = (f"attention + lse_combine of the decode step, median of {rounds} "
                   f"round-robin rounds of {reps} calls")
    return res


if __name__ == "__main__":
    main()
