"""GPU parity: latent (MLA-shaped) split-KV decode, history partials + current
partial merged by the LSE combine, against the float64 oracle."""
import numpy as np
import pytest
import torch

import paged_sliding_window_amd as psw
from oracle import lse_merge_ref
from tests.gpu_setup import (DecodeStep, GpuWorkload, assert_close, assert_lse_close, i32,
                             oracle_rows)
from workloads import make_config, make_small_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bench_decode_oracle():
    """Oracle of the decode workload as the bench runs it (history as one split
    [0, L-1), the current key [L-1, L)): per request the merged row, the
    history partial and the current partial, all 128 heads."""
    w = make_config(5, decode_splits=1)
    full, hist, cur = [], [], []
    for r in range(w.num_seqs):
        full.append(oracle_rows(w, r))
        hist.append(oracle_rows(w, r, key_range=tuple(w.key_ranges[0, r])))
        cur.append(oracle_rows(w, r, key_range=tuple(w.current_ranges[0, r])))
    return w, full, hist, cur


@pytest.mark.parametrize("pdt", [torch.bfloat16, torch.float16, torch.float32],
                         ids=["bf16", "f16", "f32"])
def test_bench_decode_step_full_size(bench_decode_oracle, pdt):
    """Exactly the decode step bench.py times (64 requests x 128 heads, one
    attention call over [history, current] key ranges, partials in pdt, LSE
    combine, V-up projection), run twice: every element of both partials and
    their LSEs, the merged output and LSE, and the projected output against the
    oracle ([DCP] stage 3 sections 3.1-3.2 and code blocks B-D; "Terms" and
    block A for the projection)."""
    from oracle import vup_projection_ref
    w, full, hist, cur = bench_decode_oracle
    ds = DecodeStep(w, partial_dtype=pdt)
    ds.run()
    ds.run()   # the step again on its own outputs: the cache write is idempotent
    torch.cuda.synchronize()
    R, H, DV = w.num_seqs, w.num_q_heads, w.head_dim_v
    po = ds.part_o.float().cpu().numpy()
    pl = ds.part_l.cpu().numpy()
    out = ds.out.float().cpu().numpy().reshape(R, H, DV)
    lse = ds.out_lse.cpu().numpy().reshape(R, H)
    merged_ref = np.zeros((R, H, DV))
    for r in range(R):
        assert_close(po[0, r], hist[r][0][0], f"history partial of {r}")
        assert_lse_close(pl[0, r], hist[r][1][0], f"history lse of {r}")
        assert_close(po[1, r], cur[r][0][0], f"current partial of {r}")
        assert_lse_close(pl[1, r], cur[r][1][0], f"current lse of {r}")
        assert_close(out[r], full[r][0][0], f"merged row of {r}")
        assert_lse_close(lse[r], full[r][1][0], f"merged lse of {r}")
        merged_ref[r] = full[r][0][0]
    proj = ds.vup_out.float().cpu().numpy().reshape(R, H, ds.dv_up)
    assert_close(proj, vup_projection_ref(merged_ref, ds.wuv_f32), "projected output")


def _decode(gw, w, partial_dtype=torch.float32):
    hist_o, hist_l = gw.attention(key_ranges=w.key_ranges, out_dtype=partial_dtype)
    cur_o, cur_l = gw.attention(key_ranges=w.current_ranges, out_dtype=partial_dtype)
    S = hist_o.shape[0]
    rows = w.num_tokens * w.num_q_heads
    outs = [hist_o[j].view(rows, w.head_dim_v) for j in range(S)] + [cur_o[0].view(rows, w.head_dim_v)]
    lses = [hist_l[j].view(rows) for j in range(S)] + [cur_l[0].view(rows)]
    lse_out = torch.empty(rows, dtype=torch.float32, device="cuda")
    out = psw.lse_combine(outs, lses, out_lse=lse_out)[0]
    return out, lse_out, hist_o, hist_l, cur_o, cur_l


def test_mla_decode_full_size():
    w = make_config(5)
    gw = GpuWorkload(w)
    out, lse, hist_o, hist_l, cur_o, cur_l = _decode(gw, w)
    out = out.float().cpu().numpy().reshape(w.num_tokens, w.num_q_heads, w.head_dim_v)
    lse = lse.cpu().numpy().reshape(w.num_tokens, w.num_q_heads)
    for r in range(w.num_seqs):
        ref_o, ref_l = oracle_rows(w, r)
        assert_close(out[r], ref_o[0], f"token {r}")
        assert_lse_close(lse[r], ref_l[0], f"token {r} lse")
    # the partials themselves, on a few requests
    ho, hl = hist_o.cpu().numpy(), hist_l.cpu().numpy()
    for r in (0, 17, 63):
        for j in range(w.key_ranges.shape[0]):
            ref_o, ref_l = oracle_rows(w, r, key_range=tuple(w.key_ranges[j, r]))
            assert_close(ho[j, r], ref_o[0], f"history split {j} of {r}")
            assert_lse_close(hl[j, r], ref_l[0], f"history split {j} of {r} lse")
        ref_o, ref_l = oracle_rows(w, r, key_range=tuple(w.current_ranges[0, r]))
        assert_close(cur_o[0, r].cpu().numpy(), ref_o[0], f"current of {r}")


@pytest.mark.parametrize("seed,pdt", [(0, torch.bfloat16), (1, torch.bfloat16), (2, torch.float16),
                                      (3, torch.float16)])
def test_small_latent_decode_half_partials(seed, pdt):
    # one new token per request: the last position of each request
    w = _small_decode_case(900 + seed)
    gw = GpuWorkload(w)
    out, lse, *_ = _decode(gw, w, partial_dtype=pdt)
    out = out.float().cpu().numpy().reshape(w.num_tokens, w.num_q_heads, w.head_dim_v)
    for r in range(w.num_seqs):
        ref_o, _ = oracle_rows(w, r)
        assert_close(out[r], ref_o[0], f"token {r}")


@pytest.mark.parametrize("P,pdt,odt", [(1, torch.float32, torch.bfloat16),
                                        (9, torch.float32, torch.bfloat16),
                                        (9, torch.bfloat16, torch.float32),
                                        (9, torch.float16, torch.bfloat16),
                                        (9, torch.float16, torch.float16),
                                        (2, torch.bfloat16, torch.float16),
                                        (64, torch.float32, torch.float32)])
def test_lse_combine_random_partials(P, pdt, odt):
    rng = np.random.default_rng(P)
    rows, dv = 777, 512 if P < 64 else 64
    outs = [rng.standard_normal((rows, dv)).astype(np.float32) for _ in range(P)]
    lses = [rng.normal(0, 4, rows).astype(np.float32) for _ in range(P)]
    for l in lses:
        l[rng.random(rows) < 0.3] = -np.inf
    lses[0][:5] = -np.inf
    for l in lses:
        l[:5] = -np.inf            # rows with every partial empty
    t_outs = [torch.from_numpy(o).cuda().to(pdt) for o in outs]
    ref_in = [t.float().cpu().numpy() for t in t_outs]   # what the kernel actually reads
    t_lses = [torch.from_numpy(l).cuda() for l in lses]
    out_lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    out, ol = psw.lse_combine(t_outs, t_lses, out_lse=out_lse, out_dtype=odt)
    ref_o, ref_l = lse_merge_ref(ref_in, lses)
    assert_close(out.float().cpu().numpy(), ref_o, "combine out")
    assert_lse_close(ol.cpu().numpy(), ref_l, "combine lse")


def _keep_last_tokens(w, k):
    """Keep the last (up to) k new tokens of every request: a decode step with
    several new tokens per request (the earlier ones become cached context)."""
    keep, qls = [], []
    for r in range(w.num_seqs):
        t0, t1 = int(w.query_start_loc[r]), int(w.query_start_loc[r + 1])
        n = min(k, t1 - t0)
        keep.extend(range(t1 - n, t1))
        qls.append(n)
    keep = np.array(keep)
    w.q_bits = w.q_bits[keep]
    w.positions = w.positions[keep]
    w.query_lens = np.array(qls, dtype=np.int64)
    w.context_lens = w.seq_lens - w.query_lens
    w.query_start_loc = np.concatenate([[0], np.cumsum(qls)]).astype(np.int32)
    return w


# Latent decode under the balanced (stream-K) schedule: blocks of 16 keys (a tile
# spans two blocks), 32 / 64 / 128 heads per KV head, sliding windows and image
# ranges (splits that the mask empties), several new tokens per request, and
# more than 1,024 (token, split) items.
@pytest.mark.parametrize("case", [
    dict(seed=951, num_seqs=6, max_len=1500, hq=128, block_size=16, window=100, max_ranges=3,
         splits=4, tokens=3),
    dict(seed=952, num_seqs=4, max_len=2500, hq=64, block_size=64, window=0, max_ranges=0,
         splits=3, tokens=2),
    dict(seed=953, num_seqs=5, max_len=900, hq=32, block_size=32, window=33, max_ranges=2,
         splits=2, tokens=4),
    dict(seed=954, num_seqs=64, max_len=400, hq=32, block_size=64, window=0, max_ranges=0,
         splits=8, tokens=3),
], ids=["bs16_window_images", "qpk64", "qpk32_window", "over_1024_items"])
def test_latent_decode_scheduling(case):
    from workloads.synth import decode_split_ranges
    c = dict(case)
    splits, tokens = c.pop("splits"), c.pop("tokens")
    w = make_small_case(c.pop("seed"), hkv=1, d=576, dv=512, causal=True, chunk=(0, -1),
                        latent=True, **c)
    w = _keep_last_tokens(w, tokens)
    w.key_ranges = decode_split_ranges(w.seq_lens, splits)
    w.current_ranges = np.stack([np.stack([w.seq_lens - 1, w.seq_lens], 1)]).astype(np.int32)
    if case["seed"] == 954:
        assert w.num_tokens * splits > 1024
    gw = GpuWorkload(w)
    out, lse, hist_o, hist_l, cur_o, cur_l = _decode(gw, w)
    out = out.float().cpu().numpy().reshape(w.num_tokens, w.num_q_heads, w.head_dim_v)
    ho, hl = hist_o.cpu().numpy(), hist_l.cpu().numpy()
    for r in range(w.num_seqs):
        t0, t1 = w.query_start_loc[r], w.query_start_loc[r + 1]
        ref_o, _ = oracle_rows(w, r)
        assert_close(out[t0:t1], ref_o, f"merged, request {r}")
        for j in range(splits):
            ref_o, ref_l = oracle_rows(w, r, key_range=tuple(w.key_ranges[j, r]))
            assert_close(ho[j, t0:t1], ref_o, f"split {j} of request {r}")
            assert_lse_close(hl[j, t0:t1], ref_l, f"split {j} of request {r} lse")


def _small_decode_case(seed, num_seqs=5, splits=4):
    from workloads.synth import decode_split_ranges
    w = make_small_case(seed, num_seqs=num_seqs, max_len=3000, hq=64, hkv=1, d=576, dv=512,
                        window=0, causal=True, chunk=(0, -1), max_ranges=0, latent=True,
                        block_size=64)
    last = w.query_start_loc[1:] - 1
    w.q_bits = w.q_bits[last]
    w.positions = (w.seq_lens - 1).astype(np.int64)
    w.context_lens = w.seq_lens - 1
    w.query_lens = np.ones(w.num_seqs, dtype=np.int64)
    w.query_start_loc = np.arange(w.num_seqs + 1, dtype=np.int32)
    w.key_ranges = decode_split_ranges(w.seq_lens, splits)
    w.current_ranges = np.stack([np.stack([w.seq_lens - 1, w.seq_lens], 1)]).astype(np.int32)
    return w


@pytest.mark.parametrize("case", ["full", "small"])
@pytest.mark.parametrize("shared", [False, True])
def test_two_stream_decode(case, shared):
    """History partials on the main stream, the current partial on a side
    stream, joined before the LSE combine ([DCP] 2.1 stream swap, 3.2, blocks C
    and D): bit-identical to the same three calls in order on one stream, with
    the current call overlapping the history call (separate workspaces) or
    ordered after it (one shared workspace), over repeated calls with other
    work in between; and the merged rows equal the oracle."""
    w = make_config(5) if case == "full" else _small_decode_case(950)
    gw = GpuWorkload(w)
    ref_out, ref_lse, ref_ho, ref_hl, ref_co, ref_cl = _decode(gw, w, partial_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    hr, cr = i32(w.key_ranges), i32(w.current_ranges)
    for rep in range(3):
        out, lse, (ho, hl), (co, cl) = psw.decode_two_streams(
            gw.q, gw.k_cache, None, gw.block_table, gw.qsl, gw.seq_lens, history_ranges=hr,
            current_ranges=cr, side_stream=side, scale=w.scale, window=w.window, causal=w.causal,
            head_dim_v=w.head_dim_v, partial_dtype=torch.bfloat16, shared_workspace=shared)
        torch.cuda.synchronize()
        for name, got, ref in (("out", out, ref_out), ("lse", lse, ref_lse), ("history", ho, ref_ho),
                               ("history lse", hl, ref_hl), ("current", co, ref_co),
                               ("current lse", cl, ref_cl)):
            assert torch.equal(got.view(-1), ref.view(-1)), f"{name} differs on call {rep}"
        # unrelated eager work on the main stream between calls
        torch.randn(1 << 20, device="cuda").sum().item()
    out = out.float().cpu().numpy().reshape(w.num_tokens, w.num_q_heads, w.head_dim_v)
    lse = lse.cpu().numpy().reshape(w.num_tokens, w.num_q_heads)
    for r in ((0, 31, 63) if case == "full" else range(w.num_seqs)):
        ref_o, ref_l = oracle_rows(w, r)
        assert_close(out[r], ref_o[0], f"token {r}")
        assert_lse_close(lse[r], ref_l[0], f"token {r} lse")


def test_two_stream_decode_on_one_stream():
    """main stream == side stream: the three steps in order on that stream."""
    w = _small_decode_case(951, num_seqs=3, splits=2)
    gw = GpuWorkload(w)
    ref_out, ref_lse, *_ = _decode(gw, w, partial_dtype=torch.bfloat16)
    main = torch.cuda.current_stream()
    out, lse, _, _ = psw.decode_two_streams(
        gw.q, gw.k_cache, None, gw.block_table, gw.qsl, gw.seq_lens,
        history_ranges=i32(w.key_ranges), current_ranges=i32(w.current_ranges), side_stream=main,
        scale=w.scale, window=w.window, causal=w.causal, head_dim_v=w.head_dim_v,
        partial_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(out.view(-1), ref_out.view(-1)) and torch.equal(lse, ref_lse)
