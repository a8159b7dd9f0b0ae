"""The bench's steps captured in a HIP graph (torch.cuda.CUDAGraph): the
decode step (slot mapping, latent KV write, one attention call with a fixed
workspace, LSE combine, V-up projection), the same decode attention through
the allocation-free entry point, and the prefill step (slot mapping, then the
attention launch with the KV-cache write fused in).  The decode of the pages
runs in graph mode, where the two partial calls share one preallocated
workspace whose address capture fixes ([DCP] stage 1, section 1.2 and figure
2; stage 2, section 2.1 keeps that capture logic unchanged); the library
allocates nothing and issues no memset, so its launches can be recorded.
Each graph is replayed several times, with eager calls and synchronisations
between the replays, and every replay must reproduce the eager step bit for
bit."""
import numpy as np
import pytest
import torch

import paged_sliding_window_amd as psw
from tests.gpu_setup import DecodeStep, GpuWorkload, bits_to_bf16
from workloads import make_config

pytestmark = pytest.mark.gpu


def _replays_match_eager(step, outs, replays=3):
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one eager call on a side stream before capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i in range(replays):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), f"replay {i}: output {j} differs from the eager step"
        step()  # the program's own eager work between replays
        torch.cuda.synchronize()
    del g


def test_decode_step_in_a_graph():
    ds = DecodeStep(make_config(5, decode_splits=1))
    _replays_match_eager(ds.run, [ds.part_o, ds.part_l, ds.out, ds.out_lse, ds.vup_out,
                                  ds.slots])


def test_noalloc_decode_attention_in_a_graph():
    ds = DecodeStep(make_config(5, decode_splits=2))
    w = ds.w

    def step():
        psw.swa_mm_attention_noalloc(ds.q, ds.cache, None, ds.bt, ds.qsl, ds.seq_lens,
                                     out=ds.part_o, lse=ds.part_l, scale=w.scale, window=0,
                                     causal=True, key_ranges=ds.kr_all, head_dim_v=w.head_dim_v)
        ds.combine()

    _replays_match_eager(step, [ds.part_o, ds.part_l, ds.out, ds.out_lse])


def test_fused_prefill_step_in_a_graph():
    w = make_config(2)
    gw = GpuWorkload(w, fill_cache=False)
    k_new = bits_to_bf16(np.concatenate(w.k_bits))
    v_new = bits_to_bf16(np.concatenate(w.v_bits))
    slots = torch.empty(w.max_num_tokens, dtype=torch.int32, device="cuda")
    out = torch.empty((w.num_tokens, w.num_q_heads, w.head_dim_v), dtype=torch.bfloat16,
                      device="cuda")
    lse = torch.empty((w.num_tokens, w.num_q_heads), dtype=torch.float32, device="cuda")

    def step():
        psw.slot_mapping(gw.qsl, gw.positions, gw.block_table, w.block_size, w.max_num_tokens,
                         out=slots)
        psw.swa_mm_attention_kv_write(gw.q, k_new, v_new, slots, gw.k_cache, gw.v_cache,
                                      gw.block_table, gw.qsl, gw.seq_lens, scale=w.scale,
                                      window=w.window, causal=w.causal, mm_ranges=gw.mm_ranges,
                                      out=out, lse=lse)

    _replays_match_eager(step, [slots, out, lse, gw.k_cache, gw.v_cache])
