"""GPU parity: psw_lse_combine_vup, the LSE merge of the latent partials and the
V-up projection of the merged rows in one launch ([DCP] code blocks D and A).

Two bars: bit for bit the two-launch chain psw_lse_combine (bf16 output) ->
psw_vup_projection on the same inputs (output, merged LSE and merged rows),
and within 2e-2 + 2e-2 |ref| of the float64 oracle lse_merge_ref ->
vup_projection_ref (the merged rows are rounded to bf16 before the projection,
as the two-launch chain does).
"""
import numpy as np
import pytest
import torch

import paged_sliding_window_amd as psw
from oracle import lse_merge_ref, vup_projection_ref
from tests.gpu_setup import assert_close, assert_lse_close, bits_to_bf16
from workloads.synth import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _inputs(seed, P, T, H, R, Dv, pdt):
    rng = np.random.default_rng(seed)
    rows = T * H
    outs = [torch.from_numpy(rng.standard_normal((T, H, R)).astype(np.float32)).cuda().to(pdt)
            for _ in range(P)]
    lses = [rng.normal(0, 4, rows).astype(np.float32) for _ in range(P)]
    for l in lses:
        l[rng.random(rows) < 0.25] = -np.inf     # empty partials
    for l in lses:
        l[:3] = -np.inf                          # rows with every partial empty
    lses = [torch.from_numpy(l).cuda() for l in lses]
    wb = f32_to_bf16_bits((rng.standard_normal((H, R, Dv)) * R ** -0.5).astype(np.float32))
    return outs, lses, bits_to_bf16(wb), bf16_bits_to_f32(wb)


CASES = [(1, torch.bfloat16, 1, 1, 128, 64), (2, torch.bfloat16, 64, 128, 512, 128),
         (2, torch.float16, 64, 128, 512, 128), (2, torch.float32, 64, 128, 512, 128),
         (3, torch.float32, 5, 3, 256, 128), (5, torch.bfloat16, 70, 4, 512, 192),
         (8, torch.float16, 130, 2, 128, 64), (9, torch.float32, 33, 16, 256, 256),
         (16, torch.bfloat16, 64, 128, 512, 128)]


@pytest.mark.parametrize("P,pdt,T,H,R,Dv", CASES)
def test_matches_two_launches_bit_for_bit(P, pdt, T, H, R, Dv):
    outs, lses, w_uv, _ = _inputs(P * 100 + T, P, T, H, R, Dv, pdt)
    rows = T * H
    flat = [o.view(rows, R) for o in outs]
    m2 = torch.empty((rows, R), dtype=torch.bfloat16, device="cuda")
    l2 = torch.empty(rows, dtype=torch.float32, device="cuda")
    psw.lse_combine(flat, lses, out=m2, out_lse=l2)
    o2 = psw.vup_projection(m2.view(T, H, R), w_uv)
    m1 = torch.full((rows, R), 7.0, dtype=torch.bfloat16, device="cuda")
    l1 = torch.full((rows,), 7.0, dtype=torch.float32, device="cuda")
    o1 = psw.lse_combine_vup(outs, lses, w_uv, out_lse=l1, merged=m1)
    torch.cuda.synchronize()
    assert torch.equal(m1, m2), "merged rows"
    assert torch.equal(l1, l2), "merged LSE"
    assert torch.equal(o1, o2), "projected output"


@pytest.mark.parametrize("P,pdt,T,H,R,Dv", [CASES[1], CASES[4], CASES[6]])
def test_against_oracle(P, pdt, T, H, R, Dv):
    outs, lses, w_uv, wf = _inputs(P * 7 + T, P, T, H, R, Dv, pdt)
    rows = T * H
    l1 = torch.empty(rows, dtype=torch.float32, device="cuda")
    got = psw.lse_combine_vup(outs, lses, w_uv, out_lse=l1).float().cpu().numpy()
    ref_x, ref_l = lse_merge_ref([o.float().cpu().numpy().reshape(rows, R) for o in outs],
                                 [l.cpu().numpy() for l in lses])
    assert_lse_close(l1.cpu().numpy(), ref_l, "merged LSE")
    assert_close(got, vup_projection_ref(ref_x.reshape(T, H, R), wf), "projected output")


def test_optional_outputs_and_errors():
    outs, lses, w_uv, _ = _inputs(3, 2, 9, 4, 256, 64, torch.bfloat16)
    o_all = psw.lse_combine_vup(outs, lses, w_uv,
                                out_lse=torch.empty(36, dtype=torch.float32, device="cuda"),
                                merged=torch.empty((36, 256), dtype=torch.bfloat16, device="cuda"))
    o_none = psw.lse_combine_vup(outs, lses, w_uv)
    assert torch.equal(o_all, o_none)
    with pytest.raises(psw.PswError):   # more partials than the fused kernel takes
        psw.lse_combine_vup(outs * 9, lses * 9, w_uv)
    with pytest.raises(psw.PswError):   # no kernel for a rank of 96
        x = [torch.zeros((2, 1, 96), dtype=torch.bfloat16, device="cuda")]
        psw.lse_combine_vup(x, [torch.zeros(2, dtype=torch.float32, device="cuda")],
                            torch.zeros((1, 96, 64), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):     # partials of another shape
        psw.lse_combine_vup([outs[0], outs[1][:4]], lses, w_uv)
