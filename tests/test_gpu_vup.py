"""GPU parity: the V-up projection of the merged latent output against the oracle.

Tolerance as for attention (bf16 inputs and result, fp32 accumulation): every
element within 2e-2 + 2e-2 |ref|.
"""
import numpy as np
import pytest
import torch

import paged_sliding_window_amd as psw
from oracle import vup_projection_ref
from tests.gpu_setup import assert_close, bits_to_bf16
from workloads.synth import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _bf16(rng, shape, scale=1.0):
    bits = f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))
    return bits, bf16_bits_to_f32(bits)


@pytest.mark.parametrize("T,H,R,Dv", [(1, 1, 128, 64), (5, 3, 256, 128), (64, 128, 512, 128),
                                      (100, 7, 512, 192), (130, 2, 128, 64), (33, 16, 256, 256)])
def test_against_oracle(T, H, R, Dv):
    rng = np.random.default_rng(T * 1000 + H * 10 + R + Dv)
    xb, xf = _bf16(rng, (T, H, R))
    wb, wf = _bf16(rng, (H, R, Dv), scale=R ** -0.5)
    got = psw.vup_projection(bits_to_bf16(xb), bits_to_bf16(wb)).float().cpu().numpy()
    assert_close(got, vup_projection_ref(xf, wf), f"vup T={T} H={H} R={R} Dv={Dv}")


def test_merged_decode_output_then_projection():
    """The decode chain: the combine's [tokens * heads, 512] output viewed as
    [tokens, heads, 512], projected per head (the shape of the latent decode
    workload: 64 tokens, 128 heads, rank 512, V head dim 128)."""
    rng = np.random.default_rng(5)
    T, H, R, Dv = 64, 128, 512, 128
    xb, xf = _bf16(rng, (T * H, R), scale=0.3)
    wb, wf = _bf16(rng, (H, R, Dv), scale=R ** -0.5)
    out = torch.empty((T, H * Dv), dtype=torch.bfloat16, device="cuda")
    psw.vup_projection(bits_to_bf16(xb), bits_to_bf16(wb), out=out)
    assert_close(out.float().cpu().numpy().reshape(T, H, Dv),
                 vup_projection_ref(xf.reshape(T, H, R), wf), "vup of merged rows")


def test_unsupported_shapes_are_rejected():
    x = torch.zeros((2, 1, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(psw.PswError):
        psw.vup_projection(x, torch.zeros((1, 96, 64), dtype=torch.bfloat16, device="cuda"))
    x = torch.zeros((2, 1, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(psw.PswError):
        psw.vup_projection(x, torch.zeros((1, 128, 48), dtype=torch.bfloat16, device="cuda"))
