"""The torch wrappers refuse inconsistent tensors before anything is enqueued:
each call below raises ValueError and leaves its (sentinel-filled) output
untouched."""
import pytest
import torch

import paged_sliding_window_amd as psw

pytestmark = pytest.mark.gpu


def _t(shape, dtype=torch.bfloat16, fill=0):
    return torch.full(shape, fill, dtype=dtype, device="cuda")


def _attn_inputs():
    return dict(q=_t((10, 8, 128)), k_cache=_t((20, 16, 2, 128)), v_cache=_t((20, 16, 2, 128)),
                block_table=_t((3, 7), torch.int32), query_start_loc=_t((4,), torch.int32),
                seq_lens=_t((3,), torch.int32))


@pytest.mark.parametrize("change", [
    dict(q=(10, 8, 64)), dict(v_cache=(20, 16, 1, 128)), dict(seq_lens=(2,)),
    dict(block_table=(2, 7)), dict(mm_ranges=(2, 2, 2)), dict(key_ranges=(2, 4, 2)),
], ids=lambda d: ",".join(d))
def test_attention_mismatch_raises_before_launch(change):
    x = _attn_inputs()
    for k, shape in change.items():
        dt = torch.int32 if k in ("seq_lens", "block_table", "mm_ranges", "key_ranges") else torch.bfloat16
        x[k] = _t(shape, dt)
    out = _t((2 if "key_ranges" in change else 1, 10, 8, 128), fill=7)
    with pytest.raises(ValueError):
        psw.swa_mm_attention(x.pop("q"), x.pop("k_cache"), x.pop("v_cache"), x.pop("block_table"),
                             x.pop("query_start_loc"), x.pop("seq_lens"), scale=0.1, window=0,
                             causal=True, out=out, **x)
    torch.cuda.synchronize()
    assert bool((out == 7).all())


def test_kv_write_mismatch_raises_before_launch():
    cache_k, cache_v = _t((4, 16, 2, 64), fill=3), _t((4, 16, 2, 64), fill=3)
    slots = torch.arange(5, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        psw.kv_cache_write(_t((5, 2, 64), fill=1), _t((5, 1, 64), fill=1), slots, cache_k, cache_v)
    with pytest.raises(ValueError):
        psw.kv_cache_write(_t((5, 2, 64), fill=1), _t((5, 2, 64), fill=1), slots,
                           _t((4, 16, 1, 64)), cache_v)
    torch.cuda.synchronize()
    assert bool((cache_k == 3).all()) and bool((cache_v == 3).all())


def test_combine_mismatch_raises_before_launch():
    parts = [_t((6, 64), torch.float32, 1.0) for _ in range(2)]
    lses = [_t((6,), torch.float32, 0.0) for _ in range(2)]
    out = _t((5, 64), fill=9)
    with pytest.raises(ValueError):
        psw.lse_combine(parts, lses, out=out)
    out = _t((6, 64), fill=9)
    with pytest.raises(ValueError):
        psw.lse_combine(parts, lses, out=out, out_lse=_t((5,), torch.float32))
    torch.cuda.synchronize()
    assert bool((out == 9).all())
    # the same call with consistent shapes runs
    got = psw.lse_combine(parts, lses, out=out, out_lse=_t((6,), torch.float32))[0]
    torch.cuda.synchronize()
    assert torch.allclose(got.float(), torch.ones_like(got.float()))
