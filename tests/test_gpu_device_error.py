"""otq_last_device_error on the GPU: kernels that meet an append position or
an attended length outside the caller's contract record it in the device
error word (and skip or clamp as documented); the call reads and clears it.
In-contract calls leave the word at zero."""
import math

import numpy as np
import pytest
import torch

import int4_kv_cache_quant_amd as otq

from gpu_common import say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _kv(B, H, T, D, seed):
    g = torch.Generator().manual_seed(seed)
    k = torch.randn((B, H, T, D), generator=g).to(torch.bfloat16).to(DEV)
    v = torch.randn((B, H, T, D), generator=g).to(torch.bfloat16).to(DEV)
    return k, v


@pytest.mark.parametrize("n_new", [1, 4, 40])
def test_append_position_out_of_range_sets_pos_flag(n_new):
    """Both append kernels (under 8 tokens: one wave per token pair; 8 and
    more: one block per tile) report a range that leaves the cache."""
    B, H, D, cap = 3, 2, 128, 128
    cache = otq.Int4KVCache(B, H, D, cap, device=DEV)
    k, v = _kv(B, H, n_new, D, seed=n_new)
    otq.otq_last_device_error()  # start from a clear word
    cache.append(k, v, torch.tensor([0, 5, 7], dtype=torch.int32, device=DEV))
    assert otq.otq_last_device_error() == 0
    for bad in ([cap - n_new + 1, 0, 0], [0, -1, 0], [0, 0, cap]):
        cache.append(k, v, torch.tensor(bad, dtype=torch.int32, device=DEV))
        flags = otq.otq_last_device_error()
        say(f"n_new={n_new} pos={bad} flags={flags}")
        assert flags == otq.OTQ_DEVERR_POS
        assert otq.otq_last_device_error() == 0  # read and cleared


@pytest.mark.parametrize("bits", [2, 3])
def test_append_position_out_of_range_b_bit(bits):
    B, H, D, cap = 2, 2, 64, 64
    cache = otq.Int4KVCache(B, H, D, cap, device=DEV, code_bits=bits)
    k, v = _kv(B, H, 3, D, seed=bits)
    otq.otq_last_device_error()
    cache.append(k, v, torch.tensor([62, 0], dtype=torch.int32, device=DEV))
    assert otq.otq_last_device_error() == otq.OTQ_DEVERR_POS


@pytest.mark.parametrize("variant,B", [(otq.OTQ_VARIANT_MFMA, 1), (otq.OTQ_VARIANT_MFMA, 3),
                                       (otq.OTQ_VARIANT_VECTOR, 1), (otq.OTQ_VARIANT_VECTOR, 3)])
@pytest.mark.parametrize("fused", [False, True])
def test_lens_out_of_range_sets_lens_flag(variant, B, fused):
    """lens[b] > max_len or < 0: clamped, reported (one sequence, and a batch
    whose split blocks take their items longest first)."""
    H, G, D, cap = 2, 2, 128, 256
    cache = otq.Int4KVCache(B, H, D, cap, device=DEV)
    k, v = _kv(B, H, cap, D, seed=3)
    cache.append(k, v, torch.zeros(B, dtype=torch.int32, device=DEV))
    q = torch.randn((B, G * H, D), generator=torch.Generator().manual_seed(4)).to(torch.bfloat16).to(DEV)
    kn, vn = k[:, :, 0].contiguous(), v[:, :, 0].contiguous()
    max_len = 200
    plan = cache.plan(G * H, max_len, chunk=128, variant=variant)

    def call(lens):
        lt = torch.tensor(lens, dtype=torch.int32, device=DEV)
        if fused:
            cache.decode_append(q, kn, vn, lt, max_len, 1.0 / math.sqrt(D), plan=plan)
        else:
            cache.decode(q, lt, max_len, 1.0 / math.sqrt(D), plan=plan)
        return otq.otq_last_device_error()

    otq.otq_last_device_error()
    good = [max_len] + [17] * (B - 1)
    assert call(good) == 0
    for bad in ([max_len + 1] + [17] * (B - 1), [-5] + [17] * (B - 1)):
        flags = call(bad)
        say(f"variant={variant} B={B} fused={fused} lens={bad} flags={flags}")
        assert flags == otq.OTQ_DEVERR_LENS
    assert otq.otq_last_device_error() == 0
