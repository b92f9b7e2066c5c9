"""otq_sdpa_int4_decode_append_noalloc: the decode step with the library's
per-device scratch array as its workspace.  It runs the same kernels with
the same plan as otq_sdpa_int4_decode_append on a caller workspace, so the
outputs and the cache bytes must be identical, bit for bit; two calls in a
row (the second on a smaller input) share the array."""
import ctypes
import math

import numpy as np
import pytest
import torch

import int4_kv_cache_quant_amd as otq

from gpu_common import say

DEV = "cuda"


def _setup(B, Hkv, G, D, cap, lens, seed):
    g = torch.Generator().manual_seed(seed)
    k = torch.randn((B, Hkv, cap, D), generator=g).to(torch.bfloat16).to(DEV)
    v = torch.randn((B, Hkv, cap, D), generator=g).to(torch.bfloat16).to(DEV)
    q = torch.randn((B, G * Hkv, D), generator=g).to(torch.bfloat16).to(DEV)
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    caches = []
    for _ in range(2):
        c = otq.Int4KVCache(B, Hkv, D, cap, device=DEV)
        c.append(k, v, torch.zeros(B, dtype=torch.int32, device=DEV))  # every slot, then overwritten
        caches.append(c)
    idx = (lens_t.long() - 1).clamp(min=0)
    ar = torch.arange(B, device=DEV)
    kn = (k[ar, :, idx] * 0.5).contiguous()  # a new token unlike the one in the slot
    vn = (v[ar, :, idx] * -2.0).contiguous()
    return caches, q, kn, vn, lens_t


def _bytes(c):
    return [t.cpu().numpy().view(np.uint8).copy() for t in (c.k_codes, c.k_scales, c.v_codes, c.v_scales)]


@pytest.mark.gpu
def test_noalloc_matches_workspace_call_twice():
    cases = [  # (B, Hkv, G, D, cap, lens): then a smaller one on the same array
        (4, 8, 8, 128, 4096, [4096, 1000, 2500, 33]),
        (2, 2, 4, 64, 512, [300, 1]),
    ]
    for i, (B, Hkv, G, D, cap, lens) in enumerate(cases):
        caches, q, kn, vn, lens_t = _setup(B, Hkv, G, D, cap, lens, seed=10 + i)
        max_len = max(lens)
        plan = caches[0].plan(G * Hkv, max_len)
        assert plan.workspace_bytes <= otq.OTQ_NOALLOC_SCRATCH_BYTES
        scale = 1.0 / math.sqrt(D)
        out_ref = caches[0].decode_append(q, kn, vn, lens_t, max_len, scale, plan=plan)
        out = torch.empty_like(out_ref)
        otq.otq_sdpa_int4_decode_append_noalloc(q, kn, vn, caches[1].desc, lens_t, max_len, scale, out,
                                                plan=plan)
        torch.cuda.synchronize()
        say(f"noalloc call {i}: B={B} Hkv={Hkv} G={G} D={D} lens={lens} workspace={plan.workspace_bytes}")
        assert torch.equal(out, out_ref)
        for a, b in zip(_bytes(caches[0]), _bytes(caches[1])):
            assert np.array_equal(a, b)


@pytest.mark.gpu
def test_noalloc_default_plan_and_limit():
    """plan = NULL takes the default plan; a plan whose workspace exceeds the
    array is refused on the host with OTQ_EWORKSPACE."""
    caches, q, kn, vn, lens_t = _setup(1, 2, 2, 128, 256, [200], seed=3)
    out = torch.empty((1, 4, 128), dtype=torch.float32, device=DEV)
    otq.otq_sdpa_int4_decode_append_noalloc(q, kn, vn, caches[1].desc, lens_t, 200, 0.1, out)
    ref = caches[0].decode_append(q, kn, vn, lens_t, 200, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    # 64 sequences x 64 query heads x 64 splits of 128 channels: 128 MiB of partials
    big = otq.Int4KVCache(64, 8, 128, 8192, device=DEV)
    p = big.plan(64, 8192, chunk=128)
    assert p.workspace_bytes > otq.OTQ_NOALLOC_SCRATCH_BYTES
    qb = torch.zeros((64, 64, 128), dtype=torch.bfloat16, device=DEV)
    kb = torch.zeros((64, 8, 128), dtype=torch.bfloat16, device=DEV)
    lb = torch.ones(64, dtype=torch.int32, device=DEV)
    ob = torch.empty((64, 64, 128), dtype=torch.float32, device=DEV)
    rc = otq.otq_sdpa_int4_decode_append_noalloc(qb, kb, kb, big.desc, lb, 8192, 0.1, ob, plan=p, check=False)
    assert rc == otq.OTQ_EWORKSPACE
