"""Graph capture and the two-phase API.

The bench replays HIP graphs of the decode step, so every path it captures is
replayed here several times, with eager work and synchronisations between the
replays, and each replay must equal the eager result bit for bit (every call
is deterministic and, repeated, rewrites the same bytes).  The two-phase API
(split, then combine) must equal the single call bit for bit."""
import math

import numpy as np
import pytest
import torch

import int4_kv_cache_quant_amd as otq
import oracle

from gpu_common import (MAX_ABS, REL_L2, build_cache, chan_scales, errors, oracle_cache, rand_signs,
                        rot_norm32, say, to_bits)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _setup(B, G, Hkv, D, cap, lens, extras, seed):
    """extras: False, True (K rotated and scaled, V rotated: the Hadamard
    kind) or "srft" (the same with the FFT kind)."""
    kind = "srft" if extras == "srft" else "srht"
    g = torch.Generator().manual_seed(seed)
    k = torch.randn((B, Hkv, cap, D), generator=g)
    v = torch.randn((B, Hkv, cap, D), generator=g)
    k[..., 5] *= 10
    k, v = k.to(torch.bfloat16), v.to(torch.bfloat16)
    q = torch.randn((B, G * Hkv, D), generator=g).to(torch.bfloat16)
    sk = rand_signs(D, seed + 1) if extras else None
    lam = chan_scales(D, seed + 2, outliers=(5,)) if extras else None
    sv = rand_signs(D, seed + 3) if extras else None
    T = max(lens)
    cache = build_cache(k[:, :, :T].to(DEV).contiguous(), v[:, :, :T].to(DEV).contiguous(), cap,
                        signs=None if sk is None else sk.to(DEV), append_last=False,
                        chan_scale=None if lam is None else lam.to(DEV),
                        v_signs=None if sv is None else sv.to(DEV), rot_kind=kind)
    return k, v, q, sk, lam, sv, cache, kind


@pytest.mark.parametrize("B,lens,extras", [(1, [700], False), (3, [700, 129, 333], False),
                                          (3, [700, 129, 333], True), (3, [700, 129, 333], "srft")])
def test_graph_replays_match_eager(B, lens, extras):
    G, Hkv, D, cap = 8, 2, 128, 768
    say(f"graph B={B} lens={lens} extras={extras}")
    seed = B + {False: 0, True: 10, "srft": 20}[extras]
    k, v, q, sk, lam, sv, cache, kind = _setup(B, G, Hkv, D, cap, lens, extras, seed=seed)
    Hq = G * Hkv
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    idx = (lens_t.long() - 1).clamp(min=0)
    ar = torch.arange(B, device=DEV)
    kn = k.to(DEV)[ar, :, idx].contiguous()
    vn = v.to(DEV)[ar, :, idx].contiguous()
    qd = q.to(DEV)
    max_len = max(lens)
    plan = cache.plan(Hq, max_len, chunk=128)
    ws = cache.workspace(Hq, max_len, plan)
    out_e = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    out_g = torch.empty_like(out_e)
    cache.decode_append(qd, kn, vn, lens_t, max_len, 0.09, out=out_e, workspace=ws, plan=plan)
    # a bulk append of the first 40 tokens, rewriting the same bytes
    kb = k[:, :, :40].to(DEV).contiguous()
    vb = v[:, :, :40].to(DEV).contiguous()
    pos0 = torch.zeros((B,), dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    snap = [t.clone() for t in (cache.k_codes, cache.k_scales, cache.v_codes, cache.v_scales)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cache.append(kb, vb, pos0)
        cache.decode_append(qd, kn, vn, lens_t, max_len, 0.09, out=out_g, workspace=ws, plan=plan)
    for r in range(3):
        out_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {r}"
        for a, b in zip(snap, (cache.k_codes, cache.k_scales, cache.v_codes, cache.v_scales)):
            assert torch.equal(a, b), f"replay {r}: cache changed"
        # eager work between the replays
        junk = torch.randn((1 << 20,), device=DEV).sum()
        cache.decode(qd, lens_t, max_len, 0.09, workspace=ws, plan=plan)
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
    # and the eager result against the oracle
    name = "bf16"
    kc, ks, vc, vs = oracle_cache(k, v, name, None if sk is None else sk.numpy(), rot_norm32(D, kind),
                                  chan_scale=None if lam is None else lam.numpy(),
                                  v_signs=None if sv is None else sv.numpy(), rot_kind=kind)
    ref = oracle.sdpa(to_bits(q), name, kc, ks, vc, vs, np.array(lens, np.int32), 0.09,
                      signs=None if sk is None else sk.numpy(), rot_norm=rot_norm32(D, kind), threads=8,
                      chan_scale=None if lam is None else lam.numpy(),
                      v_signs=None if sv is None else sv.numpy(), rot_kind=kind)
    ma, rel = errors(out_e.cpu().numpy(), ref)
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("extras", [False, True, "srft"])
@pytest.mark.parametrize("variant", [otq.OTQ_VARIANT_VECTOR, otq.OTQ_VARIANT_MFMA])
def test_two_phase_equals_single_call(extras, variant):
    B, G, Hkv, D, cap, lens = 2, 2, 2, 128, 512, [500, 77]
    say(f"two-phase variant={variant} extras={extras}")
    seed = 20 + {False: 0, True: 1, "srft": 2}[extras]
    k, v, q, sk, lam, sv, cache, kind = _setup(B, G, Hkv, D, cap, lens, extras, seed=seed)
    Hq = G * Hkv
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    qd = q.to(DEV)
    plan = cache.plan(Hq, max(lens), chunk=128, variant=variant)
    ws = cache.workspace(Hq, max(lens), plan)
    one = cache.decode(qd, lens_t, max(lens), 0.1, workspace=ws, plan=plan).clone()
    two = torch.empty_like(one)
    otq.otq_sdpa_int4_split(qd, cache.desc, lens_t, max(lens), 0.1, ws, plan)
    otq.otq_sdpa_lse_combine(Hq, cache.desc, lens_t, max(lens), ws, plan, two)
    torch.cuda.synchronize()
    assert torch.equal(one, two)
