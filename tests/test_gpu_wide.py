"""GPU parity at head_dim 192 (six groups; D/2 = 96 = 3 * 32 complex numbers),
the width the mixed-radix SRFT serves ("SRFT + int4 KV-cache" page: core
method and comparison of methods), through the C ABI.

Codes and scales must equal the oracle's bit for bit (plain, K rotated by
the mixed-radix SRFT, with K's channel scale), appended one token at a time
at odd and even positions and in chunks; outputs must be within max-abs 2e-3
and relative L2 1e-3 of the fp64 oracle for every G <= 16, ragged batches
(longest-first order) and the two-phase calls, on both split passes: the
matrix-core one (the default for a K that is not rotated) and the vector one
(asked for explicitly): the matrix-core pass is the default
for every K, the rotated one taking the query through the mixed-radix FFT
in registers."""
import math

import numpy as np
import pytest
import torch

import int4_kv_cache_quant_amd as otq
import oracle

from gpu_common import (MAX_ABS, REL_L2, chan_scales, compare_codes, errors, host_cache, oracle_cache,
                        rand_signs, rot_norm32, say, to_bits)

pytestmark = pytest.mark.gpu

DEV = "cuda"
D = 192


def _inputs(B, Hkv, T, G, seed, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    k = torch.randn((B, Hkv, T, D), generator=g)
    v = torch.randn((B, Hkv, T, D), generator=g)
    k[..., 7] *= 10
    v[..., 7] *= 10
    q = torch.randn((B, G * Hkv, D), generator=g)
    return k.to(dtype), v.to(dtype), q.to(dtype)


def _cache(B, Hkv, cap, rotate, scaled, seed):
    signs = rand_signs(D, seed) if rotate else None
    lam = chan_scales(D, seed + 1, outliers=(7,)) if scaled else None
    c = otq.Int4KVCache(B, Hkv, D, cap, device=DEV, rot_signs=None if signs is None else signs.to(DEV),
                        chan_scale=None if lam is None else lam.to(DEV), rot_kind="srft")
    return c, signs, lam


def _fill(cache, k, v, T, chunk):
    B = k.shape[0]
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        cache.append(k[:, :, t0:t1].contiguous().to(DEV), v[:, :, t0:t1].contiguous().to(DEV),
                     torch.full((B,), t0, dtype=torch.int32, device=DEV))


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("rotate,scaled", [(False, False), (True, False), (True, True), (False, True)])
@pytest.mark.parametrize("chunk", [1, 19, 64])
def test_wide_codes_bit_exact(dtype, rotate, scaled, chunk):
    B, Hkv, T, cap = 2, 3, 97, 128
    k, v, _ = _inputs(B, Hkv, T, 1, seed=chunk + 2 * rotate + scaled, dtype=dtype)
    cache, signs, lam = _cache(B, Hkv, cap, rotate, scaled, seed=5)
    say(f"wide append D={D} dtype={dtype} rotate={rotate} scaled={scaled} chunk={chunk}")
    _fill(cache, k, v, T, chunk)
    torch.cuda.synchronize()
    name = "fp16" if dtype == torch.float16 else "bf16"
    ref = oracle_cache(k, v, name, None if signs is None else signs.numpy(), rot_norm32(D, "srft"),
                       chan_scale=None if lam is None else lam.numpy(), rot_kind="srft")
    assert compare_codes(host_cache(cache), ref, T) == {"k_codes": 0, "k_scales": 0, "v_codes": 0, "v_scales": 0}
    # the slots past T are untouched (zero)
    kc, ks, vc, vs = host_cache(cache)
    assert not kc[:, :, T:].any() and not vc[:, :, T:].any() and not ks[:, :, T:].any()


def test_wide_single_tokens_scattered_keep_neighbours():
    """Single-token appends in a shuffled order: every V byte is shared by two
    tokens appended at different times."""
    B, Hkv, cap = 1, 2, 64
    k, v, _ = _inputs(B, Hkv, cap, 1, seed=3)
    cache, signs, _ = _cache(B, Hkv, cap, True, False, seed=9)
    for t in np.random.default_rng(1).permutation(cap):
        cache.append(k[:, :, t:t + 1].contiguous().to(DEV), v[:, :, t:t + 1].contiguous().to(DEV),
                      torch.full((B,), int(t), dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    ref = oracle_cache(k, v, "bf16", signs.numpy(), rot_norm32(D, "srft"), rot_kind="srft")
    assert compare_codes(host_cache(cache), ref, cap) == {"k_codes": 0, "k_scales": 0, "v_codes": 0, "v_scales": 0}


def _sdpa(B, G, Hkv, cap, lens, rotate=False, scaled=False, seed=0, chunk=0, dtype=torch.bfloat16,
          two_phase=False, variant=otq.OTQ_VARIANT_AUTO):
    T = max(lens)
    k, v, q = _inputs(B, Hkv, cap, G, seed=seed, dtype=dtype)
    cache, signs, lam = _cache(B, Hkv, cap, rotate, scaled, seed=seed + 50)
    _fill(cache, k, v, T, 1000)
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    plan = cache.plan(G * Hkv, T, chunk=chunk, variant=variant)
    assert plan.variant == (variant if variant != otq.OTQ_VARIANT_AUTO else otq.OTQ_VARIANT_MFMA)
    say(f"wide sdpa B={B} G={G} Hkv={Hkv} lens={lens[:6]} rotate={rotate} scaled={scaled} "
        f"chunk={plan.chunk} splits={plan.num_splits} variant={plan.variant}")
    scale = 1.0 / math.sqrt(D)
    if two_phase:
        ws = cache.workspace(G * Hkv, T, plan)
        out = torch.empty((B, G * Hkv, D), dtype=torch.float32, device=DEV)
        otq.otq_sdpa_int4_split(q.to(DEV), cache.desc, lens_t, T, scale, ws, plan)
        otq.otq_sdpa_lse_combine(G * Hkv, cache.desc, lens_t, T, ws, plan, out)
    else:
        out = cache.decode(q.to(DEV), lens_t, T, scale, plan=plan)
    torch.cuda.synchronize()
    name = "fp16" if dtype == torch.float16 else "bf16"
    kc, ks, vc, vs = oracle_cache(k, v, name, None if signs is None else signs.numpy(), rot_norm32(D, "srft"),
                                  chan_scale=None if lam is None else lam.numpy(), rot_kind="srft")
    ref = oracle.sdpa(to_bits(q), name, kc, ks, vc, vs, np.array(lens, np.int32), scale,
                      signs=None if signs is None else signs.numpy(), rot_norm=rot_norm32(D, "srft"),
                      threads=8, chan_scale=None if lam is None else lam.numpy(), rot_kind="srft")
    got = out.cpu().numpy()
    ma, rel = errors(got, ref)
    say(f"  max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert np.all(np.isfinite(got))
    assert ma <= MAX_ABS and rel <= REL_L2
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(got[b] == 0.0)
    return plan


VEC = otq.OTQ_VARIANT_VECTOR


@pytest.mark.parametrize("G", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("rotate,scaled,variant", [(False, False, 0), (False, False, VEC), (True, False, 0),
                                                   (True, False, VEC), (True, True, 0), (True, True, VEC),
                                                   (False, True, 0), (False, True, VEC)])
def test_wide_sdpa_parity(G, rotate, scaled, variant):
    plan = _sdpa(2, G, 2, 640, [600, 131], rotate=rotate, scaled=scaled, seed=G + 10 * rotate + scaled,
                 chunk=128, variant=variant)
    assert plan.num_splits == 5


@pytest.mark.parametrize("lens", [[0, 1], [31, 32], [33, 256], [257, 0]])
@pytest.mark.parametrize("rotate", [True, False])
def test_wide_sdpa_edge_lengths(lens, rotate):
    _sdpa(2, 4, 2, 320, lens, rotate=rotate, seed=sum(lens), chunk=128)


@pytest.mark.parametrize("rotate", [True, False])
def test_wide_sdpa_fp16_and_default_plan(rotate):
    _sdpa(1, 8, 2, 2048, [2000], rotate=rotate, seed=77, dtype=torch.float16)


@pytest.mark.parametrize("rotate", [True, False])
def test_wide_sdpa_ragged_batch_in_longest_first_order(rotate):
    lens = [0, 1, 128, 129, 383, 256, 32, 300, 127, 384, 255, 2]
    _sdpa(len(lens), 4, 2, 384, lens, rotate=rotate, seed=21, chunk=128)


@pytest.mark.parametrize("rotate,scaled", [(True, True), (False, True)])
def test_wide_two_phase_calls(rotate, scaled):
    _sdpa(3, 8, 2, 512, [500, 77, 256], rotate=rotate, scaled=scaled, seed=33, chunk=128, two_phase=True)


@pytest.mark.parametrize("rotate,variant", [(True, 0), (False, 0), (True, VEC)])
def test_wide_long_context(rotate, variant):
    """One sequence of 16384 tokens, default plan (many splits)."""
    _sdpa(1, 8, 2, 16384, [16384], rotate=rotate, seed=91, variant=variant)
