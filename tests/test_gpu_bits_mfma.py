"""GPU parity of the 2- and 3-bit split pass on the matrix cores (the
default for b-bit caches whose K is neither rotated nor channel-scaled),
through the C ABI, against the oracle's b-bit quantiser and fp64 attention.

Covers every G up to 16 at head_dim 64, 128 and 256, tails and chunk ends,
ragged batches in longest-first order, a rotated V (undone by the combine),
Inf/NaN scales and junk codes past the attended length, query rows of any
bf16 magnitude and V scaled by powers of two from 2^-100 to 2^100.
Tolerance as everywhere: max-abs <= 2e-3, relative L2 <= 1e-3."""
import math

import numpy as np
import pytest
import torch

import int4_kv_cache_quant_amd as otq
import oracle

from int4_kv_cache_quant_amd import layout

from gpu_common import MAX_ABS, REL_L2, errors, rand_signs, say, to_bits

pytestmark = pytest.mark.gpu

DEV = "cuda"
VEC, MF = otq.OTQ_VARIANT_VECTOR, otq.OTQ_VARIANT_MFMA


def _inputs(B, Hq, Hkv, D, cap, seed, dtype=torch.bfloat16, v_exp=None):
    g = torch.Generator().manual_seed(seed)
    k = torch.randn((B, Hkv, cap, D), generator=g)
    v = torch.randn((B, Hkv, cap, D), generator=g)
    k[..., 5] *= 10
    v[..., 5] *= 10
    if v_exp is not None:  # powers of two: exact in bf16, codes unchanged
        v = v * 2.0 ** v_exp
    q = torch.randn((B, Hq, D), generator=g)
    return k.to(dtype), v.to(dtype), q.to(dtype)


def _cache(k, v, v_signs=None, bits=2):
    B, H, cap, D = k.shape
    cache = otq.Int4KVCache(B, H, D, cap, device=DEV, code_bits=bits,
                            v_rot_signs=None if v_signs is None else v_signs.to(DEV))
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    cache.append(k.contiguous().to(DEV), v.contiguous().to(DEV), pos)
    torch.cuda.synchronize()
    return cache


def _ref(q, k, v, lens, scale, name="bf16", v_signs=None, bits=2):
    D = k.shape[-1]
    rn = float(np.float32(1.0 / math.sqrt(D)))
    kc, ks = oracle.quantize(to_bits(k), name, code_bits=bits)
    vc, vs = oracle.quantize(to_bits(v), name, code_bits=bits, signs=v_signs,
                             rot_norm=rn if v_signs is not None else 0.0)
    return oracle.sdpa(to_bits(q), name, kc, ks, vc, vs, np.array(lens, np.int32), scale, threads=8,
                       code_bits=bits, v_signs=v_signs, rot_norm=rn if v_signs is not None else 0.0)


def _decode(cache, q, lens, scale, chunk=0, variant=otq.OTQ_VARIANT_AUTO):
    Hq = q.shape[1]
    plan = cache.plan(Hq, max(1, max(lens)), chunk=chunk, variant=variant)
    out = cache.decode(q.to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV), max(1, max(lens)), scale,
                       plan=plan)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), plan


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_bits_mfma_parity(bits, D, G):
    B, Hkv, cap = 2, 2, 448
    lens = [437, 77]  # partial tiles, several splits of 128
    k, v, q = _inputs(B, G * Hkv, Hkv, D, cap, seed=D + G + 100 * bits)
    cache = _cache(k, v, bits=bits)
    got, plan = _decode(cache, q, lens, 1.0 / math.sqrt(D), chunk=128)
    # the default for a plain b-bit cache
    assert plan.variant == MF
    ref = _ref(q, k, v, lens, 1.0 / math.sqrt(D), bits=bits)
    ma, rel = errors(got, ref)
    say(f"b{bits} mfma D={D} G={G}: max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("lens", [[1, 2], [32, 31], [33, 128], [129, 256], [255, 384]])
def test_bits_mfma_edges(bits, lens):
    """One token, tile ends (31, 32, 33), chunk ends (128, 129, 256) and a
    full cache (384) with chunk 128; fp16 inputs."""
    k, v, q = _inputs(2, 16, 2, 128, 384, seed=sum(lens) + bits, dtype=torch.float16)
    cache = _cache(k, v, bits=bits)
    got, _ = _decode(cache, q, lens, 0.1, chunk=128, variant=MF)
    ref = _ref(q, k, v, lens, 0.1, name="fp16", bits=bits)
    ma, rel = errors(got, ref)
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("bits", [2, 3])
def test_bits_mfma_matches_vector_variant(bits):
    """The same call on both b-bit split passes: both within tolerance of the
    oracle (and of each other)."""
    k, v, q = _inputs(1, 8, 2, 128, 512, seed=3 + bits)
    cache = _cache(k, v, bits=bits)
    a, _ = _decode(cache, q, [500], 0.125, chunk=128, variant=MF)
    b, _ = _decode(cache, q, [500], 0.125, chunk=128, variant=VEC)
    ref = _ref(q, k, v, [500], 0.125, bits=bits)
    for got in (a, b):
        ma, rel = errors(got, ref)
        assert ma <= MAX_ABS and rel <= REL_L2
    assert errors(a, b)[0] <= MAX_ABS


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("B", [12, 64])
@pytest.mark.parametrize("Hkv", [1, 2])
def test_bits_mfma_ragged_batch(bits, B, Hkv):
    """A batch in longest-first order: empty sequences, one token, chunk
    multiples and partial chunks; one KV head (one per wave) and two (G = 8:
    both in one wave)."""
    rng = np.random.default_rng(B)
    lens = [int(x) for x in rng.integers(0, 385, size=B)]
    lens[0], lens[1], lens[2] = 0, 1, 384
    k, v, q = _inputs(B, 8 * Hkv, Hkv, 64, 384, seed=B + bits + Hkv)
    cache = _cache(k, v, bits=bits)
    got, plan = _decode(cache, q, lens, 0.125, chunk=128, variant=MF)
    ref = _ref(q, k, v, lens, 0.125, bits=bits)
    assert np.all(got[0] == 0.0)
    ma, rel = errors(got, ref)
    say(f"b{bits} mfma ragged B={B} Hkv={Hkv}: max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("bits", [2, 3])
def test_bits_mfma_rotated_v(bits):
    """V rotated (signs + Walsh-Hadamard, undone by the combine) keeps the
    MFMA pass; K stays plain."""
    D = 128
    k, v, q = _inputs(2, 8, 2, D, 256, seed=11 + bits)
    vs = rand_signs(D, 12)
    cache = _cache(k, v, v_signs=vs, bits=bits)
    got, plan = _decode(cache, q, [250, 100], 0.1, chunk=128)
    assert plan.variant == MF
    ref = _ref(q, k, v, [250, 100], 0.1, v_signs=vs.numpy(), bits=bits)
    ma, rel = errors(got, ref)
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("bits", [2, 3])
def test_bits_mfma_junk_past_lens(bits):
    """Inf/NaN scales and arbitrary code bytes in every slot at or past
    lens[b]: only tokens t < lens[b] may reach the output."""
    B, Hkv, G, D, cap = 3, 2, 8, 128, 320
    lens = [291, 77, 160]
    k, v, q = _inputs(B, G * Hkv, Hkv, D, cap, seed=23 + bits)
    cache = _cache(k, v, bits=bits)
    rng = np.random.default_rng(5)
    pattern = torch.tensor([float("inf"), float("nan"), -float("inf"), float("nan")], device=DEV)
    vp = layout.v_bits_tiled_to_plain(cache.v_codes.cpu().numpy(), D, bits)
    for b, f in enumerate(lens):
        n = cap - f
        idx = torch.arange(n * (D // 32), device=DEV) % 4
        cache.k_scales[b, :, f:] = pattern[idx].reshape(n, D // 32)
        cache.v_scales[b, :, f:] = pattern[(idx + 1) % 4].reshape(n, D // 32)
        cache.k_codes[b, :, f:] = torch.from_numpy(rng.integers(0, 256, size=(Hkv, n, D * bits // 8),
                                                                dtype=np.uint8)).to(DEV)
        # V: junk in the fields of tokens f.. only (a tile also holds tokens below f)
        vp[b, :, f:] = rng.integers(0, 256, size=(Hkv, n, D * bits // 8), dtype=np.uint8)
    cache.v_codes.copy_(torch.from_numpy(layout.v_bits_plain_to_tiled(vp, D, bits)).to(DEV))
    got, _ = _decode(cache, q, lens, 1.0 / math.sqrt(D), chunk=128, variant=MF)
    ref = _ref(q, k, v, lens, 1.0 / math.sqrt(D), bits=bits)
    assert np.all(np.isfinite(got))
    ma, rel = errors(got, ref)
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("bits", [2, 3])
def test_bits_mfma_query_magnitudes(bits):
    """bf16 query rows of ~1e5, ~1e-6 and both mixed in one row."""
    B, Hkv, G, D, cap = 2, 2, 8, 128, 256
    k, v, _ = _inputs(B, G * Hkv, Hkv, D, cap, seed=31)
    g = torch.Generator().manual_seed(32)
    q = torch.randn((B, G * Hkv, D), generator=g)
    kinds = torch.arange(B * G * Hkv).reshape(B, G * Hkv) % 4
    mixed = torch.where(torch.rand((B, G * Hkv, D), generator=g) < 0.5, 1e5, 1e-6)
    q = torch.where((kinds == 0)[..., None], q * 1e5, q)
    q = torch.where((kinds == 1)[..., None], q * 1e-6, q)
    q = torch.where((kinds == 2)[..., None], q.sign() * mixed, q).to(torch.bfloat16)
    cache = _cache(k, v, bits=bits)
    got, _ = _decode(cache, q, [250, 97], 1.0 / math.sqrt(D), chunk=128, variant=MF)
    ref = _ref(q, k, v, [250, 97], 1.0 / math.sqrt(D), bits=bits)
    assert np.all(np.isfinite(got))
    ma, rel = errors(got, ref)
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("kexp", [-100, -70, 20, 100])
def test_bits_mfma_value_magnitudes(bits, kexp):
    """V times 2^kexp: the output is 2^kexp times the unscaled one."""
    B, Hkv, G, D, cap = 2, 2, 8, 128, 256
    k, v, q = _inputs(B, G * Hkv, Hkv, D, cap, seed=40 + bits, v_exp=float(kexp))
    cache = _cache(k, v, bits=bits)
    got, _ = _decode(cache, q, [256, 131], 0.1, chunk=128, variant=MF)
    ref = _ref(q, k, v, [256, 131], 0.1, bits=bits)
    ma, rel = errors(got * 2.0 ** -kexp, ref * 2.0 ** -kexp)
    assert np.all(np.isfinite(got))
    assert ma <= MAX_ABS and rel <= REL_L2
