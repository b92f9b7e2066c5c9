"""GPU parity at the edges of the input ranges, through the C ABI.

* Junk past the attended length: every cache slot at or past lens[b] (and,
  for the fused decode step, the new token's own slot) holds Inf or NaN
  scales and arbitrary code bytes.  Only tokens t < lens[b] enter the
  attention, so the outputs must match the fp64 oracle on the clean cache.
* Query rows of any bf16 magnitude (elements of 1e5 or 1e-6, and rows that
  mix both), which do not fit fp16 as they are.
* V of any magnitude: V scaled by 2^k (exact in bf16, so the codes are the
  same and every scale is multiplied by 2^k: the exact output is 2^k times
  the unscaled one) for k from -100 to 100, and V whose magnitude varies by
  2^+-30 from token to token.
* lens[b] above max_len in the fused step: both phases clamp lens[b] to
  max_len first, so the call equals the one with lens[b] = max_len.

Tolerance as everywhere: max-abs <= 2e-3 and relative L2 <= 1e-3 against the
fp64 oracle (for scaled V, on outputs divided by the same power of two)."""
import math

import numpy as np
import pytest
import torch

import int4_kv_cache_quant_amd as otq
import oracle
from int4_kv_cache_quant_amd import layout

from gpu_common import (MAX_ABS, REL_L2, compare_codes, errors, host_cache, oracle_cache, rot_norm32,
                        say, to_bits)

pytestmark = pytest.mark.gpu

DEV = "cuda"
VEC, MF = otq.OTQ_VARIANT_VECTOR, otq.OTQ_VARIANT_MFMA


def _fill(cache, k, v, T):
    """Quantise tokens [0, T) of k, v [B, H, cap, D] (host) into the cache."""
    B = k.shape[0]
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    cache.append(k[:, :, :T].contiguous().to(DEV), v[:, :, :T].contiguous().to(DEV), pos)


def _poison_from(cache, first):
    """Junk in every slot t >= first[b] of sequence b: K and V scales Inf,
    -Inf or NaN, K code bytes and V nibbles arbitrary.  The V codes are
    edited in the plain layout (one row of D/2 bytes per token) and packed
    back, so a tiled V byte shared with token first[b] - 1 keeps that
    token's nibble."""
    B, H, D, cap = cache.shape
    G = D // 32
    pattern = torch.tensor([float("inf"), float("nan"), -float("inf"), float("nan")],
                           dtype=torch.float32, device=DEV)
    vplain = layout.v_tiled_to_plain(cache.v_codes.cpu().numpy(), D)
    rng = np.random.default_rng(7)
    for b in range(B):
        f = int(first[b])
        if f >= cap:
            continue
        n = cap - f
        idx = torch.arange(n * G, device=DEV) % 4
        cache.k_scales[b, :, f:] = pattern[idx].reshape(n, G)
        cache.v_scales[b, :, f:] = pattern[(idx + 1) % 4].reshape(n, G)
        cache.k_codes[b, :, f:] = torch.from_numpy(rng.integers(0, 256, size=(H, n, D // 2), dtype=np.uint8)).to(DEV)
        vplain[b, :, f:] = rng.integers(0, 256, size=(H, n, D // 2), dtype=np.uint8)
    cache.v_codes.copy_(torch.from_numpy(layout.v_plain_to_tiled(vplain, D)).to(DEV))


def _inputs(B, Hq, Hkv, D, cap, seed, dtype=torch.bfloat16, v_scale_exp=None):
    g = torch.Generator().manual_seed(seed)
    k = torch.randn((B, Hkv, cap, D), generator=g)
    v = torch.randn((B, Hkv, cap, D), generator=g)
    k[..., 5] *= 10
    v[..., 5] *= 10
    if v_scale_exp is not None:  # per-token powers of two (exact in bf16)
        v = v * torch.exp2(v_scale_exp.to(torch.float32))[None, None, :, None]
    q = torch.randn((B, Hq, D), generator=g)
    return k.to(dtype), v.to(dtype), q.to(dtype)


def _oracle_out(q, k, v, lens, scale, name, signs=None, kind="srht"):
    D = k.shape[-1]
    rn = rot_norm32(D, kind)
    kc, ks, vc, vs = oracle_cache(k, v, name, signs, rn, rot_kind=kind)
    return oracle.sdpa(to_bits(q), name, kc, ks, vc, vs, np.array(lens, np.int32), scale,
                       signs=signs, rot_norm=rn, threads=8, rot_kind=kind), (kc, ks, vc, vs)


@pytest.mark.parametrize("variant,G", [(MF, 8), (MF, 1), (MF, 16), (VEC, 2)])
@pytest.mark.parametrize("rotate", [False, True])
def test_junk_scales_past_lens_decode(variant, G, rotate):
    B, Hkv, D, cap = 3, 2, 128, 320
    Hq = G * Hkv
    lens = [291, 77, 160]  # a partial tile, a partial tile, a tile end
    k, v, q = _inputs(B, Hq, Hkv, D, cap, seed=G + 17 * rotate)
    g = torch.Generator().manual_seed(99)
    signs = torch.where(torch.rand(D, generator=g) < 0.5, -1.0, 1.0) if rotate else None
    cache = otq.Int4KVCache(B, Hkv, D, cap, device=DEV, rot_signs=None if signs is None else signs.to(DEV))
    _fill(cache, k, v, cap)
    _poison_from(cache, lens)
    plan = cache.plan(Hq, max(lens), chunk=128, variant=variant)
    say(f"junk past lens: variant={variant} G={G} rotate={rotate} lens={lens}")
    out = cache.decode(q.to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV), max(lens),
                       1.0 / math.sqrt(D), plan=plan)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref, _ = _oracle_out(q, k, v, lens, 1.0 / math.sqrt(D), "bf16",
                         None if signs is None else signs.numpy())
    ma, rel = errors(got, ref)
    say(f"  max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert np.all(np.isfinite(got))
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("variant,G", [(MF, 8), (MF, 4), (VEC, 1)])
@pytest.mark.parametrize("rotate", [False, True])
def test_junk_scales_past_lens_fused(variant, G, rotate):
    """The fused step reads the new token's slot (lens - 1) only after the
    combine has written it: Inf/NaN junk there and beyond must not reach the
    output, and the whole cache below lens must end up bit-exact."""
    B, Hkv, D, cap = 3, 2, 128, 320
    Hq = G * Hkv
    lens = [291, 78, 129]
    k, v, q = _inputs(B, Hq, Hkv, D, cap, seed=3 * G + rotate)
    g = torch.Generator().manual_seed(98)
    signs = torch.where(torch.rand(D, generator=g) < 0.5, -1.0, 1.0) if rotate else None
    cache = otq.Int4KVCache(B, Hkv, D, cap, device=DEV, rot_signs=None if signs is None else signs.to(DEV))
    _fill(cache, k, v, cap)
    _poison_from(cache, [n - 1 for n in lens])
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    idx = (lens_t.long() - 1).clamp(min=0)
    ar = torch.arange(B, device=DEV)
    kn = k.to(DEV)[ar, :, idx].contiguous()
    vn = v.to(DEV)[ar, :, idx].contiguous()
    plan = cache.plan(Hq, max(lens), chunk=128, variant=variant)
    say(f"junk past lens (fused): variant={variant} G={G} rotate={rotate} lens={lens}")
    out = cache.decode_append(q.to(DEV), kn, vn, lens_t, max(lens), 1.0 / math.sqrt(D), plan=plan)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref, ref_cache = _oracle_out(q, k, v, lens, 1.0 / math.sqrt(D), "bf16",
                                 None if signs is None else signs.numpy())
    got_cache = host_cache(cache)
    for b, n in enumerate(lens):
        sub = tuple(x[b:b + 1, :, :n] for x in got_cache)
        refb = tuple(x[b:b + 1, :, :n] for x in ref_cache)
        assert compare_codes(sub, refb, n) == {"k_codes": 0, "k_scales": 0, "v_codes": 0, "v_scales": 0}
    ma, rel = errors(got, ref)
    say(f"  max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert np.all(np.isfinite(got))
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("variant,G", [(MF, 8), (MF, 1), (VEC, 4)])
@pytest.mark.parametrize("rotate", [False, True])
@pytest.mark.parametrize("fused", [False, True])
def test_junk_scales_past_lens_head_dim_192(variant, G, rotate, fused):
    """The same junk (Inf/NaN scales, arbitrary codes) at and past lens at
    head_dim 192, K plain or SRFT-rotated, for the decode call and the decode
    step (whose token takes its own append launch at this width)."""
    B, Hkv, D, cap = 3, 2, 192, 320
    Hq = G * Hkv
    lens = [291, 78, 129]
    k, v, q = _inputs(B, Hq, Hkv, D, cap, seed=5 * G + rotate + 2 * fused)
    g = torch.Generator().manual_seed(97)
    signs = torch.where(torch.rand(D, generator=g) < 0.5, -1.0, 1.0) if rotate else None
    cache = otq.Int4KVCache(B, Hkv, D, cap, device=DEV, rot_signs=None if signs is None else signs.to(DEV),
                            rot_kind="srft")
    _fill(cache, k, v, cap)
    _poison_from(cache, [n - 1 for n in lens] if fused else lens)
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    plan = cache.plan(Hq, max(lens), chunk=128, variant=variant)
    say(f"junk past lens D=192: variant={variant} G={G} rotate={rotate} fused={fused} lens={lens}")
    if fused:
        idx = (lens_t.long() - 1).clamp(min=0)
        ar = torch.arange(B, device=DEV)
        kn = k.to(DEV)[ar, :, idx].contiguous()
        vn = v.to(DEV)[ar, :, idx].contiguous()
        out = cache.decode_append(q.to(DEV), kn, vn, lens_t, max(lens), 1.0 / math.sqrt(D), plan=plan)
    else:
        out = cache.decode(q.to(DEV), lens_t, max(lens), 1.0 / math.sqrt(D), plan=plan)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref, ref_cache = _oracle_out(q, k, v, lens, 1.0 / math.sqrt(D), "bf16",
                                 None if signs is None else signs.numpy(), kind="srft")
    if fused:
        got_cache = host_cache(cache)
        for b, n in enumerate(lens):
            sub = tuple(x[b:b + 1, :, :n] for x in got_cache)
            refb = tuple(x[b:b + 1, :, :n] for x in ref_cache)
            assert compare_codes(sub, refb, n) == {"k_codes": 0, "k_scales": 0, "v_codes": 0, "v_scales": 0}
    ma, rel = errors(got, ref)
    say(f"  max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert np.all(np.isfinite(got))
    assert ma <= MAX_ABS and rel <= REL_L2


def _query_rows(B, Hq, D, seed):
    """bf16 query rows of several magnitudes: ~1e5 (past fp16's range),
    ~1e-6 (subnormal in fp16), 1e5 and 1e-6 mixed in one row, and N(0, 1)."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, Hq, D), generator=g)
    kinds = torch.arange(B * Hq).reshape(B, Hq) % 4
    mixed = torch.where(torch.rand((B, Hq, D), generator=g) < 0.5, 1e5, 1e-6)
    q = torch.where((kinds == 0)[..., None], q * 1e5, q)
    q = torch.where((kinds == 1)[..., None], q * 1e-6, q)
    q = torch.where((kinds == 2)[..., None], q.sign() * mixed, q)
    return q.to(torch.bfloat16)


@pytest.mark.parametrize("variant,G", [(MF, 8), (MF, 2), (VEC, 2)])
@pytest.mark.parametrize("opt", ["plain", "rotated", "scaled"])
def test_query_magnitudes(variant, G, opt):
    """q elements of 1e5 (beyond fp16) and 1e-6 (fp16 subnormals) with the
    usual softmax scale: the outputs equal the oracle's (a large row selects
    its top token, a tiny one averages V), plain, with K rotated, and with
    K's per-channel scale."""
    B, Hkv, D, cap = 2, 2, 128, 256
    Hq = G * Hkv
    lens = [250, 97]
    k, v, _ = _inputs(B, Hq, Hkv, D, cap, seed=5 + G)
    q = _query_rows(B, Hq, D, seed=6 + G)
    g = torch.Generator().manual_seed(97)
    signs = torch.where(torch.rand(D, generator=g) < 0.5, -1.0, 1.0) if opt == "rotated" else None
    lam = torch.exp2(torch.rand(D, generator=g) * 4 - 2) if opt == "scaled" else None
    cache = otq.Int4KVCache(B, Hkv, D, cap, device=DEV, rot_signs=None if signs is None else signs.to(DEV),
                            chan_scale=None if lam is None else lam.to(DEV))
    _fill(cache, k, v, cap)
    plan = cache.plan(Hq, max(lens), chunk=128, variant=variant)
    scale = 1.0 / math.sqrt(D)
    say(f"query magnitudes: variant={variant} G={G} opt={opt}")
    out = cache.decode(q.to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV), max(lens), scale,
                       plan=plan)
    torch.cuda.synchronize()
    rn = rot_norm32(D)
    kc, ks, vc, vs = oracle_cache(k, v, "bf16", None if signs is None else signs.numpy(), rn,
                                  chan_scale=None if lam is None else lam.numpy())
    ref = oracle.sdpa(to_bits(q), "bf16", kc, ks, vc, vs, np.array(lens, np.int32), scale,
                      signs=None if signs is None else signs.numpy(), rot_norm=rn, threads=8,
                      chan_scale=None if lam is None else lam.numpy())
    got = out.cpu().numpy()
    ma, rel = errors(got, ref)
    say(f"  max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert np.all(np.isfinite(got))
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("G", [8, 2])
@pytest.mark.parametrize("opt", ["plain", "rotated", "scaled"])
def test_query_magnitudes_head_dim_192(G, opt):
    """The query magnitudes above on the matrix-core pass at head_dim 192
    (K plain, SRFT-rotated or channel-scaled)."""
    B, Hkv, D, cap = 2, 2, 192, 256
    Hq = G * Hkv
    lens = [250, 97]
    k, v, _ = _inputs(B, Hq, Hkv, D, cap, seed=11 + G)
    q = _query_rows(B, Hq, D, seed=16 + G)
    g = torch.Generator().manual_seed(96)
    signs = torch.where(torch.rand(D, generator=g) < 0.5, -1.0, 1.0) if opt == "rotated" else None
    lam = torch.exp2(torch.rand(D, generator=g) * 4 - 2) if opt == "scaled" else None
    cache = otq.Int4KVCache(B, Hkv, D, cap, device=DEV, rot_signs=None if signs is None else signs.to(DEV),
                            chan_scale=None if lam is None else lam.to(DEV), rot_kind="srft")
    _fill(cache, k, v, cap)
    plan = cache.plan(Hq, max(lens), chunk=128, variant=MF)
    scale = 1.0 / math.sqrt(D)
    say(f"query magnitudes D=192: G={G} opt={opt}")
    out = cache.decode(q.to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV), max(lens), scale,
                       plan=plan)
    torch.cuda.synchronize()
    rn = rot_norm32(D, "srft")
    kc, ks, vc, vs = oracle_cache(k, v, "bf16", None if signs is None else signs.numpy(), rn,
                                  chan_scale=None if lam is None else lam.numpy(), rot_kind="srft")
    ref = oracle.sdpa(to_bits(q), "bf16", kc, ks, vc, vs, np.array(lens, np.int32), scale,
                      signs=None if signs is None else signs.numpy(), rot_norm=rn, threads=8,
                      chan_scale=None if lam is None else lam.numpy(), rot_kind="srft")
    got = out.cpu().numpy()
    ma, rel = errors(got, ref)
    say(f"  max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert np.all(np.isfinite(got))
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("variant", [MF, VEC])
def test_tiny_query_large_scale(variant):
    """q ~ 1e-6 with a softmax scale of 1e6 / sqrt(D): scores of order one
    built from elements that are subnormal in fp16."""
    B, Hkv, G, D, cap = 1, 2, 2, 128, 256
    k, v, q = _inputs(B, G * Hkv, Hkv, D, cap, seed=41)
    q = (q.float() * 1e-6).to(torch.bfloat16)
    cache = otq.Int4KVCache(B, Hkv, D, cap, device=DEV)
    _fill(cache, k, v, cap)
    scale = 1e6 / math.sqrt(D)
    plan = cache.plan(G * Hkv, 240, chunk=128, variant=variant)
    out = cache.decode(q.to(DEV), torch.tensor([240], dtype=torch.int32, device=DEV), 240, scale, plan=plan)
    torch.cuda.synchronize()
    ref, _ = _oracle_out(q, k, v, [240], scale, "bf16")
    ma, rel = errors(out.cpu().numpy(), ref)
    say(f"tiny q, scale 1e6/sqrt(D): variant={variant} max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("variant,G", [(MF, 8), (MF, 1), (VEC, 2)])
@pytest.mark.parametrize("kexp", [-100, -70, 20, 60, 100])
def test_value_magnitudes(variant, G, kexp):
    """V scaled by 2^kexp: 2^20 puts p s_v past fp16's largest value, 2^-70
    below its subnormals; the output must be 2^kexp times the unscaled one."""
    B, Hkv, D, cap = 2, 2, 128, 256
    Hq = G * Hkv
    lens = [256, 131]
    k, v, q = _inputs(B, Hq, Hkv, D, cap, seed=60 + G, v_scale_exp=torch.full((cap,), float(kexp)))
    cache = otq.Int4KVCache(B, Hkv, D, cap, device=DEV)
    _fill(cache, k, v, cap)
    plan = cache.plan(Hq, max(lens), chunk=128, variant=variant)
    scale = 1.0 / math.sqrt(D)
    out = cache.decode(q.to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV), max(lens), scale,
                       plan=plan)
    torch.cuda.synchronize()
    ref, _ = _oracle_out(q, k, v, lens, scale, "bf16")
    got = out.cpu().numpy().astype(np.float64) * 2.0 ** -kexp
    ref = ref * 2.0 ** -kexp
    ma, rel = errors(got, ref)
    say(f"V x 2^{kexp}: variant={variant} G={G} max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert np.all(np.isfinite(got))
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("variant,G", [(MF, 8), (MF, 1), (VEC, 2)])
def test_value_magnitudes_per_token(variant, G):
    """V whose magnitude is 2^e_t with e_t drawn per token in [-30, 30]
    (seeded): the large tokens dominate the output, and the small ones must
    not be lost where they matter."""
    B, Hkv, D, cap = 2, 2, 128, 384
    Hq = G * Hkv
    lens = [384, 200]
    ex = torch.randint(-30, 31, (cap,), generator=torch.Generator().manual_seed(3))
    k, v, q = _inputs(B, Hq, Hkv, D, cap, seed=70 + G, v_scale_exp=ex)
    cache = otq.Int4KVCache(B, Hkv, D, cap, device=DEV)
    _fill(cache, k, v, cap)
    plan = cache.plan(Hq, max(lens), chunk=128, variant=variant)
    scale = 1.0 / math.sqrt(D)
    out = cache.decode(q.to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV), max(lens), scale,
                       plan=plan)
    torch.cuda.synchronize()
    ref, _ = _oracle_out(q, k, v, lens, scale, "bf16")
    got = out.cpu().numpy().astype(np.float64)
    # compare each row relative to its own magnitude (rows are 2^30-wide apart)
    for r in range(got.shape[0] * got.shape[1]):
        gr, rr = got.reshape(-1, D)[r], ref.reshape(-1, D)[r]
        m = np.max(np.abs(rr))
        ma, rel = errors(gr / m, rr / m)
        assert ma <= MAX_ABS and rel <= REL_L2, (r, ma, rel)
    say(f"V 2^[-30,30] per token: variant={variant} G={G} ok")


def test_fused_lens_above_max_len():
    """lens[b] > max_len (out of contract) in the fused step: the split and
    the combine clamp alike, so the call equals the one with lens[b] =
    max_len: the new token lands at max_len - 1 once and is merged once."""
    B, Hkv, G, D, cap = 2, 2, 8, 128, 256
    Hq = G * Hkv
    max_len = 200
    k, v, q = _inputs(B, Hq, Hkv, D, cap, seed=88)
    kn = torch.randn((B, Hkv, D), generator=torch.Generator().manual_seed(1)).to(torch.bfloat16).to(DEV)
    vn = torch.randn((B, Hkv, D), generator=torch.Generator().manual_seed(2)).to(torch.bfloat16).to(DEV)
    outs, caches = [], []
    for lens in ([max_len + 2, 150], [max_len, 150]):
        cache = otq.Int4KVCache(B, Hkv, D, cap, device=DEV)
        _fill(cache, k, v, cap)
        plan = cache.plan(Hq, max_len, chunk=128)
        out = cache.decode_append(q.to(DEV), kn, vn, torch.tensor(lens, dtype=torch.int32, device=DEV),
                                  max_len, 1.0 / math.sqrt(D), plan=plan)
        torch.cuda.synchronize()
        outs.append(out.cpu())
        caches.append(host_cache(cache))
    assert torch.equal(outs[0], outs[1])
    for a, b in zip(*caches):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
