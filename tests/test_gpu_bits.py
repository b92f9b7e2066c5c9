"""GPU parity of the 2- and 3-bit path (plain bit-stream K rows, V in
32-token tiles): codes and scales bit-exact against the oracle's b-bit
quantiser (its plain rows, with the V tiles converted back by layout.py),
outputs of the split + combine within the same tolerance as int4 against the
oracle's fp64 attention over the cache it quantised itself."""
import math

import numpy as np
import pytest
import torch

import int4_kv_cache_quant_amd as otq
import oracle
from int4_kv_cache_quant_amd import layout, synth

from gpu_common import MAX_ABS, REL_L2, errors, say, to_bits

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _kv(B, H, T, D, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((2, B, H, T, D), generator=g)
    x[..., 3] *= 10
    x = x.to(dtype)
    return x[0], x[1]


def _vplain(cache):
    """The cache's V codes as plain b-bit rows [B, H, C, D*b/8]."""
    D = cache.shape[2]
    return layout.v_bits_tiled_to_plain(cache.v_codes.cpu().numpy(), D, cache.code_bits)


def _set_vplain(cache, plain):
    D = cache.shape[2]
    cache.v_codes.copy_(torch.from_numpy(layout.v_bits_plain_to_tiled(plain, D, cache.code_bits)).to(DEV))


def _build(k, v, cap, bits, chunk):
    B, H, T, D = k.shape
    cache = otq.Int4KVCache(B, H, D, cap, device=DEV, code_bits=bits)
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        pos = torch.full((B,), t0, dtype=torch.int32, device=DEV)
        cache.append(k[:, :, t0:t1].to(DEV).contiguous(), v[:, :, t0:t1].to(DEV).contiguous(), pos)
    torch.cuda.synchronize()
    return cache


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("chunk", [19, 1])
def test_bits_quantize_bit_exact(bits, D, dtype, chunk):
    B, H, T, cap = 2, 3, 45, 64
    say(f"bits quantize b={bits} D={D} dtype={dtype} chunk={chunk}")
    k, v = _kv(B, H, T, D, dtype, seed=bits * 1000 + D + chunk)
    cache = _build(k, v, cap, bits, chunk)
    name = "fp16" if dtype == torch.float16 else "bf16"
    kc, ks = oracle.quantize(to_bits(k), name, code_bits=bits)
    vc, vs = oracle.quantize(to_bits(v), name, code_bits=bits)
    vp = _vplain(cache)
    got = [cache.k_codes.cpu().numpy()[:, :, :T], cache.k_scales.cpu().numpy()[:, :, :T], vp[:, :, :T],
           cache.v_scales.cpu().numpy()[:, :, :T]]
    for g, r in zip(got, (kc, ks, vc, vs)):
        if g.dtype == np.float32:
            g, r = g.view(np.uint32), r.view(np.uint32)
        assert np.array_equal(g, r)
    # tokens past the appended range stay untouched (T = 45 ends inside a V tile)
    assert not np.any(cache.k_codes.cpu().numpy()[:, :, T:]) and not np.any(cache.v_scales.cpu().numpy()[:, :, T:])
    assert not np.any(vp[:, :, T:])


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("G,D", [(1, 64), (4, 128), (8, 128), (16, 64), (2, 256)])
@pytest.mark.parametrize("variant", [otq.OTQ_VARIANT_AUTO, otq.OTQ_VARIANT_VECTOR])
def test_bits_sdpa_parity(bits, G, D, variant):
    B, Hkv, cap = 2, 2, 448
    lens = [448, 77]
    say(f"bits sdpa b={bits} G={G} D={D} variant={variant}")
    k, v = _kv(B, Hkv, cap, D, torch.bfloat16, seed=bits * 100 + G + D)
    g = torch.Generator().manual_seed(G + D)
    q = torch.randn((B, G * Hkv, D), generator=g).to(torch.bfloat16)
    cache = _build(k, v, cap, bits, 100)
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    plan = cache.plan(G * Hkv, max(lens), chunk=128, variant=variant)
    # b-bit codes default to the MFMA split pass
    mfma_ok = True
    want = otq.OTQ_VARIANT_MFMA if (mfma_ok and variant == otq.OTQ_VARIANT_AUTO) else otq.OTQ_VARIANT_VECTOR
    assert plan.variant == want
    scale = 1.0 / math.sqrt(D)
    out = cache.decode(q.to(DEV), lens_t, max(lens), scale, plan=plan)
    torch.cuda.synchronize()
    kc, ks = oracle.quantize(to_bits(k), "bf16", code_bits=bits)
    vc, vs = oracle.quantize(to_bits(v), "bf16", code_bits=bits)
    ref = oracle.sdpa(to_bits(q), "bf16", kc, ks, vc, vs, np.array(lens, np.int32), scale, threads=8,
                      code_bits=bits)
    ma, rel = errors(out.cpu().numpy(), ref)
    say(f"  max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("bits", [2, 3])
def test_bits_edge_lengths_and_ragged_batch(bits):
    B, Hkv, G, D, cap = 5, 2, 4, 128, 384
    lens = [0, 1, 256, 129, 384]
    k, v = _kv(B, Hkv, cap, D, torch.float16, seed=bits + 7)
    g = torch.Generator().manual_seed(bits)
    q = torch.randn((B, G * Hkv, D), generator=g).to(torch.float16)
    cache = _build(k, v, cap, bits, cap)
    out = cache.decode(q.to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV), cap, 0.1)
    torch.cuda.synchronize()
    kc, ks = oracle.quantize(to_bits(k), "fp16", code_bits=bits)
    vc, vs = oracle.quantize(to_bits(v), "fp16", code_bits=bits)
    ref = oracle.sdpa(to_bits(q), "fp16", kc, ks, vc, vs, np.array(lens, np.int32), 0.1, threads=8,
                      code_bits=bits)
    got = out.cpu().numpy()
    assert np.all(got[0] == 0.0)
    ma, rel = errors(got, ref)
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("bits", [2, 3])
def test_bits_full_workload_3(bits):
    """The 70B layer at 131072 tokens with b-bit codes: every code and
    scale bit-exact, every output row within tolerance."""
    w = synth.WORKLOADS[3]
    say(f"bits full workload 3 b={bits}")
    k = synth.kv(w, 0, "k", device=DEV)
    v = synth.kv(w, 0, "v", device=DEV)
    q = synth.query(w, 0, device=DEV)
    cache = otq.Int4KVCache(w.B, w.Hkv, w.D, w.capacity, device=DEV, code_bits=bits)
    for t0 in range(0, w.T, 16384):
        pos = torch.full((w.B,), t0, dtype=torch.int32, device=DEV)
        cache.append(k[:, :, t0:t0 + 16384].contiguous(), v[:, :, t0:t0 + 16384].contiguous(), pos)
    lens = synth.lens(w, 0)
    out = cache.decode(q, torch.from_numpy(lens).to(DEV), int(lens.max()), w.scale)
    torch.cuda.synchronize()
    kc, ks = oracle.quantize(to_bits(k.cpu()), w.dtype, threads=16, code_bits=bits)
    vc, vs = oracle.quantize(to_bits(v.cpu()), w.dtype, threads=16, code_bits=bits)
    T = w.T
    assert np.array_equal(cache.k_codes.cpu().numpy()[:, :, :T], kc)
    assert np.array_equal(_vplain(cache)[:, :, :T], vc)
    assert np.array_equal(cache.k_scales.cpu().numpy()[:, :, :T].view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(cache.v_scales.cpu().numpy()[:, :, :T].view(np.uint32), vs.view(np.uint32))
    ref = oracle.sdpa(to_bits(q.cpu()), w.dtype, kc, ks, vc, vs, lens, w.scale, threads=16, code_bits=bits)
    ma, rel = errors(out.cpu().numpy(), ref)
    say(f"  max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("opts", ["srht", "srft+lam", "srht+vrot", "srft+vrot+lam"])
@pytest.mark.parametrize("G,D", [(8, 128), (2, 64), (1, 256)])
def test_bits_with_rotations_and_scale(bits, opts, G, D):
    """b-bit caches with K rotated (either kind), K's channel scale and V
    rotated: codes bit-exact, outputs within tolerance (the combine brings a
    rotated V's rows back)."""
    B, Hkv, cap = 2, 2, 320
    lens = [320, 99]
    kind = "srft" if "srft" in opts else "srht"
    say(f"bits options b={bits} opts={opts} G={G} D={D}")
    k, v = _kv(B, Hkv, cap, D, torch.bfloat16, seed=bits * 31 + G + D + len(opts))
    g = torch.Generator().manual_seed(G * D + bits)
    q = torch.randn((B, G * Hkv, D), generator=g).to(torch.bfloat16)
    sk = torch.where(torch.rand(D, generator=g) < 0.5, -1.0, 1.0)
    sv = torch.where(torch.rand(D, generator=g) < 0.5, -1.0, 1.0) if "vrot" in opts else None
    lam = torch.exp2(torch.rand(D, generator=g) * 4.0 - 2.0) if "lam" in opts else None
    cache = otq.Int4KVCache(B, Hkv, D, cap, device=DEV, code_bits=bits, rot_signs=sk.to(DEV), rot_kind=kind,
                            chan_scale=None if lam is None else lam.to(DEV),
                            v_rot_signs=None if sv is None else sv.to(DEV))
    for t0 in range(0, cap, 100):
        pos = torch.full((B,), t0, dtype=torch.int32, device=DEV)
        cache.append(k[:, :, t0:t0 + 100].to(DEV).contiguous(), v[:, :, t0:t0 + 100].to(DEV).contiguous(), pos)
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    scale = 1.0 / math.sqrt(D)
    out = cache.decode(q.to(DEV), lens_t, max(lens), scale)
    torch.cuda.synchronize()
    rn = cache.rot_norm
    lam_np = None if lam is None else lam.numpy()
    sv_np = None if sv is None else sv.numpy()
    kc, ks = oracle.quantize(to_bits(k), "bf16", signs=sk.numpy(), rot_norm=rn, chan_scale=lam_np, rot_kind=kind,
                             code_bits=bits)
    vc, vs = oracle.quantize(to_bits(v), "bf16", signs=sv_np, rot_norm=rn, rot_kind=kind, code_bits=bits)
    assert np.array_equal(cache.k_codes.cpu().numpy(), kc)
    assert np.array_equal(cache.k_scales.cpu().numpy().view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(_vplain(cache), vc)
    assert np.array_equal(cache.v_scales.cpu().numpy().view(np.uint32), vs.view(np.uint32))
    ref = oracle.sdpa(to_bits(q), "bf16", kc, ks, vc, vs, np.array(lens, np.int32), scale, signs=sk.numpy(),
                      rot_norm=rn, threads=8, chan_scale=lam_np, v_signs=sv_np, rot_kind=kind, code_bits=bits)
    ma, rel = errors(out.cpu().numpy(), ref)
    say(f"  max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert ma <= MAX_ABS and rel <= REL_L2



@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("opts", ["plain", "vrot", "srht+lam", "srft+vrot"])
@pytest.mark.parametrize("G,D", [(8, 128), (4, 64), (2, 256)])
def test_bits_fused_decode_step(bits, opts, G, D):
    """One decode step of a b-bit cache in one call: the split pass covers
    [0, lens - 1), the combine quantises the token at lens - 1 into its b-bit
    rows and merges it.  The token's slot holds junk before the call (code
    bytes and Inf/NaN scales); afterwards the whole cache equals the oracle's
    quantisation bit for bit and the outputs match the fp64 oracle.  Caches
    take the MFMA split pass (a rotated or channel-scaled K with a hi + lo
    query, up to D = 128), the others the vector one."""
    B, Hkv, cap = 3, 2, 320
    lens = [301, 96, 1]  # a token inside a tile, one opening a tile, one alone
    kind = "srft" if "srft" in opts else "srht"
    say(f"bits fused b={bits} opts={opts} G={G} D={D}")
    k, v = _kv(B, Hkv, cap, D, torch.bfloat16, seed=bits * 53 + G + D + len(opts))
    g = torch.Generator().manual_seed(G * D + bits + 5)
    q = torch.randn((B, G * Hkv, D), generator=g).to(torch.bfloat16)
    sk = torch.where(torch.rand(D, generator=g) < 0.5, -1.0, 1.0) if ("srht" in opts or "srft" in opts) else None
    sv = torch.where(torch.rand(D, generator=g) < 0.5, -1.0, 1.0) if "vrot" in opts else None
    lam = torch.exp2(torch.rand(D, generator=g) * 4.0 - 2.0) if "lam" in opts else None
    cache = otq.Int4KVCache(B, Hkv, D, cap, device=DEV, code_bits=bits,
                            rot_signs=None if sk is None else sk.to(DEV), rot_kind=kind,
                            chan_scale=None if lam is None else lam.to(DEV),
                            v_rot_signs=None if sv is None else sv.to(DEV))
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    cache.append(k.to(DEV).contiguous(), v.to(DEV).contiguous(), pos)
    torch.cuda.synchronize()
    rng = np.random.default_rng(bits + D)
    vp = _vplain(cache)
    for b, n in enumerate(lens):  # junk in the new token's slot
        cache.k_codes[b, :, n - 1] = torch.from_numpy(rng.integers(0, 256, size=(Hkv, D * bits // 8),
                                                                   dtype=np.uint8)).to(DEV)
        vp[b, :, n - 1] = rng.integers(0, 256, size=(Hkv, D * bits // 8), dtype=np.uint8)
        cache.k_scales[b, :, n - 1] = float("nan")
        cache.v_scales[b, :, n - 1] = float("inf")
    _set_vplain(cache, vp)
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    idx = (lens_t.long() - 1)
    ar = torch.arange(B, device=DEV)
    kn = k.to(DEV)[ar, :, idx].contiguous()
    vn = v.to(DEV)[ar, :, idx].contiguous()
    scale = 1.0 / math.sqrt(D)
    plan = cache.plan(G * Hkv, max(lens), chunk=128)
    plain_k = sk is None and lam is None
    want = otq.OTQ_VARIANT_MFMA if (plain_k or D <= 128) else otq.OTQ_VARIANT_VECTOR
    assert plan.variant == want
    otq.otq_last_device_error()
    out = cache.decode_append(q.to(DEV), kn, vn, lens_t, max(lens), scale, plan=plan)
    torch.cuda.synchronize()
    assert otq.otq_last_device_error() == 0
    rn = cache.rot_norm
    lam_np = None if lam is None else lam.numpy()
    sk_np = None if sk is None else sk.numpy()
    sv_np = None if sv is None else sv.numpy()
    kc, ks = oracle.quantize(to_bits(k), "bf16", signs=sk_np, rot_norm=rn, chan_scale=lam_np, rot_kind=kind,
                             code_bits=bits)
    vc, vs = oracle.quantize(to_bits(v), "bf16", signs=sv_np, rot_norm=rn, rot_kind=kind, code_bits=bits)
    assert np.array_equal(cache.k_codes.cpu().numpy(), kc)
    assert np.array_equal(cache.k_scales.cpu().numpy().view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(_vplain(cache), vc)
    assert np.array_equal(cache.v_scales.cpu().numpy().view(np.uint32), vs.view(np.uint32))
    ref = oracle.sdpa(to_bits(q), "bf16", kc, ks, vc, vs, np.array(lens, np.int32), scale, signs=sk_np,
                      rot_norm=rn, threads=8, chan_scale=lam_np, v_signs=sv_np, rot_kind=kind, code_bits=bits)
    ma, rel = errors(out.cpu().numpy(), ref)
    say(f"  max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("p0,n", [(37, 100), (5, 8), (64, 64), (90, 7)])
def test_bits_append_inside_a_filled_cache(bits, D, p0, n):
    """A cache filled with one set of tokens, then n other tokens appended at
    p0 (tile-aligned or not, bulk and short appends): the new tokens' codes
    and scales are the oracle's, every other token keeps its bytes (its V
    fields share tile words with the new ones)."""
    B, H, cap = 2, 2, 192
    say(f"bits overwrite b={bits} D={D} p0={p0} n={n}")
    k, v = _kv(B, H, cap, D, torch.bfloat16, seed=bits * 7 + D + p0)
    k2, v2 = _kv(B, H, n, D, torch.bfloat16, seed=bits * 11 + D + n)
    cache = _build(k, v, cap, bits, cap)
    pos = torch.full((B,), p0, dtype=torch.int32, device=DEV)
    cache.append(k2.to(DEV).contiguous(), v2.to(DEV).contiguous(), pos)
    torch.cuda.synchronize()
    km, vm = k.clone(), v.clone()
    km[:, :, p0:p0 + n] = k2
    vm[:, :, p0:p0 + n] = v2
    kc, ks = oracle.quantize(to_bits(km), "bf16", code_bits=bits)
    vc, vs = oracle.quantize(to_bits(vm), "bf16", code_bits=bits)
    assert np.array_equal(cache.k_codes.cpu().numpy(), kc)
    assert np.array_equal(cache.k_scales.cpu().numpy().view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(_vplain(cache), vc)
    assert np.array_equal(cache.v_scales.cpu().numpy().view(np.uint32), vs.view(np.uint32))
