"""GPU parity of otq_quantize_append: codes and scales bit-exact against the
CPU oracle (the oracle sees the same 16-bit inputs; nothing it uses comes
from the GPU path)."""
import numpy as np
import pytest
import torch

import int4_kv_cache_quant_amd as otq
from int4_kv_cache_quant_amd import synth

from gpu_common import (build_cache, chan_scales, compare_codes, host_cache, oracle_cache, rand_signs,
                        rot_norm32, say, to_bits)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _rand_kv(B, H, T, D, dtype, seed, sigma=1.0, outliers=(3,)):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((2, B, H, T, D), generator=g) * sigma
    for c in outliers:
        x[..., c] *= 10
    x = x.to(dtype)
    return x[0].to(DEV), x[1].to(DEV)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("rotate", [False, True])
def test_quantize_bit_exact(D, dtype, rotate):
    B, H, T, cap = 2, 3, 77, 96
    say(f"quantize D={D} dtype={dtype} rotate={rotate}")
    k, v = _rand_kv(B, H, T, D, dtype, seed=D + 7 * rotate)
    signs = None
    if rotate:
        s = torch.where(torch.rand(D, generator=torch.Generator().manual_seed(D)) < 0.5, -1.0, 1.0)
        signs = s.to(DEV)
    cache = build_cache(k, v, cap, signs=signs, prefill_chunk=19)
    torch.cuda.synchronize()
    name = "fp16" if dtype == torch.float16 else "bf16"
    ref = oracle_cache(k.cpu(), v.cpu(), name, None if signs is None else signs.cpu().numpy(),
                       rot_norm32(D))
    bad = compare_codes(host_cache(cache), ref, T)
    assert bad == {"k_codes": 0, "k_scales": 0, "v_codes": 0, "v_scales": 0}, bad


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("rotate", [False, True])
def test_quantize_chan_scale_bit_exact(D, dtype, rotate):
    """K's per-channel scale, after the rotation: chunks of 19 tokens (the
    bulk kernel) and a last single token (the small-append kernel)."""
    B, H, T, cap = 2, 3, 77, 96
    say(f"quantize chan_scale D={D} dtype={dtype} rotate={rotate}")
    k, v = _rand_kv(B, H, T, D, dtype, seed=D + 11 * rotate + 5)
    signs = None
    if rotate:
        s = torch.where(torch.rand(D, generator=torch.Generator().manual_seed(D + 1)) < 0.5, -1.0, 1.0)
        signs = s.to(DEV)
    lam = chan_scales(D, D + rotate, outliers=(3,))
    cache = build_cache(k, v, cap, signs=signs, prefill_chunk=19, chan_scale=lam.to(DEV))
    torch.cuda.synchronize()
    name = "fp16" if dtype == torch.float16 else "bf16"
    ref = oracle_cache(k.cpu(), v.cpu(), name, None if signs is None else signs.cpu().numpy(),
                       rot_norm32(D), chan_scale=lam.numpy())
    bad = compare_codes(host_cache(cache), ref, T)
    assert bad == {"k_codes": 0, "k_scales": 0, "v_codes": 0, "v_scales": 0}, bad


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("rotate_k", [False, True])
def test_quantize_v_rotated_bit_exact(D, dtype, rotate_k):
    """V rotated with its own signs: chunks of 19 tokens (the bulk kernel's
    rotated-V form, whole and edge tiles) and a last single token."""
    B, H, T, cap = 2, 3, 77, 96
    say(f"quantize v-rotated D={D} dtype={dtype} rotate_k={rotate_k}")
    k, v = _rand_kv(B, H, T, D, dtype, seed=D + 13 * rotate_k + 3, outliers=(3, 17))
    ks = rand_signs(D, D + 2) if rotate_k else None
    vs = rand_signs(D, D + 3)
    cache = build_cache(k, v, cap, signs=None if ks is None else ks.to(DEV), prefill_chunk=19,
                        v_signs=vs.to(DEV))
    torch.cuda.synchronize()
    name = "fp16" if dtype == torch.float16 else "bf16"
    ref = oracle_cache(k.cpu(), v.cpu(), name, None if ks is None else ks.numpy(), rot_norm32(D),
                       v_signs=vs.numpy())
    bad = compare_codes(host_cache(cache), ref, T)
    assert bad == {"k_codes": 0, "k_scales": 0, "v_codes": 0, "v_scales": 0}, bad


def test_quantize_adversarial_values():
    """Ties at every half-step, zero groups, subnormal groups, -0.0, abs-max
    in every lane position, fp16 inputs."""
    D, B, H = 128, 1, 1
    rows = []
    for pos in range(32):                       # abs-max at each position of the group
        x = np.zeros(D, np.float32)
        x[:32] = (np.arange(32) % 15 - 7) / 2.0  # k/2 ties
        x[pos] = 7.0
        x[32:64] = np.float32(-0.0)             # -0 group -> zero scale
        x[64:96] = np.float32(1e-6) * (np.arange(32) - 16)   # fp16 subnormals
        x[96:128] = 3.5 * ((-1.0) ** np.arange(32))            # all ties at abs-max/2
        rows.append(x)
    x = torch.tensor(np.stack(rows), dtype=torch.float16)[None, None]   # [1,1,32,D]
    T = x.shape[2]
    k = x.to(DEV)
    v = (-x).to(DEV)
    say("quantize adversarial")
    cache = build_cache(k, v, 32, prefill_chunk=5)
    torch.cuda.synchronize()
    ref = oracle_cache(x, -x, "fp16")
    bad = compare_codes(host_cache(cache), ref, T)
    assert bad == {"k_codes": 0, "k_scales": 0, "v_codes": 0, "v_scales": 0}, bad


def test_quantize_adversarial_bf16_ranges():
    """bf16 groups across the exponent range, with ties at every half-step and
    the abs-max in every lane position: scales below 2^-90 (bf16 subnormal
    inputs among them) and above 2^100, which divide element by element, and
    scales just inside those bounds, which divide from one reciprocal."""
    D = 256
    exps = (-131, -120, -93, -87, 0, 95, 101, 120)
    rows = []
    for pos in range(32):
        x = np.zeros(D, np.float32)
        for g, e in enumerate(exps):
            grp = (np.arange(32) % 15 - 7) / 2.0
            grp[pos] = 7.0 if g % 2 == 0 else -7.0
            x[32 * g:32 * g + 32] = np.ldexp(grp, e)
        rows.append(x)
    x = torch.tensor(np.stack(rows), dtype=torch.bfloat16)[None, None]   # [1,1,32,D]
    assert torch.equal(x.float(), torch.tensor(np.stack(rows))[None, None])  # exact in bf16
    say("quantize adversarial bf16 ranges")
    cache = build_cache(x.to(DEV), (-x).to(DEV), 32, prefill_chunk=16)
    torch.cuda.synchronize()
    ref = oracle_cache(x, -x, "bf16")
    bad = compare_codes(host_cache(cache), ref, 32)
    assert bad == {"k_codes": 0, "k_scales": 0, "v_codes": 0, "v_scales": 0}, bad


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("scaled", [False, True])
@pytest.mark.parametrize("chunk", [19, 5])
def test_quantize_srft_bit_exact(D, dtype, scaled, chunk):
    """K rotated by the sign-randomised FFT (then, if scaled, by K's
    per-channel scale): chunks of 19 tokens take the bulk kernel (whole and
    edge tiles), chunks of 5 the small-append kernel; the last token comes
    alone.  Codes and scales are the oracle's bit for bit."""
    B, H, T, cap = 2, 3, 77, 96
    say(f"quantize srft D={D} dtype={dtype} scaled={scaled} chunk={chunk}")
    k, v = _rand_kv(B, H, T, D, dtype, seed=D + 23 + 2 * scaled + chunk, outliers=(3, 40))
    signs = rand_signs(D, D + 29)
    lam = chan_scales(D, D + 31, outliers=(3,)) if scaled else None
    cache = build_cache(k, v, cap, signs=signs.to(DEV), prefill_chunk=chunk,
                        chan_scale=None if lam is None else lam.to(DEV), rot_kind="srft")
    torch.cuda.synchronize()
    name = "fp16" if dtype == torch.float16 else "bf16"
    ref = oracle_cache(k.cpu(), v.cpu(), name, signs.numpy(), rot_norm32(D, "srft"),
                       chan_scale=None if lam is None else lam.numpy(), rot_kind="srft")
    bad = compare_codes(host_cache(cache), ref, T)
    assert bad == {"k_codes": 0, "k_scales": 0, "v_codes": 0, "v_scales": 0}, bad


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("rotate_k", [False, True])
def test_quantize_srft_v_rotated_bit_exact(D, dtype, rotate_k):
    """V rotated by the sign-randomised FFT (its own signs), K too or not:
    chunks of 19 (the bulk kernel's rotated-V form, whole and edge tiles) and
    a last single token."""
    B, H, T, cap = 2, 3, 77, 96
    say(f"quantize srft v-rotated D={D} dtype={dtype} rotate_k={rotate_k}")
    k, v = _rand_kv(B, H, T, D, dtype, seed=D + 17 * rotate_k + 9, outliers=(3, 17))
    ks = rand_signs(D, D + 71) if rotate_k else None
    vs = rand_signs(D, D + 73)
    cache = build_cache(k, v, cap, signs=None if ks is None else ks.to(DEV), prefill_chunk=19,
                        v_signs=vs.to(DEV), rot_kind="srft")
    torch.cuda.synchronize()
    name = "fp16" if dtype == torch.float16 else "bf16"
    ref = oracle_cache(k.cpu(), v.cpu(), name, None if ks is None else ks.numpy(), rot_norm32(D, "srft"),
                       v_signs=vs.numpy(), rot_kind="srft")
    bad = compare_codes(host_cache(cache), ref, T)
    assert bad == {"k_codes": 0, "k_scales": 0, "v_codes": 0, "v_scales": 0}, bad


@pytest.mark.parametrize("D", [64, 256])
def test_quantize_srft_exponent_ranges(D):
    """FFT-rotated bf16 vectors scaled across the exponent range: twiddle
    products in the subnormal range, scales below 2^-80 and above 2^100 (which
    divide element by element) and just inside them."""
    exps = (-131, -120, -93, -87, 0, 95, 101, 120)
    g = torch.Generator().manual_seed(D + 61)
    base = torch.randn((32, D), generator=g)
    x = torch.stack([torch.ldexp(base[t], torch.tensor(exps[t % len(exps)])) for t in range(32)])
    x = x.to(torch.bfloat16)[None, None]   # [1,1,32,D]
    signs = rand_signs(D, D + 67)
    say(f"quantize srft exponent ranges D={D}")
    cache = build_cache(x.to(DEV), (-x).to(DEV), 32, prefill_chunk=16, signs=signs.to(DEV),
                        rot_kind="srft")
    torch.cuda.synchronize()
    ref = oracle_cache(x, -x, "bf16", signs.numpy(), rot_norm32(D, "srft"), rot_kind="srft")
    bad = compare_codes(host_cache(cache), ref, 32)
    assert bad == {"k_codes": 0, "k_scales": 0, "v_codes": 0, "v_scales": 0}, bad


def test_append_preserves_neighbours_and_skips_out_of_range():
    """Single-token appends at odd and even positions keep the other nibble of
    each shared V byte; positions outside [0, capacity) are not written."""
    D, B, H, cap = 128, 3, 2, 64
    k, v = _rand_kv(B, H, cap, D, torch.bfloat16, seed=5)
    cache = otq.Int4KVCache(B, H, D, cap, device=DEV)
    order = np.random.default_rng(0).permutation(cap)      # scattered single appends
    for t in order:
        pos = torch.full((B,), int(t), dtype=torch.int32, device=DEV)
        cache.append(k[:, :, t:t + 1].contiguous(), v[:, :, t:t + 1].contiguous(), pos)
    torch.cuda.synchronize()
    ref = oracle_cache(k.cpu(), v.cpu(), "bf16")
    assert compare_codes(host_cache(cache), ref, cap) == {"k_codes": 0, "k_scales": 0, "v_codes": 0, "v_scales": 0}
    before = [t.clone() for t in (cache.k_codes, cache.k_scales, cache.v_codes, cache.v_scales)]
    # straddling the end: 4 tokens at pos cap-2 -> only cap-2, cap-1 are written
    pos = torch.tensor([cap - 2, -3, cap], dtype=torch.int32, device=DEV)
    k2, v2 = _rand_kv(B, H, 4, D, torch.bfloat16, seed=6)
    cache.append(k2, v2, pos)
    torch.cuda.synchronize()
    after = [t for t in (cache.k_codes, cache.k_scales, cache.v_codes, cache.v_scales)]
    # sequence 1 (pos -3: tokens -3..0) writes only token 0; sequence 2 writes nothing
    assert torch.equal(before[0][2], after[0][2]) and torch.equal(before[2][2], after[2][2])
    assert torch.equal(before[0][1, :, 1:], after[0][1, :, 1:])
    assert torch.equal(before[1][0, :, :cap - 2], after[1][0, :, :cap - 2])
    kk = torch.cat([k[:, :, :cap - 2].cpu(), k2[:, :, :2].cpu()], 2)[0:1]
    vv = torch.cat([v[:, :, :cap - 2].cpu(), v2[:, :, :2].cpu()], 2)[0:1]
    ref0 = oracle_cache(kk, vv, "bf16")
    got = tuple(a[0:1] for a in host_cache(cache))
    assert compare_codes(got, ref0, cap) == {"k_codes": 0, "k_scales": 0, "v_codes": 0, "v_scales": 0}
    k1 = k[1:2, :, :].cpu().clone()
    v1 = v[1:2, :, :].cpu().clone()
    k1[:, :, 0] = k2[1:2, :, 3].cpu()
    v1[:, :, 0] = v2[1:2, :, 3].cpu()
    ref1 = oracle_cache(k1, v1, "bf16")
    got = tuple(a[1:2] for a in host_cache(cache))
    assert compare_codes(got, ref1, cap) == {"k_codes": 0, "k_scales": 0, "v_codes": 0, "v_scales": 0}


@pytest.mark.parametrize("D", [64, 128, 256])
def test_bulk_append_merges_partial_tiles(D):
    """Bulk appends (8 tokens and more) at unaligned positions write exactly
    their range: whole V tiles inside it, the V words shared with older tokens
    at both ends merged, and ranges clipped to [0, capacity)."""
    B, H, cap = 3, 2, 128
    zero = {"k_codes": 0, "k_scales": 0, "v_codes": 0, "v_scales": 0}
    k, v = _rand_kv(B, H, cap, D, torch.bfloat16, seed=D)
    say(f"bulk append D={D}")
    cache = build_cache(k, v, cap, prefill_chunk=cap, append_last=False)
    kk, vv = k.cpu().clone(), v.cpu().clone()
    rng = np.random.default_rng(D)
    for step, n in enumerate([8, 9, 31, 33, 45, 64]):
        p = rng.integers(0, cap - n + 1, size=B)
        k2, v2 = _rand_kv(B, H, n, D, torch.bfloat16, seed=100 + step, outliers=(step,))
        cache.append(k2, v2, torch.tensor(p, dtype=torch.int32, device=DEV))
        for b in range(B):
            kk[b, :, p[b]:p[b] + n] = k2[b].cpu()
            vv[b, :, p[b]:p[b] + n] = v2[b].cpu()
    # straddling the end, starting below zero, starting at the capacity
    n = 20
    k2, v2 = _rand_kv(B, H, n, D, torch.bfloat16, seed=7)
    cache.append(k2, v2, torch.tensor([cap - 7, -11, cap], dtype=torch.int32, device=DEV))
    kk[0, :, cap - 7:] = k2[0, :, :7].cpu()
    vv[0, :, cap - 7:] = v2[0, :, :7].cpu()
    kk[1, :, :9] = k2[1, :, 11:].cpu()
    vv[1, :, :9] = v2[1, :, 11:].cpu()
    torch.cuda.synchronize()
    assert compare_codes(host_cache(cache), oracle_cache(kk, vv, "bf16"), cap) == zero


@pytest.mark.parametrize("cfg", [1, 4, 5])
def test_quantize_full_size_workloads(cfg):
    """Every token of one layer of the workload, at its full size."""
    w = synth.WORKLOADS[cfg]
    say(f"quantize full workload {cfg} {w.name}")
    k = synth.kv(w, 0, "k", device=DEV)
    v = synth.kv(w, 0, "v", device=DEV)
    signs = torch.from_numpy(synth.rot_signs(w, 0)).to(DEV) if w.rotate else None
    cache = build_cache(k, v, w.capacity, signs=signs, prefill_chunk=8192)
    torch.cuda.synchronize()
    ref = oracle_cache(k.cpu(), v.cpu(), w.dtype,
                       None if signs is None else signs.cpu().numpy(), rot_norm32(w.D), threads=16)
    bad = compare_codes(host_cache(cache), ref, w.T)
    assert bad == {"k_codes": 0, "k_scales": 0, "v_codes": 0, "v_scales": 0}, bad
