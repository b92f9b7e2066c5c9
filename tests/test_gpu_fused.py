"""GPU parity of otq_sdpa_int4_decode_append (one decode step: the split
pass covers the cached tokens, the combine pass quantises the new token into
the cache and merges it).

Each case prefills every sequence, then poisons the slot of its new token
(K codes and scales, the V scale and the token's own V nibble; the
neighbour's nibble is kept) and runs the fused call with that token as
k_new / v_new.  The whole cache must then equal the oracle's quantisation bit
for bit, and the outputs must be within the usual tolerance of the fp64
oracle over [0, lens[b])."""
import math

import numpy as np
import pytest
import torch

import int4_kv_cache_quant_amd as otq
import oracle
from int4_kv_cache_quant_amd import layout, synth

from gpu_common import (MAX_ABS, REL_L2, build_cache, chan_scales, compare_codes, errors, host_cache,
                        oracle_cache, rand_signs, rot_norm32, say, to_bits)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _poison(cache, lens):
    """Overwrite the slot of token lens[b] - 1 of every sequence with junk."""
    B, H, D, cap = cache.shape
    vplain = layout.v_tiled_to_plain(cache.v_codes.cpu().numpy(), D)
    for b, n in enumerate(lens):
        if n < 1:
            continue
        p = n - 1
        cache.k_codes[b, :, p] = 0x5A
        cache.k_scales[b, :, p] = 123.0
        cache.v_scales[b, :, p] = -7.0
        # token p's nibble of every channel pair: byte c // 2 of the plain row
        vplain[b, :, p] = 0xA5
    # keep the neighbours' nibbles: only token p's own nibbles change
    orig = layout.v_tiled_to_plain(cache.v_codes.cpu().numpy(), D)
    mixed = orig.copy()
    for b, n in enumerate(lens):
        if n >= 1:
            mixed[b, :, n - 1] = vplain[b, :, n - 1]
    cache.v_codes.copy_(torch.from_numpy(layout.v_plain_to_tiled(mixed, D)).to(DEV))


def _run(B, G, Hkv, D, cap, lens, dtype=torch.bfloat16, rotate=False, chunk=0, seed=0, steps=1,
         variant=otq.OTQ_VARIANT_MFMA, scaled=False, rotate_v=False, splits=0):
    """rotate: False, True (the Hadamard rotation) or "srft" (the FFT one)."""
    kind = "srft" if rotate == "srft" else "srht"
    g = torch.Generator().manual_seed(seed)
    Hq = G * Hkv
    T = max(lens) + steps - 1
    k = torch.randn((B, Hkv, cap, D), generator=g)
    v = torch.randn((B, Hkv, cap, D), generator=g)
    k[..., 3] *= 10
    v[..., 3] *= 10
    k, v = k.to(dtype), v.to(dtype)
    signs = torch.where(torch.rand(D, generator=g) < 0.5, -1.0, 1.0) if rotate else None
    lam = chan_scales(D, seed, outliers=(3,)) if scaled else None
    lam_np = None if lam is None else lam.numpy()
    vsg = rand_signs(D, seed + 1000) if rotate_v else None
    vsg_np = None if vsg is None else vsg.numpy()
    name = "fp16" if dtype == torch.float16 else "bf16"
    scale = 1.0 / math.sqrt(D)
    cache = build_cache(k[:, :, :T].to(DEV).contiguous(), v[:, :, :T].to(DEV).contiguous(), cap,
                        signs=None if signs is None else signs.to(DEV), append_last=False,
                        chan_scale=None if lam is None else lam.to(DEV),
                        v_signs=None if vsg is None else vsg.to(DEV), rot_kind=kind)
    ref_cache = oracle_cache(k, v, name, None if signs is None else signs.numpy(), rot_norm32(D, kind),
                             chan_scale=lam_np, v_signs=vsg_np, rot_kind=kind)
    for step in range(steps):
        cur = [n + step for n in lens]
        _poison(cache, cur)
        lens_t = torch.tensor(cur, dtype=torch.int32, device=DEV)
        idx = (lens_t.long() - 1).clamp(min=0)
        ar = torch.arange(B, device=DEV)
        kn = k.to(DEV)[ar, :, idx].contiguous()   # [B, Hkv, D]
        vn = v.to(DEV)[ar, :, idx].contiguous()
        q = torch.randn((B, Hq, D), generator=g).to(dtype)
        max_len = max(1, max(cur))
        plan = cache.plan(Hq, max_len, chunk=chunk, variant=variant, splits=splits)
        say(f"fused B={B} G={G} Hkv={Hkv} D={D} lens={cur} chunk={plan.chunk} rotate={rotate} "
            f"scaled={scaled} rotate_v={rotate_v}")
        out = cache.decode_append(q.to(DEV), kn, vn, lens_t, max_len, scale, plan=plan)
        torch.cuda.synchronize()
        got_cache = host_cache(cache)
        for b, n in enumerate(cur):
            if n < 1:
                continue
            sub = tuple(x[b:b + 1, :, :n] for x in got_cache)
            ref = tuple(x[b:b + 1, :, :n] for x in ref_cache)
            assert compare_codes(sub, ref, n) == {
                "k_codes": 0, "k_scales": 0, "v_codes": 0, "v_scales": 0}, f"seq {b}"
        kc, ks, vc, vs = ref_cache
        ref = oracle.sdpa(to_bits(q), name, kc, ks, vc, vs, np.array(cur, np.int32), scale,
                          signs=None if signs is None else signs.numpy(), rot_norm=rot_norm32(D, kind),
                          threads=8, chan_scale=lam_np, v_signs=vsg_np, rot_kind=kind)
        ma, rel = errors(out.cpu().numpy(), ref)
        say(f"  max_abs={ma:.3e} rel_l2={rel:.3e}")
        assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 4, 8, 16])
@pytest.mark.parametrize("rotate", [False, True])
def test_fused_append_parity(D, G, rotate):
    # new tokens at an odd and an even position, in the middle of a chunk
    _run(2, G, 2, D, 384, [351, 190], rotate=rotate, chunk=128, seed=D + G + rotate)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 8])
@pytest.mark.parametrize("rotate", [False, True])
def test_fused_append_chan_scale(D, G, rotate):
    """K with a per-channel scale: the combine quantises the new token with
    it and divides q by it for the token's score."""
    _run(2, G, 2, D, 384, [351, 190], rotate=rotate, chunk=128, seed=7 * D + G + rotate, scaled=True)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 8])
@pytest.mark.parametrize("rotate,scaled", [(False, False), (True, False), (True, True)])
def test_fused_append_v_rotated(D, G, rotate, scaled):
    """V rotated: the combine rotates the new token's V before quantising
    it and the output is brought back by the inverse rotation."""
    _run(2, G, 2, D, 384, [351, 190], rotate=rotate, chunk=128, seed=11 * D + G + rotate + scaled,
         scaled=scaled, rotate_v=True)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 8])
@pytest.mark.parametrize("scaled,rotate_v", [(False, False), (True, False), (False, True), (True, True)])
def test_fused_append_srft(D, G, scaled, rotate_v):
    """K rotated by the sign-randomised FFT: the combine rotates the new
    token's K (to the bulk kernel's bytes) and the query for its score; with
    V rotated by the same kind it also rotates the new V and brings the output
    row back by the inverse transform."""
    _run(2, G, 2, D, 384, [351, 190], rotate="srft", chunk=128, seed=13 * D + G + scaled + 2 * rotate_v,
         scaled=scaled, rotate_v=rotate_v)


@pytest.mark.parametrize("lens", [[1, 2], [129, 128], [257, 33], [32, 31]])
def test_fused_append_edges(lens):
    """lens = 1 (no cached token at all), a new token opening a chunk (129
    with chunk 128: that split has no cached token), chunk and tile ends."""
    _run(2, 8, 2, 128, 384, lens, chunk=128, seed=sum(lens))


def test_fused_append_consecutive_steps():
    """Three decode steps in a row, default plan, fp16 and rotated."""
    _run(3, 4, 2, 128, 512, [300, 77, 2], dtype=torch.float16, rotate=True, steps=3, seed=9)


@pytest.mark.parametrize("lens", [[1000], [641], [129], [1]])
def test_fused_append_interleaved_pieces(lens):
    """The fused step with fewer splits than pieces (3 splits of 128-token
    pieces): the split pass covers [0, lens - 1) over interleaved pieces,
    the combine appends the token at lens - 1."""
    _run(1, 8, 2, 128, 1024, lens, chunk=128, splits=3, seed=lens[0], rotate=True)


@pytest.mark.parametrize("G,D", [(1, 128), (2, 64)])
@pytest.mark.parametrize("scaled", [False, True])
def test_fused_append_vector_variant(G, D, scaled):
    """The same call on the vector split variant."""
    _run(2, G, 2, D, 320, [300, 77], chunk=128, seed=G + D + scaled, variant=otq.OTQ_VARIANT_VECTOR,
         scaled=scaled)


@pytest.mark.parametrize("G", [1, 4, 8, 16])
@pytest.mark.parametrize("rotate,scaled", [(False, False), ("srft", False), ("srft", True), (False, True)])
def test_fused_append_head_dim_192(G, rotate, scaled):
    """head_dim 192: the combine quantises the step's token (the mixed-radix
    FFT in every channel slice when K is rotated), writes it and merges it;
    two steps in a row, one sequence that has no token yet."""
    _run(3, G, 2, 192, 384, [351, 190, 0], rotate=rotate, chunk=128, seed=17 * G + scaled + 2 * bool(rotate),
         scaled=scaled, steps=2)


@pytest.mark.parametrize("lens", [[1, 2], [129, 32]])
def test_fused_append_head_dim_192_vector_variant(lens):
    _run(2, 8, 2, 192, 320, lens, rotate="srft", chunk=128, seed=sum(lens), variant=otq.OTQ_VARIANT_VECTOR)


# -------------------------------------------------------------- full workloads

def _full_fused(cfg):
    """One decode step of layer 0 of a full workload, in the launch
    configuration the benchmark times (the planner's default plan): every
    sequence prefilled, the slot of its new token poisoned, then the fused
    call.  The whole cache must equal the oracle's quantisation bit for bit
    and every output row must match the fp64 oracle."""
    w = synth.WORKLOADS[cfg]
    say(f"fused full workload {cfg} {w.name}")
    k = synth.kv(w, 0, "k", device=DEV)
    v = synth.kv(w, 0, "v", device=DEV)
    q = synth.query(w, 0, device=DEV)
    lens = synth.lens(w, 0)
    signs = torch.from_numpy(synth.rot_signs(w, 0)).to(DEV) if w.rotate else None
    cache = otq.Int4KVCache(w.B, w.Hkv, w.D, w.capacity, device=DEV, rot_signs=signs)
    for t0 in range(0, w.T, 16384):
        t1 = min(w.T, t0 + 16384)
        pos = torch.full((w.B,), t0, dtype=torch.int32, device=DEV)
        cache.append(k[:, :, t0:t1].contiguous(), v[:, :, t0:t1].contiguous(), pos)
    _poison(cache, [int(n) for n in lens])
    lens_t = torch.from_numpy(lens).to(DEV)
    idx = (lens_t.long() - 1).clamp(min=0)
    ar = torch.arange(w.B, device=DEV)
    kn = k[ar, :, idx].contiguous()
    vn = v[ar, :, idx].contiguous()
    max_len = int(lens.max())
    plan = cache.plan(w.Hq, max_len)
    say(f"  plan chunk={plan.chunk} splits={plan.num_splits} variant={plan.variant}")
    torch.cuda.synchronize()
    otq.otq_last_device_error()  # start from a clear word (earlier tests may leave flags)
    out = cache.decode_append(q, kn, vn, lens_t, max_len, w.scale, plan=plan)
    torch.cuda.synchronize()
    assert otq.otq_last_device_error() == 0
    ref_cache = oracle_cache(k.cpu(), v.cpu(), w.dtype, None if signs is None else signs.cpu().numpy(),
                             rot_norm32(w.D, "srht"), threads=16)
    assert compare_codes(host_cache(cache), ref_cache, w.T) == {
        "k_codes": 0, "k_scales": 0, "v_codes": 0, "v_scales": 0}
    kc, ks, vc, vs = ref_cache
    ref = oracle.sdpa(to_bits(q), w.dtype, kc, ks, vc, vs, lens, w.scale,
                      signs=None if signs is None else signs.cpu().numpy(), rot_norm=rot_norm32(w.D, "srht"),
                      threads=16)
    ma, rel = errors(out.cpu().numpy(), ref)
    say(f"  rows={w.B * w.Hq} max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert ma <= MAX_ABS and rel <= REL_L2


def test_fused_full_workload_3_llama70b_128k():
    _full_fused(3)


def test_fused_full_workload_5_ragged_rotated():
    _full_fused(5)
