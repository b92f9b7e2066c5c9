"""GPU parity of otq_sdpa_int4_decode against the fp64 CPU oracle.

Tolerance (fp32 outputs vs the fp64 oracle): max-abs <= 2e-3 and relative
L2 <= 1e-3 per checked set of rows.  The oracle reads a cache it quantised
itself from the same 16-bit inputs (after the quantiser's bit-exactness is
checked), so no oracle input comes from the GPU path."""
import math

import numpy as np
import pytest
import torch

import int4_kv_cache_quant_amd as otq
import oracle
from int4_kv_cache_quant_amd import synth

from gpu_common import (MAX_ABS, REL_L2, build_cache, chan_scales, compare_codes, errors, host_cache,
                        oracle_cache, rand_signs, rot_norm32, say, to_bits)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(B, Hq, Hkv, D, cap, dtype, seed, sigma=1.0, rotate=False, n_out=2, spikes=(), beta=0.0,
          scaled=False):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((2, B, Hkv, cap, D), generator=g) * sigma
    oc = torch.randperm(D, generator=g)[:n_out]
    x[..., oc] *= 10
    lam = chan_scales(D, seed, outliers=[int(c) for c in oc]) if scaled else None
    q = torch.randn((B, Hq, D), generator=g)
    # score spikes: K of the given tokens = beta * unit vector of the first
    # query head of the group, so that head's score there exceeds every other
    # score by ~beta |q| scale log2(e) in the base-2 exponent
    G = Hq // Hkv
    for t in spikes:
        for j in range(Hkv):
            u = q[:, j * G] / q[:, j * G].norm(dim=-1, keepdim=True)
            x[0, :, j, t] = beta * u
    x = x.to(dtype)
    q = q.to(dtype)
    signs = None
    if rotate:
        signs = torch.where(torch.rand(D, generator=g) < 0.5, -1.0, 1.0)
    return x[0], x[1], q, signs, lam


def _run(B, Hq, Hkv, D, cap, lens, dtype=torch.bfloat16, scale=None, seed=0, sigma=1.0,
         rotate=False, chunk=0, variant=otq.OTQ_VARIANT_AUTO, rows=None, spikes=(), beta=0.0,
         scaled=False, rotate_v=False, splits=0):
    """rotate: False, True (the Hadamard rotation) or "srft" (the FFT one)."""
    kind = "srft" if rotate == "srft" else "srht"
    k, v, q, signs, lam = _case(B, Hq, Hkv, D, cap, dtype, seed, sigma, bool(rotate), spikes=spikes,
                                beta=beta, scaled=scaled)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    name = "fp16" if dtype == torch.float16 else "bf16"
    lam_np = None if lam is None else lam.numpy()
    vsg = rand_signs(D, seed + 1000) if rotate_v else None
    vsg_np = None if vsg is None else vsg.numpy()
    cache = build_cache(k.to(DEV), v.to(DEV), cap, signs=None if signs is None else signs.to(DEV),
                        prefill_chunk=max(1, cap // 3), chan_scale=None if lam is None else lam.to(DEV),
                        v_signs=None if vsg is None else vsg.to(DEV), rot_kind=kind)
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    max_len = max(1, int(max(lens)))
    plan = cache.plan(Hq, max_len, chunk=chunk, variant=variant, splits=splits)
    say(f"sdpa B={B} Hq={Hq} Hkv={Hkv} D={D} cap={cap} chunk={plan.chunk} "
        f"splits={plan.num_splits} variant={plan.variant} rotate={rotate} scaled={scaled} "
        f"rotate_v={rotate_v}")
    out = cache.decode(q.to(DEV), lens_t, max_len, scale, plan=plan)
    torch.cuda.synchronize()
    ref_cache = oracle_cache(k, v, name, None if signs is None else signs.numpy(), rot_norm32(D, kind),
                             chan_scale=lam_np, v_signs=vsg_np, rot_kind=kind)
    assert compare_codes(host_cache(cache), ref_cache, cap) == {
        "k_codes": 0, "k_scales": 0, "v_codes": 0, "v_scales": 0}
    kc, ks, vc, vs = ref_cache
    ref = oracle.sdpa(to_bits(q), name, kc, ks, vc, vs, np.array(lens, np.int32), scale,
                      signs=None if signs is None else signs.numpy(), rot_norm=rot_norm32(D, kind),
                      rows=rows, threads=8, chan_scale=lam_np, v_signs=vsg_np, rot_kind=kind)
    got = out.cpu().numpy().astype(np.float64)
    if rows is not None:
        got = got.reshape(-1, D)[rows]
    return got, ref, plan


VEC, MF = otq.OTQ_VARIANT_VECTOR, otq.OTQ_VARIANT_MFMA


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 2, 4])
def test_sdpa_small_parity_vector(D, G):
    if D == 256 and G == 4:
        pytest.skip("vector variant does not build G=4 at D=256 (register file)")
    Hkv = 2
    got, ref, _ = _run(2, G * Hkv, Hkv, D, 320, [300, 77], seed=D + G, variant=VEC, chunk=128)
    ma, rel = errors(got, ref)
    say(f"  max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("rotate", [False, True])
def test_sdpa_small_parity_mfma(D, G, rotate):
    Hkv = 2
    got, ref, _ = _run(2, G * Hkv, Hkv, D, 352, [350, 45], seed=3 * D + G + rotate, variant=MF,
                       chunk=128, rotate=rotate)
    ma, rel = errors(got, ref)
    say(f"  max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("variant,G,D", [(VEC, 1, 128), (VEC, 2, 64), (VEC, 4, 128), (MF, 1, 64),
                                         (MF, 4, 128), (MF, 8, 128), (MF, 16, 64), (MF, 2, 256)])
@pytest.mark.parametrize("rotate", [False, True])
def test_sdpa_chan_scale(variant, G, D, rotate):
    """K with a per-channel scale (1/10 on its outlier channels): multi-tile
    ragged lengths, both variants, one and two heads per MFMA wave."""
    got, ref, _ = _run(2, 2 * G, 2, D, 192, [192, 77], seed=31 + G + D + rotate, rotate=rotate,
                       chunk=128, variant=variant, scaled=True)
    ma, rel = errors(got, ref)
    say(f"  max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("variant,G,D", [(VEC, 1, 128), (VEC, 4, 64), (MF, 1, 256), (MF, 8, 128),
                                         (MF, 16, 64), (MF, 2, 256)])
@pytest.mark.parametrize("rotate,scaled", [(False, False), (True, False), (True, True)])
def test_sdpa_v_rotated(variant, G, D, rotate, scaled):
    """V quantised in a rotated basis: the output is brought back by the
    inverse rotation; alone, with K rotated, and with K rotated and scaled."""
    got, ref, _ = _run(2, 2 * G, 2, D, 192, [192, 70], seed=51 + G + D + rotate + scaled, rotate=rotate,
                       chunk=128, variant=variant, scaled=scaled, rotate_v=True)
    ma, rel = errors(got, ref)
    say(f"  max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("variant,G,D", [(VEC, 1, 64), (VEC, 2, 256), (VEC, 4, 128), (MF, 1, 256),
                                         (MF, 2, 256), (MF, 4, 64), (MF, 8, 128), (MF, 16, 128),
                                         (MF, 8, 64)])
@pytest.mark.parametrize("scaled,rotate_v", [(False, False), (True, False), (False, True), (True, True)])
def test_sdpa_srft(variant, G, D, scaled, rotate_v):
    """K rotated by the sign-randomised FFT: the split kernels rotate the
    query the same way (then divide it by K's channel scale if scaled); one
    and two KV heads per MFMA wave, every head width; V rotated by the same
    kind or not (its output brought back by the inverse transform)."""
    got, ref, _ = _run(2, 2 * G, 2, D, 192, [192, 77], seed=71 + G + D + scaled + 2 * rotate_v,
                       rotate="srft", chunk=128, variant=variant, scaled=scaled, rotate_v=rotate_v)
    ma, rel = errors(got, ref)
    say(f"  max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("variant,G,D", [(VEC, 1, 128), (VEC, 2, 64), (MF, 4, 128), (MF, 8, 128),
                                         (MF, 16, 64), (MF, 8, 256)])
@pytest.mark.parametrize("rotate", [False, True])
def test_sdpa_score_spikes(variant, G, D, rotate):
    """A few tokens whose score exceeds the rest by ~140 in the base-2
    exponent, placed in every row position of the score tiles (tokens 4 r + i
    of both 16-token halves): the running maximum must be the column's true
    maximum, or exp2 of the difference overflows fp32."""
    Hkv = 2
    spikes = [6, 37, 90, 255, 301]
    got, ref, _ = _run(2, G * Hkv, Hkv, D, 320, [320, 260], seed=11 * G + D + rotate, variant=variant,
                       chunk=128, rotate=rotate, spikes=spikes, beta=100.0)
    ma, rel = errors(got, ref)
    say(f"  max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert np.all(np.isfinite(got))
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("variant,Hq", [(VEC, 4), (MF, 16)])
@pytest.mark.parametrize("lens", [[0, 5], [1, 1], [31, 32], [33, 160], [160, 0]])
def test_sdpa_edge_lengths(lens, variant, Hq):
    got, ref, _ = _run(2, Hq, 2, 128, 160, lens, seed=sum(lens), variant=variant, chunk=128)
    ma, rel = errors(got, ref)
    assert ma <= MAX_ABS and rel <= REL_L2
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(got[b] == 0.0)


@pytest.mark.parametrize("variant,Hq", [(VEC, 2), (MF, 8)])
@pytest.mark.parametrize("chunk", [128, 256, 384, 1024])
def test_sdpa_split_invariance(chunk, variant, Hq):
    got, ref, plan = _run(1, Hq, 1, 128, 1024, [1000], seed=11, chunk=chunk, variant=variant)
    ma, rel = errors(got, ref)
    assert plan.num_splits == -(-1000 // chunk)
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("D,Hq", [(64, 8), (128, 16), (128, 2), (256, 4)])
@pytest.mark.parametrize("chunk,splits,lens", [(128, 3, 1000), (256, 2, 1000), (128, 5, 641),
                                               (128, 7, 896), (128, 4, 33), (128, 8, 1)])
def test_sdpa_interleaved_pieces(D, Hq, chunk, splits, lens):
    """Fewer splits than pieces: split s takes pieces s, s + S, ...; the last
    round of pieces is partial (641, 1000), exactly full (896 = 7 x 128), or
    covers fewer splits than S (33, 1), and the sequence's last tile is
    partial."""
    got, ref, plan = _run(1, Hq, 2, D, 1024, [lens], seed=D + chunk + splits + lens, chunk=chunk,
                          variant=MF, splits=splits)
    assert (plan.chunk, plan.num_splits) == (chunk, min(splits, -(-lens // chunk)))
    ma, rel = errors(got, ref)
    say(f"  max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert ma <= MAX_ABS and rel <= REL_L2


def test_sdpa_interleaved_plan_reused_at_longer_length():
    """A plan made for a short max_len, passed to a call with a longer one:
    the call keeps its split count and interleaves the pieces."""
    k, v, q, _, _ = _case(1, 8, 2, 128, 1024, torch.bfloat16, 5)
    cache = build_cache(k.to(DEV), v.to(DEV), 1024)
    plan = cache.plan(8, 300, chunk=128)  # 3 splits
    assert plan.num_splits == 3
    ws = cache.workspace(8, 300, plan)
    out = cache.decode(q.to(DEV), torch.tensor([1000], dtype=torch.int32, device=DEV), 1000, 0.1,
                       workspace=ws, plan=plan)
    torch.cuda.synchronize()
    kc, ks, vc, vs = oracle_cache(k, v, "bf16")
    ref = oracle.sdpa(to_bits(q), "bf16", kc, ks, vc, vs, np.array([1000], np.int32), 0.1, threads=8)
    ma, rel = errors(out.cpu().numpy(), ref)
    say(f"  max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("variant,Hq,rotate", [(VEC, 4, False), (MF, 8, False), (MF, 8, True)])
def test_sdpa_ragged_batch_order(variant, Hq, rotate):
    """A batch takes its split items longest first (an order kernel writes
    the block -> item table): empty sequences, one token, exact chunk
    multiples and partial chunks of every size, in a mixed order."""
    lens = [0, 1, 128, 129, 383, 256, 32, 300, 127, 384, 255, 2]
    got, ref, plan = _run(len(lens), Hq, 2, 128, 384, lens, chunk=128, variant=variant, seed=21,
                          rotate=rotate)
    assert plan.num_splits == 3
    ma, rel = errors(got, ref)
    say(f"  max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert ma <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("B", [64, 257])
def test_sdpa_ragged_batch_sizes(B):
    """A larger batch in longest-first order (64) and one past the order
    kernel's limit of 256 (257: blocks keep the grid order)."""
    rng = np.random.default_rng(B)
    lens = [int(x) for x in rng.integers(0, 161, size=B)]
    rows = np.arange(0, B * 4, 7, dtype=np.int32)
    got, ref, plan = _run(B, 4, 1, 64, 160, lens, chunk=128, variant=MF, seed=B, rows=rows)
    ma, rel = errors(got, ref)
    say(f"  B={B} max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert ma <= MAX_ABS and rel <= REL_L2


def test_sdpa_fp16_rotated_and_scale_one():
    got, ref, _ = _run(3, 4, 2, 128, 256, [256, 200, 9], dtype=torch.float16, seed=3, rotate=True)
    ma, rel = errors(got, ref)
    assert ma <= MAX_ABS and rel <= REL_L2
    got, ref, _ = _run(1, 4, 2, 256, 512, [500], seed=4, scale=1.0, sigma=0.5)
    ma, rel = errors(got, ref)
    say(f"  scale=1 max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert ma <= MAX_ABS and rel <= REL_L2


def test_sdpa_deterministic():
    k, v, q, _, _ = _case(1, 2, 1, 128, 512, torch.bfloat16, 9)
    cache = build_cache(k.to(DEV), v.to(DEV), 512)
    lens = torch.tensor([512], dtype=torch.int32, device=DEV)
    a = cache.decode(q.to(DEV), lens, 512, 0.1)
    b = cache.decode(q.to(DEV), lens, 512, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    q8 = torch.randn((1, 8, 128), generator=torch.Generator().manual_seed(2)).to(torch.bfloat16).to(DEV)
    a = cache.decode(q8, lens, 512, 0.1)
    b = cache.decode(q8, lens, 512, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# -------------------------------------------------------------- full workloads

def _full(cfg, rows_per_seq=None, layer=0, options=False, srft=False):
    """options: K's per-channel scale and a rotated V (seeded, as bench.py
    --chan-scale --v-rotate makes them) on top of the workload's own; srft:
    K rotated by the sign-randomised FFT (with K's channel scale when options
    is set too; as bench.py --srft makes it)."""
    w = synth.WORKLOADS[cfg]
    kind = "srft" if srft else "srht"
    say(f"sdpa full workload {cfg} {w.name} options={options} srft={srft}")
    k = synth.kv(w, layer, "k", device=DEV)
    v = synth.kv(w, layer, "v", device=DEV)
    q = synth.query(w, layer, device=DEV)
    lens = synth.lens(w, layer)
    signs = torch.from_numpy(synth.rot_signs(w, layer)).to(DEV) if (w.rotate or srft) else None
    lam = synth.chan_scale(w, layer) if options else None
    vsg = synth.v_rot_signs(w, layer) if options else None
    cache = otq.Int4KVCache(w.B, w.Hkv, w.D, w.capacity, device=DEV, rot_signs=signs,
                            chan_scale=None if lam is None else torch.from_numpy(lam),
                            v_rot_signs=None if vsg is None else torch.from_numpy(vsg), rot_kind=kind)
    # prefill lens-1 tokens per sequence, then append token lens-1 (ragged-aware)
    for t0 in range(0, w.T, 8192):
        t1 = min(w.T, t0 + 8192)
        pos = torch.full((w.B,), t0, dtype=torch.int32, device=DEV)
        cache.append(k[:, :, t0:t1].contiguous(), v[:, :, t0:t1].contiguous(), pos)
    lens_t = torch.from_numpy(lens).to(DEV)
    idx = (lens_t.long() - 1).clamp(min=0)
    kn = k[torch.arange(w.B, device=DEV), :, idx][:, :, None].contiguous()
    vn = v[torch.arange(w.B, device=DEV), :, idx][:, :, None].contiguous()
    cache.append(kn, vn, (lens_t - 1).clamp(min=0))
    out = cache.decode(q, lens_t, int(lens.max()), w.scale)
    torch.cuda.synchronize()
    ref_cache = oracle_cache(k.cpu(), v.cpu(), w.dtype,
                             None if signs is None else signs.cpu().numpy(), rot_norm32(w.D, kind),
                             threads=16, chan_scale=lam, v_signs=vsg, rot_kind=kind)
    assert compare_codes(host_cache(cache), ref_cache, w.T) == {
        "k_codes": 0, "k_scales": 0, "v_codes": 0, "v_scales": 0}
    rng = np.random.default_rng(cfg)
    if rows_per_seq is None:
        rows = np.arange(w.B * w.Hq, dtype=np.int32)
    else:
        rows = np.sort(np.concatenate([b * w.Hq + rng.choice(w.Hq, rows_per_seq, replace=False)
                                       for b in range(w.B)])).astype(np.int32)
    kc, ks, vc, vs = ref_cache
    ref = oracle.sdpa(to_bits(q), w.dtype, kc, ks, vc, vs, lens, w.scale,
                      signs=None if signs is None else signs.cpu().numpy(),
                      rot_norm=rot_norm32(w.D, kind), rows=rows, threads=16, chan_scale=lam, v_signs=vsg,
                      rot_kind=kind)
    got = out.cpu().numpy().reshape(-1, w.D)[rows].astype(np.float64)
    ma, rel = errors(got, ref)
    say(f"  rows={len(rows)} max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert ma <= MAX_ABS and rel <= REL_L2


def test_full_workload_2_llama70b_32k():
    _full(2)


def test_full_workload_3_llama70b_128k():
    _full(3)


def test_full_workload_1_tiny():
    _full(1)


def test_full_workload_4_gemma_scale1():
    _full(4)


def test_full_workload_5_ragged_rotated():
    _full(5)


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_full_workload_with_options(cfg):
    """The full workloads with K's per-channel scale and a rotated V."""
    _full(cfg, options=True)


@pytest.mark.parametrize("cfg,options", [(3, False), (4, True), (5, False)])
def test_full_workload_srft(cfg, options):
    """The full workloads with K rotated by the sign-randomised FFT (workload
    5 switches from the Hadamard rotation to it); workload 4 with K's channel
    scale and V rotated by the same kind."""
    _full(cfg, options=options, srft=True)
