"""Helpers shared by the GPU parity tests (test side only)."""
import math
import sys

import numpy as np
import torch

import int4_kv_cache_quant_amd as otq
import oracle
from int4_kv_cache_quant_amd import layout, synth

# Output tolerance against the fp64 oracle: max-abs and relative L2.
MAX_ABS = 2e-3
REL_L2 = 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_bits(t):
    return synth.bits(t)


def build_cache(k, v, capacity, signs=None, prefill_chunk=None, append_last=True, chan_scale=None,
                v_signs=None, rot_kind="srht"):
    """Quantise K/V [B, H, T, D] (device) into a new cache: prefill T-1 tokens
    (optionally in chunks), then append the last token on its own."""
    B, H, T, D = k.shape
    cache = otq.Int4KVCache(B, H, D, capacity, device=k.device, rot_signs=signs,
                            chan_scale=chan_scale, v_rot_signs=v_signs, rot_kind=rot_kind)
    n_pre = T - 1 if append_last else T
    step = n_pre if prefill_chunk is None else prefill_chunk
    for t0 in range(0, n_pre, max(step, 1)):
        t1 = min(n_pre, t0 + step)
        pos = torch.full((B,), t0, dtype=torch.int32, device=k.device)
        cache.append(k[:, :, t0:t1].contiguous(), v[:, :, t0:t1].contiguous(), pos)
    if append_last:
        pos = torch.full((B,), T - 1, dtype=torch.int32, device=k.device)
        cache.append(k[:, :, T - 1:T].contiguous(), v[:, :, T - 1:T].contiguous(), pos)
    return cache


def host_cache(cache):
    """(k_codes, k_scales, v_codes_plain, v_scales) as numpy arrays."""
    D = cache.shape[2]
    return (layout.k_rows_to_plain(cache.k_codes.cpu().numpy(), D), cache.k_scales.cpu().numpy(),
            layout.v_tiled_to_plain(cache.v_codes.cpu().numpy(), D), cache.v_scales.cpu().numpy())


def oracle_cache(k, v, dtype, signs=None, rot_norm=0.0, threads=8, chan_scale=None, v_signs=None,
                 rot_kind="srht"):
    kb, vb = to_bits(k), to_bits(v)
    kc, ks = oracle.quantize(kb, dtype, signs=signs, rot_norm=rot_norm, threads=threads,
                             chan_scale=chan_scale, rot_kind=rot_kind)
    vc, vs = oracle.quantize(vb, dtype, signs=v_signs, rot_norm=rot_norm, threads=threads, rot_kind=rot_kind)
    return kc, ks, vc, vs


def compare_codes(gpu, ref, T):
    """Bit-exact comparison over the first T tokens; returns mismatch counts."""
    names = ("k_codes", "k_scales", "v_codes", "v_scales")
    bad = {}
    for n, g, r in zip(names, gpu, ref):
        g = g[:, :, :T]
        r = r[:, :, :T]
        if g.dtype == np.float32:
            g, r = g.view(np.uint32), r.view(np.uint32)
        bad[n] = int(np.count_nonzero(g != r))
    return bad


def errors(out, ref):
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    max_abs = float(np.max(np.abs(out - ref))) if out.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(out - ref) / den) if den > 0 else float(np.linalg.norm(out - ref))
    return max_abs, rel


def rot_norm32(D, rot_kind="srht"):
    """fp32(1/sqrt(n)): n = D for the Hadamard rotation, D/2 (complex
    numbers) for the FFT one."""
    n = D // 2 if rot_kind == "srft" else D
    return float(np.float32(1.0 / math.sqrt(n)))


def rand_signs(D, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.where(torch.rand(D, generator=g) < 0.5, -1.0, 1.0).to(torch.float32)


def chan_scales(D, seed, outliers=()):
    """A per-channel scale for K: log-uniform in [1/4, 4], and 1/10 on the
    given outlier channels (whose values the tests multiply by 10)."""
    g = torch.Generator().manual_seed(seed)
    lam = torch.exp2(torch.rand(D, generator=g) * 4.0 - 2.0)
    for c in outliers:
        lam[c] = 0.1
    return lam.to(torch.float32)
