"""Seeded synthetic inputs for the five decode workloads.

This module only draws random numbers and shapes them; it holds none of the
quantisation or attention arithmetic, so both the GPU path and the CPU
reference can be fed from it.

The workloads stand in for the models the Open-TQ-Metal abstract measures
(Llama 3.1 70B at 128K context; Gemma-family layers with attention scale 1.0):
only the attention shapes matter for the kernels, so K/V/q are Gaussian with a
few amplified "outlier" channels, as described per workload below.

Recipe (all workloads):
  * K, V ~ N(0, sigma) drawn in fp32 from a seeded generator, outlier channels
    multiplied, then rounded to the workload's dtype (round-to-nearest-even).
  * The outlier channel set is the first n_out entries of a seeded permutation
    of 0..D-1, shared by K and V, all heads and all tokens.
  * q ~ N(0, 1) in the same dtype; rotation signs are a seeded +-1 vector.
  * seed = 20260000 + 1000 * workload + 10 * layer + slot, slot in
    {K: 0, V: 1, q: 2, lens: 3, signs: 4, outliers: 5, channel scales: 6,
    V signs: 7}.
  * K's per-channel scale, where a run asks for one: log-uniform in [1/4, 4]
    per channel, and 1 / the outlier multiplier on the outlier channels.
  * "T cached tokens" is the attended length: the cache is prefilled with T-1
    tokens, one token is appended at position T-1, and attention runs with
    lens = T.
"""
import math
from dataclasses import dataclass, field

import numpy as np
import torch

SLOT = {"k": 0, "v": 1, "q": 2, "lens": 3, "signs": 4, "outliers": 5, "chan_scale": 6, "v_signs": 7}


@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    T: int               # attended tokens (max over the batch when ragged)
    dtype: str           # "fp16" | "bf16"
    sigma: float
    n_out: int
    out_mult: float
    scale: float
    rotate: bool
    layers: int          # distinct caches the bench cycles through
    ragged: bool = False
    lens_lo: int = 0
    notes: str = field(default="", compare=False)

    @property
    def G(self):
        return self.Hq // self.Hkv

    @property
    def capacity(self):
        # every workload's T is already a multiple of 32
        return self.T


WORKLOADS = {
    1: Workload(1, "tiny-4h-d128-4k-fp16", 1, 4, 4, 128, 4096, "fp16", 1.0, 4, 8.0,
                1.0 / math.sqrt(128), False, 80),
    2: Workload(2, "llama70b-layer-32k-bf16", 1, 64, 8, 128, 32768, "bf16", 1.0, 1, 10.0,
                1.0 / math.sqrt(128), False, 80),
    3: Workload(3, "llama70b-layer-128k-bf16", 1, 64, 8, 128, 131072, "bf16", 1.0, 1, 10.0,
                1.0 / math.sqrt(128), False, 80),
    4: Workload(4, "gemma-layer-d256-64k-scale1", 1, 32, 16, 256, 65536, "bf16", 0.5, 3, 10.0,
                1.0, False, 16),
    5: Workload(5, "ragged-32seq-1k-32k-rotated", 32, 32, 8, 128, 32768, "bf16", 1.0, 1, 10.0,
                1.0 / math.sqrt(128), True, 16, ragged=True, lens_lo=1024),
}


def seed(cfg: int, layer: int, slot: str) -> int:
    return 20260000 + 1000 * cfg + 10 * layer + SLOT[slot]


def torch_dtype(name: str):
    return {"fp16": torch.float16, "bf16": torch.bfloat16}[name]


def outlier_channels(w: Workload, layer: int) -> np.ndarray:
    rng = np.random.default_rng(seed(w.cfg, layer, "outliers"))
    return np.sort(rng.permutation(w.D)[: w.n_out])


def chan_scale(w: Workload, layer: int) -> np.ndarray:
    """A per-channel scale for K [D] float32 (an input: seeded, not fitted)."""
    rng = np.random.default_rng(seed(w.cfg, layer, "chan_scale"))
    lam = np.exp2(rng.uniform(-2.0, 2.0, w.D))
    lam[outlier_channels(w, layer)] = 1.0 / w.out_mult
    return lam.astype(np.float32)


def rot_signs(w: Workload, layer: int) -> np.ndarray:
    rng = np.random.default_rng(seed(w.cfg, layer, "signs"))
    return np.where(rng.integers(0, 2, w.D) == 1, 1.0, -1.0).astype(np.float32)


def v_rot_signs(w: Workload, layer: int) -> np.ndarray:
    """Signs for V's rotation, where a run asks for one."""
    rng = np.random.default_rng(seed(w.cfg, layer, "v_signs"))
    return np.where(rng.integers(0, 2, w.D) == 1, 1.0, -1.0).astype(np.float32)


def lens(w: Workload, layer: int) -> np.ndarray:
    if not w.ragged:
        return np.full(w.B, w.T, np.int32)
    rng = np.random.default_rng(seed(w.cfg, layer, "lens"))
    return rng.integers(w.lens_lo, w.T + 1, w.B).astype(np.int32)


def _gen(device, s):
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def kv(w: Workload, layer: int, which: str, T: int = None, device="cpu",
       sigma: float = None, chunk_tokens: int = 8192) -> torch.Tensor:
    """K or V for all heads: [B, Hkv, T, D] in the workload dtype.

    Drawn chunk by chunk along tokens from one generator so that big caches
    never need a full fp32 copy; the values depend only on (seed, T, device).
    """
    T = w.T if T is None else T
    sigma = w.sigma if sigma is None else sigma
    dt = torch_dtype(w.dtype)
    out = torch.empty((w.B, w.Hkv, T, w.D), dtype=dt, device=device)
    g = _gen(device, seed(w.cfg, layer, which))
    mult = torch.ones(w.D, dtype=torch.float32, device=device)
    oc = outlier_channels(w, layer)
    if len(oc):
        mult[torch.as_tensor(oc, device=device)] = w.out_mult
    mult *= sigma
    for t0 in range(0, T, chunk_tokens):
        t1 = min(T, t0 + chunk_tokens)
        x = torch.randn((w.B, w.Hkv, t1 - t0, w.D), generator=g, dtype=torch.float32,
                        device=device)
        out[:, :, t0:t1, :] = (x * mult).to(dt)
    return out


def query(w: Workload, layer: int, device="cpu") -> torch.Tensor:
    g = _gen(device, seed(w.cfg, layer, "q"))
    x = torch.randn((w.B, w.Hq, w.D), generator=g, dtype=torch.float32, device=device)
    return x.to(torch_dtype(w.dtype))


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 bit patterns of an fp16/bf16 tensor (host copy)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def small(w: Workload, **kw) -> Workload:
    """A shrunken copy of a workload for oracle-speed tests."""
    d = {f: getattr(w, f) for f in w.__dataclass_fields__}
    d.update(kw)
    return Workload(**d)
