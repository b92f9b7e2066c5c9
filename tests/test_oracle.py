"""Pins for the CPU oracle: each check ties it to something other than itself
(a library routine, a closed form, an invariant, or brute force), chosen so
that a dropped term, a wrong sign or index, or a swapped operand fails."""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _codes(packed, D):
    """Unpack nibble bytes to signed ints (test-side, plain numpy)."""
    p = np.asarray(packed, np.uint8)
    lo = (p & 0xF).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    c = np.stack([lo, hi], -1).reshape(p.shape[:-1] + (p.shape[-1] * 2,))
    return np.where(c >= 8, c - 16, c)


# ------------------------------------------------------------------ widening

def test_f16_widening_matches_numpy_for_every_pattern():
    lib = oracle._load()
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float32)
    got = np.array([lib.oracle_f16_to_f32(int(p)) for p in pats], np.float32)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def test_bf16_widening_matches_torch_for_every_pattern():
    lib = oracle._load()
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = np.array([lib.oracle_bf16_to_f32(int(p)) for p in pats], np.float32)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))


# ------------------------------------------------------------------ quantiser

def test_golden_special_case():
    g = json.load(open(os.path.join(GOLDEN, "quant_special_case.json")))
    codes, scales = oracle.quantize_vector(np.array(g["x"], np.float32))
    assert scales.tolist() == [g["scale"]]
    assert codes.tolist() == g["bytes"]
    assert _codes(codes, 32).tolist() == g["codes"]


def test_unit_scale_group_is_numpy_rint():
    # abs-max 7 -> scale exactly 1 -> codes are round-half-even of x itself.
    rng = np.random.default_rng(1)
    for _ in range(200):
        x = (rng.integers(-14, 15, 32) / 2.0).astype(np.float32)  # many .5 ties
        x[rng.integers(32)] = 7.0 * rng.choice([-1, 1])
        codes, s = oracle.quantize_vector(x)
        assert s[0] == 1.0
        assert np.array_equal(_codes(codes, 32), np.rint(x).astype(int))


def test_power_of_two_scale_is_exact_rint():
    rng = np.random.default_rng(2)
    for k in range(-20, 20, 3):
        x = (rng.standard_normal(64) * 2.0 ** k).astype(np.float32)
        for g in range(2):
            x[32 * g + rng.integers(32)] = np.float32(7.0 * 2.0 ** k) * rng.choice([-1, 1])
            x[32 * g:32 * g + 32] = np.clip(x[32 * g:32 * g + 32], -7.0 * 2.0 ** k, 7.0 * 2.0 ** k)
        codes, s = oracle.quantize_vector(x)
        assert np.all(s == np.float32(2.0 ** k))
        assert np.array_equal(_codes(codes, 64), np.rint(x / np.float32(2.0 ** k)).astype(int))


def _brute_code(q):
    """Nearest code in [-8, 7] to the real number q, ties to the even code."""
    best = None
    for c in range(-8, 8):
        d = abs(q - c)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def test_codes_brute_force_tiny():
    rng = np.random.default_rng(3)
    for dt in (np.float16, np.float32):
        for _ in range(60):
            x = rng.standard_normal(32).astype(dt).astype(np.float32)
            codes, s = oracle.quantize_vector(x)
            c = _codes(codes, 32)
            # the fp32 quotient x/s is one IEEE division: numpy computes the same
            q = (x / s[0]).astype(np.float64)
            assert [_brute_code(v) for v in q] == c.tolist()


def test_scale_is_nearest_fp32_to_absmax_over_7():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((500, 32)) * np.exp(rng.uniform(-30, 30, (500, 1)))).astype(np.float32)
    for row in x:
        _, s = oracle.quantize_vector(row)
        a = float(np.max(np.abs(row)))
        exact = a / 7.0
        s = float(s[0])
        ulp = float(np.spacing(np.float32(s)))
        assert abs(s - exact) <= ulp / 2 * (1 + 1e-12)


def _gauss_rows(n, D, dtype, outliers=()):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((n, D)).astype(np.float32)
    for c in outliers:
        x[:, c] *= 10
    t = torch.from_numpy(x).to(torch.float16 if dtype == "fp16" else torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16), t.float().numpy()


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_quantiser_invariants(dtype, D):
    bits, x = _gauss_rows(400, D, dtype, outliers=(3,))
    codes, scales = oracle.quantize(bits, dtype)
    c = _codes(codes, D).reshape(400, D // 32, 32)
    s = scales.astype(np.float64)[..., None]
    xg = x.reshape(400, D // 32, 32).astype(np.float64)
    assert np.all(np.abs(c) <= 7)
    nz = scales > 0
    assert np.all(np.abs(c).max(-1)[nz] == 7)
    assert np.all((np.sign(c) == np.sign(xg)) | (c == 0))
    err = np.abs(xg - c * s)
    assert np.all(err <= s * (0.5 + 7 * 2.0 ** -23))


def test_zero_and_subnormal_groups():
    x = np.zeros(64, np.float32)
    tiny = np.float32(2) * np.float32(1.4e-45)  # 2 ulp of the subnormal range
    x[40] = tiny                        # abs-max 2 ulp: /7 rounds to zero
    codes, s = oracle.quantize_vector(x)
    assert s[0] == 0.0 and np.all(codes[:16] == 0)
    assert s[1] == 0.0 and np.all(codes[16:] == 0)   # s == 0 although a != 0
    x[40] = np.float32(7) * np.float32(1.4e-45)      # 7 ulp: /7 is exactly 1 ulp
    codes, s = oracle.quantize_vector(x)
    assert s[1] == np.float32(1.4e-45) and _codes(codes, 64)[40] == 7
    x[40] = np.float32(-3e-39)          # subnormal abs-max with a subnormal scale
    codes, s = oracle.quantize_vector(x)
    assert s[1] > 0 and _codes(codes, 64)[40] == -7
    x2 = np.full(32, -0.0, np.float32)
    codes, s = oracle.quantize_vector(x2)
    assert s[0] == 0.0 and np.all(codes == 0)


def test_nibble_order_low_first():
    x = np.zeros(32, np.float32)
    x[0], x[1] = 7.0, -7.0
    codes, _ = oracle.quantize_vector(x)
    assert codes[0] == (7 | (9 << 4))   # -7 & 15 = 9 in the high nibble


# ------------------------------------------------------------------ rotation

@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_srht_matches_explicit_hadamard(D):
    rng = np.random.default_rng(6)
    H = scipy.linalg.hadamard(D).astype(np.float64)
    s = np.where(rng.integers(0, 2, D) == 1, 1.0, -1.0).astype(np.float32)
    c = 1.0 / math.sqrt(D)
    for _ in range(5):
        x = rng.standard_normal(D).astype(np.float32)
        ref = c * (H @ (s.astype(np.float64) * x.astype(np.float64)))
        y64 = oracle.srht_f64(x, s, c)
        assert np.max(np.abs(y64 - ref)) < 1e-12
        y32 = oracle.srht_f32(x, s, np.float32(c))
        assert np.max(np.abs(y32 - ref)) < 1e-5 * math.sqrt(D)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_srht_closed_forms(D):
    c = np.float32(1.0 / math.sqrt(D))
    ones = np.ones(D, np.float32)
    y = oracle.srht_f32(ones, ones, c)              # H 1 = D e0
    assert y[0] == np.float32(D) * c and np.all(y[1:] == 0)
    codes, s = oracle.quantize_vector(y)
    cc = _codes(codes, D)
    assert cc[0] == 7 and np.all(cc[1:] == 0) and np.all(s[1:] == 0)
    rng = np.random.default_rng(7)
    sg = np.where(rng.integers(0, 2, D) == 1, 1.0, -1.0).astype(np.float32)
    e0 = np.zeros(D, np.float32)
    e0[0] = 1
    y = oracle.srht_f32(e0, sg, c)                  # H D e0 = s0 * 1
    assert np.all(y == sg[0] * c)
    assert np.all(_codes(oracle.quantize_vector(y)[0], D) == 7 * int(sg[0]))


def test_srht_involution_and_inner_product():
    D = 128
    rng = np.random.default_rng(8)
    x = rng.standard_normal(D)
    ones = np.ones(D, np.float32)
    twice = oracle.srht_f64(oracle.srht_f64(x, ones, 1.0), ones, 1.0)
    assert np.max(np.abs(twice - D * x)) < 1e-10    # H H = D I
    s = np.where(rng.integers(0, 2, D) == 1, 1.0, -1.0).astype(np.float32)
    c = 1 / math.sqrt(D)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    assert abs(oracle.srht_f64(q, s, c) @ oracle.srht_f64(k, s, c) - q @ k) < 1e-10


# ------------------------------------------------------------------ attention

def _random_cache(rng, B, Hkv, cap, D, dtype="bf16"):
    bits, _ = (None, None)
    x = rng.standard_normal((2, B, Hkv, cap, D)).astype(np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16 if dtype == "bf16" else torch.float16)
    b = t.view(torch.int16).numpy().view(np.uint16)
    kc, ks = oracle.quantize(b[0], dtype)
    vc, vs = oracle.quantize(b[1], dtype)
    return kc, ks, vc, vs


def _q(rng, B, Hq, D, dtype="bf16"):
    t = torch.from_numpy(rng.standard_normal((B, Hq, D)).astype(np.float32))
    t = t.to(torch.bfloat16 if dtype == "bf16" else torch.float16)
    return t.view(torch.int16).numpy().view(np.uint16), t.double()


@pytest.mark.parametrize("B,Hq,Hkv,D", [(2, 4, 4, 64), (1, 8, 2, 128), (3, 8, 1, 256)])
def test_sdpa_matches_torch_fp64(B, Hq, Hkv, D):
    rng = np.random.default_rng(9)
    cap = 37
    kc, ks, vc, vs = _random_cache(rng, B, Hkv, cap, D)
    qb, qt = _q(rng, B, Hq, D)
    lens = rng.integers(1, cap + 1, B).astype(np.int32)
    scale = 1 / math.sqrt(D)
    out = oracle.sdpa(qb, "bf16", kc, ks, vc, vs, lens, scale, threads=2)
    K = torch.from_numpy(oracle.dequantize(kc, ks))
    V = torch.from_numpy(oracle.dequantize(vc, vs))
    G = Hq // Hkv
    for b in range(B):
        T = int(lens[b])
        Kb = K[b, :, :T].repeat_interleave(G, 0)
        Vb = V[b, :, :T].repeat_interleave(G, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt[b][:, None, :], Kb, Vb, scale=scale)[:, 0]
        assert torch.max(torch.abs(torch.from_numpy(out[b]) - ref)) < 1e-12


def test_sdpa_zero_query_is_mean_of_values():
    rng = np.random.default_rng(10)
    kc, ks, vc, vs = _random_cache(rng, 1, 2, 50, 128)
    q = np.zeros((1, 2, 128), np.uint16)           # +0.0 in both formats
    out = oracle.sdpa(q, "bf16", kc, ks, vc, vs, np.array([33], np.int32), 0.1)
    V = oracle.dequantize(vc, vs)
    for h in range(2):
        assert np.max(np.abs(out[0, h] - V[0, h, :33].mean(0))) < 1e-12


def test_sdpa_dominant_score_selects_row():
    D = 64
    kc = np.zeros((1, 1, 20, D // 2), np.uint8)
    ks = np.ones((1, 1, 20, D // 32), np.float32)
    kc[0, 0, 13, 0] = 0x07                          # K^[13][0] = 7, every other K^ = 0
    rng = np.random.default_rng(11)
    _, _, vc, vs = _random_cache(rng, 1, 1, 20, D)
    q = torch.zeros((1, 1, D), dtype=torch.bfloat16)
    q[0, 0, 0] = 1.0
    qb = q.view(torch.int16).numpy().view(np.uint16)
    out = oracle.sdpa(qb, "bf16", kc, ks, vc, vs, np.array([20], np.int32), 200.0)
    V = oracle.dequantize(vc, vs)
    assert np.max(np.abs(out[0, 0] - V[0, 0, 13])) < 1e-12   # other weights e^-1400


def test_sdpa_weights_sum_to_one_and_edge_lengths():
    rng = np.random.default_rng(12)
    kc, ks, _, _ = _random_cache(rng, 2, 1, 40, 128)
    vc = np.full((2, 1, 40, 64), 0x77, np.uint8)    # every V code 7
    vs = np.full((2, 1, 40, 4), 0.25, np.float32)   # V^ = 1.75 everywhere
    qb, _ = _q(rng, 2, 1, 128)
    out = oracle.sdpa(qb, "bf16", kc, ks, vc, vs, np.array([40, 0], np.int32), 1.0)
    assert np.max(np.abs(out[0, 0] - 1.75)) < 1e-13     # sum of weights is 1
    assert np.all(out[1, 0] == 0.0)                      # lens 0 -> zeros
    _, _, vc2, vs2 = _random_cache(rng, 2, 1, 40, 128)
    out = oracle.sdpa(qb, "bf16", kc, ks, vc2, vs2, np.array([1, 1], np.int32), 1.0)
    V = oracle.dequantize(vc2, vs2)
    assert np.max(np.abs(out[:, 0] - V[:, 0, 0])) < 1e-13


def test_sdpa_rotated_query_matches_torch():
    D, T = 128, 29
    rng = np.random.default_rng(13)
    s = np.where(rng.integers(0, 2, D) == 1, 1.0, -1.0).astype(np.float32)
    c = np.float32(1 / math.sqrt(D))
    x = torch.from_numpy(rng.standard_normal((2, 1, 2, T, D)).astype(np.float32)).to(torch.bfloat16)
    b = x.view(torch.int16).numpy().view(np.uint16)
    kc, ks = oracle.quantize(b[0], "bf16", signs=s, rot_norm=c)
    vc, vs = oracle.quantize(b[1], "bf16")
    # the rotated cache is quantise(c H (s . k)): check one row by hand
    krow = oracle.srht_f32(x[0, 0, 0, 5].float().numpy(), s, c)
    assert np.array_equal(oracle.quantize_vector(krow)[0], kc[0, 0, 5])
    qb, qt = _q(rng, 1, 4, D)
    lens = np.array([T], np.int32)
    out = oracle.sdpa(qb, "bf16", kc, ks, vc, vs, lens, 0.09, signs=s, rot_norm=c)
    K = torch.from_numpy(oracle.dequantize(kc, ks))[0].repeat_interleave(2, 0)
    V = torch.from_numpy(oracle.dequantize(vc, vs))[0].repeat_interleave(2, 0)
    H = torch.from_numpy(scipy.linalg.hadamard(D).astype(np.float64))
    qr = (float(c) * (H @ (torch.from_numpy(s).double()[:, None] * qt[0].T))).T
    ref = torch.nn.functional.scaled_dot_product_attention(qr[:, None, :], K, V, scale=0.09)[:, 0]
    assert torch.max(torch.abs(torch.from_numpy(out[0]) - ref)) < 1e-12


def test_sdpa_row_subset_and_threads_agree():
    rng = np.random.default_rng(14)
    kc, ks, vc, vs = _random_cache(rng, 2, 2, 64, 128)
    qb, _ = _q(rng, 2, 8, 128)
    lens = np.array([64, 17], np.int32)
    full = oracle.sdpa(qb, "bf16", kc, ks, vc, vs, lens, 0.1, threads=1)
    rows = np.array([15, 0, 9], np.int32)
    sub = oracle.sdpa(qb, "bf16", kc, ks, vc, vs, lens, 0.1, rows=rows, threads=3)
    assert np.array_equal(sub, full.reshape(16, 128)[rows])


# ------------------------------------------------------------------ per-channel scale

def _rows(rng, shape, dtype, outliers=(), factor=1.0):
    x = rng.standard_normal(shape).astype(np.float32)
    for c in outliers:
        x[..., c] *= factor
    t = torch.from_numpy(x).to(torch.bfloat16 if dtype == "bf16" else torch.float16)
    return t.view(torch.int16).numpy().view(np.uint16), t.float().numpy()


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("rotate", [False, True])
def test_chan_scale_power_of_two_per_group_is_exact(dtype, D, rotate):
    """lambda = 2^k_g, constant within each group: every product is exact, so
    the codes are those without lambda and each scale is multiplied by 2^k_g;
    attention, which divides lambda back out, is then bit-identical."""
    rng = np.random.default_rng(D + rotate)
    bits, _ = _rows(rng, (2, 3, 40, D), dtype, outliers=(5,), factor=8.0)
    k = rng.integers(-6, 7, D // 32)
    lam = np.repeat(np.ldexp(1.0, k), 32).astype(np.float32)
    sg = np.where(rng.integers(0, 2, D) == 1, 1.0, -1.0).astype(np.float32) if rotate else None
    c = np.float32(1 / math.sqrt(D))
    c0, s0 = oracle.quantize(bits, dtype, signs=sg, rot_norm=c)
    c1, s1 = oracle.quantize(bits, dtype, signs=sg, rot_norm=c, chan_scale=lam)
    assert np.array_equal(c0, c1)
    assert np.array_equal(s1, (s0 * np.ldexp(1.0, k)).astype(np.float32))
    qb, _ = _q(rng, 2, 6, D, dtype)
    vc, vs = oracle.quantize(bits[::-1].copy(), dtype)
    lens = np.array([40, 23], np.int32)
    o0 = oracle.sdpa(qb, dtype, c0, s0, vc, vs, lens, 0.1, signs=sg, rot_norm=c)
    o1 = oracle.sdpa(qb, dtype, c1, s1, vc, vs, lens, 0.1, signs=sg, rot_norm=c, chan_scale=lam)
    assert np.array_equal(o0, o1)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_chan_scale_codes_bound_the_scaled_vector(dtype):
    """With any positive lambda the codes quantise z = fp32(lambda x): the
    error bound, the sign rule and max |c| = 7 hold against z, channel by
    channel (a lambda applied to the wrong channel breaks them)."""
    D = 128
    rng = np.random.default_rng(21)
    bits, x = _rows(rng, (300, D), dtype, outliers=(7, 70), factor=12.0)
    lam = rng.uniform(0.25, 4.0, D).astype(np.float32)
    codes, scales = oracle.quantize(bits, dtype, chan_scale=lam)
    z = (x * lam).astype(np.float32).reshape(300, D // 32, 32).astype(np.float64)
    cc = _codes(codes, D).reshape(300, D // 32, 32)
    s = scales.astype(np.float64)[..., None]
    assert np.all(np.abs(z - cc * s) <= s * (0.5 + 7 * 2.0 ** -23))
    assert np.all(np.abs(cc).max(-1)[scales > 0] == 7)
    assert np.all((np.sign(cc) == np.sign(z)) | (cc == 0))


@pytest.mark.parametrize("rotate", [False, True])
def test_sdpa_chan_scale_matches_torch(rotate):
    D, T, B, Hq, Hkv = 128, 33, 2, 4, 2
    rng = np.random.default_rng(22 + rotate)
    bits, _ = _rows(rng, (2, B, Hkv, T, D), "bf16")
    lam = rng.uniform(0.5, 2.0, D).astype(np.float32)
    sg = np.where(rng.integers(0, 2, D) == 1, 1.0, -1.0).astype(np.float32) if rotate else None
    c = np.float32(1 / math.sqrt(D))
    kc, ks = oracle.quantize(bits[0], "bf16", signs=sg, rot_norm=c, chan_scale=lam)
    vc, vs = oracle.quantize(bits[1], "bf16")
    qb, qt = _q(rng, B, Hq, D)
    lens = np.array([T, 19], np.int32)
    out = oracle.sdpa(qb, "bf16", kc, ks, vc, vs, lens, 0.11, signs=sg, rot_norm=c, chan_scale=lam)
    K = torch.from_numpy(oracle.dequantize(kc, ks) / lam.astype(np.float64))
    V = torch.from_numpy(oracle.dequantize(vc, vs))
    if rotate:
        H = torch.from_numpy(scipy.linalg.hadamard(D).astype(np.float64))
        qt = float(c) * (qt * torch.from_numpy(sg).double()) @ H.T
    for b in range(B):
        n = int(lens[b])
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt[b][:, None, :], K[b, :, :n].repeat_interleave(2, 0), V[b, :, :n].repeat_interleave(2, 0),
            scale=0.11)[:, 0]
        assert torch.max(torch.abs(torch.from_numpy(out[b]) - ref)) < 1e-12


def test_chan_scale_evens_out_outlier_channels():
    """What the scale is for: with three K channels 20x larger than the rest,
    lambda = 1/20 on them brings the attention on the quantised cache closer
    to attention on the unquantised K."""
    D, T = 128, 256
    rng = np.random.default_rng(23)
    out_ch = (3, 40, 100)
    bits, x = _rows(rng, (1, 1, T, D), "bf16", outliers=out_ch, factor=20.0)
    lam = np.ones(D, np.float32)
    lam[list(out_ch)] = np.float32(1 / 20)
    vbits, _ = _rows(rng, (1, 1, T, D), "bf16")
    vc, vs = oracle.quantize(vbits, "bf16")
    qb, qt = _q(rng, 1, 8, D)
    lens = np.array([T], np.int32)
    Kt = torch.from_numpy(x.astype(np.float64))[0].repeat_interleave(8, 0)
    V = torch.from_numpy(oracle.dequantize(vc, vs))[0].repeat_interleave(8, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt[0][:, None, :], Kt, V, scale=0.3)[:, 0].numpy()
    errs = []
    for ls in (None, lam):
        kc, ks = oracle.quantize(bits, "bf16", chan_scale=ls)
        out = oracle.sdpa(qb, "bf16", kc, ks, vc, vs, lens, 0.3, chan_scale=ls)
        errs.append(np.linalg.norm(out[0] - ref) / np.linalg.norm(ref))
    assert errs[1] < 0.5 * errs[0], errs


# ------------------------------------------------------------------ rotated V

@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_unrotate_is_the_inverse_rotation(D):
    """s (.) (c H y) against the explicit fp64 matrix S H c, and as the
    inverse of the forward rotation c H (s (.) x)."""
    rng = np.random.default_rng(40 + D)
    s = np.where(rng.integers(0, 2, D) == 1, 1.0, -1.0).astype(np.float32)
    c = 1 / math.sqrt(D)
    y = rng.standard_normal(D)
    H = scipy.linalg.hadamard(D).astype(np.float64)
    assert np.max(np.abs(oracle.unrotate_f64(y, s, c) - s * (c * (H @ y)))) < 1e-12
    x = rng.standard_normal(D)
    assert np.max(np.abs(oracle.unrotate_f64(oracle.srht_f64(x, s, c), s, c) - x)) < 1e-12


@pytest.mark.parametrize("rotate_k", [False, True])
def test_sdpa_rotated_v_matches_torch(rotate_k):
    """V quantised in the rotated basis; attention returns to the original
    basis: PyTorch fp64 SDPA on V^_t = S H c (code * s) per token."""
    D, T, B, Hq, Hkv = 128, 35, 2, 4, 2
    rng = np.random.default_rng(41 + rotate_k)
    bits, _ = _rows(rng, (2, B, Hkv, T, D), "bf16")
    c = np.float32(1 / math.sqrt(D))
    sk = np.where(rng.integers(0, 2, D) == 1, 1.0, -1.0).astype(np.float32) if rotate_k else None
    sv = np.where(rng.integers(0, 2, D) == 1, 1.0, -1.0).astype(np.float32)
    kc, ks = oracle.quantize(bits[0], "bf16", signs=sk, rot_norm=c)
    vc, vs = oracle.quantize(bits[1], "bf16", signs=sv, rot_norm=c)
    qb, qt = _q(rng, B, Hq, D)
    lens = np.array([T, 21], np.int32)
    out = oracle.sdpa(qb, "bf16", kc, ks, vc, vs, lens, 0.12, signs=sk, rot_norm=c, v_signs=sv)
    H = torch.from_numpy(scipy.linalg.hadamard(D).astype(np.float64))
    K = torch.from_numpy(oracle.dequantize(kc, ks))
    V = (torch.from_numpy(oracle.dequantize(vc, vs)) @ H.T) * float(c) * torch.from_numpy(sv).double()
    if rotate_k:
        qt = float(c) * (qt * torch.from_numpy(sk).double()) @ H.T
    for b in range(B):
        n = int(lens[b])
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt[b][:, None, :], K[b, :, :n].repeat_interleave(2, 0), V[b, :, :n].repeat_interleave(2, 0),
            scale=0.12)[:, 0]
        assert torch.max(torch.abs(torch.from_numpy(out[b]) - ref)) < 1e-12


def test_rotated_v_spreads_outlier_channels():
    """What rotating V is for: with three V channels 20x larger than the
    rest, quantising V in the rotated basis brings the attention output on
    the quantised cache closer to attention on the unquantised V."""
    D, T = 128, 256
    rng = np.random.default_rng(42)
    kbits, _ = _rows(rng, (1, 1, T, D), "bf16")
    vbits, v = _rows(rng, (1, 1, T, D), "bf16", outliers=(5, 50, 99), factor=20.0)
    kc, ks = oracle.quantize(kbits, "bf16")
    qb, qt = _q(rng, 1, 8, D)
    lens = np.array([T], np.int32)
    K = torch.from_numpy(oracle.dequantize(kc, ks))[0].repeat_interleave(8, 0)
    Vt = torch.from_numpy(v.astype(np.float64))[0].repeat_interleave(8, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt[0][:, None, :], K, Vt, scale=0.1)[:, 0].numpy()
    c = np.float32(1 / math.sqrt(D))
    sv = np.where(rng.integers(0, 2, D) == 1, 1.0, -1.0).astype(np.float32)
    errs = []
    for signs in (None, sv):
        vc, vs = oracle.quantize(vbits, "bf16", signs=signs, rot_norm=c)
        out = oracle.sdpa(qb, "bf16", kc, ks, vc, vs, lens, 0.1, rot_norm=c, v_signs=signs)
        errs.append(np.linalg.norm(out[0] - ref) / np.linalg.norm(ref))
    assert errs[1] < 0.6 * errs[0], errs   # 0.44 here; 0.43-0.44 over other seeds


# ------------------------------------------------------------------ closed forms

def test_closed_form_storage_figures():
    g = json.load(open(os.path.join(GOLDEN, "storage_closed_forms.json")))
    L = g["llama31_70b_128k"]
    n = L["layers"] * L["kv_heads"] * L["head_dim"] * L["tokens"] * 2
    assert n * 2 == L["fp16_bytes"] == 40 * 2 ** 30
    # one packed row of D codes is D/2 bytes and D/32 fp32 scales
    D = L["head_dim"]
    codes, scales = oracle.quantize_vector(np.ones(D, np.float32))
    per_vec = codes.nbytes + scales.nbytes
    assert n // D * per_vec == L["int4_bytes"] == int(12.5 * 2 ** 30)
    assert L["fp16_bytes"] / L["int4_bytes"] == L["ratio"]
    A = g["adaptq_4h_d128_4096"]
    m = A["heads"] * A["head_dim"] * A["tokens"] * 2
    assert m * 2 == A["fp16_bytes"] and m // A["head_dim"] * codes.nbytes == A["codes_only_bytes"]
