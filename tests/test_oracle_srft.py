"""Pins for the oracle's SRFT rotation (the sign-randomised FFT that may take
the place of the Hadamard rotation on the "SRFT + int4 KV-cache" page, core
method).  The transform is pinned to the DFT's definition on tiny inputs, to
numpy's FFT at the cache widths, to closed forms that are exact in fp32, and
its fp32 twiddles to values computed here from a 50-digit series."""
import cmath
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle


def _bitrev(k, bits):
    r = 0
    for _ in range(bits):
        r = (r << 1) | (k & 1)
        k >>= 1
    return r


def _dft_definition(x, signs):
    """c * DFT(z), z_j = s_2j x_2j + i s_2j+1 x_2j+1, coefficient bitrev(k)
    placed at position k; plain sums of the definition."""
    D = len(x)
    N = D // 2
    bits = N.bit_length() - 1
    z = [complex(signs[2 * j] * x[2 * j], signs[2 * j + 1] * x[2 * j + 1]) for j in range(N)]
    out = np.zeros(D)
    for k in range(N):
        f = _bitrev(k, bits)
        acc = sum(z[j] * cmath.exp(-2j * math.pi * j * f / N) for j in range(N))
        acc /= math.sqrt(N)
        out[2 * k], out[2 * k + 1] = acc.real, acc.imag
    return out


def _numpy_srft(x, signs):
    D = x.shape[-1]
    N = D // 2
    bits = N.bit_length() - 1
    xs = x * signs
    F = np.fft.fft(xs[0::2] + 1j * xs[1::2]) / math.sqrt(N)
    perm = np.array([_bitrev(k, bits) for k in range(N)])
    Z = F[perm]
    out = np.empty(D)
    out[0::2], out[1::2] = Z.real, Z.imag
    return out


def _signs(D, seed):
    return np.where(np.random.default_rng(seed).random(D) < 0.5, -1.0, 1.0).astype(np.float32)


@pytest.mark.parametrize("D", [4, 8, 16, 32])
def test_srft_tiny_matches_dft_definition(D):
    rng = np.random.default_rng(D)
    for trial in range(3):
        x = rng.standard_normal(D)
        s = _signs(D, 100 * D + trial)
        got = oracle.srft_f64(x, s, 1.0 / math.sqrt(D // 2))
        assert np.allclose(got, _dft_definition(x, s), rtol=0, atol=1e-12)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_srft_f64_matches_numpy_fft(D):
    rng = np.random.default_rng(7 + D)
    x = rng.standard_normal(D) * 3.0
    s = _signs(D, D)
    got = oracle.srft_f64(x, s, 1.0 / math.sqrt(D // 2))
    assert np.allclose(got, _numpy_srft(x, s), rtol=0, atol=1e-12)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_srft_f32_close_to_f64(D):
    rng = np.random.default_rng(11 + D)
    s = _signs(D, 3 * D)
    c32 = np.float32(1.0 / math.sqrt(D // 2))
    for _ in range(20):
        x = rng.standard_normal(D).astype(np.float32)
        x[rng.integers(D)] *= 40.0  # an outlier channel
        y32 = oracle.srft_f32(x, s, c32).astype(np.float64)
        y64 = oracle.srft_f64(x.astype(np.float64), s, float(c32))
        # each of the log2(D/2) stages adds a few fp32 roundings per element
        bound = 8 * math.log2(D // 2) * 2.0 ** -24 * np.linalg.norm(x)
        assert np.max(np.abs(y32 - y64)) <= bound


@pytest.mark.parametrize("D", [64, 128, 256])
def test_srft_orthogonal_and_keeps_dot_products(D):
    rng = np.random.default_rng(5 * D)
    s = _signs(D, 9 * D)
    c = 1.0 / math.sqrt(D // 2)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    qr, kr = oracle.srft_f64(q, s, c), oracle.srft_f64(k, s, c)
    assert abs(np.linalg.norm(qr) - np.linalg.norm(q)) < 1e-12 * np.linalg.norm(q)
    assert abs(qr @ kr - q @ k) < 1e-12 * np.linalg.norm(q) * np.linalg.norm(k)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_srft_closed_forms_exact_in_fp32(D):
    N = D // 2
    c = np.float32(1.0 / math.sqrt(N))
    ones = np.ones(D, np.float32)
    # z = delta_0: every coefficient is 1, so y = c (1, 0, 1, 0, ...)
    e0 = np.zeros(D, np.float32)
    e0[0] = 1.0
    y = oracle.srft_f32(e0, ones, c)
    want = np.zeros(D, np.float32)
    want[0::2] = c
    assert np.array_equal(y.view(np.uint32), want.view(np.uint32))
    # z = i delta_0: y = c (0, 1, 0, 1, ...)
    e1 = np.zeros(D, np.float32)
    e1[1] = 1.0
    y = oracle.srft_f32(e1, ones, c)
    want = np.zeros(D, np.float32)
    want[1::2] = c
    assert np.array_equal(y.view(np.uint32), want.view(np.uint32))
    # z = 1 everywhere: only the zero frequency, N c, at position 0
    dc = np.zeros(D, np.float32)
    dc[0::2] = 1.0
    y = oracle.srft_f32(dc, ones, c)
    want = np.zeros(D, np.float32)
    want[0] = np.float32(N) * c
    assert np.array_equal(y.view(np.uint32), want.view(np.uint32))
    # the signs enter before the transform: s = -1 on element 0 negates e0's image
    s = ones.copy()
    s[0] = -1.0
    assert np.array_equal(oracle.srft_f32(e0, s, c), -oracle.srft_f32(e0, ones, c))


@pytest.mark.parametrize("D", [64, 128])
def test_srft_pure_tone_lands_at_bit_reversed_position(D):
    N = D // 2
    bits = N.bit_length() - 1
    for m in (1, 3, N // 2 - 1, N - 2):
        z = np.exp(2j * np.pi * m * np.arange(N) / N)
        x = np.empty(D)
        x[0::2], x[1::2] = z.real, z.imag
        y = oracle.srft_f64(x, np.ones(D, np.float32), 1.0 / math.sqrt(N))
        pos = [k for k in range(N) if _bitrev(k, bits) == m][0]
        want = np.zeros(D)
        want[2 * pos] = math.sqrt(N)
        assert np.allclose(y, want, rtol=0, atol=1e-11)


# -------------------------------------------------------------- twiddles

getcontext().prec = 60
_PI = Decimal("3.14159265358979323846264338327950288419716939937510582097494459")


def _dcos_sin(theta):
    """cos and sin of a Decimal angle by their Taylor series (|theta| <= pi)."""
    c, s = Decimal(0), Decimal(0)
    term_c, term_s = Decimal(1), theta
    for n in range(60):
        c += term_c
        s += term_s
        term_c = -term_c * theta * theta / ((2 * n + 1) * (2 * n + 2))
        term_s = -term_s * theta * theta / ((2 * n + 2) * (2 * n + 3))
    return c, s


def _round_f32_with_margin(v):
    """The fp32 nearest to Decimal v and v's distance, relative, to the
    nearest rounding midpoint (inf for values fp32 holds exactly)."""
    f = np.float32(float(v))
    if Decimal(float(f)) == v:
        return f, math.inf
    lo = np.nextafter(f, np.float32(-np.inf))
    hi = np.nextafter(f, np.float32(np.inf))
    m1 = (Decimal(float(lo)) + Decimal(float(f))) / 2
    m2 = (Decimal(float(f)) + Decimal(float(hi))) / 2
    assert m1 < v < m2, "the double guess must round to the nearest fp32"
    margin = min(v - m1, m2 - v) / abs(v)
    return f, float(margin)


@pytest.mark.parametrize("N", [32, 64, 128])
def test_srft_twiddles_are_correctly_rounded_with_margin(N):
    for t in range(N):
        theta = 2 * _PI * t / N
        # reduce to |theta| <= pi for the series
        if theta > _PI:
            theta -= 2 * _PI
        cv, sv = _dcos_sin(theta)
        # quarter turns are exact
        if (4 * t) % N == 0:
            cv = Decimal(round(float(cv)))
            sv = Decimal(round(float(sv)))
        wr_ref, m_r = _round_f32_with_margin(cv) if cv != 0 else (np.float32(0.0), math.inf)
        wi_ref, m_i = _round_f32_with_margin(-sv) if sv != 0 else (np.float32(0.0), math.inf)
        wr, wi = oracle.twiddle_f32(t, N)
        assert wr.view(np.uint32) == wr_ref.view(np.uint32), (t, N)
        assert wi.view(np.uint32) == wi_ref.view(np.uint32), (t, N)
        # far from every midpoint: any evaluation within 2^-40 rounds alike
        assert m_r > 2.0 ** -40 and m_i > 2.0 ** -40, (t, N)


# -------------------------------------------------------------- quantise and attend

@pytest.mark.parametrize("D", [64, 128, 256])
def test_srft_quantise_closed_form(D):
    """x = e_0 in bf16 with all signs +1 rotates to c (1, 0, 1, 0, ...): every
    group has abs-max c, codes 7 on even channels and 0 on odd ones."""
    N = D // 2
    c = np.float32(1.0 / math.sqrt(N))
    bits = np.zeros((1, D), np.uint16)
    bits[0, 0] = 0x3F80  # bf16 1.0
    codes, scales = oracle.quantize(bits, "bf16", signs=np.ones(D, np.float32), rot_norm=c,
                                    rot_kind="srft")
    lo, hi = codes[0] & 0xF, codes[0] >> 4
    assert np.all(lo == 7) and np.all(hi == 0)
    assert np.all(scales[0] == np.float32(c / np.float32(7.0)))


def test_srft_quantise_differs_from_srht_and_matches_rows():
    rng = np.random.default_rng(3)
    D = 128
    x = torch.from_numpy(rng.standard_normal((6, D)).astype(np.float32)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    s = _signs(D, 21)
    c = np.float32(1.0 / math.sqrt(D // 2))
    codes, scales = oracle.quantize(bits, "bf16", signs=s, rot_norm=c, rot_kind="srft")
    codes_h, _ = oracle.quantize(bits, "bf16", signs=s, rot_norm=c, rot_kind="srht")
    assert not np.array_equal(codes, codes_h)
    for n in range(6):
        y = oracle.srft_f32(x[n].float().numpy(), s, c)
        cv, sv = oracle.quantize_vector(y)
        assert np.array_equal(cv, codes[n]) and np.array_equal(sv, scales[n])


def test_sdpa_srft_query_matches_torch():
    """Attention over an SRFT-rotated cache equals torch's fp64 attention with
    the query rotated by numpy's FFT (a library routine) and the dequantised
    rotated keys."""
    rng = np.random.default_rng(17)
    B, Hq, Hkv, D, T = 1, 4, 2, 128, 70
    k = torch.from_numpy(rng.standard_normal((B, Hkv, T, D)).astype(np.float32)).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((B, Hkv, T, D)).astype(np.float32)).to(torch.bfloat16)
    q = torch.from_numpy(rng.standard_normal((B, Hq, D)).astype(np.float32)).to(torch.bfloat16)
    s = _signs(D, 33)
    c = np.float32(1.0 / math.sqrt(D // 2))
    u16 = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    kc, ks = oracle.quantize(u16(k), "bf16", signs=s, rot_norm=c, rot_kind="srft")
    vc, vs = oracle.quantize(u16(v), "bf16")
    lens = np.array([T], np.int32)
    scale = 1.0 / math.sqrt(D)
    got = oracle.sdpa(u16(q), "bf16", kc, ks, vc, vs, lens, scale, signs=s, rot_norm=c,
                      rot_kind="srft")
    kd = torch.from_numpy(oracle.dequantize(kc, ks))
    vd = torch.from_numpy(oracle.dequantize(vc, vs))
    qn = q.double().numpy()
    qr = np.stack([[_numpy_srft(qn[b, h], s) * (float(c) * math.sqrt(D // 2))
                    for h in range(Hq)] for b in range(B)])
    qt = torch.from_numpy(qr)
    G = Hq // Hkv
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt.unsqueeze(2), kd.repeat_interleave(G, 1), vd.repeat_interleave(G, 1),
        scale=scale).squeeze(2)
    assert np.allclose(got, ref.numpy(), rtol=0, atol=1e-10)


# -------------------------------------------------------------- rotated V

@pytest.mark.parametrize("D", [8, 64, 128, 256])
def test_unsrft_inverts_srft_and_matches_numpy_ifft(D):
    rng = np.random.default_rng(41 + D)
    s = _signs(D, 43 + D)
    c = 1.0 / math.sqrt(D // 2)
    x = rng.standard_normal(D)
    assert np.allclose(oracle.unsrft_f64(oracle.srft_f64(x, s, c), s, c), x, rtol=0, atol=1e-12)
    # the inverse of y: undo the bit-reversed order, inverse DFT (numpy), signs
    N = D // 2
    bits = N.bit_length() - 1
    y = rng.standard_normal(D)
    Z = np.empty(N, complex)
    for k in range(N):
        Z[_bitrev(k, bits)] = y[2 * k] + 1j * y[2 * k + 1]
    z = np.fft.ifft(Z) * math.sqrt(N)
    want = np.empty(D)
    want[0::2], want[1::2] = z.real, z.imag
    assert np.allclose(oracle.unsrft_f64(y, s, c), want * s, rtol=0, atol=1e-12)


def test_sdpa_srft_rotated_v_matches_torch():
    """V quantised after the SRFT rotation (its own signs): attention equals
    torch's fp64 SDPA with every dequantised V row brought back by numpy's
    inverse FFT; K rotated by SRFT as well."""
    rng = np.random.default_rng(19)
    B, Hq, Hkv, D, T = 1, 4, 2, 64, 50
    k = torch.from_numpy(rng.standard_normal((B, Hkv, T, D)).astype(np.float32)).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((B, Hkv, T, D)).astype(np.float32)).to(torch.bfloat16)
    q = torch.from_numpy(rng.standard_normal((B, Hq, D)).astype(np.float32)).to(torch.bfloat16)
    s, sv = _signs(D, 51), _signs(D, 52)
    N = D // 2
    bits = N.bit_length() - 1
    c = np.float32(1.0 / math.sqrt(N))
    u16 = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    kc, ks = oracle.quantize(u16(k), "bf16", signs=s, rot_norm=c, rot_kind="srft")
    vc, vs = oracle.quantize(u16(v), "bf16", signs=sv, rot_norm=c, rot_kind="srft")
    lens = np.array([T], np.int32)
    scale = 1.0 / math.sqrt(D)
    got = oracle.sdpa(u16(q), "bf16", kc, ks, vc, vs, lens, scale, signs=s, rot_norm=c,
                      v_signs=sv, rot_kind="srft")
    kd = torch.from_numpy(oracle.dequantize(kc, ks))
    vr = oracle.dequantize(vc, vs)  # rotated basis
    Z = np.empty(vr.shape[:-1] + (N,), complex)
    for kk in range(N):
        Z[..., _bitrev(kk, bits)] = vr[..., 2 * kk] + 1j * vr[..., 2 * kk + 1]
    z = np.fft.ifft(Z, axis=-1) * N * float(c)
    vb = np.empty(vr.shape)
    vb[..., 0::2], vb[..., 1::2] = z.real, z.imag
    vd = torch.from_numpy(vb * sv.astype(np.float64))
    qn = q.double().numpy()
    qt = torch.from_numpy(np.stack([[_numpy_srft(qn[b, h], s) * (float(c) * math.sqrt(N))
                                     for h in range(Hq)] for b in range(B)]))
    G = Hq // Hkv
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt.unsqueeze(2), kd.repeat_interleave(G, 1), vd.repeat_interleave(G, 1),
        scale=scale).squeeze(2)
    assert np.allclose(got, ref.numpy(), rtol=0, atol=1e-10)
