"""Pins for the oracle's mixed-radix SRFT: head widths whose D/2 complex
numbers are three times a power of two (D = 12, 24, ..., 192, 384), where
the FFT form of the rotation serves and the Hadamard form cannot ("SRFT +
int4 KV-cache" page: core method, and the comparison of methods, where the
FFT's freedom from powers of two is its advantage).

The transform is pinned to the DFT's definition written out as sums on tiny
inputs, to numpy's FFT (a library routine) at D = 96, 192 and 384, to
closed forms exact in fp32, and its constants (the twiddles of N = 96 and
sqrt(3)/2) to values computed here from 60-digit series.  The output order
is derived here from the decimation-in-frequency split, independently of
the oracle: the radix-3 stage sorts the frequencies by their residue m mod
3 into blocks of M = N/3, and each block is then a radix-2 FFT of M points,
which leaves its k-th frequency at the bit-reversed position."""
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


def _frequency_at(N):
    """freq[P]: the DFT coefficient the in-place transform leaves at
    position P (N = 2^b or 3 * 2^b)."""
    if N % 3:
        b = N.bit_length() - 1
        return np.array([_bitrev(P, b) for P in range(N)])
    M = N // 3
    b = M.bit_length() - 1
    return np.array([3 * _bitrev(P % M, b) + P // M for P in range(N)])


def _dft_definition(x, signs):
    """c * DFT(z), z_j = s_2j x_2j + i s_2j+1 x_2j+1, as plain sums, in the
    transform's output order."""
    D = len(x)
    N = D // 2
    freq = _frequency_at(N)
    z = [complex(signs[2 * j] * x[2 * j], signs[2 * j + 1] * x[2 * j + 1]) for j in range(N)]
    out = np.zeros(D)
    for P in range(N):
        f = freq[P]
        acc = sum(z[j] * cmath.exp(-2j * math.pi * j * f / N) for j in range(N)) / math.sqrt(N)
        out[2 * P], out[2 * P + 1] = acc.real, acc.imag
    return out


def _numpy_srft(x, signs):
    D = x.shape[-1]
    N = D // 2
    xs = x * signs
    F = np.fft.fft(xs[..., 0::2] + 1j * xs[..., 1::2], axis=-1) / math.sqrt(N)
    Z = F[..., _frequency_at(N)]
    out = np.empty(x.shape)
    out[..., 0::2], out[..., 1::2] = Z.real, Z.imag
    return out


def _signs(D, seed):
    return np.where(np.random.default_rng(seed).random(D) < 0.5, -1.0, 1.0).astype(np.float32)


def test_frequency_order_is_a_permutation():
    for N in (6, 12, 48, 96, 192):
        f = _frequency_at(N)
        assert sorted(f) == list(range(N))
        # position 0 of every block holds the block's residue, frequency m
        M = N // 3
        assert list(f[[0, M, 2 * M]]) == [0, 1, 2]


@pytest.mark.parametrize("D", [12, 24, 48])
def test_mixed_tiny_matches_dft_definition(D):
    rng = np.random.default_rng(D)
    for trial in range(3):
        x = rng.standard_normal(D)
        s = _signs(D, 100 * D + trial)
        got = oracle.srft_f64(x, s, 1.0 / math.sqrt(D // 2))
        assert np.allclose(got, _dft_definition(x, s), rtol=0, atol=1e-12)


@pytest.mark.parametrize("D", [96, 192, 384])
def test_mixed_f64_matches_numpy_fft(D):
    rng = np.random.default_rng(7 + D)
    x = rng.standard_normal(D) * 3.0
    s = _signs(D, D)
    got = oracle.srft_f64(x, s, 1.0 / math.sqrt(D // 2))
    assert np.allclose(got, _numpy_srft(x, s), rtol=0, atol=1e-12)


@pytest.mark.parametrize("D", [96, 192])
def test_mixed_f32_close_to_f64(D):
    rng = np.random.default_rng(11 + D)
    s = _signs(D, 3 * D)
    c32 = np.float32(1.0 / math.sqrt(D // 2))
    for _ in range(20):
        x = rng.standard_normal(D).astype(np.float32)
        x[rng.integers(D)] *= 40.0
        y32 = oracle.srft_f32(x, s, c32).astype(np.float64)
        y64 = oracle.srft_f64(x.astype(np.float64), s, float(c32))
        # a few fp32 roundings per element per stage (1 radix-3 + log2(N/3) radix-2)
        stages = 1 + math.log2(D // 6)
        assert np.max(np.abs(y32 - y64)) <= 8 * stages * 2.0 ** -24 * np.linalg.norm(x)


def test_mixed_orthogonal_inverse_and_dot_products():
    D = 192
    rng = np.random.default_rng(5)
    s = _signs(D, 9)
    c = 1.0 / math.sqrt(D // 2)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    qr, kr = oracle.srft_f64(q, s, c), oracle.srft_f64(k, s, c)
    assert abs(np.linalg.norm(qr) - np.linalg.norm(q)) < 1e-12 * np.linalg.norm(q)
    assert abs(qr @ kr - q @ k) < 1e-12 * np.linalg.norm(q) * np.linalg.norm(k)
    assert np.allclose(oracle.unsrft_f64(qr, s, c), q, rtol=0, atol=1e-12)


@pytest.mark.parametrize("D", [12, 192])
def test_mixed_unsrft_matches_numpy_ifft(D):
    """The inverse: undo the output order, numpy's inverse DFT, the signs."""
    rng = np.random.default_rng(43 + D)
    s = _signs(D, 44 + D)
    N = D // 2
    c = 1.0 / math.sqrt(N)
    y = rng.standard_normal(D)
    Z = np.empty(N, complex)
    Z[_frequency_at(N)] = y[0::2] + 1j * y[1::2]
    z = np.fft.ifft(Z) * math.sqrt(N)
    want = np.empty(D)
    want[0::2], want[1::2] = z.real, z.imag
    assert np.allclose(oracle.unsrft_f64(y, s, c), want * s, rtol=0, atol=1e-12)


@pytest.mark.parametrize("D", [96, 192])
def test_mixed_closed_forms_exact_in_fp32(D):
    N = D // 2
    c = np.float32(1.0 / math.sqrt(N))
    ones = np.ones(D, np.float32)
    # delta_0: every coefficient is 1, y = c (1, 0, 1, 0, ...)
    e0 = np.zeros(D, np.float32)
    e0[0] = 1.0
    want = np.zeros(D, np.float32)
    want[0::2] = c
    y = oracle.srft_f32(e0, ones, c)
    assert np.array_equal(y, want) and np.array_equal(y[0::2].view(np.uint32), want[0::2].view(np.uint32))
    # i delta_0: y = c (0, 1, 0, 1, ...)
    e1 = np.zeros(D, np.float32)
    e1[1] = 1.0
    want = np.zeros(D, np.float32)
    want[1::2] = c
    y = oracle.srft_f32(e1, ones, c)
    assert np.array_equal(y, want) and np.array_equal(y[1::2].view(np.uint32), want[1::2].view(np.uint32))
    # the all-ones real signal: only frequency 0, N c, at position 0
    dc = np.zeros(D, np.float32)
    dc[0::2] = 1.0
    want = np.zeros(D, np.float32)
    want[0] = np.float32(N) * c
    y = oracle.srft_f32(dc, ones, c)
    assert np.array_equal(y, want) and y[0].view(np.uint32) == want[0].view(np.uint32)
    # a negated sign negates the image
    s = ones.copy()
    s[0] = -1.0
    assert np.array_equal(oracle.srft_f32(e0, s, c), -oracle.srft_f32(e0, ones, c))


@pytest.mark.parametrize("D", [48, 192])
def test_mixed_pure_tone_lands_at_its_position(D):
    N = D // 2
    freq = _frequency_at(N)
    for f in (1, 2, 3, N // 3 + 1, N - 1):
        z = np.exp(2j * np.pi * f * np.arange(N) / N)
        x = np.empty(D)
        x[0::2], x[1::2] = z.real, z.imag
        y = oracle.srft_f64(x, np.ones(D, np.float32), 1.0 / math.sqrt(N))
        want = np.zeros(D)
        want[2 * int(np.nonzero(freq == f)[0][0])] = math.sqrt(N)
        assert np.allclose(y, want, rtol=0, atol=1e-11)


# -------------------------------------------------------------- constants

getcontext().prec = 60
_PI = Decimal("3.14159265358979323846264338327950288419716939937510582097494459")


def _dcos_sin(theta):
    c, s = Decimal(0), Decimal(0)
    term_c, term_s = Decimal(1), theta
    for n in range(60):
        c += term_c
        s += term_s
        term_c = -term_c * theta * theta / ((2 * n + 1) * (2 * n + 2))
        term_s = -term_s * theta * theta / ((2 * n + 2) * (2 * n + 3))
    return c, s


def _round_f32_with_margin(v):
    f = np.float32(float(v))
    if Decimal(float(f)) == v:
        return f, math.inf
    lo = np.nextafter(f, np.float32(-np.inf))
    hi = np.nextafter(f, np.float32(np.inf))
    m1 = (Decimal(float(lo)) + Decimal(float(f))) / 2
    m2 = (Decimal(float(f)) + Decimal(float(hi))) / 2
    assert m1 < v < m2
    return f, float(min(v - m1, m2 - v) / abs(v))


def test_twiddles_of_96_points_are_correctly_rounded_with_margin():
    N = 96
    for t in range(N):
        theta = 2 * _PI * t / N
        if theta > _PI:
            theta -= 2 * _PI
        cv, sv = _dcos_sin(theta)
        if (4 * t) % N == 0:  # quarter turns are exact
            cv, sv = Decimal(round(float(cv))), Decimal(round(float(sv)))
        wr_ref, m_r = _round_f32_with_margin(cv) if cv != 0 else (np.float32(0.0), math.inf)
        wi_ref, m_i = _round_f32_with_margin(-sv) if sv != 0 else (np.float32(0.0), math.inf)
        wr, wi = oracle.twiddle_f32(t, N)
        assert wr.view(np.uint32) == wr_ref.view(np.uint32), t
        assert wi.view(np.uint32) == wi_ref.view(np.uint32), t
        assert m_r > 2.0 ** -40 and m_i > 2.0 ** -40, t


def test_radix3_constant_is_correctly_rounded():
    """c3 = sqrt(3)/2: the fp32 transform's only other constant.  The radix-3
    butterfly of a0 = 0, a1 = 1, a2 = 0 gives t = c3 exactly, so the image of
    z_M = 1 at D = 12 carries it: position M (block 1, frequency 1) holds
    c (m - i t) = c (-1/2, -c3) for j = 0."""
    root3 = Decimal(3).sqrt() / 2
    ref, margin = _round_f32_with_margin(root3)
    assert margin > 2.0 ** -30
    D, N = 12, 6
    M = N // 3
    x = np.zeros(D, np.float32)
    x[2 * M] = 1.0  # z_M = 1
    y = oracle.srft_f32(x, np.ones(D, np.float32), np.float32(1.0))
    # the radix-3 stage leaves b1 = (-1/2, -c3) at position M (twiddle W^0),
    # and the radix-2 stage of block 1 (2 points: b1 and the zero at M + 1)
    # copies it to position M
    assert y[2 * M] == np.float32(-0.5)
    assert y[2 * M + 1].view(np.uint32) == (-ref).view(np.uint32)


# -------------------------------------------------------------- quantise and attend

def test_mixed_quantise_closed_form():
    """x = e_0 rotates to c (1, 0, 1, 0, ...) at D = 192: every group has
    abs-max c, codes 7 on even channels and 0 on odd ones."""
    D = 192
    c = np.float32(1.0 / math.sqrt(D // 2))
    bits = np.zeros((1, D), np.uint16)
    bits[0, 0] = 0x3F80  # bf16 1.0
    codes, scales = oracle.quantize(bits, "bf16", signs=np.ones(D, np.float32), rot_norm=c, rot_kind="srft")
    assert np.all(codes[0] & 0xF == 7) and np.all(codes[0] >> 4 == 0)
    assert np.all(scales[0] == np.float32(c / np.float32(7.0)))


def test_srht_needs_a_power_of_two():
    bits = np.zeros((1, 192), np.uint16)
    with pytest.raises(Exception):
        oracle.quantize(bits, "bf16", signs=np.ones(192, np.float32), rot_norm=0.1, rot_kind="srht")


@pytest.mark.parametrize("rot", [False, True])
def test_sdpa_d192_matches_torch(rot):
    """Attention at D = 192 (six groups): unrotated, and with K and V rotated
    by the mixed-radix SRFT, against torch's fp64 SDPA with the query rotated
    by numpy's FFT and every V row brought back by numpy's inverse FFT."""
    rng = np.random.default_rng(23 + rot)
    B, Hq, Hkv, D, T = 2, 4, 2, 192, 45
    N = D // 2
    k = torch.from_numpy(rng.standard_normal((B, Hkv, T, D)).astype(np.float32)).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((B, Hkv, T, D)).astype(np.float32)).to(torch.bfloat16)
    q = torch.from_numpy(rng.standard_normal((B, Hq, D)).astype(np.float32)).to(torch.bfloat16)
    s, sv = (_signs(D, 61), _signs(D, 62)) if rot else (None, None)
    c = np.float32(1.0 / math.sqrt(N))
    u16 = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    kw = dict(signs=s, rot_norm=c, rot_kind="srft") if rot else {}
    vw = dict(signs=sv, rot_norm=c, rot_kind="srft") if rot else {}
    kc, ks = oracle.quantize(u16(k), "bf16", **kw)
    vc, vs = oracle.quantize(u16(v), "bf16", **vw)
    lens = np.array([T, 30], np.int32)
    scale = 1.0 / math.sqrt(D)
    got = oracle.sdpa(u16(q), "bf16", kc, ks, vc, vs, lens, scale, signs=s, rot_norm=c, v_signs=sv,
                      rot_kind="srft")
    kd = oracle.dequantize(kc, ks)
    vd = oracle.dequantize(vc, vs)
    qn = q.double().numpy()
    if rot:
        qn = _numpy_srft(qn, s) * (float(c) * math.sqrt(N))
        Z = np.empty(vd.shape[:-1] + (N,), complex)
        Z[..., _frequency_at(N)] = vd[..., 0::2] + 1j * vd[..., 1::2]
        z = np.fft.ifft(Z, axis=-1) * N * float(c)
        vb = np.empty(vd.shape)
        vb[..., 0::2], vb[..., 1::2] = z.real, z.imag
        vd = vb * sv.astype(np.float64)
    G = Hq // Hkv
    for b in range(B):
        n = int(lens[b])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qn[b:b + 1]).unsqueeze(2),
            torch.from_numpy(kd[b:b + 1, :, :n]).repeat_interleave(G, 1),
            torch.from_numpy(vd[b:b + 1, :, :n]).repeat_interleave(G, 1), scale=scale).squeeze(2)
        assert np.allclose(got[b], ref.numpy()[0], rtol=0, atol=1e-10)
