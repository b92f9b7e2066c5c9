"""Pins for the oracle's 2- and 3-bit codes (the same group quantiser with
the symmetric range of b bits, s = abs-max / (2^(b-1) - 1), element i at
bits [b i, b i + b) of a row's little-endian bit stream).  Checked against
the int4 path at b = 4, hand-packed bytes, numpy's rint on tiny inputs, the
quantiser's invariants, and torch's fp64 attention."""
import math

import numpy as np
import pytest
import torch

import oracle


def _unpack(codes, D, b):
    """Test-side unpacker: one element at a time from its bit offsets."""
    out = np.zeros(D, np.int64)
    for i in range(D):
        u = 0
        for k in range(b):
            pos = i * b + k
            u |= ((int(codes[pos // 8]) >> (pos % 8)) & 1) << k
        out[i] = u - (1 << b) if u >= (1 << (b - 1)) else u
    return out


@pytest.mark.parametrize("D", [64, 128])
def test_four_bits_is_the_int4_path(D):
    rng = np.random.default_rng(D)
    for _ in range(20):
        x = (rng.standard_normal(D) * rng.choice([1e-3, 1.0, 300.0])).astype(np.float32)
        c4, s4 = oracle.quantize_vector(x)
        cb, sb = oracle.quantize_vector_bits(x, 4)
        assert np.array_equal(c4, cb) and np.array_equal(s4.view(np.uint32), sb.view(np.uint32))


def test_hand_packed_bytes():
    # three bits: abs-max 3 gives s = 1, so the codes are the inputs
    x = np.zeros(32, np.float32)
    x[:8] = [1, -1, 2, 3, 0, -3, -2, -1]
    c, s = oracle.quantize_vector_bits(x, 3)
    assert s[0] == 1.0
    assert list(c[:3]) == [0xB9, 0x86, 0xFA] and not np.any(c[3:])
    # two bits: abs-max 1 gives s = 1
    x = np.zeros(32, np.float32)
    x[:8] = [1, -1, 0, 1, -1, -1, 0, 0]
    c, s = oracle.quantize_vector_bits(x, 2)
    assert s[0] == 1.0
    assert list(c[:2]) == [0x4D, 0x0F] and not np.any(c[2:])


@pytest.mark.parametrize("b,group,want", [
    (3, [3, 2.5, -2.5, 0.5, 1.5, -3, 1.4, -0.6], [3, 2, -2, 0, 2, -3, 1, -1]),
    (2, [1, 0.5, -0.5, -1, 0.4, -0.6, 0.51, -0.49], [1, 0, 0, -1, 0, -1, 1, 0]),
])
def test_unit_scale_group_is_rint_half_even(b, group, want):
    x = np.zeros(64, np.float32)
    x[:8] = group
    c, s = oracle.quantize_vector_bits(x, b)
    assert s[0] == 1.0 and s[1] == 0.0
    got = _unpack(c, 64, b)
    assert list(got[:8]) == want and not np.any(got[8:])


@pytest.mark.parametrize("b", [2, 3])
def test_codes_brute_force_tiny(b):
    rng = np.random.default_rng(b)
    qmax = (1 << (b - 1)) - 1
    for _ in range(200):
        x = (rng.standard_normal(32) * rng.choice([1e-30, 1e-3, 1.0, 1e20])).astype(np.float32)
        c, s = oracle.quantize_vector_bits(x, b)
        sref = np.float32(np.max(np.abs(x)) / np.float32(qmax))
        assert s[0].view(np.uint32) == sref.view(np.uint32)
        want = np.clip(np.rint(x / sref), -qmax - 1, qmax).astype(np.int64) if sref != 0 else np.zeros(32)
        assert np.array_equal(_unpack(c, 32, b), want)


@pytest.mark.parametrize("b", [2, 3, 4])
def test_invariants(b):
    rng = np.random.default_rng(10 + b)
    qmax = (1 << (b - 1)) - 1
    D = 128
    x = rng.standard_normal((50, D)).astype(np.float32)
    x[:, 7] *= 20
    for row in x:
        c, s = oracle.quantize_vector_bits(row, b)
        codes = _unpack(c, D, b).reshape(-1, 32)
        assert np.all(np.abs(codes) <= qmax)
        assert np.all(np.max(np.abs(codes), axis=1) == qmax)
        xs = row.reshape(-1, 32).astype(np.float64)
        assert np.all(np.sign(codes) * np.sign(xs) >= 0)
        err = np.abs(xs - codes * s[:, None].astype(np.float64))
        assert np.all(err <= s[:, None] * (0.5 + 2.0 ** -20))


@pytest.mark.parametrize("b", [2, 3])
def test_sdpa_bits_matches_torch_and_bits_matter(b):
    rng = np.random.default_rng(40 + b)
    B, Hq, Hkv, D, T = 2, 4, 2, 64, 90
    k = torch.from_numpy(rng.standard_normal((B, Hkv, T, D)).astype(np.float32)).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((B, Hkv, T, D)).astype(np.float32)).to(torch.bfloat16)
    q = torch.from_numpy(rng.standard_normal((B, Hq, D)).astype(np.float32)).to(torch.bfloat16)
    u16 = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    lens = np.array([T, 41], np.int32)
    scale = 1.0 / math.sqrt(D)
    errs = {}
    ref_exact = None
    for bits in (b, 4):
        kc, ks = oracle.quantize(u16(k), "bf16", code_bits=bits)
        vc, vs = oracle.quantize(u16(v), "bf16", code_bits=bits)
        assert kc.shape == (B, Hkv, T, D * bits // 8)
        got = oracle.sdpa(u16(q), "bf16", kc, ks, vc, vs, lens, scale, code_bits=bits)
        kd = np.zeros((B, Hkv, T, D))
        vd = np.zeros((B, Hkv, T, D))
        for bb in range(B):
            for h in range(Hkv):
                for t in range(T):
                    kd[bb, h, t] = _unpack(kc[bb, h, t], D, bits) * np.repeat(ks[bb, h, t], 32)
                    vd[bb, h, t] = _unpack(vc[bb, h, t], D, bits) * np.repeat(vs[bb, h, t], 32)
        assert np.allclose(oracle.dequantize(kc, ks, code_bits=bits), kd, rtol=0, atol=0)
        G = Hq // Hkv
        for bb in range(B):
            n = int(lens[bb])
            ref = torch.nn.functional.scaled_dot_product_attention(
                q[bb:bb + 1].double().unsqueeze(2),
                torch.from_numpy(kd[bb:bb + 1, :, :n]).repeat_interleave(G, 1),
                torch.from_numpy(vd[bb:bb + 1, :, :n]).repeat_interleave(G, 1), scale=scale).squeeze(2)
            assert np.allclose(got[bb], ref[0].numpy(), rtol=0, atol=1e-10)
        if ref_exact is None:
            G = Hq // Hkv
            ref_exact = [torch.nn.functional.scaled_dot_product_attention(
                q[bb:bb + 1].double().unsqueeze(2),
                k[bb:bb + 1, :, :int(lens[bb])].double().repeat_interleave(G, 1),
                v[bb:bb + 1, :, :int(lens[bb])].double().repeat_interleave(G, 1),
                scale=scale).squeeze(2)[0].numpy() for bb in range(B)]
        errs[bits] = max(float(np.linalg.norm(got[bb] - ref_exact[bb]) / np.linalg.norm(ref_exact[bb]))
                         for bb in range(B))
    assert errs[b] > 1.5 * errs[4]   # fewer bits, larger error against unquantised K and V
