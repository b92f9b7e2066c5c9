"""numpy front end of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the bench's
CPU-baseline leg may import this module; the product library never does.

Arrays are plain numpy arrays in the *plain* cache layout:
codes uint8 [..., T, D/2] (element 2j in the low nibble of byte j) and
scales float32 [..., T, D/32].  16-bit inputs are passed as their raw bit
patterns (uint16) together with a dtype tag: "fp16" or "bf16".
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

DTYPES = {"fp16": 0, "bf16": 1}
# K rotation kinds: the sign-randomised Hadamard and Fourier transforms
ROT_KINDS = {"srht": 0, "srft": 1}


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f32.restype = ctypes.c_float
    lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f32.restype = ctypes.c_float
    lib.oracle_srht_f32.argtypes = [P, P, ctypes.c_int, ctypes.c_float]
    lib.oracle_srht_f32.restype = None
    lib.oracle_srht_f64.argtypes = [P, P, ctypes.c_int, ctypes.c_double]
    lib.oracle_srht_f64.restype = None
    lib.oracle_unrotate_f64.argtypes = [P, P, ctypes.c_int, ctypes.c_double]
    lib.oracle_unrotate_f64.restype = None
    lib.oracle_srft_f32.argtypes = [P, P, ctypes.c_int, ctypes.c_float]
    lib.oracle_srft_f32.restype = None
    lib.oracle_srft_f64.argtypes = [P, P, ctypes.c_int, ctypes.c_double]
    lib.oracle_srft_f64.restype = None
    lib.oracle_unsrft_f64.argtypes = [P, P, ctypes.c_int, ctypes.c_double]
    lib.oracle_unsrft_f64.restype = None
    lib.oracle_twiddle_f32.argtypes = [ctypes.c_int, ctypes.c_int, P, P]
    lib.oracle_twiddle_f32.restype = None
    lib.oracle_quantize_vector.argtypes = [P, ctypes.c_int, P, P]
    lib.oracle_quantize_vector.restype = None
    lib.oracle_quantize_vector_bits.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P]
    lib.oracle_quantize_vector_bits.restype = None
    lib.oracle_quantize_rows.argtypes = [P, ctypes.c_int, ctypes.c_long, ctypes.c_int,
                                         P, ctypes.c_float, ctypes.c_int, P, ctypes.c_int, P, P,
                                         ctypes.c_int]
    lib.oracle_quantize_rows.restype = ctypes.c_int
    lib.oracle_attend_row.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P, P, P,
                                      ctypes.c_long, ctypes.c_double, P, ctypes.c_float,
                                      ctypes.c_int, P, P, ctypes.c_int, P, P]
    lib.oracle_attend_row.restype = None
    lib.oracle_sdpa.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                ctypes.c_int, ctypes.c_long, P, P, P, P, P,
                                ctypes.c_double, P, ctypes.c_float, ctypes.c_int, P, P,
                                ctypes.c_int, P, ctypes.c_long, P, ctypes.c_int]
    lib.oracle_sdpa.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def f16_to_f32(bits):
    lib = _load()
    return np.array([lib.oracle_f16_to_f32(int(b)) for b in np.ravel(bits)],
                    dtype=np.float32).reshape(np.shape(bits))


def bf16_to_f32(bits):
    lib = _load()
    return np.array([lib.oracle_bf16_to_f32(int(b)) for b in np.ravel(bits)],
                    dtype=np.float32).reshape(np.shape(bits))


def srht_f32(x, signs, rot_norm):
    """fp32 sign-randomised Walsh-Hadamard rotation of one vector."""
    lib = _load()
    y = _c(x, np.float32).copy()
    s = _c(signs, np.float32)
    lib.oracle_srht_f32(_ptr(y), _ptr(s), y.shape[-1], float(np.float32(rot_norm)))
    return y


def srht_f64(x, signs, c):
    lib = _load()
    y = _c(x, np.float64).copy()
    s = _c(signs, np.float32)
    lib.oracle_srht_f64(_ptr(y), _ptr(s), y.shape[-1], float(c))
    return y


def srft_f32(x, signs, rot_norm):
    """fp32 sign-randomised FFT rotation of one vector (in-place radix-2
    decimation-in-frequency order over the (even, odd) complex pairs)."""
    lib = _load()
    y = _c(x, np.float32).copy()
    s = _c(signs, np.float32)
    lib.oracle_srft_f32(_ptr(y), _ptr(s), y.shape[-1], float(np.float32(rot_norm)))
    return y


def srft_f64(x, signs, c):
    lib = _load()
    y = _c(x, np.float64).copy()
    s = _c(signs, np.float32)
    lib.oracle_srft_f64(_ptr(y), _ptr(s), y.shape[-1], float(c))
    return y


def unsrft_f64(y, signs, c):
    """The inverse of srft_f64: s (.) (c U y), U the stages undone in reverse."""
    lib = _load()
    y = _c(y, np.float64).copy()
    s = _c(signs, np.float32)
    lib.oracle_unsrft_f64(_ptr(y), _ptr(s), y.shape[-1], float(c))
    return y


def twiddle_f32(t, N):
    """The fp32 twiddle (cos, -sin) of 2 pi t / N the fp32 SRFT uses."""
    lib = _load()
    wr, wi = ctypes.c_float(), ctypes.c_float()
    lib.oracle_twiddle_f32(int(t), int(N), ctypes.byref(wr), ctypes.byref(wi))
    return np.float32(wr.value), np.float32(wi.value)


def _kind(rot_kind):
    return ROT_KINDS[rot_kind] if isinstance(rot_kind, str) else int(rot_kind)


def unrotate_f64(y, signs, c):
    """The inverse rotation s (.) (c H y) in fp64."""
    lib = _load()
    y = _c(y, np.float64).copy()
    s = _c(signs, np.float32)
    lib.oracle_unrotate_f64(_ptr(y), _ptr(s), y.shape[-1], float(c))
    return y


def quantize_vector(x):
    """One fp32 vector -> (codes uint8[D/2], scales float32[D/32])."""
    lib = _load()
    x = _c(x, np.float32)
    D = x.shape[-1]
    codes = np.zeros(D // 2, np.uint8)
    scales = np.zeros(D // 32, np.float32)
    lib.oracle_quantize_vector(_ptr(x), D, _ptr(codes), _ptr(scales))
    return codes, scales


def quantize_vector_bits(x, nbits):
    """One fp32 vector -> (b-bit codes uint8[D b / 8], scales float32[D/32])."""
    lib = _load()
    x = _c(x, np.float32)
    D = x.shape[-1]
    codes = np.zeros(D * nbits // 8, np.uint8)
    scales = np.zeros(D // 32, np.float32)
    lib.oracle_quantize_vector_bits(_ptr(x), D, int(nbits), _ptr(codes), _ptr(scales))
    return codes, scales


def quantize(bits, dtype, signs=None, rot_norm=0.0, threads=1, chan_scale=None, rot_kind="srht",
             code_bits=4):
    """[..., D] 16-bit rows -> codes [..., D code_bits / 8], scales [..., D/32].

    rot_kind: "srht" or "srft", the rotation applied when signs is given;
    chan_scale: per-channel scale lambda [D] applied after the rotation
    (the cache then holds lambda (.) y), or None; code_bits: 4, 3 or 2."""
    lib = _load()
    bits = _c(bits, np.uint16)
    D = bits.shape[-1]
    N = bits.size // D
    codes = np.zeros(bits.shape[:-1] + (D * code_bits // 8,), np.uint8)
    scales = np.zeros(bits.shape[:-1] + (D // 32,), np.float32)
    s = None if signs is None else _c(signs, np.float32)
    lam = None if chan_scale is None else _c(chan_scale, np.float32)
    rc = lib.oracle_quantize_rows(_ptr(bits), DTYPES[dtype], N, D, _ptr(s),
                                  float(np.float32(rot_norm)), _kind(rot_kind), _ptr(lam), int(code_bits),
                                  _ptr(codes), _ptr(scales), int(threads))
    if rc != 0:
        raise ValueError("oracle_quantize_rows rejected its arguments")
    return codes, scales


def attend_row(q_bits, dtype, kc, ks, vc, vs, T, scale, signs=None, rot_norm=0.0, chan_scale=None,
               v_signs=None, rot_kind="srht", code_bits=4):
    lib = _load()
    q_bits = _c(q_bits, np.uint16)
    D = q_bits.shape[-1]
    kc, vc = _c(kc, np.uint8), _c(vc, np.uint8)
    ks, vs = _c(ks, np.float32), _c(vs, np.float32)
    s = None if signs is None else _c(signs, np.float32)
    lam = None if chan_scale is None else _c(chan_scale, np.float32)
    vsg = None if v_signs is None else _c(v_signs, np.float32)
    work = np.zeros(max(int(T), 1), np.float64)
    out = np.zeros(D, np.float64)
    lib.oracle_attend_row(_ptr(q_bits), DTYPES[dtype], D, _ptr(kc), _ptr(ks), _ptr(vc),
                          _ptr(vs), int(T), float(scale), _ptr(s),
                          float(np.float32(rot_norm)), _kind(rot_kind), _ptr(lam), _ptr(vsg),
                          int(code_bits), _ptr(work), _ptr(out))
    return out


def sdpa(q_bits, dtype, k_codes, k_scales, v_codes, v_scales, lens, scale,
         signs=None, rot_norm=0.0, rows=None, threads=1, chan_scale=None, v_signs=None,
         rot_kind="srht", code_bits=4):
    """Decode attention over a plain-layout cache.

    q_bits [B, Hq, D] uint16; k/v codes [B, Hkv, cap, D code_bits / 8]; scales
    [B, Hkv, cap, D/32]; lens [B]; rot_kind: "srht" or "srft", the kind of
    K's rotation (signs) and of V's (v_signs); chan_scale: the K cache's per-channel
    scale lambda [D] or None; v_signs: the signs V was rotated with (same
    rot_norm as K) or None.  Returns float64 [B, Hq, D], or [len(rows), D]
    for the listed rows (row = b * Hq + h).
    """
    lib = _load()
    q_bits = _c(q_bits, np.uint16)
    B, Hq, D = q_bits.shape
    kc, vc = _c(k_codes, np.uint8), _c(v_codes, np.uint8)
    ks, vs = _c(k_scales, np.float32), _c(v_scales, np.float32)
    Hkv, cap = kc.shape[1], kc.shape[2]
    lens = _c(lens, np.int32)
    s = None if signs is None else _c(signs, np.float32)
    lam = None if chan_scale is None else _c(chan_scale, np.float32)
    vsg = None if v_signs is None else _c(v_signs, np.float32)
    if rows is None:
        out = np.zeros((B, Hq, D), np.float64)
        r = None
        nrows = 0
    else:
        r = _c(rows, np.int32)
        nrows = r.size
        out = np.zeros((nrows, D), np.float64)
    rc = lib.oracle_sdpa(_ptr(q_bits), DTYPES[dtype], B, Hq, Hkv, D, cap, _ptr(kc), _ptr(ks),
                         _ptr(vc), _ptr(vs), _ptr(lens), float(scale), _ptr(s),
                         float(np.float32(rot_norm)), _kind(rot_kind), _ptr(lam), _ptr(vsg),
                         int(code_bits), _ptr(r), nrows,
                         _ptr(out), int(threads))
    if rc != 0:
        raise ValueError("oracle_sdpa rejected its arguments")
    return out


def dequantize(codes, scales, code_bits=4):
    """Exact fp64 dequantisation code * scale of a plain-layout array."""
    codes = np.asarray(codes, np.uint8)
    # element i at bits [b i, b i + b) of the row's little-endian bit stream
    bitstream = np.unpackbits(codes, axis=-1, bitorder="little")
    n = bitstream.shape[-1] // code_bits
    b = bitstream.reshape(codes.shape[:-1] + (n, code_bits)).astype(np.int16)
    u = (b << np.arange(code_bits, dtype=np.int16)).sum(axis=-1)
    c = np.where(u >= (1 << (code_bits - 1)), u - (1 << code_bits), u).astype(np.float64)
    s = np.repeat(np.asarray(scales, np.float64), 32, axis=-1)
    return c * s
