"""CPU tests of libotq's C ABI: it loads, exports every declared symbol, and
rejects bad arguments on the host (no GPU is touched by these calls)."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import int4_kv_cache_quant_amd as otq
from int4_kv_cache_quant_amd import layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "otq.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")

FAKE = 0x10000  # never dereferenced: every call below fails host validation first


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(otq_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = otq.lib()
    names = _declared_functions()
    assert set(names) == set(otq.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.otq_abi_version() == 8


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5):
        assert otq.status_str(s).startswith("OTQ_")
    assert "unknown" in otq.status_str(7)


def _desc(B=1, H=2, D=128, cap=64, signs=None):
    return otq.otq_cache(B, H, D, cap, FAKE, FAKE, FAKE, FAKE, signs, 0.0883883)


def test_cache_bytes_closed_form_llama70b_128k():
    g = json.load(open(os.path.join(GOLDEN, "storage_closed_forms.json")))["llama31_70b_128k"]
    per_layer = otq.otq_cache_bytes(1, g["kv_heads"], g["head_dim"], g["tokens"], 4)
    assert per_layer * g["layers"] == g["int4_bytes"]
    fp16 = g["layers"] * g["kv_heads"] * g["head_dim"] * g["tokens"] * 2 * 2
    assert fp16 / (per_layer * g["layers"]) == g["ratio"]
    cb, sb = otq.otq_cache_array_bytes(1, 8, 128, 131072)
    assert 2 * cb == 134217728 and 2 * sb == 33554432   # K + V codes, K + V scales


def test_cache_bytes_rejects_bad_dims():
    lib = otq.lib()
    c, s = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.otq_cache_array_bytes(1, 1, 96, 64, 4, ctypes.byref(c), ctypes.byref(s)) == otq.OTQ_EUNSUPPORTED
    assert lib.otq_cache_array_bytes(1, 1, 128, 48, 4, ctypes.byref(c), ctypes.byref(s)) == otq.OTQ_EINVAL
    assert lib.otq_cache_array_bytes(0, 1, 128, 64, 4, ctypes.byref(c), ctypes.byref(s)) == otq.OTQ_EINVAL
    for bits in (1, 5, 8, -4):
        assert lib.otq_cache_array_bytes(1, 1, 128, 64, bits, ctypes.byref(c), ctypes.byref(s)) == otq.OTQ_EINVAL
        assert lib.otq_cache_bytes(1, 1, 128, 64, bits) == 0
    assert lib.otq_cache_bytes(1, 1, 100, 64, 4) == 0


@pytest.mark.parametrize("bits", [0, 2, 3, 4])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_cache_bytes_by_code_width(bits, D):
    """Codes take D * b / 8 bytes per token and head (b = 4 for code_bits 0),
    scales D / 32 fp32 words whatever the width."""
    B, H, cap = 3, 5, 96
    cb, sb = otq.otq_cache_array_bytes(B, H, D, cap, bits)
    b = bits or 4
    assert cb == B * H * cap * D * b // 8
    assert sb == B * H * cap * (D // 32) * 4
    assert otq.otq_cache_bytes(B, H, D, cap, bits) == 2 * (cb + sb)


def test_query_and_output_alignment():
    """q is read and out written 16 bytes at a time: a misaligned pointer is
    rejected on the host by every attention entry point."""
    lib = otq.lib()
    d = _desc(B=2, H=2, D=128, cap=256)
    p = otq.otq_sdpa_plan(4, d, 256)
    P = ctypes.c_void_p
    wsb = p.workspace_bytes
    for off_q, off_o in ((8, 0), (2, 0), (0, 4), (0, 8)):
        q, o = FAKE + off_q, FAKE + off_o
        assert lib.otq_sdpa_int4_decode(P(q), 1, 4, ctypes.byref(d), P(FAKE), 256, 0.1, P(o), P(4096), wsb,
                                        None) == otq.OTQ_EINVAL
        assert lib.otq_sdpa_int4_decode_planned(P(q), 1, 4, ctypes.byref(d), P(FAKE), 256, 0.1, P(o), P(4096),
                                                wsb, ctypes.byref(p), None) == otq.OTQ_EINVAL
        assert lib.otq_sdpa_int4_decode_append(P(q), P(FAKE), P(FAKE), 1, 4, ctypes.byref(d), P(FAKE), 256,
                                               0.1, P(o), P(4096), wsb, ctypes.byref(p), None) == otq.OTQ_EINVAL
        if off_q:
            assert lib.otq_sdpa_int4_split(P(q), 1, 4, ctypes.byref(d), P(FAKE), 256, 0.1, P(4096), wsb,
                                           ctypes.byref(p), None) == otq.OTQ_EINVAL
        if off_o:
            assert lib.otq_sdpa_lse_combine(4, ctypes.byref(d), P(FAKE), 256, P(4096), wsb, ctypes.byref(p),
                                            P(o), None) == otq.OTQ_EINVAL


def test_last_device_error_rejects_null_flags():
    assert otq.lib().otq_last_device_error(None, None) == otq.OTQ_EINVAL


def test_quantize_append_host_errors():
    lib = otq.lib()
    d = _desc()
    P = ctypes.c_void_p
    call = lambda k, v, dt, n, desc, pos: lib.otq_quantize_append(P(k), P(v), dt, n, ctypes.byref(desc), P(pos), None)
    assert call(0, FAKE, 1, 1, d, FAKE) == otq.OTQ_EINVAL
    assert call(FAKE, FAKE, 1, 1, d, 0) == otq.OTQ_EINVAL
    assert call(FAKE, FAKE, 1, 0, d, FAKE) == otq.OTQ_EINVAL
    assert call(FAKE + 2, FAKE, 1, 1, d, FAKE) == otq.OTQ_EINVAL   # k, v read 16 bytes at a time
    assert call(FAKE, FAKE + 8, 1, 1, d, FAKE) == otq.OTQ_EINVAL
    for field in ("k_rot_signs", "k_chan_scale", "v_rot_signs"):   # read 16 bytes at a time
        mis = _desc()
        setattr(mis, field, FAKE + 4)
        assert call(FAKE, FAKE, 1, 1, mis, FAKE) == otq.OTQ_EINVAL
        assert otq.lib().otq_sdpa_plan(16, ctypes.byref(mis), 64, 0, 0, 0, ctypes.byref(otq.otq_plan())) == otq.OTQ_EINVAL
    assert call(FAKE, FAKE, 2, 1, d, FAKE) == otq.OTQ_EUNSUPPORTED
    assert call(FAKE, FAKE, 1, 65, d, FAKE) == otq.OTQ_ECAPACITY
    assert call(FAKE, FAKE, 1, 1, _desc(D=96), FAKE) == otq.OTQ_EUNSUPPORTED
    assert call(FAKE, FAKE, 1, 1, _desc(D=160), FAKE) == otq.OTQ_EUNSUPPORTED
    assert call(FAKE, FAKE, 1, 1, _desc(cap=40), FAKE) == otq.OTQ_EINVAL
    bad = _desc()
    bad.v_scales = None
    assert call(FAKE, FAKE, 1, 1, bad, FAKE) == otq.OTQ_EINVAL
    assert lib.otq_quantize_append(P(FAKE), P(FAKE), 1, 1, None, P(FAKE), None) == otq.OTQ_EINVAL


def test_rotation_kind_host_checks():
    """The rotations' kind is read only with K or V signs, and must be SRHT or
    SRFT; either kind serves K and V."""
    lib = otq.lib()
    P = ctypes.c_void_p
    call = lambda desc: lib.otq_quantize_append(P(FAKE), P(FAKE), 1, 1, ctypes.byref(desc), P(FAKE), None)
    plan = lambda desc: lib.otq_sdpa_plan(16, ctypes.byref(desc), 64, 0, 0, 0, ctypes.byref(otq.otq_plan()))
    d = _desc()
    d.rot_kind = 7                        # ignored without signs
    assert plan(d) == otq.OTQ_OK
    for k_signs, v_signs in ((FAKE, None), (None, FAKE), (FAKE, FAKE)):
        d = _desc(signs=k_signs)
        d.v_rot_signs = v_signs
        for kind, want in ((otq.OTQ_ROT_SRHT, otq.OTQ_OK), (otq.OTQ_ROT_SRFT, otq.OTQ_OK), (2, otq.OTQ_EINVAL),
                           (-1, otq.OTQ_EINVAL)):
            d.rot_kind = kind
            assert plan(d) == want, (k_signs, v_signs, kind)
            if want != otq.OTQ_OK:
                assert call(d) == want


def test_plan_batch_order_table():
    """A batch of 2..256 sequences plans finer chunks (its split blocks take
    their items longest first) and its workspace ends with the item table,
    8 bytes per split block; one sequence, or more than 256, has no table."""
    ru = lambda x: -(-x // 256) * 256
    for B, table in ((1, False), (2, True), (32, True), (256, True), (257, False)):
        d = _desc(B=B, H=8, D=128, cap=32768)
        p = otq.otq_sdpa_plan(32, d, 32768)
        rows = B * 32 * p.num_splits
        want = ru(rows * 128 * 4) + ru(rows * 8) + (p.num_splits * 8 * B * 8 if table else 0)
        assert p.workspace_bytes == want, (B, p.workspace_bytes, want)
    # the ragged workload's shape: chunk 2048 (8x the waves of one sequence)
    assert otq.otq_sdpa_plan(32, _desc(B=32, H=8, D=128, cap=32768), 32768).chunk == 2048
    assert otq.otq_sdpa_plan(32, _desc(B=1, H=8, D=128, cap=32768), 32768).chunk == 512


def test_plan_defaults_and_errors():
    d = _desc(B=1, H=8, D=128, cap=131072)
    p = otq.otq_sdpa_plan(64, d, 131072)
    assert p.variant == otq.OTQ_VARIANT_MFMA
    assert otq.otq_sdpa_plan(16, d, 131072).variant == otq.OTQ_VARIANT_MFMA  # G = 2 too
    assert p.chunk % 128 == 0 and p.num_splits == -(-131072 // p.chunk)
    rows = 64 * p.num_splits
    assert p.workspace_bytes == -(-rows * 128 * 4 // 256) * 256 + rows * 8
    assert otq.otq_sdpa_workspace_bytes(64, d, 131072) == p.workspace_bytes
    assert otq.otq_sdpa_plan(64, d, 100, variant=otq.OTQ_VARIANT_VECTOR, check=False)[0] == otq.OTQ_EUNSUPPORTED
    assert otq.otq_sdpa_plan(8, d, 100, variant=otq.OTQ_VARIANT_MFMA).variant == otq.OTQ_VARIANT_MFMA  # G = 1
    p = otq.otq_sdpa_plan(8, d, 1000, chunk=256, variant=otq.OTQ_VARIANT_VECTOR, check=False)[1]
    assert (p.chunk, p.num_splits, p.variant) == (256, 4, otq.OTQ_VARIANT_VECTOR)
    rc = lambda *a, **k: otq.otq_sdpa_plan(*a, check=False, **k)[0]
    assert rc(60, d, 100) == otq.OTQ_EINVAL              # Hq % Hkv
    assert rc(8 * 17, d, 100) == otq.OTQ_EUNSUPPORTED    # G > 16
    assert rc(16, d, 131073) == otq.OTQ_ECAPACITY
    assert rc(16, d, 0) == otq.OTQ_EINVAL
    assert rc(16, d, 100, chunk=100) == otq.OTQ_EINVAL
    assert rc(16, d, 100, variant=7) == otq.OTQ_EINVAL
    assert otq.otq_sdpa_workspace_bytes(60, d, 100) == 0


def test_decode_host_errors():
    lib = otq.lib()
    d = _desc(B=2, H=2, D=128, cap=256)
    p = otq.otq_sdpa_plan(4, d, 256)
    P = ctypes.c_void_p

    def call(q=FAKE, dt=1, Hq=4, desc=d, lens=FAKE, max_len=256, scale=0.1, out=FAKE, ws=4096,
             wsb=None):
        wsb = p.workspace_bytes if wsb is None else wsb
        return lib.otq_sdpa_int4_decode(P(q), dt, Hq, ctypes.byref(desc), P(lens), max_len, scale,
                                        P(out), P(ws), wsb, None)
    assert call(q=0) == otq.OTQ_EINVAL
    assert call(lens=0) == otq.OTQ_EINVAL
    assert call(out=0) == otq.OTQ_EINVAL
    assert call(dt=3) == otq.OTQ_EUNSUPPORTED
    assert call(max_len=257) == otq.OTQ_ECAPACITY
    assert call(Hq=3) == otq.OTQ_EINVAL
    assert call(scale=float("nan")) == otq.OTQ_EINVAL
    assert call(ws=0) == otq.OTQ_EWORKSPACE
    assert call(wsb=p.workspace_bytes - 1) == otq.OTQ_EWORKSPACE
    assert call(ws=4096 + 4) == otq.OTQ_EWORKSPACE       # workspace must be 256-byte aligned
    assert lib.otq_sdpa_int4_decode_planned(P(FAKE), 1, 4, ctypes.byref(d), P(FAKE), 256, 0.1,
                                            P(FAKE), P(4096), p.workspace_bytes, None, None) == otq.OTQ_EINVAL
    sp = lambda q=FAKE, lens=FAKE, ws=4096, wsb=p.workspace_bytes, plan=p, scale=0.1: lib.otq_sdpa_int4_split(
        P(q), 1, 4, ctypes.byref(d), P(lens), 256, scale, P(ws), wsb,
        None if plan is None else ctypes.byref(plan), None)
    assert sp(q=0) == otq.OTQ_EINVAL and sp(lens=0) == otq.OTQ_EINVAL and sp(plan=None) == otq.OTQ_EINVAL
    assert sp(wsb=16) == otq.OTQ_EWORKSPACE and sp(scale=float("inf")) == otq.OTQ_EINVAL
    cb = lambda out=FAKE, lens=FAKE, ws=4096, wsb=p.workspace_bytes: lib.otq_sdpa_lse_combine(
        4, ctypes.byref(d), P(lens), 256, P(ws), wsb, ctypes.byref(p), P(out), None)
    assert cb(out=0) == otq.OTQ_EINVAL and cb(lens=0) == otq.OTQ_EINVAL and cb(ws=0) == otq.OTQ_EWORKSPACE
    fa = lambda q=FAKE, kn=FAKE, vn=FAKE, lens=FAKE, out=FAKE, ws=4096, wsb=p.workspace_bytes, plan=p, dt=1: \
        lib.otq_sdpa_int4_decode_append(P(q), P(kn), P(vn), dt, 4, ctypes.byref(d), P(lens), 256, 0.1,
                                        P(out), P(ws), wsb, None if plan is None else ctypes.byref(plan), None)
    assert fa(q=0) == otq.OTQ_EINVAL and fa(kn=0) == otq.OTQ_EINVAL and fa(vn=0) == otq.OTQ_EINVAL
    assert fa(lens=0) == otq.OTQ_EINVAL and fa(out=0) == otq.OTQ_EINVAL and fa(dt=2) == otq.OTQ_EUNSUPPORTED
    assert fa(ws=0) == otq.OTQ_EWORKSPACE and fa(wsb=16) == otq.OTQ_EWORKSPACE
    assert fa(plan=otq.otq_plan(100, 3, 1, 0, 0)) == otq.OTQ_EINVAL   # chunk not a multiple of 128
    bad = otq.otq_plan(100, 3, 1, 0, 0)            # chunk not a multiple of 128
    assert lib.otq_sdpa_lse_combine(4, ctypes.byref(d), P(FAKE), 256, P(4096), 1 << 20,
                                    ctypes.byref(bad), P(FAKE), None) == otq.OTQ_EINVAL


@pytest.mark.parametrize("D", [64, 128, 256])
def test_v_layout_roundtrip_and_fixed_points(D):
    rng = np.random.default_rng(0)
    plain = rng.integers(0, 256, (2, 3, 64, D // 2), dtype=np.uint8)
    tiled = layout.v_plain_to_tiled(plain, D)
    assert tiled.shape == (2, 3, 2, 16 * D)
    assert np.array_equal(layout.v_tiled_to_plain(tiled, D), plain)
    # hand-worked positions: token u=0, channel 0 -> word 0 byte 0 low nibble;
    # u=1 -> same byte, high nibble; u=16 (slot 4) -> byte 2; u=4 (quarter 1)
    # -> word (1*16 + 0)*4 = 64; channel 17 (cb 1, n 1) -> word 1*4 + 1 = 5.
    p = np.zeros((32, D // 2), np.uint8)
    p[0, 0] = 0x03          # token 0: ch0 = 3, ch1 = 0
    p[1, 0] = 0x05          # token 1: ch0 = 5
    p[16, 0] = 0x07         # token 16: ch0 = 7
    p[4, 0] = 0x01          # token 4: ch0 = 1
    p[0, 8] = 0x20          # token 0: ch17 = 2
    t = layout.v_plain_to_tiled(p, D)[0]
    assert t[0] == 0x53 and t[2] == 0x07 and t[64 * 4] == 0x01 and t[5 * 4] == 0x02
    assert np.count_nonzero(t) == 4


@pytest.mark.parametrize("D", [64, 128, 256])
def test_k_row_layout_roundtrip_and_fixed_points(D):
    rng = np.random.default_rng(1)
    plain = rng.integers(0, 256, (3, 5, D // 2), dtype=np.uint8)
    rows = layout.k_plain_to_rows(plain, D)
    assert np.array_equal(layout.k_rows_to_plain(rows, D), plain)
    NG = D // 32
    # hand-worked: channel 8 (group 0, quarter 1, k 0) -> word NG -> byte 4*NG;
    # channel 33 (group 1, quarter 0, k 1) -> word 1, byte 4, high nibble.
    p = np.zeros((1, D // 2), np.uint8)
    p[0, 4] = 0x05            # channel 8 = 5
    p[0, 16] = 0x30           # channel 33 = 3
    r = layout.k_plain_to_rows(p, D)[0]
    assert r[4 * NG] == 0x05 and r[4] == 0x30 and np.count_nonzero(r) == 2


def test_code_bits_host_checks():
    """code_bits 0 or 4 is int4, 2 and 3 the b-bit path (vector split pass, no
    fused append; rotations and the channel scale allowed); other values are
    invalid."""
    lib = otq.lib()
    P = ctypes.c_void_p
    plan = lambda desc, variant=0: lib.otq_sdpa_plan(16, ctypes.byref(desc), 64, 0, variant, 0,
                                                     ctypes.byref(otq.otq_plan()))
    for bits, want in ((0, otq.OTQ_OK), (4, otq.OTQ_OK), (2, otq.OTQ_OK), (3, otq.OTQ_OK),
                       (1, otq.OTQ_EINVAL), (5, otq.OTQ_EINVAL), (-3, otq.OTQ_EINVAL)):
        d = _desc()
        d.code_bits = bits
        assert plan(d) == want, bits
    d = _desc()
    d.code_bits = 3
    p = otq.otq_plan()
    assert lib.otq_sdpa_plan(16, ctypes.byref(d), 64, 0, 0, 0, ctypes.byref(p)) == otq.OTQ_OK
    assert p.variant == otq.OTQ_VARIANT_MFMA
    assert plan(d, otq.OTQ_VARIANT_MFMA) == otq.OTQ_OK
    assert plan(d, otq.OTQ_VARIANT_VECTOR) == otq.OTQ_OK
    for field in ("k_rot_signs", "v_rot_signs", "k_chan_scale"):
        e = _desc()
        e.code_bits = 2
        setattr(e, field, FAKE)
        assert plan(e) == otq.OTQ_OK, field
    # the fused step takes b-bit caches too; here it stops at the host checks
    # (an input dtype it does not read), before any launch
    ws = lib.otq_sdpa_workspace_bytes(16, ctypes.byref(d), 64)
    rc = lib.otq_sdpa_int4_decode_append(P(FAKE), P(FAKE), P(FAKE), 7, 16, ctypes.byref(d), P(FAKE), 64,
                                         ctypes.c_float(0.1), P(FAKE), P(FAKE), ctypes.c_size_t(ws), None,
                                         None)
    assert rc == otq.OTQ_EUNSUPPORTED
    rc = lib.otq_sdpa_int4_decode_append(P(FAKE + 8), P(FAKE), P(FAKE), 1, 16, ctypes.byref(d), P(FAKE), 64,
                                         ctypes.c_float(0.1), P(FAKE), P(FAKE), ctypes.c_size_t(ws), None,
                                         None)
    assert rc == otq.OTQ_EINVAL  # q not 16-byte aligned



def test_noalloc_scratch_limit_on_host():
    """The scratch-array decode step refuses, before any HIP call, a plan
    whose workspace exceeds OTQ_NOALLOC_SCRATCH_BYTES, and validates its
    arguments like the workspace call."""
    lib = otq.lib()
    P = ctypes.c_void_p
    d = _desc(B=64, H=8, D=128, cap=8192)
    p = otq.otq_sdpa_plan(64, d, 8192, chunk=128)
    assert p.workspace_bytes > otq.OTQ_NOALLOC_SCRATCH_BYTES
    call = lambda q=FAKE, plan=p: lib.otq_sdpa_int4_decode_append_noalloc(
        P(q), P(FAKE), P(FAKE), 1, 64, ctypes.byref(d), P(FAKE), 8192, 0.1, P(FAKE),
        None if plan is None else ctypes.byref(plan), None)
    assert call() == otq.OTQ_EWORKSPACE
    bad = otq.otq_plan(100, 3, otq.OTQ_VARIANT_MFMA, 0, 0)  # chunk not a multiple of 128
    assert call(plan=bad) == otq.OTQ_EINVAL
    small = _desc(B=1, H=2, D=128, cap=256)
    ps = otq.otq_sdpa_plan(4, small, 256)
    assert lib.otq_sdpa_int4_decode_append_noalloc(P(0), P(FAKE), P(FAKE), 1, 4, ctypes.byref(small), P(FAKE),
                                                   256, 0.1, P(FAKE), ctypes.byref(ps), None) == otq.OTQ_EINVAL


def test_head_dim_192_host_checks():
    """head_dim 192 (D/2 = 3 * 32): int4 only, K rotated by the FFT kind only
    (the Hadamard form needs a power of two), V unrotated; the matrix-core
    split pass by default, the vector one when asked for; the decode step
    passes the host checks; sizes by the int4 closed form."""
    lib = otq.lib()
    P = ctypes.c_void_p
    cb, sb = otq.otq_cache_array_bytes(2, 3, 192, 64, 4)
    assert cb == 2 * 3 * 64 * 96 and sb == 2 * 3 * 64 * 6 * 4
    assert lib.otq_cache_bytes(1, 1, 192, 64, 2) == 0   # no b-bit codes at this width
    plan = lambda desc, variant=0: otq.otq_sdpa_plan(8, desc, 64, variant=variant, check=False)
    d = _desc(D=192)
    rc, p = plan(d)
    assert rc == otq.OTQ_OK and p.variant == otq.OTQ_VARIANT_MFMA
    rc, p = plan(d, otq.OTQ_VARIANT_VECTOR)
    assert rc == otq.OTQ_OK and p.variant == otq.OTQ_VARIANT_VECTOR
    sc = _desc(D=192)
    sc.k_chan_scale = FAKE
    rc, p = plan(sc)
    assert rc == otq.OTQ_OK and p.variant == otq.OTQ_VARIANT_MFMA
    r = _desc(D=192, signs=FAKE)
    r.rot_kind = otq.OTQ_ROT_SRFT
    rc, p = plan(r)
    assert rc == otq.OTQ_OK and p.variant == otq.OTQ_VARIANT_MFMA
    rc, p = plan(r, otq.OTQ_VARIANT_VECTOR)
    assert rc == otq.OTQ_OK and p.variant == otq.OTQ_VARIANT_VECTOR
    rc, p = otq.otq_sdpa_plan(32, d, 64, variant=otq.OTQ_VARIANT_MFMA, check=False)  # G = 16
    assert rc == otq.OTQ_OK and p.variant == otq.OTQ_VARIANT_MFMA
    r.rot_kind = otq.OTQ_ROT_SRHT
    assert plan(r)[0] == otq.OTQ_EUNSUPPORTED
    vr = _desc(D=192)
    vr.v_rot_signs = FAKE
    vr.rot_kind = otq.OTQ_ROT_SRFT
    assert plan(vr)[0] == otq.OTQ_EUNSUPPORTED
    b3 = _desc(D=192)
    b3.code_bits = 3
    assert plan(b3)[0] == otq.OTQ_EUNSUPPORTED
    ws = lib.otq_sdpa_workspace_bytes(8, ctypes.byref(d), 64)
    assert ws > 0
    # accepted up to the workspace check (a byte short), which comes before any HIP call
    rc = lib.otq_sdpa_int4_decode_append(P(FAKE), P(FAKE), P(FAKE), 1, 8, ctypes.byref(d), P(FAKE), 64,
                                         ctypes.c_float(0.1), P(FAKE), P(FAKE), ctypes.c_size_t(ws - 1), None, None)
    assert rc == otq.OTQ_EWORKSPACE
    for bad in (96, 160, 320):
        assert lib.otq_cache_bytes(1, 1, bad, 64, 4) == 0


def test_stream_read_probe_host_checks():
    lib = otq.lib()
    P = ctypes.c_void_p
    assert lib.otq_stream_read_probe(P(0), 1024, P(FAKE), 4, None) == otq.OTQ_EINVAL
    assert lib.otq_stream_read_probe(P(FAKE), 1000, P(FAKE), 4, None) == otq.OTQ_EINVAL
    assert lib.otq_stream_read_probe(P(FAKE + 8), 1024, P(FAKE), 4, None) == otq.OTQ_EINVAL
    assert lib.otq_stream_read_probe(P(FAKE), 1024, P(0), 4, None) == otq.OTQ_EINVAL
    assert lib.otq_stream_read_probe(P(FAKE), 1024, P(FAKE), 0, None) == otq.OTQ_EINVAL
    assert lib.otq_stream_read_probe(P(FAKE), 0, P(FAKE), 4, None) == otq.OTQ_EINVAL


def test_plan_interleaved_pieces():
    """A split count below ceil(max_len / chunk) interleaves the pieces: kept
    for the MFMA variant on one sequence with 2^k tiles per piece, replaced by
    ceil(max_len / chunk) elsewhere; the workspace follows the split count."""
    one = _desc(B=1, H=8, D=128, cap=131072)
    p = otq.otq_sdpa_plan(64, one, 131072, chunk=256, splits=32)
    assert (p.chunk, p.num_splits, p.variant) == (256, 32, otq.OTQ_VARIANT_MFMA)
    rows = 64 * 32
    assert p.workspace_bytes == -(-rows * 128 * 4 // 256) * 256 + rows * 8
    # more splits than pieces: one piece each
    assert otq.otq_sdpa_plan(64, one, 1000, chunk=256, splits=64).num_splits == 4
    # 3 tiles per piece, the vector variant, a batch: no interleaving
    assert otq.otq_sdpa_plan(64, one, 131072, chunk=384, splits=32).num_splits == -(-131072 // 384)
    pv = otq.otq_sdpa_plan(8, one, 4096, chunk=256, variant=otq.OTQ_VARIANT_VECTOR, splits=4)
    assert (pv.chunk, pv.num_splits) == (256, 16)
    batch = _desc(B=4, H=8, D=128, cap=32768)
    assert otq.otq_sdpa_plan(32, batch, 32768, chunk=256, splits=8).num_splits == 128
    # 2- and 3-bit caches take one piece per split
    b3 = _desc(B=1, H=8, D=128, cap=32768)
    b3.code_bits = 3
    assert otq.otq_sdpa_plan(32, b3, 32768, chunk=256, splits=8).num_splits == 128
    assert otq.otq_sdpa_plan(64, one, 1000, splits=-1, check=False)[0] == otq.OTQ_EINVAL
    # the default plans take one piece per split
    for desc in (one, batch):
        d = otq.otq_sdpa_plan(32 if desc is batch else 64, desc, 32768)
        assert d.num_splits == -(-32768 // d.chunk)


def test_plan_variants_of_b_bit_caches():
    """b-bit caches take the MFMA split pass by default, with a rotated or
    channel-scaled K up to D = 128 too; at D = 256 such a K takes the vector
    pass, and forcing MFMA there is OTQ_EUNSUPPORTED."""
    lib = otq.lib()
    plain2 = _desc(B=1, H=8, D=128, cap=4096)
    plain2.code_bits = 2
    assert otq.otq_sdpa_plan(64, plain2, 4096).variant == otq.OTQ_VARIANT_MFMA
    assert otq.otq_sdpa_plan(64, plain2, 4096, variant=otq.OTQ_VARIANT_VECTOR).variant == otq.OTQ_VARIANT_VECTOR
    rot2 = _desc(B=1, H=8, D=128, cap=4096, signs=FAKE)
    rot2.code_bits = 2
    assert otq.otq_sdpa_plan(64, rot2, 4096).variant == otq.OTQ_VARIANT_MFMA
    lam2 = _desc(B=1, H=8, D=128, cap=4096)
    lam2.code_bits = 2
    lam2.k_chan_scale = FAKE
    assert otq.otq_sdpa_plan(64, lam2, 4096).variant == otq.OTQ_VARIANT_MFMA
    rot256 = _desc(B=1, H=8, D=256, cap=4096, signs=FAKE)
    rot256.code_bits = 2
    assert otq.otq_sdpa_plan(64, rot256, 4096).variant == otq.OTQ_VARIANT_VECTOR
    assert otq.otq_sdpa_plan(64, rot256, 4096, variant=otq.OTQ_VARIANT_MFMA, check=False)[0] == \
        otq.OTQ_EUNSUPPORTED
    three = _desc(B=1, H=8, D=128, cap=4096)
    three.code_bits = 3
    assert otq.otq_sdpa_plan(64, three, 4096).variant == otq.OTQ_VARIANT_MFMA
    wide3 = _desc(B=1, H=8, D=256, cap=4096)
    wide3.code_bits = 3
    assert otq.otq_sdpa_plan(64, wide3, 4096).variant == otq.OTQ_VARIANT_MFMA
    wide3r = _desc(B=1, H=8, D=256, cap=4096, signs=FAKE)
    wide3r.code_bits = 3
    assert otq.otq_sdpa_plan(64, wide3r, 4096, variant=otq.OTQ_VARIANT_MFMA, check=False)[0] == otq.OTQ_EUNSUPPORTED
    # the MFMA 2-bit plan: one KV head per block, four waves per chunk round
    p = otq.otq_sdpa_plan(64, _desc(B=1, H=8, D=128, cap=131072), 131072)
    p2 = otq.otq_sdpa_plan(64, plain2, 4096)
    assert p2.chunk % 128 == 0 and p2.num_splits == -(-4096 // p2.chunk)
    assert p.variant == otq.OTQ_VARIANT_MFMA


# ---------------------------------------------------------------- b-bit V tiles
def _one_code_plain(D, bits, u, c, code):
    """Plain rows of one 32-token tile with a single non-zero field."""
    rows = np.zeros((32, D * bits), np.uint8)
    for i in range(bits):
        rows[u, c * bits + i] = (code >> i) & 1
    return np.packbits(rows, axis=-1, bitorder="little")


def _set_bits(tiled):
    bits = np.unpackbits(tiled.reshape(-1), bitorder="little")
    return [int(x) for x in np.nonzero(bits)[0]]


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("bits", [2, 3])
def test_v_bits_tile_layout_is_a_permutation(D, bits):
    """The b-bit V tile map is a bijection on a tile's bits and round-trips."""
    src = layout._vbits_map(D, bits)
    assert src.min() == 0 and np.array_equal(np.sort(src), np.arange(32 * D * bits))
    rng = np.random.default_rng(D + bits)
    plain = rng.integers(0, 256, size=(2, 3, 96, D * bits // 8), dtype=np.uint8)
    tiled = layout.v_bits_plain_to_tiled(plain, D, bits)
    assert tiled.shape == (2, 3, 3, 32 * D * bits // 8)
    assert np.array_equal(layout.v_bits_tiled_to_plain(tiled, D, bits), plain)


def test_v_bits_tile_layout_positions():
    """Field positions worked out by hand from the layout rule in otq.h."""
    # 2 bits, D = 128: token 21 (h 1, r 1, m 1), channel 37 (cb 2, n 5):
    # lane 21, word 21 * 4 + 1 = 85, bit 16 + 0 + 2 = 18; code -1 = 0b11
    t = layout.v_bits_plain_to_tiled(_one_code_plain(128, 2, 21, 37, 0b11)[None], 128, 2)
    assert _set_bits(t) == [32 * 85 + 18, 32 * 85 + 19]
    # same token, channel 53 (cb 3: the upper byte of the same word)
    t = layout.v_bits_plain_to_tiled(_one_code_plain(128, 2, 21, 53, 0b01)[None], 128, 2)
    assert _set_bits(t) == [32 * 85 + 26]
    # 3 bits, D = 64: token 6 (h 0, r 1, m 2), channel 35 (cb 2, n 3): lane 19,
    # words 19 * 3 + 0..2, cb % 4 = 2 < 3: word 59, bit 6; code 0b101
    t = layout.v_bits_plain_to_tiled(_one_code_plain(64, 3, 6, 35, 0b101)[None], 64, 3)
    assert _set_bits(t) == [32 * 59 + 6, 32 * 59 + 8]
    # channel 51 (cb 3, n 3: the top nibbles): chunk bits p = 6, 7, 8 -> word
    # 57 + 1 bits 14, 15 and word 57 + 2 bit 12; code 0b101 sets p = 6 and 8
    t = layout.v_bits_plain_to_tiled(_one_code_plain(64, 3, 6, 51, 0b101)[None], 64, 3)
    assert _set_bits(t) == [32 * 58 + 14, 32 * 59 + 12]
    # token 22 (h 1, r 1, m 2), same channel: 16 bits higher
    t = layout.v_bits_plain_to_tiled(_one_code_plain(64, 3, 22, 51, 0b111)[None], 64, 3)
    assert _set_bits(t) == [32 * 58 + 30, 32 * 58 + 31, 32 * 59 + 28]
