"""Python binding of libotq: int4 KV-cache quantisation and decode attention
on the packed cache, for AMD MI355X (gfx950).

This module only marshals arguments: every step of the path runs in the HIP
kernels of libotq.so (built in-tree by ``build.py``).  PyTorch is used for
device memory and streams.  If the library is missing, importing the native
entry points raises: there is no CPU or PyTorch fallback.

The names mirror the C ABI in include/otq.h:
``otq_quantize_append``, ``otq_sdpa_int4_decode``, ``otq_sdpa_plan``, ...
``Int4KVCache`` is a convenience owner of the four cache arrays.
"""
import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libotq.so")

OTQ_OK, OTQ_EINVAL, OTQ_ECAPACITY, OTQ_EUNSUPPORTED, OTQ_EWORKSPACE, OTQ_EDEVICE = 0, -1, -2, -3, -4, -5
OTQ_F16, OTQ_BF16 = 0, 1
OTQ_VARIANT_AUTO, OTQ_VARIANT_VECTOR, OTQ_VARIANT_MFMA = 0, 1, 2
OTQ_GROUP, OTQ_TILE = 32, 32
OTQ_ROT_SRHT, OTQ_ROT_SRFT = 0, 1
ROT_KINDS = {"srht": OTQ_ROT_SRHT, "srft": OTQ_ROT_SRFT}

OTQ_DEVERR_POS, OTQ_DEVERR_LENS = 1, 2

EXPORTED = [
    "otq_status_str", "otq_abi_version", "otq_cache_array_bytes", "otq_cache_bytes",
    "otq_last_device_error", "otq_stream_read_probe",
    "otq_quantize_append", "otq_sdpa_plan", "otq_sdpa_workspace_bytes",
    "otq_sdpa_int4_decode", "otq_sdpa_int4_decode_planned", "otq_sdpa_int4_decode_append",
    "otq_sdpa_int4_decode_append_noalloc",
    "otq_sdpa_int4_split", "otq_sdpa_lse_combine",
]


class OtqError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} ({status})")


class otq_cache(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("capacity", ctypes.c_int32),
        ("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
        ("k_rot_signs", ctypes.c_void_p), ("rot_norm", ctypes.c_float),
        ("k_chan_scale", ctypes.c_void_p), ("v_rot_signs", ctypes.c_void_p),
        ("rot_kind", ctypes.c_int32), ("code_bits", ctypes.c_int32),
    ]


class otq_plan(ctypes.Structure):
    _fields_ = [("chunk", ctypes.c_int32), ("num_splits", ctypes.c_int32),
                ("variant", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t)]


_lib = None


def lib():
    """The loaded libotq.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libotq.so not built at {LIB_PATH}: run int4_kv_cache_quant_amd/build.py "
                          "(or __graft_entry__.build()); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    P, I, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    CP = ctypes.POINTER(otq_cache)
    L.otq_status_str.argtypes = [ctypes.c_int]
    L.otq_status_str.restype = ctypes.c_char_p
    L.otq_abi_version.argtypes = []
    L.otq_abi_version.restype = ctypes.c_int
    L.otq_cache_array_bytes.argtypes = [I, I, I, I, I, ctypes.POINTER(S), ctypes.POINTER(S)]
    L.otq_cache_array_bytes.restype = ctypes.c_int
    L.otq_cache_bytes.argtypes = [I, I, I, I, I]
    L.otq_cache_bytes.restype = S
    L.otq_last_device_error.argtypes = [P, ctypes.POINTER(ctypes.c_uint32)]
    L.otq_last_device_error.restype = ctypes.c_int
    L.otq_stream_read_probe.argtypes = [P, S, P, I, P]
    L.otq_stream_read_probe.restype = ctypes.c_int
    L.otq_quantize_append.argtypes = [P, P, I, I, CP, P, P]
    L.otq_quantize_append.restype = ctypes.c_int
    L.otq_sdpa_plan.argtypes = [I, CP, I, I, I, I, ctypes.POINTER(otq_plan)]
    L.otq_sdpa_plan.restype = ctypes.c_int
    L.otq_sdpa_workspace_bytes.argtypes = [I, CP, I]
    L.otq_sdpa_workspace_bytes.restype = S
    L.otq_sdpa_int4_decode.argtypes = [P, I, I, CP, P, I, ctypes.c_float, P, P, S, P]
    L.otq_sdpa_int4_decode.restype = ctypes.c_int
    L.otq_sdpa_int4_decode_planned.argtypes = [P, I, I, CP, P, I, ctypes.c_float, P, P, S,
                                               ctypes.POINTER(otq_plan), P]
    L.otq_sdpa_int4_decode_planned.restype = ctypes.c_int
    L.otq_sdpa_int4_decode_append.argtypes = [P, P, P, I, I, CP, P, I, ctypes.c_float, P, P, S,
                                              ctypes.POINTER(otq_plan), P]
    L.otq_sdpa_int4_decode_append.restype = ctypes.c_int
    L.otq_sdpa_int4_decode_append_noalloc.argtypes = [P, P, P, I, I, CP, P, I, ctypes.c_float, P,
                                                      ctypes.POINTER(otq_plan), P]
    L.otq_sdpa_int4_decode_append_noalloc.restype = ctypes.c_int
    L.otq_sdpa_int4_split.argtypes = [P, I, I, CP, P, I, ctypes.c_float, P, S,
                                      ctypes.POINTER(otq_plan), P]
    L.otq_sdpa_int4_split.restype = ctypes.c_int
    L.otq_sdpa_lse_combine.argtypes = [I, CP, P, I, P, S, ctypes.POINTER(otq_plan), P, P]
    L.otq_sdpa_lse_combine.restype = ctypes.c_int
    _lib = L
    return L


def status_str(status):
    return lib().otq_status_str(int(status)).decode()


def _check(rc, what):
    if rc != OTQ_OK:
        raise OtqError(rc, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def dtype_code(dt):
    if dt == torch.float16:
        return OTQ_F16
    if dt == torch.bfloat16:
        return OTQ_BF16
    raise TypeError(f"unsupported dtype {dt}: fp16 or bf16 only")


# ---------------------------------------------------------------- raw ABI
def otq_cache_array_bytes(batch, num_kv_heads, head_dim, capacity, code_bits=4):
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().otq_cache_array_bytes(batch, num_kv_heads, head_dim, capacity, code_bits,
                                       ctypes.byref(cb), ctypes.byref(sb)), "otq_cache_array_bytes")
    return cb.value, sb.value


def otq_cache_bytes(batch, num_kv_heads, head_dim, capacity, code_bits=4):
    return lib().otq_cache_bytes(batch, num_kv_heads, head_dim, capacity, code_bits)


def otq_stream_read_probe(buf, sink, nbytes=None, blocks=None, stream=None):
    """Read every byte of the device tensor buf once (the streaming-read
    reference); sink: device uint32 tensor with one word per block."""
    nbytes = buf.numel() * buf.element_size() if nbytes is None else nbytes
    blocks = sink.numel() if blocks is None else blocks
    _check(lib().otq_stream_read_probe(_ptr(buf), nbytes, _ptr(sink), blocks, _stream(stream)),
           "otq_stream_read_probe")


def otq_last_device_error(stream=None):
    """Device-side contract violations (OTQ_DEVERR_* bits) recorded on the
    current device since the previous call (which this one clears)."""
    flags = ctypes.c_uint32()
    _check(lib().otq_last_device_error(_stream(stream), ctypes.byref(flags)), "otq_last_device_error")
    return flags.value


def otq_quantize_append(k, v, cache_desc, pos, n_new=None, dtype=None, stream=None, check=True):
    """k, v: device [B, Hkv, n_new, D] fp16/bf16; pos: device int32 [B]."""
    n_new = k.shape[2] if n_new is None else n_new
    dtype = dtype_code(k.dtype) if dtype is None else dtype
    rc = lib().otq_quantize_append(_ptr(k), _ptr(v), dtype, n_new, ctypes.byref(cache_desc),
                                   _ptr(pos), _stream(stream))
    if check:
        _check(rc, "otq_quantize_append")
    return rc


def otq_sdpa_plan(num_q_heads, cache_desc, max_len, chunk=0, variant=OTQ_VARIANT_AUTO, check=True, splits=0):
    p = otq_plan()
    rc = lib().otq_sdpa_plan(num_q_heads, ctypes.byref(cache_desc), max_len, chunk, variant, splits,
                             ctypes.byref(p))
    if check:
        _check(rc, "otq_sdpa_plan")
        return p
    return rc, p


def otq_sdpa_workspace_bytes(num_q_heads, cache_desc, max_len):
    return lib().otq_sdpa_workspace_bytes(num_q_heads, ctypes.byref(cache_desc), max_len)


def otq_sdpa_int4_decode(q, cache_desc, lens, max_len, scale, out, workspace, plan=None,
                         num_q_heads=None, dtype=None, workspace_bytes=None, stream=None,
                         check=True):
    """q: device [B, Hq, D]; lens: device int32 [B]; out: device fp32 [B, Hq, D]."""
    Hq = q.shape[1] if num_q_heads is None else num_q_heads
    dtype = dtype_code(q.dtype) if dtype is None else dtype
    wsb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    if plan is None:
        rc = lib().otq_sdpa_int4_decode(_ptr(q), dtype, Hq, ctypes.byref(cache_desc), _ptr(lens),
                                        max_len, float(scale), _ptr(out), _ptr(workspace), wsb,
                                        _stream(stream))
    else:
        rc = lib().otq_sdpa_int4_decode_planned(_ptr(q), dtype, Hq, ctypes.byref(cache_desc),
                                                _ptr(lens), max_len, float(scale), _ptr(out),
                                                _ptr(workspace), wsb, ctypes.byref(plan),
                                                _stream(stream))
    if check:
        _check(rc, "otq_sdpa_int4_decode")
    return rc


def otq_sdpa_int4_decode_append(q, k_new, v_new, cache_desc, lens, max_len, scale, out, workspace,
                                plan=None, num_q_heads=None, dtype=None, workspace_bytes=None,
                                stream=None, check=True):
    """One decode step: quantise k_new, v_new (device [B, Hkv, D]) into the
    cache at position lens[b] - 1 and attend over [0, lens[b])."""
    Hq = q.shape[1] if num_q_heads is None else num_q_heads
    dtype = dtype_code(q.dtype) if dtype is None else dtype
    wsb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    rc = lib().otq_sdpa_int4_decode_append(_ptr(q), _ptr(k_new), _ptr(v_new), dtype, Hq,
                                           ctypes.byref(cache_desc), _ptr(lens), max_len,
                                           float(scale), _ptr(out), _ptr(workspace), wsb,
                                           None if plan is None else ctypes.byref(plan),
                                           _stream(stream))
    if check:
        _check(rc, "otq_sdpa_int4_decode_append")
    return rc


OTQ_NOALLOC_SCRATCH_BYTES = 16 << 20


def otq_sdpa_int4_decode_append_noalloc(q, k_new, v_new, cache_desc, lens, max_len, scale, out,
                                        plan=None, num_q_heads=None, dtype=None, stream=None, check=True):
    """otq_sdpa_int4_decode_append with the library's per-device scratch
    array as the workspace (no allocation by the caller or the call)."""
    Hq = q.shape[1] if num_q_heads is None else num_q_heads
    dtype = dtype_code(q.dtype) if dtype is None else dtype
    rc = lib().otq_sdpa_int4_decode_append_noalloc(_ptr(q), _ptr(k_new), _ptr(v_new), dtype, Hq,
                                                   ctypes.byref(cache_desc), _ptr(lens), max_len,
                                                   float(scale), _ptr(out),
                                                   None if plan is None else ctypes.byref(plan),
                                                   _stream(stream))
    if check:
        _check(rc, "otq_sdpa_int4_decode_append_noalloc")
    return rc


def otq_sdpa_int4_split(q, cache_desc, lens, max_len, scale, workspace, plan, num_q_heads=None,
                        dtype=None, workspace_bytes=None, stream=None, check=True):
    """Split pass only: partials into the workspace (layout in include/otq.h)."""
    Hq = q.shape[1] if num_q_heads is None else num_q_heads
    dtype = dtype_code(q.dtype) if dtype is None else dtype
    wsb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    rc = lib().otq_sdpa_int4_split(_ptr(q), dtype, Hq, ctypes.byref(cache_desc), _ptr(lens),
                                   max_len, float(scale), _ptr(workspace), wsb,
                                   ctypes.byref(plan), _stream(stream))
    if check:
        _check(rc, "otq_sdpa_int4_split")
    return rc


def otq_sdpa_lse_combine(num_q_heads, cache_desc, lens, max_len, workspace, plan, out,
                         workspace_bytes=None, stream=None, check=True):
    """Combine pass only: merge the partials in the workspace into out."""
    wsb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    rc = lib().otq_sdpa_lse_combine(num_q_heads, ctypes.byref(cache_desc), _ptr(lens), max_len,
                                    _ptr(workspace), wsb, ctypes.byref(plan), _ptr(out),
                                    _stream(stream))
    if check:
        _check(rc, "otq_sdpa_lse_combine")
    return rc


# ---------------------------------------------------------------- owner
class Int4KVCache:
    """Owns the four device arrays of one layer's cache and its descriptor.

    ``rot_signs`` (device float32 [D] of +-1) turns on the K rotation:
    ``rot_kind`` "srht" (Walsh-Hadamard, normalisation fp32(1/sqrt(D))) or
    "srft" (FFT over the (even, odd) complex pairs, normalisation
    fp32(1/sqrt(D/2))), the kind of V's rotation too.  ``chan_scale`` (float32 [D], > 0)
    turns on K's per-channel scale, applied after the rotation.
    ``v_rot_signs`` (float32 [D] of +-1) turns on V's rotation, whose inverse
    the attention calls apply to their outputs.
    """

    def __init__(self, batch, num_kv_heads, head_dim, capacity, device="cuda", rot_signs=None,
                 chan_scale=None, v_rot_signs=None, rot_kind="srht", code_bits=4):
        # the library sizes the arrays; the tensors only give them a shape
        cb, sb = otq_cache_array_bytes(batch, num_kv_heads, head_dim, capacity, code_bits)
        self.shape = (batch, num_kv_heads, head_dim, capacity)
        self.code_bits = code_bits
        rows = batch * num_kv_heads * capacity
        self.k_scales = torch.zeros(sb // 4, dtype=torch.float32, device=device).view(
            batch, num_kv_heads, capacity, sb // 4 // rows)
        self.v_scales = torch.zeros_like(self.k_scales)
        # K in rows of one token; V in tiles of 32 tokens (int4 and b-bit alike)
        self.k_codes = torch.zeros(cb, dtype=torch.uint8, device=device).view(batch, num_kv_heads, capacity, -1)
        self.v_codes = torch.zeros(cb, dtype=torch.uint8, device=device).view(
            batch, num_kv_heads, capacity // OTQ_TILE, -1)
        self.rot_signs = None if rot_signs is None else rot_signs.to(device=device, dtype=torch.float32).contiguous()
        self.rot_kind = ROT_KINDS[rot_kind]
        n = head_dim // 2 if self.rot_kind == OTQ_ROT_SRFT else head_dim
        self.rot_norm = float(torch.tensor(1.0 / math.sqrt(n), dtype=torch.float32))
        self.chan_scale = (None if chan_scale is None
                           else chan_scale.to(device=device, dtype=torch.float32).contiguous())
        self.v_rot_signs = (None if v_rot_signs is None
                            else v_rot_signs.to(device=device, dtype=torch.float32).contiguous())
        self.desc = otq_cache(batch, num_kv_heads, head_dim, capacity,
                              self.k_codes.data_ptr(), self.k_scales.data_ptr(),
                              self.v_codes.data_ptr(), self.v_scales.data_ptr(),
                              None if self.rot_signs is None else self.rot_signs.data_ptr(),
                              self.rot_norm,
                              None if self.chan_scale is None else self.chan_scale.data_ptr(),
                              None if self.v_rot_signs is None else self.v_rot_signs.data_ptr(),
                              self.rot_kind, code_bits)

    @property
    def nbytes(self):
        return sum(t.numel() * t.element_size() for t in (self.k_codes, self.k_scales, self.v_codes, self.v_scales))

    def append(self, k, v, pos, stream=None):
        return otq_quantize_append(k, v, self.desc, pos, stream=stream)

    def plan(self, num_q_heads, max_len, chunk=0, variant=OTQ_VARIANT_AUTO, splits=0):
        return otq_sdpa_plan(num_q_heads, self.desc, max_len, chunk, variant, splits=splits)

    def workspace(self, num_q_heads, max_len, plan=None):
        n = (plan.workspace_bytes if plan is not None
             else otq_sdpa_workspace_bytes(num_q_heads, self.desc, max_len))
        if n == 0:
            raise OtqError(OTQ_EINVAL, "workspace size")
        return torch.empty(n, dtype=torch.uint8, device=self.k_codes.device)

    def decode(self, q, lens, max_len, scale, out=None, workspace=None, plan=None, stream=None):
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = self.workspace(q.shape[1], max_len, plan)
        otq_sdpa_int4_decode(q, self.desc, lens, max_len, scale, out, workspace, plan=plan, stream=stream)
        return out

    def decode_append(self, q, k_new, v_new, lens, max_len, scale, out=None, workspace=None,
                      plan=None, stream=None):
        """Append the token at lens[b] - 1 (k_new, v_new: [B, Hkv, D]) and
        attend over [0, lens[b]) in one pass."""
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = self.workspace(q.shape[1], max_len, plan)
        otq_sdpa_int4_decode_append(q, k_new, v_new, self.desc, lens, max_len, scale, out,
                                    workspace, plan=plan, stream=stream)
        return out
