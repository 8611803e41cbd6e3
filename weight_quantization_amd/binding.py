"""ctypes binding of libhlwq (declared in include/hlwq.h).

Argument marshalling only: every function below checks the torch tensors it
is given, passes their device pointers, sizes and the current HIP stream to the
C function of the same name, and raises on a non-zero status.  All compute runs
in the HIP kernels of libhlwq.so; there is no fallback of any kind.  torch is
used for device memory and streams.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhlwq.so")
HEADER_PATH = os.path.join(os.path.dirname(HERE), "include", "hlwq.h")

HLWQ_OK = 0
BLOCK = 128
KV_DIM = 256


class HLWQError(RuntimeError):
    def __init__(self, func: str, status: int, text: str):
        super().__init__(f"{func} failed: {text} (status {status})")
        self.status = status


class Int4Desc(ctypes.Structure):
    _fields_ = [
        ("packed", ctypes.c_void_p),
        ("norms", ctypes.c_void_p),
        ("q4", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("zeros", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("in_", ctypes.c_int64),
    ]


class MatDesc(ctypes.Structure):
    _fields_ = [
        ("w", ctypes.c_void_p),
        ("packed", ctypes.c_void_p),
        ("norms", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("in_", ctypes.c_int64),
    ]


_lib = None

_i64 = ctypes.c_int64
_int = ctypes.c_int
_vp = ctypes.c_void_p

_SIGNATURES = {
    "hlwq_quantize": (_int, [_vp, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp]),
    "hlwq_dequantize": (_int, [_vp, _vp, _i64, _i64, _i64, _int, _int, _vp, _vp]),
    "hlwq_quantize_grouped": (_int, [ctypes.POINTER(MatDesc), _int, _int, _vp]),
    "hlwq_dequantize_grouped": (_int, [ctypes.POINTER(MatDesc), _int, _int, _vp]),
    "hlwq_kv_quantize": (_int, [_vp, _i64, _i64, _i64, _int, _int, _i64, _vp, _vp, _vp]),
    "hlwq_kv_dequantize": (_int, [_vp, _vp, _i64, _i64, _i64, _int, _int, _i64, _vp, _vp]),
    "hlwq_kv_append": (_int, [_vp, _i64, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _int, _int, _vp]),
    "hlwq_dequantize_int4": (_int, [_vp, _vp, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp]),
    "hlwq_dequantize_int4_grouped": (_int, [ctypes.POINTER(Int4Desc), _int, _int, _vp]),
    "hlwq_quantize_codes8": (_int, [_vp, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp]),
    "hlwq_dequantize_codes8": (_int, [_vp, _vp, _i64, _i64, _i64, _int, _int, _vp, _vp]),
    "hlwq_tq3_signs": (_int, [ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint32)]),
    "hlwq_tq3_quantize": (_int, [_vp, _i64, _i64, _i64, _int, ctypes.c_uint64, _vp, _vp, _vp]),
    "hlwq_tq3_dequantize": (_int, [_vp, _vp, _i64, _i64, _i64, _int, ctypes.c_uint64, _vp, _vp]),
    "hlwq_tq3_quantize_grouped": (_int, [ctypes.POINTER(MatDesc), _int, ctypes.c_uint64, _vp]),
    "hlwq_tq3_dequantize_grouped": (_int, [ctypes.POINTER(MatDesc), _int, ctypes.c_uint64, _vp]),
    "hlwq_packed_bytes": (ctypes.c_size_t, [_i64, _i64, _int, _int]),
    "hlwq_norm_count": (ctypes.c_size_t, [_i64, _i64, _int]),
    "hlwq_search_table": (_int, [_int, ctypes.POINTER(ctypes.c_uint8), _int, ctypes.POINTER(ctypes.c_uint32),
                                 ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_uint32)]),
    "hlwq_status_string": (ctypes.c_char_p, [_int]),
}
_SIGNATURES["hlwq_centroids"] = (_int, [_int, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float)])


def declared_functions(header: str = HEADER_PATH) -> list[str]:
    """Names of the functions include/hlwq.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hlwq_[a-z_0-9]+)\s*\(", text)))


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libhlwq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m weight_quantization_amd.build` "
            "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(func: str, status: int):
    if status != HLWQ_OK:
        raise HLWQError(func, status, hlwq_status_string(status))


# --------------------------------------------------------------------------
# host-only helpers
# --------------------------------------------------------------------------

def hlwq_status_string(status: int) -> str:
    return load_library().hlwq_status_string(int(status)).decode()


def hlwq_packed_bytes(rows: int, n_in: int, block: int = BLOCK, bits: int = 5) -> int:
    return int(load_library().hlwq_packed_bytes(rows, n_in, block, bits))


def hlwq_norm_count(rows: int, n_in: int, block: int = BLOCK) -> int:
    return int(load_library().hlwq_norm_count(rows, n_in, block))


def hlwq_centroids(bits: int):
    """(centroids float32[2^bits], thresholds float32[2^bits - 1]) used by the kernels."""
    K = 1 << bits
    c = (ctypes.c_float * K)()
    t = (ctypes.c_float * max(K - 1, 1))()
    _check("hlwq_centroids", load_library().hlwq_centroids(bits, c, t))
    return np.frombuffer(c, dtype=np.float32).copy(), np.frombuffer(t, dtype=np.float32)[:K - 1].copy()


TQ3_SEED = 42  # the quantizer state's seed (bits 3, group 128)


def hlwq_tq3_signs(seed: int = TQ3_SEED):
    """TQ3's sign vectors for `seed` as two int8 arrays of +-1 (D1, D2), from the library."""
    import numpy as np
    words = (ctypes.c_uint32 * 8)()
    _check("hlwq_tq3_signs", load_library().hlwq_tq3_signs(seed & (2 ** 64 - 1), words))
    bits = np.array([(words[i >> 5] >> (i & 31)) & 1 for i in range(256)], dtype=np.int8)
    s = (1 - 2 * bits).astype(np.int8)
    return s[:128].copy(), s[128:].copy()


def hlwq_search_table(kind: int):
    """(bucket bytes uint8[n], entries uint32[K, 2] = {threshold bits, b}, scale, bias bits)."""
    lib = load_library()
    scale = ctypes.c_float()
    bias = ctypes.c_uint32()
    n = lib.hlwq_search_table(kind, None, 0, None, ctypes.byref(scale), ctypes.byref(bias))
    if n < 0:
        _check("hlwq_search_table", n)
    K = {0: 32, 1: 8, 2: 8, 3: 4}.get(kind, 8)
    buckets = (ctypes.c_uint8 * n)()
    entries = (ctypes.c_uint32 * (2 * K))()
    lib.hlwq_search_table(kind, buckets, n, entries, ctypes.byref(scale), ctypes.byref(bias))
    return (np.frombuffer(buckets, dtype=np.uint8).copy(), np.frombuffer(entries, dtype=np.uint32).reshape(K, 2).copy(),
            float(scale.value), int(bias.value))


# --------------------------------------------------------------------------
# device calls (torch tensors in device memory)
# --------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_handle(stream=None, *tensors) -> int:
    """The stream to launch on.  The library launches on the current device,
    so the stream and every tensor of the call must be on it."""
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    if torch.cuda.device_count() > 1 or stream is not None:  # with one device nothing else can be current
        cur = torch.cuda.current_device()
        if s.device_index != cur:
            raise ValueError(f"stream is on cuda:{s.device_index}, the current device is cuda:{cur}")
        for t in tensors:
            if t is not None and t.get_device() != cur:
                raise ValueError(f"a tensor is on cuda:{t.get_device()}, the current device is cuda:{cur}; "
                                 f"call under torch.cuda.device({t.get_device()})")
    return int(s.cuda_stream)


def _ptr(t) -> int:
    return int(t.data_ptr()) if t is not None and t.numel() > 0 else 0


def _need(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be in device memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def packed_shape(w_shape, bits: int):
    *lead, n_in = w_shape
    nb = -(-n_in // BLOCK)
    return (*lead, nb, 16 * bits), (*lead, nb)


def hlwq_quantize(w, bits: int = 5, packed=None, norms=None, stream=None):
    """Quantize a bf16 [out, in] or [n_mats, out, in] tensor; returns (packed u8, norms fp16)."""
    torch = _torch()
    _need(w, torch.bfloat16, "w")
    if w.dim() not in (2, 3):
        raise ValueError("w must be [out, in] or [n_mats, out, in]")
    n_mats, out, n_in = (1, *w.shape) if w.dim() == 2 else tuple(w.shape)
    pshape, nshape = packed_shape(tuple(w.shape), bits)
    if packed is None:
        packed = torch.empty(pshape, dtype=torch.uint8, device=w.device)
    if norms is None:
        norms = torch.empty(nshape, dtype=torch.float16, device=w.device)
    _need(packed, torch.uint8, "packed")
    _need(norms, torch.float16, "norms")
    if tuple(packed.shape) != pshape or tuple(norms.shape) != nshape:
        raise ValueError("packed / norms shape mismatch")
    st = load_library().hlwq_quantize(_ptr(w), n_mats, out, n_in, BLOCK, bits, _ptr(packed), _ptr(norms),
                                      _stream_handle(stream, w, packed, norms))
    _check("hlwq_quantize", st)
    return packed, norms


def hlwq_dequantize(packed, norms, n_in: int, bits: int = 5, out=None, stream=None):
    """Inverse of hlwq_quantize; returns bf16 [.., out, in]."""
    torch = _torch()
    _need(packed, torch.uint8, "packed")
    _need(norms, torch.float16, "norms")
    if packed.dim() not in (3, 4) or packed.shape[-1] != 16 * bits:
        raise ValueError("packed must be [.., out, nb, 16*bits]")
    lead = tuple(packed.shape[:-2])
    nb = packed.shape[-2]
    if nb != -(-n_in // BLOCK) or tuple(norms.shape) != lead + (nb,):
        raise ValueError("packed / norms / in mismatch")
    n_mats, rows = (1, lead[0]) if len(lead) == 1 else lead
    if out is None:
        out = torch.empty(lead + (n_in,), dtype=torch.bfloat16, device=packed.device)
    _need(out, torch.bfloat16, "out")
    if tuple(out.shape) != lead + (n_in,):
        raise ValueError("out shape mismatch")
    st = load_library().hlwq_dequantize(_ptr(packed), _ptr(norms), n_mats, rows, n_in, BLOCK, bits, _ptr(out),
                                        _stream_handle(stream, packed, norms, out))
    _check("hlwq_dequantize", st)
    return out


def hlwq_quantize_codes8(w, bits: int = 5, codes=None, norms=None, stream=None):
    """Quantize with one code per byte; returns (codes u8 [.., nb, 128], norms fp16 [.., nb])."""
    torch = _torch()
    _need(w, torch.bfloat16, "w")
    if w.dim() not in (2, 3):
        raise ValueError("w must be [out, in] or [n_mats, out, in]")
    n_mats, out, n_in = (1, *w.shape) if w.dim() == 2 else tuple(w.shape)
    pshape, nshape = packed_shape(tuple(w.shape), 8)
    codes = torch.empty(pshape, dtype=torch.uint8, device=w.device) if codes is None else codes
    norms = torch.empty(nshape, dtype=torch.float16, device=w.device) if norms is None else norms
    _need(codes, torch.uint8, "codes")
    _need(norms, torch.float16, "norms")
    if tuple(codes.shape) != pshape or tuple(norms.shape) != nshape:
        raise ValueError("codes / norms shape mismatch")
    st = load_library().hlwq_quantize_codes8(_ptr(w), n_mats, out, n_in, BLOCK, bits, _ptr(codes), _ptr(norms),
                                             _stream_handle(stream, w, codes, norms))
    _check("hlwq_quantize_codes8", st)
    return codes, norms


def hlwq_dequantize_codes8(codes, norms, n_in: int, bits: int = 5, out=None, stream=None):
    """Inverse of hlwq_quantize_codes8; returns bf16 [.., out, in]."""
    torch = _torch()
    _need(codes, torch.uint8, "codes")
    _need(norms, torch.float16, "norms")
    if codes.dim() not in (3, 4) or codes.shape[-1] != BLOCK:
        raise ValueError("codes must be [.., out, nb, 128]")
    lead = tuple(codes.shape[:-2])
    nb = codes.shape[-2]
    if nb != -(-n_in // BLOCK) or tuple(norms.shape) != lead + (nb,):
        raise ValueError("codes / norms / in mismatch")
    n_mats, rows = (1, lead[0]) if len(lead) == 1 else lead
    out = torch.empty(lead + (n_in,), dtype=torch.bfloat16, device=codes.device) if out is None else out
    _need(out, torch.bfloat16, "out")
    if tuple(out.shape) != lead + (n_in,):
        raise ValueError("out shape mismatch")
    st = load_library().hlwq_dequantize_codes8(_ptr(codes), _ptr(norms), n_mats, rows, n_in, BLOCK, bits, _ptr(out),
                                               _stream_handle(stream, codes, norms, out))
    _check("hlwq_dequantize_codes8", st)
    return out


def hlwq_tq3_quantize(w, seed: int = TQ3_SEED, packed=None, norms=None, stream=None):
    """TQ3-quantize a bf16 [out, in] or [n_mats, out, in] tensor; returns (packed u8 [.., ng, 48], norms fp32 [.., ng])."""
    torch = _torch()
    _need(w, torch.bfloat16, "w")
    if w.dim() not in (2, 3):
        raise ValueError("w must be [out, in] or [n_mats, out, in]")
    n_mats, out, n_in = (1, *w.shape) if w.dim() == 2 else tuple(w.shape)
    pshape, nshape = packed_shape(tuple(w.shape), 3)
    packed = torch.empty(pshape, dtype=torch.uint8, device=w.device) if packed is None else packed
    norms = torch.empty(nshape, dtype=torch.float32, device=w.device) if norms is None else norms
    _need(packed, torch.uint8, "packed")
    _need(norms, torch.float32, "norms")
    if tuple(packed.shape) != pshape or tuple(norms.shape) != nshape:
        raise ValueError("packed / norms shape mismatch")
    st = load_library().hlwq_tq3_quantize(_ptr(w), n_mats, out, n_in, BLOCK, seed & (2 ** 64 - 1), _ptr(packed),
                                          _ptr(norms), _stream_handle(stream, w, packed, norms))
    _check("hlwq_tq3_quantize", st)
    return packed, norms


def hlwq_tq3_dequantize(packed, norms, n_in: int, seed: int = TQ3_SEED, out=None, stream=None):
    """Inverse of hlwq_tq3_quantize; returns bf16 [.., out, in]."""
    torch = _torch()
    _need(packed, torch.uint8, "packed")
    _need(norms, torch.float32, "norms")
    if packed.dim() not in (3, 4) or packed.shape[-1] != 48:
        raise ValueError("packed must be [.., out, ng, 48]")
    lead = tuple(packed.shape[:-2])
    nb = packed.shape[-2]
    if nb != -(-n_in // BLOCK) or tuple(norms.shape) != lead + (nb,):
        raise ValueError("packed / norms / in mismatch")
    n_mats, rows = (1, lead[0]) if len(lead) == 1 else lead
    out = torch.empty(lead + (n_in,), dtype=torch.bfloat16, device=packed.device) if out is None else out
    _need(out, torch.bfloat16, "out")
    if tuple(out.shape) != lead + (n_in,):
        raise ValueError("out shape mismatch")
    st = load_library().hlwq_tq3_dequantize(_ptr(packed), _ptr(norms), n_mats, rows, n_in, BLOCK,
                                            seed & (2 ** 64 - 1), _ptr(out),
                                            _stream_handle(stream, packed, norms, out))
    _check("hlwq_tq3_dequantize", st)
    return out


def hlwq_dequantize_int4(packed, norms, n_in: int, bits: int = 5, q4=None, scales=None, zeros=None, stream=None):
    """Dequantize to INT4 with a scale and zero point per 128-column group;
    returns (q4 uint8 [.., out, in / 2], scales float32 [.., out, in / 128],
    zeros uint8 [.., out, in / 128])."""
    torch = _torch()
    _need(packed, torch.uint8, "packed")
    _need(norms, torch.float16, "norms")
    if packed.dim() not in (3, 4) or packed.shape[-1] != 16 * bits:
        raise ValueError("packed must be [.., out, nb, 16*bits]")
    if n_in % BLOCK:
        raise ValueError("in must be a multiple of 128")
    lead = tuple(packed.shape[:-2])
    nb = packed.shape[-2]
    if nb != n_in // BLOCK or tuple(norms.shape) != lead + (nb,):
        raise ValueError("packed / norms / in mismatch")
    n_mats, rows = (1, lead[0]) if len(lead) == 1 else lead
    dev = packed.device
    q4 = torch.empty(lead + (n_in // 2,), dtype=torch.uint8, device=dev) if q4 is None else q4
    scales = torch.empty(lead + (nb,), dtype=torch.float32, device=dev) if scales is None else scales
    zeros = torch.empty(lead + (nb,), dtype=torch.uint8, device=dev) if zeros is None else zeros
    _need(q4, torch.uint8, "q4")
    _need(scales, torch.float32, "scales")
    _need(zeros, torch.uint8, "zeros")
    if tuple(q4.shape) != lead + (n_in // 2,) or tuple(scales.shape) != lead + (nb,) or \
            tuple(zeros.shape) != lead + (nb,):
        raise ValueError("q4 / scales / zeros shape mismatch")
    st = load_library().hlwq_dequantize_int4(_ptr(packed), _ptr(norms), n_mats, rows, n_in, BLOCK, bits, _ptr(q4),
                                             _ptr(scales), _ptr(zeros),
                                             _stream_handle(stream, packed, norms, q4, scales, zeros))
    _check("hlwq_dequantize_int4", st)
    return q4, scales, zeros


def hlwq_dequantize_int4_grouped(items, bits: int = 5, stream=None):
    """items: list of (packed u8 [.., out, nb, 16*bits], norms fp16 [.., out, nb],
    q4 u8 [.., out, in / 2], scales fp32 [.., out, nb], zeros u8 [.., out, nb])
    tuples, all preallocated; in = 128 nb.  One launch for up to 16 matrices."""
    torch = _torch()
    arr = (Int4Desc * max(len(items), 1))()
    for i, (p, n, q4, sc, z) in enumerate(items):
        _need(p, torch.uint8, "packed")
        _need(n, torch.float16, "norms")
        _need(q4, torch.uint8, "q4")
        _need(sc, torch.float32, "scales")
        _need(z, torch.uint8, "zeros")
        if p.dim() < 2 or p.shape[-1] != 16 * bits:
            raise ValueError("packed must be [.., out, nb, 16*bits]")
        lead, nb = tuple(p.shape[:-2]), p.shape[-2]
        if tuple(n.shape) != lead + (nb,) or tuple(sc.shape) != lead + (nb,) or tuple(z.shape) != lead + (nb,) or \
                tuple(q4.shape) != lead + (nb * BLOCK // 2,):
            raise ValueError("packed / norms / q4 / scales / zeros shape mismatch")
        rows = int(np.prod(lead)) if lead else 1
        arr[i] = Int4Desc(_ptr(p), _ptr(n), _ptr(q4), _ptr(sc), _ptr(z), rows, nb * BLOCK)
    st = load_library().hlwq_dequantize_int4_grouped(arr, len(items), bits,
                                                     _stream_handle(stream, *[t for item in items for t in item]))
    _check("hlwq_dequantize_int4_grouped", st)


def _descs(items):
    arr = (MatDesc * max(len(items), 1))()
    for i, (w, p, n) in enumerate(items):
        n_in = w.shape[-1]
        rows = w.numel() // n_in if n_in else 0
        arr[i] = MatDesc(_ptr(w), _ptr(p), _ptr(n), rows, n_in)
    return arr


def hlwq_quantize_grouped(items, bits: int = 5, stream=None):
    """items: list of (w bf16, packed u8, norms fp16) triples, all preallocated."""
    torch = _torch()
    for w, p, n in items:
        _need(w, torch.bfloat16, "w")
        _need(p, torch.uint8, "packed")
        _need(n, torch.float16, "norms")
        ps, ns = packed_shape(tuple(w.shape), bits)
        if tuple(p.shape) != ps or tuple(n.shape) != ns:
            raise ValueError("packed / norms shape mismatch")
    arr = _descs(items)
    st = load_library().hlwq_quantize_grouped(arr, len(items), bits,
                                              _stream_handle(stream, *[t for item in items for t in item]))
    _check("hlwq_quantize_grouped", st)


def hlwq_dequantize_grouped(items, bits: int = 5, stream=None):
    """items: list of (w_out bf16, packed u8, norms fp16) triples, all preallocated."""
    torch = _torch()
    for w, p, n in items:
        _need(w, torch.bfloat16, "w")
        _need(p, torch.uint8, "packed")
        _need(n, torch.float16, "norms")
        ps, ns = packed_shape(tuple(w.shape), bits)
        if tuple(p.shape) != ps or tuple(n.shape) != ns:
            raise ValueError("packed / norms shape mismatch")
    arr = _descs(items)
    st = load_library().hlwq_dequantize_grouped(arr, len(items), bits,
                                                _stream_handle(stream, *[t for item in items for t in item]))
    _check("hlwq_dequantize_grouped", st)


def _check_tq3_items(items):
    torch = _torch()
    for w, p, n in items:
        _need(w, torch.bfloat16, "w")
        _need(p, torch.uint8, "packed")
        _need(n, torch.float32, "norms")
        ps, ns = packed_shape(tuple(w.shape), 3)
        if tuple(p.shape) != ps or tuple(n.shape) != ns:
            raise ValueError("packed / norms shape mismatch")


def hlwq_tq3_quantize_grouped(items, seed: int = TQ3_SEED, stream=None):
    """items: list of (w bf16, packed u8, norms fp32) triples, all preallocated."""
    _check_tq3_items(items)
    st = load_library().hlwq_tq3_quantize_grouped(_descs(items), len(items), seed & (2 ** 64 - 1),
                                                  _stream_handle(stream, *[t for item in items for t in item]))
    _check("hlwq_tq3_quantize_grouped", st)


def hlwq_tq3_dequantize_grouped(items, seed: int = TQ3_SEED, stream=None):
    """items: list of (w_out bf16, packed u8, norms fp32) triples, all preallocated."""
    _check_tq3_items(items)
    st = load_library().hlwq_tq3_dequantize_grouped(_descs(items), len(items), seed & (2 ** 64 - 1),
                                                    _stream_handle(stream, *[t for item in items for t in item]))
    _check("hlwq_tq3_dequantize_grouped", st)


def hlwq_kv_quantize(kv, n_residual: int = 128, bits: int = 3, packed=None, norms=None, stream=None):
    """Quantize a bf16 KV cache [B, H, T, 256] (bits 3 or 2); returns
    (packed [B, H, Tq, 32 * bits], norms [B, H, Tq])."""
    torch = _torch()
    _need(kv, torch.bfloat16, "kv")
    if kv.dim() != 4:
        raise ValueError("kv must be [batch, heads, tokens, head_dim]")
    B, H, T, D = kv.shape
    tq = max(T - n_residual, 0)
    if packed is None:
        packed = torch.empty((B, H, tq, D * bits // 8), dtype=torch.uint8, device=kv.device)
    if norms is None:
        norms = torch.empty((B, H, tq), dtype=torch.float16, device=kv.device)
    _need(packed, torch.uint8, "packed")
    _need(norms, torch.float16, "norms")
    if tuple(packed.shape) != (B, H, tq, D * bits // 8) or tuple(norms.shape) != (B, H, tq):
        raise ValueError("packed / norms shape mismatch")
    st = load_library().hlwq_kv_quantize(_ptr(kv), B, H, T, D, bits, n_residual, _ptr(packed), _ptr(norms),
                                         _stream_handle(stream, kv, packed, norms))
    _check("hlwq_kv_quantize", st)
    return packed, norms


def hlwq_kv_append(new_kv, window, packed, norms, tokens: int, n_residual: int = 128, bits: int = 3, stream=None):
    """Append new_kv [B, H, n_new, 256] to a streaming cache holding `tokens`
    tokens: window [B, H, n_residual, 256] (ring, token t in slot
    t % n_residual), packed [B, H, capacity, 32 * bits], norms [B, H, capacity]."""
    torch = _torch()
    _need(new_kv, torch.bfloat16, "new_kv")
    if new_kv.dim() != 4:
        raise ValueError("new_kv must be [batch, heads, n_new, head_dim]")
    B, H, n_new, D = new_kv.shape
    if window is not None:
        _need(window, torch.bfloat16, "window")
        if tuple(window.shape) != (B, H, n_residual, D):
            raise ValueError("window shape mismatch")
    elif n_residual:
        raise ValueError("a window is needed when n_residual > 0")
    _need(packed, torch.uint8, "packed")
    _need(norms, torch.float16, "norms")
    capacity = packed.shape[2]
    if tuple(packed.shape) != (B, H, capacity, D * bits // 8) or tuple(norms.shape) != (B, H, capacity):
        raise ValueError("packed / norms shape mismatch")
    st = load_library().hlwq_kv_append(_ptr(new_kv), B, H, n_new, tokens, _ptr(window) if window is not None else None,
                                       n_residual, _ptr(packed), _ptr(norms), capacity, D, bits,
                                       _stream_handle(stream, new_kv, window, packed, norms))
    _check("hlwq_kv_append", st)
    return tokens + n_new


def hlwq_kv_dequantize(packed, norms, kv_out, n_residual: int = 128, bits: int = 3, stream=None):
    """Write tokens t < T - n_residual of kv_out [B, H, T, 256] from packed / norms."""
    torch = _torch()
    _need(packed, torch.uint8, "packed")
    _need(norms, torch.float16, "norms")
    _need(kv_out, torch.bfloat16, "kv_out")
    B, H, T, D = kv_out.shape
    tq = max(T - n_residual, 0)
    if tuple(packed.shape) != (B, H, tq, D * bits // 8) or tuple(norms.shape) != (B, H, tq):
        raise ValueError("packed / norms shape mismatch")
    st = load_library().hlwq_kv_dequantize(_ptr(packed), _ptr(norms), B, H, T, D, bits, n_residual, _ptr(kv_out),
                                           _stream_handle(stream, packed, norms, kv_out))
    _check("hlwq_kv_dequantize", st)
    return kv_out
