"""TurboQuant KV-cache codec for AMD MI355X (gfx950).

Python binding of the C ABI in ``include/tq.h`` (library ``libtq.so`` built
from the sources in ``csrc/`` by ``build.py``). This module only allocates
outputs with torch and marshals pointers; every step runs in the HIP
kernels. If the library is not built, every call raises ``RuntimeError``.

Functions follow the page "@mlx-bun/inference 0.0.0-stage -> 1.0.0", ops.ts:
``encode_kv`` (encodeKeys / encodeValues + packBits), ``decode_kv``
(unpackBits + decodeKeys / decodeValues, or decodeValuesRotated with
``rotated_v=True``), ``unrotate_values`` (unrotateValues),
``attention_decode`` (attention over the packed cache, values as
decodeValuesRotated) and ``packed_dim`` (packedDim); the page "mlx-bun
0.0.9 -> 0.0.11": ``merge_rows``, ``extend_rows``, ``extract_row``,
``filter_rows`` (batched-quant.ts) and ``lloyd_max_fit`` (the LLOYD_MAX
tables' fit).
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; TQ_LIBRARY may name another build of the same sources
LIB_PATH = os.environ.get("TQ_LIBRARY") or os.path.join(_HERE, "libtq.so")

BLOCK = 32
HEAD_DIMS = (64, 128, 256, 512)
VALUE_BITS = (2, 3, 4, 5, 8)
KEY_BITS = (2, 3, 4, 5, 8)

TQ_OK, TQ_E_NULL, TQ_E_HEAD_DIM, TQ_E_BITS, TQ_E_ALIGN, TQ_E_DTYPE, TQ_E_SHAPE, TQ_E_HIP, TQ_E_CAPTURE, \
    TQ_E_SCRATCH = range(10)
TQ_F32, TQ_BF16 = 0, 1
TQ_DECODE_ROTATED_V = 1

# every symbol include/tq.h declares
EXPORTS = (
    "tq_packed_dim", "tq_status_string", "tq_encode_kv", "tq_decode_kv", "tq_unrotate_values",
    "tq_lloyd_max_table", "tq_sign_vector", "tq_value_bin_host", "tq_quotient_host",
    "tq_merge_rows", "tq_extend_rows", "tq_extract_row", "tq_filter_rows",
    "tq_lloyd_max_workspace_bytes", "tq_lloyd_max_fit",
    "tq_attention_workspace_bytes", "tq_attention_decode", "tq_attention_decode_static",
    "tq_time_next_call",
)


class TQConfig(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("k_bits", ctypes.c_int32),
                ("v_bits", ctypes.c_int32), ("k_signed", ctypes.c_int32)]


class TQPackedKV(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("k_zero", ctypes.c_void_p),
                ("v_codes", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


class TQError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises RuntimeError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP codec library not built ({LIB_PATH}); run "
                               "`python -m kv_cache_quantization_tq_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        sig = {
            "tq_packed_dim": (i64, [i32, i32]),
            "tq_status_string": (ctypes.c_char_p, [i32]),
            "tq_time_next_call": (i32, [P, P]),
            "tq_encode_kv": (i32, [P, P, i32, i64, i32, ctypes.POINTER(TQConfig), ctypes.POINTER(TQPackedKV), P]),
            "tq_decode_kv": (i32, [ctypes.POINTER(TQPackedKV), i64, i32, ctypes.POINTER(TQConfig), P, P, i32, i32, P]),
            "tq_unrotate_values": (i32, [P, P, i32, i64, i32, P]),
            "tq_lloyd_max_table": (i32, [i32, P, P]),
            "tq_sign_vector": (i32, [i32, P]),
            "tq_value_bin_host": (i32, [i32, P, i64, P]),
            "tq_quotient_host": (i32, [P, P, i64, P]),
            "tq_merge_rows": (i32, [ctypes.POINTER(TQPackedKV), P, i32, i64, i32, ctypes.POINTER(TQConfig),
                                    ctypes.POINTER(TQPackedKV), P, P]),
            "tq_extend_rows": (i32, [ctypes.POINTER(TQPackedKV), i32, i64, P, ctypes.POINTER(TQPackedKV), i64,
                                     i64, i32, ctypes.POINTER(TQConfig), ctypes.POINTER(TQPackedKV), P, P]),
            "tq_extract_row": (i32, [ctypes.POINTER(TQPackedKV), i32, i64, i32, i64, i32,
                                     ctypes.POINTER(TQConfig), ctypes.POINTER(TQPackedKV), P]),
            "tq_filter_rows": (i32, [ctypes.POINTER(TQPackedKV), i32, i64, P, i32, i32,
                                     ctypes.POINTER(TQConfig), ctypes.POINTER(TQPackedKV), P]),
            "tq_lloyd_max_workspace_bytes": (i64, [i64]),
            "tq_attention_workspace_bytes": (i64, [i32, i32, i32, i32, i64]),
            "tq_attention_decode": (i32, [P, i32, ctypes.POINTER(TQPackedKV), i32, i64, P, i32, i32,
                                          ctypes.POINTER(TQConfig), ctypes.c_float, P, i32, P, i64, P]),
            "tq_attention_decode_static": (i32, [P, i32, ctypes.POINTER(TQPackedKV), i32, i64, P, i32, i32,
                                                 ctypes.POINTER(TQConfig), ctypes.c_float, P, i32, P]),
            "tq_lloyd_max_fit": (i32, [P, i64, i32, P, i32, P, P, P, i64, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().tq_status_string(status).decode()


def _event_handle(e):
    """A hipEvent_t as an int: a raw handle, or an object holding one as `ev`."""
    if e is None:
        return None
    ev = getattr(e, "ev", e)
    return ev.value if isinstance(ev, ctypes.c_void_p) else int(ev)


def time_next_call(start, stop) -> None:
    """Bind caller-owned HIP events to the end of the last kernel (`stop`)
    and, unless `start` is None, the start of the first kernel of the next
    library call on this thread (tq_time_next_call); None, None disarms."""
    st = lib().tq_time_next_call(_event_handle(start), _event_handle(stop))
    if st:
        raise TQError(st, "time_next_call")


def packed_dim(dim: int, bits: int) -> int:
    r = lib().tq_packed_dim(dim, bits)
    if r < 0:
        raise TQError(-r, f"packed_dim(dim={dim}, bits={bits})")
    return int(r)


def lloyd_max_table(bits: int):
    import numpy as np
    c = np.zeros(1 << bits if 1 <= bits <= 8 else 1, np.float32)
    b = np.zeros(max(c.size - 1, 1), np.float32)
    st = lib().tq_lloyd_max_table(bits, c.ctypes.data, b.ctypes.data)
    if st:
        raise TQError(st, f"lloyd_max_table(bits={bits})")
    return c, b[: c.size - 1]


def sign_vector(head_dim: int):
    import numpy as np
    s = np.zeros(max(head_dim, 1), np.float32)
    st = lib().tq_sign_vector(head_dim, s.ctypes.data)
    if st:
        raise TQError(st, f"sign_vector(head_dim={head_dim})")
    return s


def value_bin_host(bits: int, z):
    """The kernels' bin search evaluated on the host (for CPU checks)."""
    import numpy as np
    z = np.ascontiguousarray(z, dtype=np.float32).ravel()
    out = np.zeros(z.size, np.uint8)
    st = lib().tq_value_bin_host(bits, z.ctypes.data, z.size, out.ctypes.data)
    if st:
        raise TQError(st, f"value_bin_host(bits={bits})")
    return out


def quotient_host(a, b):
    """The kernels' exact quotient a / b evaluated on the host (for CPU checks)."""
    import numpy as np
    a = np.ascontiguousarray(a, dtype=np.float32).ravel()
    b = np.ascontiguousarray(b, dtype=np.float32).ravel()
    if a.size != b.size:
        raise ValueError("quotient_host: a and b differ in size")
    out = np.zeros(a.size, np.float32)
    st = lib().tq_quotient_host(a.ctypes.data, b.ctypes.data, a.size, out.ctypes.data)
    if st:
        raise TQError(st, "quotient_host")
    return out


# ------------------------------------------------------------ torch helpers

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return TQ_F32
    if t.dtype == torch.bfloat16:
        return TQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _stream_handle(stream) -> Optional[int]:
    """A torch stream, a raw hipStream_t handle (int), or None for torch's
    current stream."""
    if isinstance(stream, int):
        return stream
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def plane_shapes(rows: int, head_dim: int, k_bits: int, v_bits: int) -> Dict[str, Tuple[Tuple[int, int], str]]:
    g = head_dim // BLOCK
    return {
        "k_codes": ((rows, head_dim * k_bits // 8), "uint8"),
        "k_scale": ((rows, g), "uint16"),
        "k_zero": ((rows, g), "uint16"),
        "v_codes": ((rows, head_dim * v_bits // 8), "uint8"),
        "v_scale": ((rows, g), "uint16"),
    }


def empty_planes(rows: int, head_dim: int, k_bits: int, v_bits: int, device, keys=True, values=True):
    """Allocate the five planes; fp16 planes are int16 tensors holding fp16 bits."""
    torch = _torch()
    out = {}
    for name, (shape, kind) in plane_shapes(rows, head_dim, k_bits, v_bits).items():
        if (name.startswith("k_") and not keys) or (name.startswith("v_") and not values):
            continue
        dt = torch.uint8 if kind == "uint8" else torch.int16
        out[name] = torch.empty(shape, dtype=dt, device=device)
    return out


def _packed(planes: Dict) -> TQPackedKV:
    return TQPackedKV(*[_ptr(planes.get(n)) for n in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale")])


class PreparedCall:
    """A stream call of the library with its arguments marshalled once.
    Calling it enqueues the same call again (same buffers, same stream) and
    returns what the keyword function returns; TQError on a nonzero status.
    For launch loops whose host time per call matters: ~3 us of Python per
    call instead of ~9 us through the keyword functions. The buffers and
    the host structures the call points to are held for its lifetime."""

    __slots__ = ("_fn", "_args", "_what", "_keep", "_result")

    def __init__(self, name, args, keep, result):
        self._fn = getattr(lib(), name)
        self._args = tuple(args)
        self._what = name
        self._keep = keep
        self._result = result

    def __call__(self):
        st = self._fn(*self._args)
        if st:
            raise TQError(st, self._what)
        return self._result

    def on(self, stream) -> "PreparedCall":
        """The same call on another stream (a hipStream_t handle, an int)."""
        return PreparedCall(self._what, self._args[:-1] + (stream,), self._keep, self._result)


def _issue(name, args, keep, result, prepare):
    """Make the C call now, or return it prepared (the stream is the last
    argument of every call made this way)."""
    call = PreparedCall(name, args, keep, result)
    return call if prepare else call()


def encode_kv(k, v, *, v_bits: int, k_bits: int, k_signed: bool = False, out: Optional[Dict] = None,
              stream=None, prepare: bool = False) -> Dict:
    """Encode K and/or V ([tokens, heads, head_dim], float32 or bfloat16, contiguous,
    on the GPU) into the packed planes. Either of k, v may be None. With
    prepare=True, returns a PreparedCall of the encode instead of making it."""
    ref = k if k is not None else v
    if ref is None:
        raise ValueError("encode_kv needs k or v")
    if k is not None and v is not None and (k.shape != v.shape or k.dtype != v.dtype):
        raise ValueError("k and v must share shape and dtype")
    if ref.dim() < 2:
        raise ValueError("expected [tokens, heads, head_dim] (or [rows, head_dim])")
    d = ref.shape[-1]
    heads = ref.shape[-2] if ref.dim() >= 3 else 1
    tokens = ref.numel() // (d * heads) if d * heads else 0
    for t in (k, v):
        if t is not None and not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    rows = tokens * heads
    if out is None:
        out = empty_planes(rows, d, k_bits, v_bits, ref.device, keys=k is not None, values=v is not None)
    cfg = TQConfig(d, k_bits, v_bits, int(bool(k_signed)))
    pk = _packed(out)
    return _issue("tq_encode_kv", (_ptr(k), _ptr(v), _dtype_code(ref), tokens, heads, ctypes.byref(cfg),
                                   ctypes.byref(pk), _stream_handle(stream)), (k, v, cfg, pk), out, prepare)


def decode_kv(planes: Dict, *, tokens: int, heads: int, head_dim: int, v_bits: int, k_bits: int,
              k_signed: bool = False, out_dtype=None, keys: bool = True, values: bool = True,
              rotated_v: bool = False, k_out=None, v_out=None, stream=None, prepare: bool = False):
    """Decode planes back to (K, V) of shape [tokens, heads, head_dim]. With
    prepare=True, returns a PreparedCall of the decode instead of making it."""
    torch = _torch()
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    ref = next(p for p in planes.values() if p is not None)
    if keys and k_out is None:
        k_out = torch.empty((tokens, heads, head_dim), dtype=out_dtype, device=ref.device)
    if values and v_out is None:
        v_out = torch.empty((tokens, heads, head_dim), dtype=out_dtype, device=ref.device)
    if not keys:
        k_out = None
    if not values:
        v_out = None
    dcode = _dtype_code(k_out if k_out is not None else v_out)
    cfg = TQConfig(head_dim, k_bits, v_bits, int(bool(k_signed)))
    pk = _packed(planes)
    flags = TQ_DECODE_ROTATED_V if rotated_v else 0
    return _issue("tq_decode_kv", (ctypes.byref(pk), tokens, heads, ctypes.byref(cfg), _ptr(k_out), _ptr(v_out),
                                   dcode, flags, _stream_handle(stream)), (planes, cfg, pk), (k_out, v_out), prepare)


def unrotate_values(x, out=None, stream=None, prepare: bool = False):
    """Inverse rotation of rows [..., head_dim] (attention outputs computed on
    rotated values), in x's dtype. With prepare=True, returns a
    PreparedCall instead of making the call."""
    torch = _torch()
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    d = x.shape[-1]
    if out is None:
        out = torch.empty_like(x)
    return _issue("tq_unrotate_values", (_ptr(x), _ptr(out), _dtype_code(x), x.numel() // d if d else 0, d,
                                         _stream_handle(stream)), (x,), out, prepare)


# ------------------------------------------------- token-axis batching ops
#
# Plane dicts as above; a batch of b sequences of width W holds b * W tokens
# (b * W * heads rows per plane). The planes handled are those present in
# the source dicts; outputs are allocated with the same set.

def _like(planes: Dict, tokens: int, heads: int, head_dim: int, k_bits: int, v_bits: int):
    ref = next(p for p in planes.values() if p is not None)
    full = empty_planes(tokens * heads, head_dim, k_bits, v_bits, ref.device)
    return {n: full[n] for n in planes}


def _i64(vals):
    import numpy as np
    return np.ascontiguousarray(np.asarray(vals, dtype=np.int64))


def merge_rows(caches, lens, *, heads: int, head_dim: int, k_bits: int, v_bits: int, k_signed: bool = False,
               width: Optional[int] = None, out: Optional[Dict] = None, stream=None):
    """Stack caches (plane dicts, cache i holding lens[i] tokens) into one
    left-padded batch, written to `out` (planes for n * width tokens;
    allocated when None). Returns (planes, left_pad, width)."""
    n = len(caches)
    lens_a = _i64(lens)
    width = int(lens_a.max()) if width is None and n else int(width or 0)
    dst = _like(caches[0], n * width, heads, head_dim, k_bits, v_bits) if out is None else out
    srcs = (TQPackedKV * max(n, 1))(*[_packed(c) for c in caches])
    pad = _i64([0] * max(n, 1))
    cfg = TQConfig(head_dim, k_bits, v_bits, int(bool(k_signed)))
    st = lib().tq_merge_rows(srcs, lens_a.ctypes.data, n, width, heads, ctypes.byref(cfg),
                             ctypes.byref(_packed(dst)), pad.ctypes.data, _stream_handle(stream))
    if st:
        raise TQError(st, "tq_merge_rows")
    return dst, [int(x) for x in pad[:n]], width


def extend_rows(batch, b: int, width: int, left_pad, row, row_len: int, *, heads: int, head_dim: int,
                k_bits: int, v_bits: int, k_signed: bool = False, new_width: Optional[int] = None, stream=None):
    """Append cache `row` (row_len tokens) to a batch of b sequences of width
    `width`. Returns (planes, left_pad, new_width)."""
    new_width = max(width, row_len) if new_width is None else int(new_width)
    dst = _like(row, (b + 1) * new_width, heads, head_dim, k_bits, v_bits)
    pin = _i64(list(left_pad) + [0])
    pout = _i64([0] * (b + 1))
    cfg = TQConfig(head_dim, k_bits, v_bits, int(bool(k_signed)))
    bp = _packed(batch) if batch is not None else TQPackedKV()
    st = lib().tq_extend_rows(ctypes.byref(bp), b, width, pin.ctypes.data, ctypes.byref(_packed(row)), row_len,
                              new_width, heads, ctypes.byref(cfg), ctypes.byref(_packed(dst)), pout.ctypes.data,
                              _stream_handle(stream))
    if st:
        raise TQError(st, "tq_extend_rows")
    return dst, [int(x) for x in pout], new_width


def extract_row(batch, b: int, width: int, i: int, left_pad: int, *, heads: int, head_dim: int, k_bits: int,
                v_bits: int, k_signed: bool = False, stream=None):
    """Sequence i of a batch, past its left pad, as a cache of width - left_pad tokens."""
    dst = _like(batch, width - left_pad, heads, head_dim, k_bits, v_bits)
    cfg = TQConfig(head_dim, k_bits, v_bits, int(bool(k_signed)))
    st = lib().tq_extract_row(ctypes.byref(_packed(batch)), b, width, i, left_pad, heads, ctypes.byref(cfg),
                              ctypes.byref(_packed(dst)), _stream_handle(stream))
    if st:
        raise TQError(st, "tq_extract_row")
    return dst


def filter_rows(batch, b: int, width: int, keep, *, heads: int, head_dim: int, k_bits: int, v_bits: int,
                k_signed: bool = False, stream=None):
    """Sequences keep[j] of a batch, in that order, as a batch of len(keep)."""
    import numpy as np
    keep_a = np.ascontiguousarray(np.asarray(keep, dtype=np.int32))
    dst = _like(batch, len(keep_a) * width, heads, head_dim, k_bits, v_bits)
    cfg = TQConfig(head_dim, k_bits, v_bits, int(bool(k_signed)))
    st = lib().tq_filter_rows(ctypes.byref(_packed(batch)), b, width, keep_a.ctypes.data if keep_a.size else None,
                              len(keep_a), heads, ctypes.byref(cfg), ctypes.byref(_packed(dst)),
                              _stream_handle(stream))
    if st:
        raise TQError(st, "tq_filter_rows")
    return dst


# ------------------------------------------------------- Lloyd-Max fitting

def lloyd_max_fit(samples, levels: int, init, iterations: int = 500, workspace=None, stream=None):
    """Fit `levels` Lloyd-Max levels to `samples` (a float32 device tensor)
    from the ascending initial centroids `init`. Returns (centroids,
    boundaries) as float64 numpy arrays. Waits for the stream."""
    import numpy as np
    torch = _torch()
    if samples.dtype != torch.float32 or not samples.is_contiguous():
        raise ValueError("samples must be a contiguous float32 tensor")
    init_a = np.ascontiguousarray(np.asarray(init, dtype=np.float64))
    if init_a.size != levels:
        raise ValueError("init must hold `levels` values")
    nbytes = int(lib().tq_lloyd_max_workspace_bytes(samples.numel()))
    if nbytes < 0:
        raise TQError(-nbytes, f"lloyd_max_fit: {samples.numel()} samples")
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=samples.device)
    c = np.zeros(levels, np.float64)
    b = np.zeros(max(levels - 1, 1), np.float64)
    st = lib().tq_lloyd_max_fit(_ptr(samples), samples.numel(), levels, init_a.ctypes.data, iterations,
                                c.ctypes.data, b.ctypes.data, _ptr(workspace), workspace.numel(),
                                _stream_handle(stream))
    if st:
        raise TQError(st, "tq_lloyd_max_fit")
    return c, b[: levels - 1]


# ------------------------------------------------ attention over the cache

def attention_decode(q, cache, *, batch: int, width: int, kv_heads: int, head_dim: int, k_bits: int, v_bits: int,
                     k_signed: bool = False, left_pad=None, scale: Optional[float] = None, out_dtype=None,
                     out=None, workspace=None, stream=None, prepare: bool = False):
    """Attention of q [batch, q_heads, head_dim] over a packed batch of
    `batch` sequences of width `width` (plane dict, as the batching ops
    lay it out), decoding inside the kernel; left_pad is a device int32
    tensor [batch] or None. Returns out [batch, q_heads, head_dim], or with
    prepare=True a PreparedCall of the attention."""
    import math
    torch = _torch()
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    q_heads = q.shape[1]
    if out is None:
        out = torch.empty((batch, q_heads, head_dim), dtype=out_dtype or torch.float32, device=q.device)
    nbytes = int(lib().tq_attention_workspace_bytes(batch, kv_heads, q_heads, head_dim, width))
    if nbytes < 0:
        raise TQError(-nbytes, "tq_attention_workspace_bytes")
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if left_pad is not None and (left_pad.dtype != torch.int32 or not left_pad.is_cuda):
        raise ValueError("left_pad must be a device int32 tensor")
    cfg = TQConfig(head_dim, k_bits, v_bits, int(bool(k_signed)))
    sc = 1.0 / math.sqrt(head_dim) if scale is None else float(scale)
    pk = _packed(cache)
    return _issue("tq_attention_decode", (_ptr(q), _dtype_code(q), ctypes.byref(pk), batch, width,
                                          _ptr(left_pad), kv_heads, q_heads, ctypes.byref(cfg), sc, _ptr(out),
                                          _dtype_code(out), _ptr(workspace),
                                          0 if workspace is None else workspace.numel(), _stream_handle(stream)),
                  (q, cache, left_pad, workspace, cfg, pk), out, prepare)


def attention_decode_static(q, cache, *, batch: int, width: int, kv_heads: int, head_dim: int, k_bits: int,
                            v_bits: int, k_signed: bool = False, left_pad=None, scale: Optional[float] = None,
                            out=None, stream=None):
    """attention_decode through tq_attention_decode_static: no workspace,
    the split partials go to the library's static per-GPU buffer. `out`
    must be given (this path allocates nothing)."""
    import math
    if out is None:
        raise ValueError("attention_decode_static needs `out` (it allocates nothing)")
    if not q.is_contiguous() or not out.is_contiguous():
        raise ValueError("q and out must be contiguous")
    torch = _torch()
    if left_pad is not None and (left_pad.dtype != torch.int32 or not left_pad.is_cuda):
        raise ValueError("left_pad must be a device int32 tensor")
    cfg = TQConfig(head_dim, k_bits, v_bits, int(bool(k_signed)))
    sc = 1.0 / math.sqrt(head_dim) if scale is None else float(scale)
    st = lib().tq_attention_decode_static(_ptr(q), _dtype_code(q), ctypes.byref(_packed(cache)), batch, width,
                                          _ptr(left_pad), kv_heads, q.shape[1], ctypes.byref(cfg), sc, _ptr(out),
                                          _dtype_code(out), _stream_handle(stream))
    if st:
        raise TQError(st, "tq_attention_decode_static")
    return out
