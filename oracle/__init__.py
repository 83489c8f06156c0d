"""CPU oracle of the TurboQuant KV-cache codec -- TEST INFRASTRUCTURE.

A plain scalar binary32 C implementation (``tq_oracle.c``) of what the codec
computes, written from the pages:

* "@mlx-bun/inference 0.0.0-stage -> 1.0.0", ops.ts (``fwht``, ``encodeKeys``,
  ``decodeKeys``, ``encodeValues``, ``decodeValues``, ``decodeValuesRotated``,
  ``unrotateValues``, ``packedDim``, the bit-packing section);
* "mlx-bun 0.0.9 -> 0.0.11", turboquant-tables.ts (``SIGN_VECTORS``,
  ``LLOYD_MAX``).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP codec shares no code with it.
This module only marshals numpy arrays into the C functions.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tq_oracle.c")
_LIB = os.path.join(_HERE, "libtq_oracle.so")

F32, BF16 = 0, 1
BLOCK = 32
HEAD_DIMS = (64, 128, 256, 512)
VALUE_BITS = (2, 3, 4, 5, 8)
KEY_BITS = (2, 3, 4, 5, 8)

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared"]


def build() -> str:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        sig = {
            "tqo_f32_to_f16": (ctypes.c_uint16, [f32]),
            "tqo_f16_to_f32": (f32, [ctypes.c_uint16]),
            "tqo_f32_to_bf16": (ctypes.c_uint16, [f32]),
            "tqo_bf16_to_f32": (f32, [ctypes.c_uint16]),
            "tqo_signs": (ctypes.POINTER(f32), [i32]),
            "tqo_lloyd_max": (i32, [i32, ctypes.POINTER(ctypes.POINTER(f32)), ctypes.POINTER(ctypes.POINTER(f32))]),
            "tqo_packed_dim": (i64, [i32, i32]),
            "tqo_hadamard_scale": (f32, [i32]),
            "tqo_hadamard": (None, [P, i32]),
            "tqo_fwht": (i32, [P, i32, i32]),
            "tqo_bin_index": (i32, [f32, i32]),
            "tqo_value_encode_row": (i32, [P, i32, i32, P, P, P]),
            "tqo_value_dequant_rotated_row": (i32, [P, P, i32, i32, P]),
            "tqo_value_decode_row": (i32, [P, P, i32, i32, P]),
            "tqo_key_encode_row": (i32, [P, i32, i32, i32, P, P, P]),
            "tqo_key_decode_row": (i32, [P, P, P, i32, i32, P]),
            "tqo_pack_bits": (i32, [P, i64, i32, P]),
            "tqo_unpack_bits": (i32, [P, i64, i32, P]),
            "tqo_encode_kv": (i32, [P, P, i32, i64, i32, i32, i32, i32, P, P, P, P, P]),
            "tqo_decode_kv": (i32, [P, P, P, P, P, i64, i32, i32, i32, i32, P, P, i32, i32]),
            "tqo_unrotate": (i32, [P, P, i32, i64, i32]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(st, what):
    if st != 0:
        raise ValueError(f"oracle {what}: invalid argument (status {st})")


# --------------------------------------------------------------------- tables

def signs(d: int) -> np.ndarray:
    ptr = lib().tqo_signs(d)
    if not ptr:
        raise ValueError(f"no sign vector for head_dim {d}")
    return np.ctypeslib.as_array(ptr, shape=(d,)).copy()


def lloyd_max(bits: int):
    c = ctypes.POINTER(ctypes.c_float)()
    b = ctypes.POINTER(ctypes.c_float)()
    n = lib().tqo_lloyd_max(bits, ctypes.byref(c), ctypes.byref(b))
    if n == 0:
        raise ValueError(f"no Lloyd-Max table for bits={bits}")
    return (np.ctypeslib.as_array(c, shape=(n,)).copy(),
            np.ctypeslib.as_array(b, shape=(n - 1,)).copy())


def packed_dim(dim: int, bits: int) -> int:
    r = lib().tqo_packed_dim(dim, bits)
    if r < 0:
        raise ValueError(f"packed_dim: dim={dim} * bits={bits} is not byte-aligned")
    return int(r)


def hadamard_scale(d: int) -> np.float32:
    return np.float32(lib().tqo_hadamard_scale(d))


# ---------------------------------------------------------------- conversions

def f32_to_f16_bits(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    f = lib().tqo_f32_to_f16
    return np.array([f(float(v)) for v in x], dtype=np.uint16)


def f32_to_bf16_bits(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    f = lib().tqo_f32_to_bf16
    return np.array([f(float(v)) for v in x], dtype=np.uint16)


def f16_bits_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16).ravel()
    f = lib().tqo_f16_to_f32
    return np.array([f(int(v)) for v in h], dtype=np.float32)


# ------------------------------------------------------------------ step API

def hadamard(x) -> np.ndarray:
    y = np.array(x, dtype=np.float32, copy=True)
    lib().tqo_hadamard(_p(y), y.shape[-1])
    return y


def fwht(x, encode: bool) -> np.ndarray:
    y = np.array(x, dtype=np.float32, copy=True)
    _check(lib().tqo_fwht(_p(y), y.shape[-1], int(encode)), "fwht")
    return y


def bin_index(z, bits: int) -> np.ndarray:
    z = np.ascontiguousarray(z, dtype=np.float32).ravel()
    f = lib().tqo_bin_index
    return np.array([f(float(v), bits) for v in z], dtype=np.int32)


def value_encode_row(x, bits: int):
    x = np.ascontiguousarray(x, dtype=np.float32)
    d = x.shape[-1]
    idx = np.zeros(d, np.uint8)
    sc = np.zeros(d // BLOCK, np.uint16)
    z = np.zeros(d, np.float32)
    _check(lib().tqo_value_encode_row(_p(x), d, bits, _p(idx), _p(sc), _p(z)), "value_encode_row")
    return idx, sc, z


def value_decode_row(idx, scale16, bits: int, rotated: bool = False) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.uint8)
    scale16 = np.ascontiguousarray(scale16, dtype=np.uint16)
    d = idx.shape[-1]
    out = np.zeros(d, np.float32)
    fn = lib().tqo_value_dequant_rotated_row if rotated else lib().tqo_value_decode_row
    _check(fn(_p(idx), _p(scale16), d, bits, _p(out)), "value_decode_row")
    return out


def key_encode_row(x, bits: int, signed: bool):
    x = np.ascontiguousarray(x, dtype=np.float32)
    d = x.shape[-1]
    q = np.zeros(d, np.uint8)
    sc = np.zeros(d // BLOCK, np.uint16)
    zp = np.zeros(d // BLOCK, np.uint16)
    _check(lib().tqo_key_encode_row(_p(x), d, bits, int(signed), _p(q), _p(sc), _p(zp)), "key_encode_row")
    return q, sc, zp


def key_decode_row(q, scale16, zero16, signed: bool) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    d = q.shape[-1]
    out = np.zeros(d, np.float32)
    _check(lib().tqo_key_decode_row(_p(q), _p(np.ascontiguousarray(scale16, np.uint16)),
                                    _p(np.ascontiguousarray(zero16, np.uint16)), d, int(signed), _p(out)),
           "key_decode_row")
    return out


def pack_bits(vals, bits: int) -> np.ndarray:
    vals = np.ascontiguousarray(vals, dtype=np.uint8).ravel()
    n = vals.size
    out = np.zeros((n * bits) // 8, np.uint8)
    _check(lib().tqo_pack_bits(_p(vals), n, bits, _p(out)), "pack_bits")
    return out


def unpack_bits(packed, n: int, bits: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8).ravel()
    out = np.zeros(n, np.uint8)
    _check(lib().tqo_unpack_bits(_p(packed), n, bits, _p(out)), "unpack_bits")
    return out


# ---------------------------------------------------------- whole-tensor API

def _as_rows(a, d):
    """numpy view of K/V as [rows, d]: float32 stays float32, uint16 is bf16 bits."""
    if a is None:
        return None, None
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a.reshape(-1, d), F32
    if a.dtype == np.uint16:
        return a.reshape(-1, d), BF16
    raise TypeError("oracle inputs are float32 or uint16 (bf16 bit patterns)")


def encode_kv(k, v, *, head_dim: int, k_bits: int, v_bits: int, k_signed: bool = False) -> dict:
    """Encode K and/or V of shape [..., head_dim] (float32, or uint16 bf16 bits).

    Returns the five planes flattened over rows: k_codes [R, d*k_bits/8] u8,
    k_scale/k_zero [R, d/32] u16 (fp16 bits), v_codes [R, d*v_bits/8] u8,
    v_scale [R, d/32] u16.
    """
    d = head_dim
    kr, kdt = _as_rows(k, d)
    vr, vdt = _as_rows(v, d)
    dt = kdt if kdt is not None else vdt
    if kdt is not None and vdt is not None and kdt != vdt:
        raise TypeError("K and V must share a dtype")
    R = (kr if kr is not None else vr).shape[0]
    G = d // BLOCK
    out = {}
    if kr is not None:
        out["k_codes"] = np.zeros((R, packed_dim(d, k_bits)), np.uint8)
        out["k_scale"] = np.zeros((R, G), np.uint16)
        out["k_zero"] = np.zeros((R, G), np.uint16)
    if vr is not None:
        out["v_codes"] = np.zeros((R, packed_dim(d, v_bits)), np.uint8)
        out["v_scale"] = np.zeros((R, G), np.uint16)
    st = lib().tqo_encode_kv(_p(kr), _p(vr), dt, R, d, k_bits, int(k_signed), v_bits,
                             _p(out.get("k_codes")), _p(out.get("k_scale")), _p(out.get("k_zero")),
                             _p(out.get("v_codes")), _p(out.get("v_scale")))
    _check(st, "encode_kv")
    return out


def decode_kv(planes: dict, *, rows: int, head_dim: int, k_bits: int, v_bits: int,
              k_signed: bool = False, out_dtype: str = "bf16", keys: bool = True,
              values: bool = True, rotated_v: bool = False):
    """Decode the planes to (K, V) rows [R, d]: float32, or uint16 bf16 bits."""
    d = head_dim
    odt = BF16 if out_dtype == "bf16" else F32
    npdt = np.uint16 if odt == BF16 else np.float32
    ko = np.zeros((rows, d), npdt) if keys else None
    vo = np.zeros((rows, d), npdt) if values else None

    def g(name, dt):
        a = planes.get(name)
        return None if a is None else np.ascontiguousarray(a, dtype=dt)

    kc, ks, kz = g("k_codes", np.uint8), g("k_scale", np.uint16), g("k_zero", np.uint16)
    vc, vs = g("v_codes", np.uint8), g("v_scale", np.uint16)
    st = lib().tqo_decode_kv(_p(kc), _p(ks), _p(kz), _p(vc), _p(vs), rows, d, k_bits,
                             int(k_signed), v_bits, _p(ko), _p(vo), odt, int(rotated_v))
    _check(st, "decode_kv")
    return ko, vo


def unrotate(x, head_dim: int):
    x = np.ascontiguousarray(x)
    dt = BF16 if x.dtype == np.uint16 else F32
    if dt == F32:
        x = x.astype(np.float32)
    out = np.zeros_like(x)
    R = x.size // head_dim
    _check(lib().tqo_unrotate(_p(x), _p(out), dt, R, head_dim), "unrotate")
    return out
