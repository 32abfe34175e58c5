"""Seeded synthetic inputs shared by the CPU oracle and the GPU library.

This module holds no attention arithmetic: it only turns a seed and a token's
identity into normally distributed numbers, so that both sides can be fed the
same values without either one importing the other.

Definition (implemented three times from the same published sources: here in
numpy, in ``synth_host.c`` for fast host-side generation, and in
``synth_rng.h`` for device-side bulk fills):

* splitmix64 (S. Vigna, "splitmix64.c", public domain): the n-th output
  (n >= 1) of a stream whose state starts at ``s`` is ``mix(s + n*GAMMA)``,
  with ``GAMMA = 0x9E3779B97F4A7C15`` and ``mix`` the variant-13 finaliser
  ``z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
  z *= 0x94D049BB133111EB; z ^= z >> 31``.
* A row's stream state is a hash chain over its identity fields:
  ``h = seed; for f in fields: h = mix(h + GAMMA + f)`` with the fields
  ``(layer, kind, a, b, which, head)``; ``which`` is 0 for K, 1 for V, 2 for Q.
* Element pair ``e`` of the row uses outputs ``2e+1`` and ``2e+2``:
  ``u1 = ((r1 >> 11) + 1) * 2**-53`` in (0, 1], ``u2 = (r2 >> 11) * 2**-53``
  in [0, 1), then Box and Muller (1958): ``rho = sqrt(-2 ln u1)``,
  element ``2e`` is ``rho*cos(2 pi u2)`` and ``2e+1`` is ``rho*sin(2 pi u2)``.
* Storage values: fp32 is the round-to-nearest-even float of that double;
  bf16 rounds that float again to bf16 (nearest-even). Both sides use the same
  two-step rounding, so they agree whenever their libm results agree.

Token identity (``kind``, ``a``, ``b``): PROMPT (0, i, 0), TEXT (1, j, 0) with
``j`` the generated-token index, PAUSE (2, block, k). Query rows use the same
identity with ``which = 2``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_U64 = np.uint64

PROMPT, TEXT, PAUSE = 0, 1, 2
WHICH_K, WHICH_V, WHICH_Q = 0, 1, 2


def mix64(z):
    """splitmix64 output finaliser on a uint64 array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=_U64)
    z = z ^ (z >> _U64(30))
    z = z * _U64(_M1)
    z = z ^ (z >> _U64(27))
    z = z * _U64(_M2)
    return z ^ (z >> _U64(31))


def splitmix64_stream(state: int, n: int) -> np.ndarray:
    """First ``n`` outputs of splitmix64 started at ``state`` (uint64)."""
    idx = np.arange(1, n + 1, dtype=_U64)
    with np.errstate(over="ignore"):
        return mix64(_U64(state) + idx * _U64(GAMMA))


def row_keys(seed, layer, kind, a, b, which, head):
    """Stream state of every row identity (broadcast over array arguments)."""
    fields = np.broadcast_arrays(
        *(np.asarray(f, dtype=np.int64) for f in (layer, kind, a, b, which, head)))
    h = np.full(fields[0].shape, seed & 0xFFFFFFFFFFFFFFFF, dtype=_U64)
    with np.errstate(over="ignore"):
        for f in fields:
            h = mix64(h + _U64(GAMMA) + f.astype(_U64))
    return h


def normals_from_keys(keys, d: int) -> np.ndarray:
    """``d`` N(0,1) doubles per key (``d`` even): shape keys.shape + (d,)."""
    assert d % 2 == 0
    keys = np.asarray(keys, dtype=_U64)[..., None]
    e = np.arange(d // 2, dtype=_U64)
    with np.errstate(over="ignore"):
        r1 = mix64(keys + (_U64(2) * e + _U64(1)) * _U64(GAMMA))
        r2 = mix64(keys + (_U64(2) * e + _U64(2)) * _U64(GAMMA))
    u1 = ((r1 >> _U64(11)) + _U64(1)).astype(np.float64) * 2.0 ** -53
    u2 = (r2 >> _U64(11)).astype(np.float64) * 2.0 ** -53
    rho = np.sqrt(-2.0 * np.log(u1))
    out = np.empty(keys.shape[:-1] + (d,), dtype=np.float64)
    out[..., 0::2] = rho * np.cos(2.0 * np.pi * u2)
    out[..., 1::2] = rho * np.sin(2.0 * np.pi * u2)
    return out


def bf16_bits_from_f32(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Storage rounding of generated doubles; returns doubles exactly
    representable in ``dtype`` ('f32' or 'bf16')."""
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return x32.astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(bf16_bits_from_f32(x32))
    raise ValueError(dtype)


_HERE = os.path.dirname(os.path.abspath(__file__))
_CLIB_PATH = os.path.join(_HERE, "libsynth.so")
_clib = None


def build_c(verbose: bool = False) -> str:
    """Compile the C implementation (gcc, OpenMP)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", _CLIB_PATH + ".tmp",
           os.path.join(_HERE, "synth_host.c"), "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(_CLIB_PATH + ".tmp", _CLIB_PATH)
    return _CLIB_PATH


def _c():
    global _clib
    if _clib is None:
        if not os.path.exists(_CLIB_PATH):
            build_c()
        L = ctypes.CDLL(_CLIB_PATH)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        L.synth_rows_c.argtypes = [ctypes.c_uint64, i64, i64, vp, vp, i64, i64, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_double, vp]
        L.synth_rows_c.restype = None
        _clib = L
    return _clib


def rows(seed, layer, kind, a, b, which, heads: int, d: int, dtype: str, scale: float = 1.0):
    """Values of token rows: shape [len(a), heads, d] (doubles exactly
    representable in ``dtype``). ``a`` and ``b`` broadcast against each other;
    ``scale`` multiplies the normals before storage rounding. Computed by the C
    implementation (``synth_host.c``); :func:`rows_numpy` is the same generator
    in numpy."""
    a = np.ascontiguousarray(np.atleast_1d(np.asarray(a, dtype=np.int64)))
    b = np.ascontiguousarray(np.broadcast_to(np.asarray(b, dtype=np.int64), a.shape))
    if dtype not in ("f32", "bf16"):
        raise ValueError(dtype)
    out = np.empty((len(a), heads, d), dtype=np.float64)
    _c().synth_rows_c(seed & 0xFFFFFFFFFFFFFFFF, layer, kind, a.ctypes.data, b.ctypes.data, len(a),
                      which, heads, d, int(dtype == "bf16"), scale, out.ctypes.data)
    return out


def rows_numpy(seed, layer, kind, a, b, which, heads: int, d: int, dtype: str, scale: float = 1.0):
    """numpy implementation of :func:`rows`."""
    a = np.atleast_1d(np.asarray(a, dtype=np.int64))
    b = np.broadcast_to(np.asarray(b, dtype=np.int64), a.shape)
    h = np.arange(heads, dtype=np.int64)
    keys = row_keys(seed, layer, kind, a[:, None], b[:, None], which, h[None, :])
    z = normals_from_keys(keys, d)
    if scale != 1.0:
        z = z * scale
    return to_storage(z, dtype)
