"""CPU oracle of the FP4Quant compress / decompress transform -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library's product path never does, and
this package never imports the library: the two share no code.

The arithmetic lives in ``fp4q_oracle.c`` (plain C, binary32 in the order the
method states, binary64 for the receiver-side reduce); this module only marshals
numpy arrays through ctypes and computes the relative RMSE in binary64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp4q_oracle.c")
_LIB = os.path.join(_HERE, "libfp4q_oracle.so")
GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-Wall", "-shared", "-fPIC"]

BLOCK = 256
GROUP = 16


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (binary32 semantics: no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


# A test may point the loader at another build of the oracle (the mutation check
# of tests/test_oracle_mutations.py loads copies with one planted mistake each).
LIB_ENV = "FP4Q_ORACLE_LIB"


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get(LIB_ENV)
        if not path:
            path = build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        L.fp4q_ref_set_threads.argtypes = [I]
        L.fp4q_ref_max_threads.restype = I
        L.fp4q_ref_e2m1_decode.argtypes = [I]
        L.fp4q_ref_e2m1_decode.restype = ctypes.c_float
        L.fp4q_ref_e2m1_encode.argtypes = [ctypes.c_float]
        L.fp4q_ref_e2m1_encode.restype = I
        L.fp4q_ref_e4m3_decode.argtypes = [I]
        L.fp4q_ref_e4m3_decode.restype = ctypes.c_float
        L.fp4q_ref_e4m3_encode.argtypes = [ctypes.c_float]
        L.fp4q_ref_e4m3_encode.restype = I
        L.fp4q_ref_compress.argtypes = [P, I64, I, P, P, P, P, P]
        L.fp4q_ref_decompress.argtypes = [P, P, P, I64, I, P]
        L.fp4q_ref_decompress_f64.argtypes = [P, P, P, I64, I, P]
        L.fp4q_ref_accumulate_f64.argtypes = [I, P, P, P, I64, I, P]
        L.fp4q_ref_e2m1_encode_n.argtypes = [P, I64, P]
        L.fp4q_ref_e4m3_encode_n.argtypes = [P, I64, P]
        L.fp4q_ref_fwht256_n.argtypes = [P, I64]
        L.fp4q_ref_bf16_round.argtypes = [ctypes.c_float]
        L.fp4q_ref_bf16_round.restype = ctypes.c_uint16
        L.fp4q_ref_bf16_round_n.argtypes = [P, I64, P]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def set_threads(n: int) -> None:
    lib().fp4q_ref_set_threads(int(n))


def max_threads() -> int:
    return int(lib().fp4q_ref_max_threads())


def _check_shape(x: np.ndarray):
    if x.ndim != 2 or x.shape[1] % BLOCK != 0:
        raise ValueError("expected [rows, row_len] with row_len a multiple of 256")


def compress(x_bf16: np.ndarray, fwht: bool = True, debug: bool = False):
    """bf16 bit patterns [rows, L] -> dict(codes [rows, L/2] u8, micro [rows, L/16] u8,
    block [rows, L/256] f32) plus, with ``debug``, v [rows, L] f32 and t [rows, L/16] f32."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    _check_shape(x)
    rows, L = x.shape
    nb = rows * L // BLOCK
    codes = np.empty((rows, L // 2), np.uint8)
    micro = np.empty((rows, L // GROUP), np.uint8)
    block = np.empty((rows, L // BLOCK), np.float32)
    v = np.empty((rows, L), np.float32) if debug else None
    t = np.empty((rows, L // GROUP), np.float32) if debug else None
    lib().fp4q_ref_compress(_ptr(x), nb, int(bool(fwht)), _ptr(codes), _ptr(micro), _ptr(block),
                            _ptr(v) if debug else None, _ptr(t) if debug else None)
    out = {"codes": codes, "micro": micro, "block": block}
    if debug:
        out["v"] = v
        out["t"] = t
    return out


def decompress(codes, micro, block, fwht: bool = True) -> np.ndarray:
    """Payload -> fp32 [rows, L], in binary32 with the same operation order as compress."""
    codes = np.ascontiguousarray(codes, np.uint8)
    micro = np.ascontiguousarray(micro, np.uint8)
    block = np.ascontiguousarray(block, np.float32)
    rows, half = codes.shape
    L = 2 * half
    out = np.empty((rows, L), np.float32)
    lib().fp4q_ref_decompress(_ptr(codes), _ptr(micro), _ptr(block), rows * L // BLOCK,
                              int(bool(fwht)), _ptr(out))
    return out


def decompress_f64(codes, micro, block, fwht: bool = True) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    micro = np.ascontiguousarray(micro, np.uint8)
    block = np.ascontiguousarray(block, np.float32)
    rows, half = codes.shape
    L = 2 * half
    out = np.empty((rows, L), np.float64)
    lib().fp4q_ref_decompress_f64(_ptr(codes), _ptr(micro), _ptr(block), rows * L // BLOCK,
                                  int(bool(fwht)), _ptr(out))
    return out


def accumulate_f64(payloads, fwht: bool = True) -> np.ndarray:
    """Sum of k peers' decompressed payloads, all in binary64.  ``payloads`` is a
    list of (codes, micro, block) triples of one shape."""
    k = len(payloads)
    cs = [np.ascontiguousarray(p[0], np.uint8) for p in payloads]
    ms = [np.ascontiguousarray(p[1], np.uint8) for p in payloads]
    bs = [np.ascontiguousarray(p[2], np.float32) for p in payloads]
    rows, half = cs[0].shape
    L = 2 * half
    PA = ctypes.c_void_p * k
    out = np.empty((rows, L), np.float64)
    lib().fp4q_ref_accumulate_f64(k, PA(*[c.ctypes.data for c in cs]),
                                  PA(*[m.ctypes.data for m in ms]),
                                  PA(*[b.ctypes.data for b in bs]), rows * L // BLOCK,
                                  int(bool(fwht)), _ptr(out))
    return out


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().fp4q_ref_e2m1_encode_n(_ptr(v), v.size, _ptr(out))
    return out


def e4m3_encode(t: np.ndarray) -> np.ndarray:
    t = np.ascontiguousarray(t, np.float32)
    out = np.empty(t.shape, np.uint8)
    lib().fp4q_ref_e4m3_encode_n(_ptr(t), t.size, _ptr(out))
    return out


def e2m1_decode(c: int) -> float:
    return float(lib().fp4q_ref_e2m1_decode(int(c)))


def e4m3_decode(c: int) -> float:
    return float(lib().fp4q_ref_e4m3_decode(int(c)))


def fwht256(y: np.ndarray) -> np.ndarray:
    """Forward (= inverse) normalised FWHT of every 256-block of a float32 array."""
    y = np.array(y, dtype=np.float32, copy=True, order="C")
    if y.size % BLOCK:
        raise ValueError("size must be a multiple of 256")
    lib().fp4q_ref_fwht256_n(_ptr(y), y.size // BLOCK)
    return y


def round_bf16(x: np.ndarray) -> np.ndarray:
    """The bfloat16 output option: float32 values rounded to the nearer
    neighbouring bfloat16 (ties to even), as uint16 bit patterns."""
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().fp4q_ref_bf16_round_n(_ptr(x), x.size, _ptr(out))
    return out


def widen(x_bf16: np.ndarray) -> np.ndarray:
    return (np.asarray(x_bf16, np.uint16).astype(np.uint32) << 16).view(np.float32)


def rel_rmse(x_bf16: np.ndarray, xhat: np.ndarray) -> float:
    """||xhat - x||_2 / ||x||_2 in binary64 over the whole tensor."""
    x = widen(x_bf16).astype(np.float64)
    d = np.asarray(xhat, np.float64) - x
    nx = float(np.sqrt(np.sum(x * x)))
    return float(np.sqrt(np.sum(d * d))) / nx if nx > 0 else 0.0


def requantize(payloads, debug: bool = False, local=None, fwht: bool = True):
    """Sum of k payloads in the transform domain (fp32, peer order), quantised again;
    with ``local`` (bf16 bit patterns of the same shape) the accumulator starts at
    that slice transformed as compress transforms it (as is when ``fwht`` is off).
    Returns dict(codes, micro, block[, v, t]) of the same shape as the inputs."""
    k = len(payloads)
    if k:
        rows, half = np.asarray(payloads[0][0]).shape
        L = 2 * half
    else:
        if local is None:
            raise ValueError("requantize needs a payload or a local slice")
        rows, L = np.asarray(local).shape
    if local is not None:
        local = np.ascontiguousarray(local, dtype=np.uint16)
        _check_shape(local)
        if local.shape != (rows, L):
            raise ValueError("local slice shape differs from the payloads'")
    cs = [np.ascontiguousarray(p[0], np.uint8) for p in payloads]
    ms = [np.ascontiguousarray(p[1], np.uint8) for p in payloads]
    bs = [np.ascontiguousarray(p[2], np.float32) for p in payloads]
    nb = rows * L // BLOCK
    codes = np.empty((rows, L // 2), np.uint8)
    micro = np.empty((rows, L // GROUP), np.uint8)
    block = np.empty((rows, L // BLOCK), np.float32)
    v = np.empty((rows, L), np.float32) if debug else None
    t = np.empty((rows, L // GROUP), np.float32) if debug else None
    PA = ctypes.c_void_p * max(k, 1)
    f = lib().fp4q_ref_requantize_ex
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p]
    f(k, PA(*[c.ctypes.data for c in cs]), PA(*[m.ctypes.data for m in ms]),
      PA(*[b.ctypes.data for b in bs]), _ptr(local) if local is not None else None,
      int(bool(fwht)), nb, _ptr(codes), _ptr(micro), _ptr(block),
      _ptr(v) if debug else None, _ptr(t) if debug else None)
    out = {"codes": codes, "micro": micro, "block": block}
    if debug:
        out["v"] = v
        out["t"] = t
    return out


def compress_mx(x_bf16: np.ndarray, fwht: bool = True, debug: bool = False):
    """MXFP4-style payload: dict(codes [rows, L/2] u8, scales [rows, L/32] u8 (E8M0)[, v])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    _check_shape(x)
    rows, L = x.shape
    codes = np.empty((rows, L // 2), np.uint8)
    scales = np.empty((rows, L // 32), np.uint8)
    v = np.empty((rows, L), np.float32) if debug else None
    f = lib().fp4q_ref_compress_mx
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p]
    f(_ptr(x), rows * L // BLOCK, int(bool(fwht)), _ptr(codes), _ptr(scales), _ptr(v) if debug else None)
    out = {"codes": codes, "scales": scales}
    if debug:
        out["v"] = v
    return out


def decompress_mx(codes, scales, fwht: bool = True) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    rows, half = codes.shape
    L = 2 * half
    out = np.empty((rows, L), np.float32)
    f = lib().fp4q_ref_decompress_mx
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    f(_ptr(codes), _ptr(scales), rows * L // BLOCK, int(bool(fwht)), _ptr(out))
    return out
