"""fp4q: MI355X-native FP4 compression of tensor-parallel communication.

Thin ctypes binding over ``libfp4q.so`` (C ABI in ``include/fp4q.h``): the
functions below carry the C entry points' names and only marshal arguments --
torch tensors in, device pointers and the current HIP stream out.  Every step
of the transform runs in the library's HIP kernels; there is no fallback, and
a missing library raises.

Method: "FP4Quant: Efficient 4-Bit Communication Compression for Model-Parallel
LLM Training" (abstract).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4q.so")

FP4Q_BLOCK = 256
FP4Q_GROUP = 16
FP4Q_MAX_PEERS = 16
FP4Q_OUT_F32 = 0
FP4Q_OUT_BF16 = 1
FP4Q_FLAG_NO_FWHT = 1
FP4Q_OK = 0
FP4Q_ERR_NULL = 1
FP4Q_ERR_SHAPE = 2
FP4Q_ERR_ALIGN = 3
FP4Q_ERR_K = 4
FP4Q_ERR_ARG = 5
FP4Q_ERR_LAUNCH = 6


class Fp4qError(RuntimeError):
    def __init__(self, status: int):
        super().__init__("fp4q: %s (status %d)" % (fp4q_status_str(status), status))
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library, built first (hipcc, gfx950) if it is not there yet;
    raises if it can be neither found nor built.  There is no other path."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import _build
            try:
                _build.build(force=False)
            except Exception as e:  # noqa: BLE001 - reported with the cause
                raise ImportError("fp4q: %s is missing and could not be built: %s" % (LIB_PATH, e)) from e
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, U32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint32
        PP = ctypes.POINTER(ctypes.c_void_p)
        SZ = ctypes.POINTER(ctypes.c_size_t)
        L.fp4q_payload_bytes.argtypes = [I64, I64, SZ, SZ, SZ]
        L.fp4q_compress.argtypes = [P, I64, I64, P, P, P, P]
        L.fp4q_compress_ex.argtypes = [P, I64, I64, P, P, P, U32, P]
        L.fp4q_decompress.argtypes = [P, P, P, I64, I64, P, P]
        L.fp4q_decompress_ex.argtypes = [P, P, P, I64, I64, P, I, U32, P]
        L.fp4q_decompress_accumulate.argtypes = [I, PP, PP, PP, I64, I64, P, I, P]
        L.fp4q_decompress_accumulate_ex.argtypes = [I, PP, PP, PP, I64, I64, P, I, U32, P]
        L.fp4q_reduce_requantize.argtypes = [I, PP, PP, PP, I64, I64, P, P, P, P]
        L.fp4q_reduce_requantize_ex.argtypes = [I, PP, PP, PP, P, I64, I64, P, P, P, U32, P]
        L.fp4q_compress_mx.argtypes = [P, I64, I64, P, P, U32, P]
        L.fp4q_decompress_mx.argtypes = [P, P, I64, I64, P, I, U32, P]
        L.fp4q_status_str.argtypes = [I]
        L.fp4q_status_str.restype = ctypes.c_char_p
        for f in ("fp4q_payload_bytes", "fp4q_compress", "fp4q_compress_ex", "fp4q_decompress",
                  "fp4q_decompress_ex", "fp4q_decompress_accumulate",
                  "fp4q_decompress_accumulate_ex", "fp4q_reduce_requantize", "fp4q_reduce_requantize_ex",
                  "fp4q_compress_mx", "fp4q_decompress_mx"):
            getattr(L, f).restype = I
        _lib = L
    return _lib


def fp4q_status_str(status: int) -> str:
    return lib().fp4q_status_str(int(status)).decode()


def _check(status: int) -> None:
    if status != FP4Q_OK:
        raise Fp4qError(status)


def fp4q_payload_bytes(rows: int, row_len: int):
    c, m, b = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().fp4q_payload_bytes(rows, row_len, ctypes.byref(c), ctypes.byref(m),
                                    ctypes.byref(b)))
    return c.value, m.value, b.value


def _stream(stream, device):
    """The HIP stream to launch on: the given torch stream, else the current
    stream of the tensors' device (a stream belongs to one device)."""
    import torch
    s = torch.cuda.current_stream(device) if stream is None else stream
    if s.device != device:
        raise ValueError("fp4q: stream is on %s, tensors on %s" % (s.device, device))
    return ctypes.c_void_p(s.cuda_stream)


def _empty(shape, dtype, device, stream):
    """An output tensor allocated for the stream the kernel will run on, so that
    torch's caching allocator does not hand its memory to other work while that
    stream may still be writing it."""
    import torch
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dims(x):
    if x.dim() != 2:
        raise ValueError("fp4q: expected a 2-D tensor [rows, row_len]")
    if not x.is_contiguous():
        raise ValueError("fp4q: expected a contiguous tensor")
    return int(x.shape[0]), int(x.shape[1])


_BF16_BITS = ("bfloat16", "int16", "uint16")
_DTYPES = {}


def _dtypes(names):
    """The torch dtypes named (cached: the check runs on every call)."""
    d = _DTYPES.get(names)
    if d is None:
        import torch
        d = _DTYPES[names] = frozenset(getattr(torch, n) for n in names)
    return d


def _arg(t, name, numel, dtypes):
    """Check one tensor argument before its address goes to the library, which
    sees only pointers: its type, element type, contiguity and element count (a
    buffer too small or strided would otherwise be read or written out of bounds
    by a kernel).  _on_gpu checks the devices afterwards."""
    try:
        ok = t.dtype in _dtypes(dtypes)
    except AttributeError:
        raise TypeError("fp4q: %s must be a torch tensor" % name) from None
    if not ok:
        raise TypeError("fp4q: %s must be %s, got %s" % (name, " or ".join(dtypes), t.dtype))
    if not t.is_contiguous():
        raise ValueError("fp4q: %s must be contiguous" % name)
    if t.numel() != numel:
        raise ValueError("fp4q: %s must hold %d elements, has %d" % (name, numel, t.numel()))
    return t


def _on_gpu(*tensors):
    """Every tensor argument in device memory, all on the same GPU; returns it."""
    dev = tensors[0].device
    for t in tensors:
        if t.device.type != "cuda" or t.device != dev:
            raise ValueError("fp4q: every tensor must be on the same GPU (%s, %s)" % (dev, t.device))
    return dev


def _payload_args(codes, micro, block, n, who):
    _arg(codes, who + " codes", n // 2, ("uint8",))
    _arg(micro, who + " micro-scales", n // FP4Q_GROUP, ("uint8",))
    _arg(block, who + " block scales", n // FP4Q_BLOCK, ("float32",))
    return [codes, micro, block]


def fp4q_compress(x, codes=None, micro_scales=None, block_scales=None, flags: int = 0,
                  stream=None):
    """bf16 [rows, row_len] (CUDA) -> (codes u8 [rows, L/2], micro u8 [rows, L/16],
    block f32 [rows, L/256]).  Output tensors are allocated when not given."""
    import torch
    rows, L = _dims(x)
    _arg(x, "input", rows * L, _BF16_BITS)
    dev = x.device
    if codes is None:
        codes = _empty((rows, L // 2), torch.uint8, dev, stream)
    if micro_scales is None:
        micro_scales = _empty((rows, L // 16), torch.uint8, dev, stream)
    if block_scales is None:
        block_scales = _empty((rows, L // 256), torch.float32, dev, stream)
    gpu = _on_gpu(x, *_payload_args(codes, micro_scales, block_scales, rows * L, "output"))
    _check(lib().fp4q_compress_ex(_ptr(x), rows, L, _ptr(codes), _ptr(micro_scales),
                                  _ptr(block_scales), flags, _stream(stream, gpu)))
    return codes, micro_scales, block_scales


def _out_dtype_code(dtype):
    import torch
    if dtype == torch.float32:
        return FP4Q_OUT_F32
    if dtype == torch.bfloat16:
        return FP4Q_OUT_BF16
    raise TypeError("fp4q: output dtype must be float32 or bfloat16")


def fp4q_decompress(codes, micro_scales, block_scales, out=None, out_dtype=None, flags: int = 0,
                    stream=None):
    """Payload -> [rows, row_len] float32 (or bfloat16)."""
    import torch
    rows, half = _dims(codes)
    L = 2 * half
    pay = _payload_args(codes, micro_scales, block_scales, rows * L, "payload")
    if out is None:
        out = _empty((rows, L), out_dtype or torch.float32, codes.device, stream)
    gpu = _on_gpu(*pay, _arg(out, "output", rows * L, ("float32", "bfloat16")))
    _check(lib().fp4q_decompress_ex(_ptr(codes), _ptr(micro_scales), _ptr(block_scales), rows, L,
                                    _ptr(out), _out_dtype_code(out.dtype), flags,
                                    _stream(stream, gpu)))
    return out


def fp4q_decompress_accumulate(payloads, out=None, out_dtype=None, flags: int = 0, stream=None):
    """Sum of k peers' payloads [(codes, micro, block), ...] -> float32 (or bf16)."""
    import torch
    k = len(payloads)
    if not 1 <= k <= FP4Q_MAX_PEERS:
        raise Fp4qError(FP4Q_ERR_K)
    rows, half = _dims(payloads[0][0])
    L = 2 * half
    dev = payloads[0][0].device
    ins = []
    for i, (c, m, b) in enumerate(payloads):
        ins += _payload_args(c, m, b, rows * L, "peer %d" % i)
    if out is None:
        out = _empty((rows, L), out_dtype or torch.float32, dev, stream)
    gpu = _on_gpu(*ins, _arg(out, "output", rows * L, ("float32", "bfloat16")))
    PA = ctypes.c_void_p * max(k, 1)
    cs = PA(*[p[0].data_ptr() for p in payloads])
    ms = PA(*[p[1].data_ptr() for p in payloads])
    bs = PA(*[p[2].data_ptr() for p in payloads])
    cast = lambda a: ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p))
    _check(lib().fp4q_decompress_accumulate_ex(k, cast(cs), cast(ms), cast(bs), rows, L,
                                               _ptr(out), _out_dtype_code(out.dtype), flags,
                                               _stream(stream, gpu)))
    return out


def fp4q_reduce_requantize(payloads, codes=None, micro_scales=None, block_scales=None,
                           local=None, flags: int = 0, stream=None):
    """Sum k peers' payloads [(codes, micro, block), ...] in the transform domain,
    starting from the transformed local bf16 slice when ``local`` is given, and
    quantise the sum again -> (codes, micro, block) of the same shape."""
    import torch
    k = len(payloads)
    if k > FP4Q_MAX_PEERS or (k == 0 and local is None):
        raise Fp4qError(FP4Q_ERR_K)
    if k:
        rows, half = _dims(payloads[0][0])
        L = 2 * half
        dev = payloads[0][0].device
    else:
        rows, L = _dims(local)
        dev = local.device
    ins = []
    for i, (c, m, b) in enumerate(payloads):
        ins += _payload_args(c, m, b, rows * L, "peer %d" % i)
    if local is not None:
        ins.append(_arg(local, "local slice", rows * L, _BF16_BITS))
    if codes is None:
        codes = _empty((rows, L // 2), torch.uint8, dev, stream)
    if micro_scales is None:
        micro_scales = _empty((rows, L // 16), torch.uint8, dev, stream)
    if block_scales is None:
        block_scales = _empty((rows, L // 256), torch.float32, dev, stream)
    gpu = _on_gpu(*ins, *_payload_args(codes, micro_scales, block_scales, rows * L, "output"))
    PA = ctypes.c_void_p * max(k, 1)
    cast = lambda a: ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p))
    cs = PA(*[p[0].data_ptr() for p in payloads])
    ms = PA(*[p[1].data_ptr() for p in payloads])
    bs = PA(*[p[2].data_ptr() for p in payloads])
    _check(lib().fp4q_reduce_requantize_ex(
        k, cast(cs), cast(ms), cast(bs), _ptr(local) if local is not None else None, rows, L,
        _ptr(codes), _ptr(micro_scales), _ptr(block_scales), flags, _stream(stream, gpu)))
    return codes, micro_scales, block_scales


def fp4q_compress_mx(x, codes=None, scales=None, flags: int = 0, stream=None):
    """MXFP4-style: bf16 [rows, L] -> (codes u8 [rows, L/2], E8M0 scales u8 [rows, L/32])."""
    import torch
    rows, L = _dims(x)
    _arg(x, "input", rows * L, _BF16_BITS)
    if codes is None:
        codes = _empty((rows, L // 2), torch.uint8, x.device, stream)
    if scales is None:
        scales = _empty((rows, L // 32), torch.uint8, x.device, stream)
    gpu = _on_gpu(x, _arg(codes, "output codes", rows * L // 2, ("uint8",)),
            _arg(scales, "output scales", rows * L // 32, ("uint8",)))
    _check(lib().fp4q_compress_mx(_ptr(x), rows, L, _ptr(codes), _ptr(scales), flags,
                                  _stream(stream, gpu)))
    return codes, scales


def fp4q_decompress_mx(codes, scales, out=None, out_dtype=None, flags: int = 0, stream=None):
    """MXFP4-style payload -> [rows, row_len] float32 (or bfloat16)."""
    import torch
    rows, half = _dims(codes)
    L = 2 * half
    _arg(codes, "codes", rows * L // 2, ("uint8",))
    _arg(scales, "scales", rows * L // 32, ("uint8",))
    if out is None:
        out = _empty((rows, L), out_dtype or torch.float32, codes.device, stream)
    gpu = _on_gpu(codes, scales, _arg(out, "output", rows * L, ("float32", "bfloat16")))
    _check(lib().fp4q_decompress_mx(_ptr(codes), _ptr(scales), rows, L, _ptr(out),
                                    _out_dtype_code(out.dtype), flags, _stream(stream, gpu)))
    return out
