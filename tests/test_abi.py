"""C-ABI checks that need no GPU: the library loads, exports every declared
entry point, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import fp4_communication_compression_amd as fp4q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4q.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4q_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = fp4q.lib()
    names = declared_functions()
    assert names == sorted(["fp4q_payload_bytes", "fp4q_compress", "fp4q_compress_ex",
                            "fp4q_decompress", "fp4q_decompress_ex", "fp4q_decompress_accumulate",
                            "fp4q_decompress_accumulate_ex", "fp4q_reduce_requantize",
                            "fp4q_reduce_requantize_ex",
                            "fp4q_compress_mx", "fp4q_decompress_mx", "fp4q_status_str"])
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for s in range(7):
        assert fp4q.fp4q_status_str(s)
    assert fp4q.fp4q_status_str(99) == "unknown status"


def test_payload_bytes():
    assert fp4q.fp4q_payload_bytes(32768, 4096) == (67108864, 8388608, 2097152)
    assert fp4q.fp4q_payload_bytes(4096, 11008) == (22544384, 2818048, 704512)
    assert fp4q.fp4q_payload_bytes(0, 256) == (0, 0, 0)
    for rows, L in ((1, 255), (1, 0), (-1, 256), (1, 300), (1 << 62, 256)):
        with pytest.raises(fp4q.Fp4qError) as e:
            fp4q.fp4q_payload_bytes(rows, L)
        assert e.value.status == fp4q.FP4Q_ERR_SHAPE


# Fake device addresses: validation must reject them before touching the GPU.
# Where a GPU is visible these tests do not run: a validation regression would
# then launch a kernel on unmapped memory.  (The host-only sanitizer build makes
# the same rejected calls with no device at all.)
A = 1 << 20  # 16-byte aligned
NULL = None


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0   # counts devices without initialising one
    except Exception:
        return False


fake_addresses = pytest.mark.skipif(_gpu_visible(), reason="fake device addresses: CPU-only host")


def comp(x, rows, L, c, m, b, flags=0):
    return fp4q.lib().fp4q_compress_ex(x, rows, L, c, m, b, flags, None)


def decomp(c, m, b, rows, L, out, dt=0, flags=0):
    return fp4q.lib().fp4q_decompress_ex(c, m, b, rows, L, out, dt, flags, None)


def acc(k, cs, ms, bs, rows, L, out, dt=0, flags=0):
    PA = ctypes.c_void_p * max(len(cs), 1)
    cast = lambda a: ctypes.cast(PA(*a), ctypes.POINTER(ctypes.c_void_p))
    return fp4q.lib().fp4q_decompress_accumulate_ex(k, cast(cs), cast(ms), cast(bs), rows, L,
                                                    out, dt, flags, None)


@fake_addresses
def test_compress_validation_order():
    big = 1 << 30
    assert comp(A, 1, 300, A + big, A + 2 * big, A + 3 * big) == fp4q.FP4Q_ERR_SHAPE
    assert comp(A, -1, 256, A + big, A + 2 * big, A + 3 * big) == fp4q.FP4Q_ERR_SHAPE
    assert comp(A, 1 << 60, 256, A + big, A + 2 * big, A + 3 * big) == fp4q.FP4Q_ERR_SHAPE
    assert comp(A, 1, 256, A + big, A + 2 * big, A + 3 * big, flags=2) == fp4q.FP4Q_ERR_ARG
    assert comp(NULL, 0, 256, NULL, NULL, NULL) == fp4q.FP4Q_OK          # empty: no launch
    assert comp(NULL, 1, 256, A + big, A + 2 * big, A + 3 * big) == fp4q.FP4Q_ERR_NULL
    assert comp(A, 1, 256, NULL, A + 2 * big, A + 3 * big) == fp4q.FP4Q_ERR_NULL
    assert comp(A, 1, 256, A + big, NULL, A + 3 * big) == fp4q.FP4Q_ERR_NULL
    assert comp(A, 1, 256, A + big, A + 2 * big, NULL) == fp4q.FP4Q_ERR_NULL
    assert comp(A + 2, 1, 256, A + big, A + 2 * big, A + 3 * big) == fp4q.FP4Q_ERR_ALIGN
    assert comp(A, 1, 256, A + big + 4, A + 2 * big, A + 3 * big) == fp4q.FP4Q_ERR_ALIGN
    assert comp(A, 1, 256, A + big, A + 2 * big + 2, A + 3 * big) == fp4q.FP4Q_ERR_ALIGN
    assert comp(A, 1, 256, A + big, A + 2 * big + 4, A + 3 * big) == fp4q.FP4Q_ERR_ALIGN  # micro: 16
    assert comp(A, 1, 256, A + big, A + 2 * big, A + 3 * big + 1) == fp4q.FP4Q_ERR_ALIGN
    # overlaps: codes inside the input, micro on codes, block on micro
    assert comp(A, 4, 256, A + 16, A + 2 * big, A + 3 * big) == fp4q.FP4Q_ERR_ARG
    assert comp(A, 4, 256, A + big, A + big + 16, A + 3 * big) == fp4q.FP4Q_ERR_ARG
    assert comp(A, 4, 256, A + big, A + 2 * big, A + 2 * big + 4) == fp4q.FP4Q_ERR_ARG


@fake_addresses
def test_decompress_validation_order():
    big = 1 << 30
    args = (A, A + big, A + 2 * big)
    assert decomp(*args, 1, 128, A + 3 * big) == fp4q.FP4Q_ERR_SHAPE
    assert decomp(*args, 1, 256, A + 3 * big, dt=2) == fp4q.FP4Q_ERR_ARG
    assert decomp(*args, 1, 256, A + 3 * big, flags=4) == fp4q.FP4Q_ERR_ARG
    assert decomp(NULL, NULL, NULL, 0, 256, NULL) == fp4q.FP4Q_OK
    assert decomp(A, A + big, A + 2 * big, 1, 256, NULL) == fp4q.FP4Q_ERR_NULL
    assert decomp(NULL, A + big, A + 2 * big, 1, 256, A + 3 * big) == fp4q.FP4Q_ERR_NULL
    assert decomp(*args, 1, 256, A + 3 * big + 8) == fp4q.FP4Q_ERR_ALIGN
    assert decomp(A + 8, A + big, A + 2 * big, 1, 256, A + 3 * big) == fp4q.FP4Q_ERR_ALIGN
    assert decomp(A, A + big + 4, A + 2 * big, 1, 256, A + 3 * big) == fp4q.FP4Q_ERR_ALIGN
    assert decomp(*args, 4, 256, A + 64) == fp4q.FP4Q_ERR_ARG        # output over the codes


@fake_addresses
def test_accumulate_validation_order():
    big = 1 << 30
    cs, ms, bs = [A], [A + big], [A + 2 * big]
    out = A + 3 * big
    assert acc(1, cs, ms, bs, 1, 100, out) == fp4q.FP4Q_ERR_SHAPE
    assert acc(0, cs, ms, bs, 1, 256, out) == fp4q.FP4Q_ERR_K
    assert acc(17, cs * 17, ms * 17, bs * 17, 1, 256, out) == fp4q.FP4Q_ERR_K
    assert acc(1, cs, ms, bs, 1, 256, out, dt=7) == fp4q.FP4Q_ERR_ARG
    assert acc(1, cs, ms, bs, 1, 256, out, flags=8) == fp4q.FP4Q_ERR_ARG
    assert acc(1, cs, ms, bs, 0, 256, out) == fp4q.FP4Q_OK
    assert acc(1, cs, ms, bs, 1, 256, NULL) == fp4q.FP4Q_ERR_NULL
    assert acc(2, cs + [NULL], ms * 2, bs * 2, 1, 256, out) == fp4q.FP4Q_ERR_NULL
    assert acc(1, cs, ms, bs, 1, 256, out + 4) == fp4q.FP4Q_ERR_ALIGN
    assert acc(2, cs + [A + 4], ms * 2, bs * 2, 1, 256, out) == fp4q.FP4Q_ERR_ALIGN
    assert acc(2, cs * 2, ms + [A + big + 8], bs * 2, 1, 256, out) == fp4q.FP4Q_ERR_ALIGN
    assert acc(1, [out + 16], ms, bs, 4, 256, out) == fp4q.FP4Q_ERR_ARG   # overlap with out


def req(k, cs, ms, bs, rows, L, oc, om, ob):
    PA = ctypes.c_void_p * max(len(cs), 1)
    cast = lambda a: ctypes.cast(PA(*a), ctypes.POINTER(ctypes.c_void_p))
    return fp4q.lib().fp4q_reduce_requantize(k, cast(cs), cast(ms), cast(bs), rows, L, oc, om, ob,
                                             None)


@fake_addresses
def test_requantize_validation_order():
    big = 1 << 30
    cs, ms, bs = [A], [A + big], [A + 2 * big]
    outs = (A + 3 * big, A + 4 * big, A + 5 * big)
    assert req(1, cs, ms, bs, 1, 200, *outs) == fp4q.FP4Q_ERR_SHAPE
    assert req(0, cs, ms, bs, 1, 256, *outs) == fp4q.FP4Q_ERR_K
    assert req(17, cs * 17, ms * 17, bs * 17, 1, 256, *outs) == fp4q.FP4Q_ERR_K
    assert req(1, cs, ms, bs, 0, 256, *outs) == fp4q.FP4Q_OK
    assert req(1, cs, ms, bs, 1, 256, NULL, outs[1], outs[2]) == fp4q.FP4Q_ERR_NULL
    assert req(2, cs + [NULL], ms * 2, bs * 2, 1, 256, *outs) == fp4q.FP4Q_ERR_NULL
    assert req(1, cs, ms, bs, 1, 256, outs[0] + 8, outs[1], outs[2]) == fp4q.FP4Q_ERR_ALIGN
    assert req(1, cs, ms, bs, 1, 256, outs[0], outs[1] + 2, outs[2]) == fp4q.FP4Q_ERR_ALIGN
    assert req(1, cs, ms, bs, 1, 256, outs[0], outs[1] + 4, outs[2]) == fp4q.FP4Q_ERR_ALIGN
    assert req(1, cs, [A + big + 4], bs, 1, 256, *outs) == fp4q.FP4Q_ERR_ALIGN
    assert req(1, cs, ms, bs, 4, 256, A + 16, outs[1], outs[2]) == fp4q.FP4Q_ERR_ARG   # over input codes
    assert req(1, cs, ms, bs, 4, 256, outs[0], outs[0] + 16, outs[2]) == fp4q.FP4Q_ERR_ARG


def req_ex(k, cs, ms, bs, local, rows, L, oc, om, ob, flags=0):
    PA = ctypes.c_void_p * max(len(cs), 1)
    cast = lambda a: ctypes.cast(PA(*a), ctypes.POINTER(ctypes.c_void_p))
    return fp4q.lib().fp4q_reduce_requantize_ex(k, cast(cs), cast(ms), cast(bs), local, rows, L,
                                                oc, om, ob, flags, None)


@fake_addresses
def test_requantize_ex_validation_order():
    big = 1 << 30
    cs, ms, bs = [A], [A + big], [A + 2 * big]
    outs = (A + 3 * big, A + 4 * big, A + 5 * big)
    local = A + 6 * big
    assert req_ex(1, cs, ms, bs, local, 1, 100, *outs) == fp4q.FP4Q_ERR_SHAPE
    assert req_ex(0, [], [], [], NULL, 1, 256, *outs) == fp4q.FP4Q_ERR_K      # k = 0 needs local
    assert req_ex(-1, [], [], [], local, 1, 256, *outs) == fp4q.FP4Q_ERR_K
    assert req_ex(17, cs * 17, ms * 17, bs * 17, local, 1, 256, *outs) == fp4q.FP4Q_ERR_K
    assert req_ex(1, cs, ms, bs, local, 1, 256, *outs, flags=2) == fp4q.FP4Q_ERR_ARG
    assert req_ex(0, [], [], [], local, 0, 256, *outs) == fp4q.FP4Q_OK        # empty: no launch
    assert req_ex(0, [], [], [], local, 1, 256, NULL, outs[1], outs[2]) == fp4q.FP4Q_ERR_NULL
    assert req_ex(2, cs + [NULL], ms * 2, bs * 2, local, 1, 256, *outs) == fp4q.FP4Q_ERR_NULL
    assert req_ex(0, [], [], [], local + 8, 1, 256, *outs) == fp4q.FP4Q_ERR_ALIGN
    assert req_ex(1, cs, ms, bs, local, 1, 256, outs[0], outs[1] + 4, outs[2]) == fp4q.FP4Q_ERR_ALIGN
    # local slice over an output, or an output over the local slice
    assert req_ex(0, [], [], [], outs[0], 4, 256, *outs) == fp4q.FP4Q_ERR_ARG
    assert req_ex(0, [], [], [], local, 4, 256, local + 256, outs[1], outs[2]) == fp4q.FP4Q_ERR_ARG
    assert req_ex(1, cs, ms, bs, local, 4, 256, A + 16, outs[1], outs[2]) == fp4q.FP4Q_ERR_ARG


@fake_addresses
def test_mx_validation_order():
    big = 1 << 30
    c = fp4q.lib().fp4q_compress_mx
    d = fp4q.lib().fp4q_decompress_mx
    assert c(A, 1, 300, A + big, A + 2 * big, 0, None) == fp4q.FP4Q_ERR_SHAPE
    assert c(A, 1, 256, A + big, A + 2 * big, 2, None) == fp4q.FP4Q_ERR_ARG
    assert c(NULL, 0, 256, NULL, NULL, 0, None) == fp4q.FP4Q_OK
    assert c(A, 1, 256, A + big, NULL, 0, None) == fp4q.FP4Q_ERR_NULL
    assert c(A, 1, 256, A + big, A + 2 * big + 4, 0, None) == fp4q.FP4Q_ERR_ALIGN
    assert c(A, 4, 256, A + 64, A + 2 * big, 0, None) == fp4q.FP4Q_ERR_ARG
    assert d(A, A + big, 1, 256, A + 2 * big, 3, 0, None) == fp4q.FP4Q_ERR_ARG
    assert d(A, A + big, 1, 256, NULL, 0, 0, None) == fp4q.FP4Q_ERR_NULL
    assert d(A, A + big + 4, 1, 256, A + 2 * big, 0, 0, None) == fp4q.FP4Q_ERR_ALIGN
    assert d(A, A + big, 4, 256, A + 16, 0, 0, None) == fp4q.FP4Q_ERR_ARG
