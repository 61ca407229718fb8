"""The Python binding rejects tensor arguments the C library cannot check (it sees
only pointers) before any library call: wrong element type, strided, too few or
too many elements, host memory, wrong peer count.  Runs without a GPU."""
import pytest

torch = pytest.importorskip("torch")

import fp4_communication_compression_amd as fp4q


def bf16(rows, L):
    return torch.zeros((rows, L), dtype=torch.bfloat16)


def payload(rows, L):
    n = rows * L
    return (torch.zeros((rows, L // 2), dtype=torch.uint8),
            torch.zeros((rows, L // 16), dtype=torch.uint8),
            torch.zeros((rows, L // 256), dtype=torch.float32))


def test_compress_arguments():
    with pytest.raises(TypeError):
        fp4q.fp4q_compress(torch.zeros((4, 256), dtype=torch.float32))
    with pytest.raises(ValueError, match="contiguous"):
        fp4q.fp4q_compress(bf16(256, 4).t())
    with pytest.raises(ValueError, match="2-D"):
        fp4q.fp4q_compress(torch.zeros(1024, dtype=torch.bfloat16))
    c, m, b = payload(4, 256)
    with pytest.raises(ValueError, match="elements"):
        fp4q.fp4q_compress(bf16(4, 256), c[:2], m, b)              # codes too small
    with pytest.raises(TypeError):
        fp4q.fp4q_compress(bf16(4, 256), c, m, b.double())         # block scales not fp32
    with pytest.raises(ValueError, match="GPU"):
        fp4q.fp4q_compress(bf16(4, 256))                            # host memory


def test_decompress_arguments():
    c, m, b = payload(4, 512)
    with pytest.raises(ValueError, match="elements"):
        fp4q.fp4q_decompress(c, torch.zeros((4, 8), dtype=torch.uint8), b)
    with pytest.raises(ValueError, match="elements"):
        fp4q.fp4q_decompress(c, m, b, out=torch.zeros((4, 256), dtype=torch.float32))
    with pytest.raises(TypeError):
        fp4q.fp4q_decompress(c, m, b, out=torch.zeros((4, 512), dtype=torch.float16))
    with pytest.raises(ValueError, match="contiguous"):
        fp4q.fp4q_decompress(c, m, b, out=torch.zeros((512, 4), dtype=torch.float32).t())
    with pytest.raises(ValueError, match="GPU"):
        fp4q.fp4q_decompress(c, m, b)


def test_accumulate_and_requantize_arguments():
    p = payload(2, 1024)
    with pytest.raises(fp4q.Fp4qError) as e:
        fp4q.fp4q_decompress_accumulate([])
    assert e.value.status == fp4q.FP4Q_ERR_K
    with pytest.raises(fp4q.Fp4qError) as e:
        fp4q.fp4q_decompress_accumulate([p] * 17)
    assert e.value.status == fp4q.FP4Q_ERR_K
    with pytest.raises(ValueError, match="peer 1"):
        fp4q.fp4q_decompress_accumulate([p, payload(1, 1024)])      # peers of different sizes
    with pytest.raises(fp4q.Fp4qError) as e:
        fp4q.fp4q_reduce_requantize([])                            # no peer and no local slice
    assert e.value.status == fp4q.FP4Q_ERR_K
    with pytest.raises(ValueError, match="local"):
        fp4q.fp4q_reduce_requantize([p], local=bf16(2, 512))
    with pytest.raises(TypeError):
        fp4q.fp4q_reduce_requantize([p], local=torch.zeros((2, 1024), dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU"):
        fp4q.fp4q_reduce_requantize([p], local=bf16(2, 1024))


def test_mx_arguments():
    with pytest.raises(ValueError, match="elements"):
        fp4q.fp4q_compress_mx(bf16(4, 256), torch.zeros((4, 128), dtype=torch.uint8),
                              torch.zeros((4, 4), dtype=torch.uint8))
    with pytest.raises(ValueError, match="elements"):
        fp4q.fp4q_decompress_mx(torch.zeros((4, 128), dtype=torch.uint8),
                                torch.zeros((4, 16), dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU"):
        fp4q.fp4q_decompress_mx(torch.zeros((4, 128), dtype=torch.uint8),
                                torch.zeros((4, 8), dtype=torch.uint8))


def test_missing_library_that_cannot_be_built_fails_loudly(tmp_path, monkeypatch):
    """No library and no way to build one: the binding raises instead of falling
    back to anything else."""
    from fp4_communication_compression_amd import _build
    missing = str(tmp_path / "libfp4q.so")
    monkeypatch.setattr(fp4q, "_lib", None)
    monkeypatch.setattr(fp4q, "LIB_PATH", missing)
    monkeypatch.setattr(_build, "LIB", missing)
    monkeypatch.setattr(_build, "HIPCC", "/bin/false")
    with pytest.raises(ImportError, match="could not be built"):
        fp4q.lib()
