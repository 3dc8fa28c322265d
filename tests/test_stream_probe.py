"""The cold read-stream probe (libmla_stream.so, csrc/stream_read.hip) that
bench.py times as the practical read ceiling: it loads, exports its entry
point and rejects bad arguments before any device call (CPU); on a GPU it
reads a buffer, ragged sizes included."""
import ctypes
import os

import pytest

from mla_token_decode_amd import build as hipbuild


def _lib():
    if not os.path.exists(hipbuild.STREAM_LIB):
        pytest.fail(f"{hipbuild.STREAM_LIB} is missing: run the build first")
    lib = ctypes.CDLL(hipbuild.STREAM_LIB)
    lib.mla_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_void_p]
    lib.mla_stream_read.restype = ctypes.c_int
    return lib


def test_probe_rejects_bad_arguments_before_touching_a_device():
    lib = _lib()
    fake = 1 << 40  # never dereferenced: every call below fails its argument check
    sink = fake + 64
    assert lib.mla_stream_read(None, 1024, sink, 64, 0, None) == -1
    assert lib.mla_stream_read(fake, 1024, None, 64, 0, None) == -1
    assert lib.mla_stream_read(fake, 0, sink, 64, 0, None) == -1
    assert lib.mla_stream_read(fake, 1000, sink, 64, 0, None) == -1      # not a multiple of 16
    assert lib.mla_stream_read(fake + 8, 1024, sink, 64, 1, None) == -1  # not 16-byte aligned
    assert lib.mla_stream_read(fake, 1024, sink, 0, 0, None) == -1
    assert lib.mla_stream_read(fake, 1024, sink, 65537, 1, None) == -1
    assert lib.mla_stream_read(fake, 1024, sink, 64, 2, None) == -1      # no such layout


@pytest.mark.gpu
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (16, 8), (1 << 20, 64), ((1 << 20) + 48, 1024),
                                           (3 << 24, 4096)])
def test_probe_reads_a_buffer(nbytes, blocks, layout):
    import torch
    lib = _lib()
    buf = torch.arange(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    rc = lib.mla_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, layout,
                             torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    # the sink is written only by a lane whose XOR fold hits one fixed value
    assert int(sink.item()) in (0, 0x9E3779B9 - (1 << 32))
