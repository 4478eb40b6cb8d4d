"""The streaming-read probe that bench.py --ceilings loads (libmoe_fp4_probe.so): it
refuses arguments that would read past the caller's buffer before it launches
anything, and on a GPU one small launch completes without touching its sink."""
import ctypes
import os

import pytest

from conftest import ROOT

PROBE = os.path.join(ROOT, "block_scaled_fp4_05_amd", "libmoe_fp4_probe.so")


def _probe():
    if not os.path.exists(PROBE):
        from block_scaled_fp4_05_amd import build
        build.build_probe()
    L = ctypes.CDLL(PROBE)
    fn = L.moe_fp4_stream_probe
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return fn


# (buf_bytes, per_wave, stages, waves, layout, nt): each is refused on the host.
REFUSED = [
    (0, 32768, 2, 4, 0, 0),                      # empty buffer
    (1 << 31, 1 << 20, 2, 4, 0, 0),              # beyond one buffer resource
    (1 << 20, 32768, 1, 4, 0, 0),                # fewer than two stages
    (1 << 20, 32768, 2, 3, 0, 0),                # waves not a multiple of 4
    (1 << 20, 32768, 2, 0, 0, 0),                # no waves
    (1 << 20, 32768, 2, 4, 2, 0),                # unknown layout
    (1 << 20, 32768, 2, 4, 0, 2),                # unknown hint
    (1 << 20, 16384, 2, 4, 0, 0),                # region shorter than its stages
    (4 * 32768 - 1, 32768, 2, 4, 0, 0),          # regions past the buffer's end
    (4 * 2 * 16384 - 1, 0, 2, 4, 1, 0),          # interleaved pieces past the end
]


@pytest.mark.parametrize("args", REFUSED)
def test_probe_refuses_out_of_range_arguments(args):
    fn = _probe()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every case fails validation first
    assert fn(fake, *args, fake, None) == 1


def test_probe_refuses_null_pointers():
    fn = _probe()
    fake = ctypes.c_void_p(0x1000)
    assert fn(None, 1 << 20, 32768, 2, 4, 0, 0, fake, None) == 1
    assert fn(fake, 1 << 20, 32768, 2, 4, 0, 0, None, None) == 1


@pytest.mark.gpu
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("nt", [0, 1])
def test_probe_runs_on_a_small_buffer(layout, nt):
    import torch
    fn = _probe()
    waves, stages, per_wave = 8, 4, 4 * 16384
    buf = torch.arange(waves * per_wave, dtype=torch.int64, device="cuda").to(torch.uint8)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert fn(buf.data_ptr(), buf.numel(), per_wave, stages, waves, layout, nt,
              sink.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
