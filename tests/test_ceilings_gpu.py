"""The measurement kernels of libsinkattn_ceilings (include/sinkattn_ceilings.h) launch and finish on
the GPU at small sizes: every entry point returns 0, the stream completes without an error, the
read kernels leave the output word untouched (it is written only for a value their fills cannot
produce), and the issue-cost loops record nonzero cycle and tick counts for every work-group.
bench.py times them at full size; these runs only show that each launch is well-formed."""
from __future__ import annotations

import ctypes
import os

import pytest
import torch

from gqa_learned_softmax_amd import _lib

LIB = os.path.join(os.path.dirname(_lib.DEFAULT_LIB_PATH), "libsinkattn_ceilings.so")

pytestmark = pytest.mark.gpu


def _lib_and_stream():
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required")
    lib = ctypes.CDLL(LIB)
    V, I = ctypes.c_void_p, ctypes.c_int
    lib.sinkattn_ceiling_stream_read.argtypes = [V, ctypes.c_uint64, I, V, V]
    lib.sinkattn_ceiling_stream_read_slices.argtypes = [V, V, I, I, I, I, V, V]
    lib.sinkattn_ceiling_mfma_bf16.argtypes = [I, I, V, V]
    lib.sinkattn_ceiling_mfma_bf16_random.argtypes = [I, I, V, V]
    lib.sinkattn_ceiling_issue.argtypes = [I, I, I, V, V, V]
    return lib, V(torch.cuda.current_stream().cuda_stream)


def test_read_kernels_launch_and_leave_the_output_word_alone():
    lib, stream = _lib_and_stream()
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    buf = torch.full((1 << 20,), 1, dtype=torch.uint8, device="cuda")
    assert lib.sinkattn_ceiling_stream_read(buf.data_ptr(), buf.numel(), 64, out.data_ptr(), stream) == 0
    # 2 sequences x 2 chunks x 64 rows of 1 KB in K and in V: 16 work-groups of 512 threads.
    k = torch.full((2 * 2 * 64 * 1024,), 1, dtype=torch.uint8, device="cuda")
    v = torch.full_like(k, 2)
    assert lib.sinkattn_ceiling_stream_read_slices(k.data_ptr(), v.data_ptr(), 2, 2, 64, 1024, out.data_ptr(),
                                                   stream) == 0
    torch.cuda.synchronize()
    assert int(out.item()) == 0


def test_mfma_loops_launch():
    lib, stream = _lib_and_stream()
    out = torch.zeros(1, dtype=torch.float32, device="cuda")
    assert lib.sinkattn_ceiling_mfma_bf16(8, 10, out.data_ptr(), stream) == 0
    assert lib.sinkattn_ceiling_mfma_bf16_random(8, 10, out.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    assert float(out.item()) == 0.0


@pytest.mark.parametrize("kind", range(8))
def test_issue_loops_record_their_clocks(kind):
    lib, stream = _lib_and_stream()
    blocks = 8
    clk = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
    out = torch.zeros(1, dtype=torch.float32, device="cuda")
    assert lib.sinkattn_ceiling_issue(kind, blocks, 10, clk.data_ptr(), out.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    c = clk.cpu().view(blocks, 2)
    assert bool((c[:, 0] > 0).all()), "shader-clock cycles"
    assert bool((c[:, 1] >= 0).all()), "100 MHz ticks"
