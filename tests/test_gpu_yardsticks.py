"""The measurement yardsticks of qgemm_probe.h run and report sane figures.

They compute nothing that is compared with the oracle: the read kernels must
leave their sink untouched, the MFMA issue loop must record a shader clock
between 100 MHz and 5 GHz for every workgroup (s_memtime against the 100 MHz
s_memrealtime counter) and leave its sink untouched, and the empty kernel must
launch in every shape the benchmark uses.
"""
import pytest
import torch

import grouped_gemm_qgemm_amd as q
from gpu_util import say

pytestmark = pytest.mark.gpu


def test_read_kernels_leave_sink(gpu):
    sink = torch.zeros(4, dtype=torch.int32, device=gpu)
    src = torch.arange(1 << 20, dtype=torch.int32, device=gpu)
    q.read_contiguous(src, sink, 512)
    q.read_strips(src.view(1024, 1024), 64, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_mfma_loop_clocks(gpu, kind):
    wg = 256
    say(f"[yardstick] mfma_loop kind {kind}")
    clocks = torch.zeros(2 * wg, dtype=torch.int64, device=gpu)
    sink = torch.zeros(4, dtype=torch.int32, device=gpu)
    q.mfma_loop(kind, 64, wg, clocks, sink)
    torch.cuda.synchronize()
    c = clocks.view(wg, 2).cpu().double()
    assert bool((c > 0).all())
    mhz = c[:, 0] / c[:, 1] * 100.0
    assert bool(((mhz > 100) & (mhz < 5000)).all()), (float(mhz.min()), float(mhz.max()))
    assert int(sink.abs().sum()) == 0


@pytest.mark.parametrize("shape", [(256, 512), (1, 64), (1024, 1024)])
def test_empty_launch(gpu, shape):
    q.empty_launch(*shape)
    torch.cuda.synchronize()
