"""mx_prefetch reads and discards: the data and every result computed from it
are unchanged, on the launch stream and on a side stream, for ragged sizes."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp8xfp4_amd import mxmoe
from gpu_common import dev, host

pytestmark = pytest.mark.gpu


def test_prefetch_leaves_data_and_results_unchanged():
    rng = np.random.default_rng(1)
    a = rng.standard_normal((16, 1024)).astype(np.float32)
    w = (rng.standard_normal((512, 1024)) * 0.02).astype(np.float32)
    aq, asc = oracle.quantize_e4m3(a)
    wq, wsc = oracle.quantize_e4m3(w)
    da, dasc, dw, dwsc = dev(aq), dev(asc), dev(wq), dev(wsc)
    before = host(dw).copy()
    y0 = torch.empty((16, 512), dtype=torch.float32, device="cuda")
    mxmoe.fp8_block_gemm(da, dasc, dw, dwsc, y0, mxmoe.MX_OUT_F32)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mxmoe.prefetch(dw, 16 * 1024)                            # one 16-row slice per workgroup
        mxmoe.prefetch(dwsc, 0)
        mxmoe.prefetch(dw, 48, nbytes=dw.numel() - 8)            # ragged: the trailing partial unit is skipped
    torch.cuda.current_stream().wait_stream(side)
    mxmoe.prefetch(dw)
    y1 = torch.empty_like(y0)
    mxmoe.fp8_block_gemm(da, dasc, dw, dwsc, y1, mxmoe.MX_OUT_F32)
    assert np.array_equal(host(dw), before)
    assert torch.equal(y0, y1)
