"""The requant of the FFN intermediate converts with the hardware (clamp to
+-448, round to nearest even, OCP E4M3); the quantize kernels encode with
integer rounding.  Every finite float, with both signs, gets the same code
from both: the first is then exactly the E4M3 encoding the oracle pins
(post #6 "Why TileLang": FP8 quantization; OCP MX v1.0 "Conversion")."""
import pytest

from block_scaled_fp8xfp4_amd import mxmoe

pytestmark = pytest.mark.gpu


def test_hardware_requant_equals_the_encoder_on_every_finite_float():
    import torch
    mxmoe.load()
    n = torch.zeros(1, dtype=torch.int64, device="cuda")
    mxmoe.check_requant(0, 0x44000000, n)            # |x| < 512: every value the requant sees
    torch.cuda.synchronize()
    assert int(n.item()) == 0
    mxmoe.check_requant(0x44000000, 0x7F800000, n)   # the rest of the finite floats (saturate)
    torch.cuda.synchronize()
    assert int(n.item()) == 0
