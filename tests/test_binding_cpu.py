"""The Python binding's argument checks run on the host before any launch: an
output of the wrong shape, dtype or layout, or a bias of the wrong length, is
refused -- shape and dtype before anything touches a device (no GPU here)."""
import pytest
import torch

import microscaling_quantized_dit_amd as mxq


def test_outputs_checked_before_device():
    good = [("q", torch.uint8, (4, 64)), ("scales", torch.uint8, (4, 2))]
    with pytest.raises(ValueError, match="shape"):
        mxq._outputs((torch.empty((4, 63), dtype=torch.uint8), torch.empty((4, 2), dtype=torch.uint8)), good, None)
    with pytest.raises(TypeError, match="uint8"):
        mxq._outputs((torch.empty((4, 64), dtype=torch.float32), torch.empty((4, 2), dtype=torch.uint8)), good, None)
    with pytest.raises(ValueError, match="must hold 2"):
        mxq._outputs((torch.empty((4, 64), dtype=torch.uint8),), good, None)
    # the right shape and dtype reach the residency check (a CPU tensor here)
    with pytest.raises(ValueError, match="GPU"):
        mxq._outputs((torch.empty((4, 64), dtype=torch.uint8), torch.empty((4, 2), dtype=torch.uint8)), good, None)


def test_bias_length_checked():
    with pytest.raises(ValueError, match="GPU"):
        mxq._bias(torch.empty((256,), dtype=torch.bfloat16), 256, None)
    with pytest.raises(TypeError, match="bfloat16"):
        mxq._bias(torch.empty((256,), dtype=torch.float32), 256, None)


def test_need_checks_shape_before_residency():
    with pytest.raises(ValueError, match="shape"):
        mxq._need(torch.empty((3, 5), dtype=torch.uint8), torch.uint8, "w_q", None, (3, 4))
    with pytest.raises(ValueError, match="GPU"):
        mxq._need(torch.empty((3, 4), dtype=torch.uint8), torch.uint8, "w_q", None, (3, 4))


def test_entry_points_refuse_non_2d_and_cpu_inputs():
    with pytest.raises(ValueError, match="2-D"):
        mxq.quantize_mxfp8(torch.empty((4, 4, 4), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="GPU"):
        mxq.quantize_nvfp4(torch.empty((4, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="2-D"):
        mxq.gemm_mxfp8(torch.empty((128,), dtype=torch.uint8), None, None, None)
