"""Host-side checks of the MXFP8 linear layer (no GPU needed: they fail before
any kernel is launched)."""

import pytest
import torch

from mxfp8_block_scaled_quantize_amd.linear import MXFP8LinearFunction


@pytest.mark.parametrize("M,K,N", [(100, 128, 128), (128, 96, 128), (128, 128, 160)])
def test_rejects_shapes_not_multiple_of_128(M, K, N):
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    w = torch.zeros((N, K), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        MXFP8LinearFunction.apply(x, w, False)


def test_rejects_non_bf16_and_mismatched_weight():
    with pytest.raises(TypeError):
        MXFP8LinearFunction.apply(torch.zeros((128, 128)), torch.zeros((128, 128), dtype=torch.bfloat16), False)
    with pytest.raises(ValueError):
        MXFP8LinearFunction.apply(torch.zeros((128, 128), dtype=torch.bfloat16),
                                  torch.zeros((128, 256), dtype=torch.bfloat16), False)
