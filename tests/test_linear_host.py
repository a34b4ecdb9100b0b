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


def test_helpers_reject_bad_tensors_before_any_launch():
    """The allocating helpers check dtype, shape, contiguity and device on the
    host (CPU tensors are refused before the library is called)."""
    import pytest
    import torch

    import mxfp8_block_scaled_quantize_amd as mx
    x = torch.zeros((64, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="CUDA"):
        mx.quantize(x)
    with pytest.raises(ValueError, match="BF16"):
        mx.quantize(x.float())
    with pytest.raises(ValueError, match="unit column stride"):
        mx.quantize(torch.zeros((64, 128), dtype=torch.bfloat16)[:, ::2])
    a = torch.zeros((64, 128), dtype=torch.uint8)
    p = torch.zeros((1, 64), dtype=torch.int32)
    with pytest.raises(ValueError, match="CUDA"):
        mx.gemm(a, p, a, p)
    with pytest.raises(ValueError, match="2-D"):
        mx.gemm(a[0], p, a, p)
    with pytest.raises(ValueError, match="CUDA"):
        mx.grouped_gemm(a, p, a.reshape(1, 64, 128), p, torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError, match="uint8"):
        mx.pack_scales(torch.zeros((64, 4), dtype=torch.int32))


def test_module_weight_cache_key(monkeypatch):
    """MXFP8Linear.quantized_weight quantizes again exactly when the weight's
    version counter, storage or shape changes (host logic only: the quantizer
    is replaced by a stub that records its calls)."""
    import mxfp8_block_scaled_quantize_amd.linear as lin
    calls = []

    def stub(t, **kw):
        calls.append(t.data_ptr())
        return {"q_row": t, "p_row": t, "q_colT": t, "p_colT": t}

    monkeypatch.setattr(lin, "quantize", stub)
    layer = lin.MXFP8Linear(128, 256)
    first = layer.quantized_weight()
    assert layer.quantized_weight() is first and len(calls) == 1
    with torch.no_grad():
        layer.weight.add_(1.0)                  # in-place update: version counter moves
    assert layer.quantized_weight() is not first and len(calls) == 2
    again = layer.quantized_weight()
    assert len(calls) == 2
    layer.weight.data = torch.zeros((256, 128), dtype=torch.bfloat16)   # new storage
    assert layer.quantized_weight() is not again and len(calls) == 3


def test_bias_is_checked_before_any_launch():
    """A bias must be BF16 with one value per output feature; the GEMM helpers
    refuse a bias together with accumulate (host checks only)."""
    import mxfp8_block_scaled_quantize_amd as mx
    x = torch.zeros((128, 128), dtype=torch.bfloat16)
    w = torch.zeros((256, 128), dtype=torch.bfloat16)
    for bad in (torch.zeros(256), torch.zeros(128, dtype=torch.bfloat16), torch.zeros((1, 256), dtype=torch.bfloat16)):
        with pytest.raises(ValueError, match="bias"):
            MXFP8LinearFunction.apply(x, w, False, None, bad)
    a = torch.zeros((64, 128), dtype=torch.uint8)
    p = torch.zeros((1, 64), dtype=torch.int32)
    with pytest.raises(ValueError):
        mx.gemm(a, p, a, p, out=torch.zeros((64, 64), dtype=torch.bfloat16), accumulate=True,
                bias=torch.zeros(64, dtype=torch.bfloat16))


def test_module_with_bias_has_a_bias_parameter():
    import mxfp8_block_scaled_quantize_amd.linear as lin
    layer = lin.MXFP8Linear(128, 256, bias=True)
    assert layer.bias is not None and layer.bias.dtype == torch.bfloat16 and tuple(layer.bias.shape) == (256,)
    assert {n for n, _ in layer.named_parameters()} == {"weight", "bias"}
    assert lin.MXFP8Linear(128, 256).bias is None


def test_inference_without_a_cached_weight_quantizes_rowwise_only(monkeypatch):
    """mxfp8_linear_inference with no weight quantization given makes only
    the rowwise copies of x and W (host logic: quantize and gemm are stubs)."""
    import mxfp8_block_scaled_quantize_amd.linear as lin
    calls = []

    def stub_quantize(t, **kw):
        calls.append((tuple(t.shape), kw.get("rowwise"), bool(kw.get("colwise"))))
        return {"q_row": t, "p_row": t}

    monkeypatch.setattr(lin, "quantize", stub_quantize)
    monkeypatch.setattr(lin, "gemm", lambda a, pa, b, pb, bias=None: torch.zeros((a.shape[0], b.shape[0])))
    x = torch.zeros((128, 256), dtype=torch.bfloat16)
    w = torch.zeros((384, 256), dtype=torch.bfloat16)
    y = lin.mxfp8_linear_inference(x, w)
    assert tuple(y.shape) == (128, 384)
    assert calls == [((128, 256), True, False), ((384, 256), True, False)], calls
