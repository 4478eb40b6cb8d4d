"""The Python binding checks every tensor before its pointer reaches the library:
dtype, shape, layout and device (CPU only: the checks run before any library
call, so wrong arguments never reach a kernel)."""
import pytest
import torch

from block_scaled_fp4_05_amd import moe_fp4

U8, F32, I32, BF16 = torch.uint8, torch.float32, torch.int32, torch.bfloat16


def _gemm_args(E=2, n=64, k=256, a_rows=4):
    return dict(a_q=torch.zeros(a_rows, k // 2, dtype=U8), a_sf=torch.zeros(a_rows, k // 16, dtype=U8),
                a_scale=torch.ones(1), w_q=torch.zeros(E, n, k // 2, dtype=U8),
                w_sf=torch.zeros(E, n, k // 16, dtype=U8), w_scale=torch.ones(E),
                offsets=torch.zeros(E + 1, dtype=I32))


@pytest.mark.parametrize("change,message", [
    (dict(a_sf=torch.zeros(4, 15, dtype=U8)), "a_sf: shape"),
    (dict(a_q=torch.zeros(4, 128, dtype=torch.int8)), "a_q: dtype"),
    (dict(w_sf=torch.zeros(2, 64, 16, dtype=U8)[:, ::2]), "w_sf: shape"),
    (dict(w_q=torch.zeros(2, 128, 64, dtype=U8).transpose(1, 2)), "w_q: must be contiguous"),
    (dict(w_scale=torch.ones(3)), "w_scale: shape"),
    (dict(offsets=torch.zeros(3, dtype=torch.int64)), "offsets: dtype"),
    (dict(a_scale=torch.ones(1, dtype=torch.float64)), "a_scale: dtype"),
    ({}, "must be a CUDA tensor"),
])
def test_grouped_gemm_checks_its_tensors(change, message):
    args = _gemm_args()
    args.update(change)
    with pytest.raises(ValueError, match=message):
        moe_fp4.grouped_gemm(**args)


def test_grouped_gemm_checks_the_row_index_and_output():
    args = _gemm_args()
    with pytest.raises(ValueError, match="a_row_index: dtype"):
        moe_fp4.grouped_gemm(**args, a_row_index=torch.zeros(8, dtype=torch.int64))
    with pytest.raises(ValueError, match="out: shape"):
        moe_fp4.grouped_gemm(**args, out=torch.zeros(3, 64, dtype=BF16))
    with pytest.raises(ValueError, match="out: rows must have unit column stride"):
        moe_fp4.grouped_gemm(**args, out=torch.zeros(64, 4, dtype=BF16).t())


def test_quantize_checks_its_buffers():
    x = torch.zeros(4, 64, dtype=BF16)
    with pytest.raises(ValueError, match="q: shape"):
        moe_fp4.quantize(x, q=torch.zeros(4, 31, dtype=U8))
    with pytest.raises(ValueError, match="sf: dtype"):
        moe_fp4.quantize(x, sf=torch.zeros(4, 4, dtype=torch.int8))
    with pytest.raises(ValueError, match="tensor_scale: dtype"):
        moe_fp4.quantize(x, torch.ones(1, dtype=torch.float64))
    with pytest.raises(ValueError, match="must be a CUDA tensor"):
        moe_fp4.quantize(x)


def test_swiglu_finalize_combine_and_pack_check_their_tensors():
    args = _gemm_args()
    with pytest.raises(ValueError, match="h_q: shape"):
        moe_fp4.grouped_gemm_swiglu(**args, h_scale=torch.ones(1), h_q=torch.zeros(4, 15, dtype=U8))
    with pytest.raises(ValueError, match="out_token: shape"):
        moe_fp4.grouped_gemm_finalize(**args, out_token=torch.zeros(5, dtype=I32),
                                      row_weight=torch.zeros(4), out=torch.zeros(8, 64))
    with pytest.raises(ValueError, match="token_weights: shape"):
        moe_fp4.combine(torch.zeros(8, 64, dtype=BF16), torch.zeros(4, 2, dtype=I32),
                        torch.zeros(4, 3))
    with pytest.raises(ValueError, match="out: dtype"):
        moe_fp4.combine(torch.zeros(8, 64, dtype=BF16), torch.zeros(4, 2, dtype=I32),
                        torch.zeros(4, 2), out=torch.zeros(4, 64, dtype=torch.float16))
    with pytest.raises(ValueError, match="out: shape"):
        moe_fp4.pack_weights(torch.zeros(2, 64, 128, dtype=U8), out=torch.zeros(2, 64, 64, dtype=U8))
    with pytest.raises(ValueError, match="must be a CUDA tensor"):
        moe_fp4.unpack_weights(torch.zeros(2, 64, 128, dtype=U8))


def test_the_launch_stream_must_be_on_the_tensors_device():
    class FakeStream:
        device_index, cuda_stream = 1, 0

    with pytest.raises(ValueError, match="stream on cuda:1, tensors on cuda:0"):
        moe_fp4._stream(FakeStream(), 0)
    assert moe_fp4._stream(FakeStream(), 1).value is None
