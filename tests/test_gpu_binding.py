"""The Python binding checks every tensor it hands to the library against
the dimensions of the call: the C ABI sees only pointers and row strides,
so a view with fewer rows or columns than the call needs would be read or
written past its end.  Each case below must raise before any launch."""
import pytest
import torch

import block_scaled_fp8_02_amd as fb

pytestmark = pytest.mark.gpu


def z(*shape, dtype=torch.uint8):
    return torch.zeros(shape, dtype=dtype, device="cuda")


def bf(rows, cols):
    """rows x cols bf16 view with the row stride padded to 16 bytes, as the
    quantizers require."""
    return z(rows, (cols + 7) // 8 * 8, dtype=torch.bfloat16)[:, :cols]


def test_quantizer_outputs_are_checked():
    x = bf(256, 300)
    with pytest.raises(ValueError):
        fb.fp8_quantize_act_1x128(x, q=z(255, 384))                          # a row short
    with pytest.raises(ValueError):
        fb.fp8_quantize_act_1x128(x, q=z(256, 300))                          # padding columns missing
    with pytest.raises(TypeError):
        fb.fp8_quantize_act_1x128(x, s=z(256, 3, dtype=torch.float16))
    with pytest.raises(ValueError):
        fb.fp8_quantize_weight_128x128(x, qT=z(300, 128))                    # transposed copy too short
    with pytest.raises(ValueError):
        fb.fp8_quantize_transposed(x, sT=z(300, 1, dtype=torch.float32))     # needs ceil(256/128) = 2
    with pytest.raises(ValueError):
        fb.fp8_mx_quantize_1x32(x, q=z(256, 384), e=z(256, 11))              # needs 384/32 = 12
    with pytest.raises(ValueError):
        fb.fp8_quantize_transposed_grouped(x, torch.tensor([0, 256], dtype=torch.int64, device="cuda"))


def test_gemm_operands_are_checked():
    x = bf(256, 300)
    w = bf(384, 300)
    xq, xs = fb.fp8_quantize_act_1x128(x)
    wq, ws, wqT = fb.fp8_quantize_weight_128x128(w)
    fb.fp8_gemm_fprop(xq, xs, wq, ws, 256, 384, 300)                        # the well-formed call runs
    with pytest.raises(ValueError):
        fb.fp8_gemm_fprop(xq[:100], xs, wq, ws, 256, 384, 300)              # N larger than the codes
    with pytest.raises(ValueError):
        fb.fp8_gemm_fprop(xq, xs, wq, ws, 256, 384, 512)                    # K larger than the codes
    with pytest.raises(ValueError):
        fb.fp8_gemm_fprop(xq, xs, wq, ws, 256, 384, 300, y=z(256, 383, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        fb.fp8_gemm_dgrad(xq, xs, wqT, ws[:1], 256, 384, 300)               # 128x128 grid needs 3 rows
    with pytest.raises(TypeError):
        fb.fp8_gemm_wgrad(wqT, z(300, 3, dtype=torch.float16), wqT, z(300, 3, dtype=torch.float32),
                          384, 300, 300)
    mq, me, _, _ = fb.fp8_mx_quantize_1x32(x, colwise=False)
    mw, mwe, _, _ = fb.fp8_mx_quantize_1x32(w, colwise=False)
    with pytest.raises(ValueError):
        fb.fp8_mx_gemm_fprop(mq, me[:, :5], mw, mwe, 256, 384, 300)          # E8M0 columns missing


def test_grouped_and_dequant_operands_are_checked():
    offs = torch.tensor([0, 100, 256], dtype=torch.int32, device="cuda")
    x = bf(256, 300)
    w2 = bf(2 * 384, 300)                                                  # two experts stacked
    xq, xs = fb.fp8_quantize_act_1x128(x)
    wq, ws, _ = fb.fp8_quantize_weight_128x128(w2, transpose=False)
    fb.fp8_gemm_fprop_grouped(xq, xs, wq, 384 * wq.stride(0), ws, 3 * ws.stride(0), offs, 256, 384, 300)
    with pytest.raises(ValueError):                                          # the second expert is missing
        fb.fp8_gemm_fprop_grouped(xq, xs, wq[:384], 384 * wq.stride(0), ws, 3 * ws.stride(0), offs,
                                  256, 384, 300)
    with pytest.raises(ValueError):
        fb.fp8_dequantize_bf16(xq, xs[:, :2], fb.FP8B_SCALE_ROWS_1X128, 300)  # needs 3 scale columns
    with pytest.raises(ValueError):
        fb.fp8_dequant_gemm_dgrad(z(256, 384, dtype=torch.bfloat16), wq[:384], ws[:3],
                                  fb.FP8B_SCALE_BLOCKS_128X128, 256, 384, 300,
                                  work=z(384, 200, dtype=torch.bfloat16))
