"""The binding rejects caller buffers that are too small or of the wrong type before any C call.

The C ABI takes raw pointers and cannot see buffer sizes, so these checks are
what keeps a mis-sized tensor from becoming an out-of-bounds device access.
They run before the device check, so CPU tensors exercise them here.
"""
from __future__ import annotations

import pytest
import torch

import quantization_aware_amd as qa

pytestmark = pytest.mark.filterwarnings("ignore")


def u8(n):
    return torch.zeros(n, dtype=torch.uint8)


def f32(n):
    return torch.zeros(n, dtype=torch.float32)


def gemm_args(m=40, n=24, k=256):
    return dict(a=u8(qa.operand_bytes(m, k)), a_scale=f32(m), m=m, a_bits=4, b=u8(qa.operand_bytes(n, k)),
                b_scale=f32(n), n=n, b_bits=4, k=k)


def test_gemm_well_sized_cpu_buffers_reach_the_device_check():
    with pytest.raises(ValueError, match="GPU tensor"):
        qa.gemm(**gemm_args())


@pytest.mark.parametrize("field,value,exc,msg", [
    ("a", u8(qa.operand_bytes(40, 256) - 1), ValueError, "a too small"),
    ("b", u8(qa.operand_bytes(24, 256) - 16), ValueError, "b too small"),
    ("a_scale", f32(39), ValueError, "a_scale too small"),
    ("b_scale", f32(23), ValueError, "b_scale too small"),
    ("a_scale", torch.zeros(40, dtype=torch.float64), TypeError, "a_scale must be"),
    ("b", torch.zeros(qa.operand_bytes(24, 256), dtype=torch.int8), TypeError, "b must be"),
])
def test_gemm_rejects_bad_operands(field, value, exc, msg):
    args = gemm_args()
    args[field] = value
    with pytest.raises(exc, match=msg):
        qa.gemm(**args)


def test_gemm_rejects_small_or_mistyped_out():
    with pytest.raises(ValueError, match="out too small"):
        qa.gemm(**gemm_args(), out=torch.zeros((40, 23), dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="out must be"):
        qa.gemm(**gemm_args(), out=torch.zeros((40, 24), dtype=torch.float16))


def test_gemm_larger_k_needs_larger_operands():
    args = gemm_args(k=256)
    with pytest.raises(ValueError, match="a too small"):
        qa.gemm(**{**args, "k": 384})


def test_fwd_op_rejects_small_operand_and_scale():
    x = torch.zeros((33, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="operand too small"):
        qa.quantize_fwd_op(x, 128, 4, operand=u8(qa.operand_bytes(32, 256)))
    with pytest.raises(ValueError, match="scale too small"):
        qa.quantize_fwd_op(x, 128, 4, scale=f32(32))
    with pytest.raises(TypeError, match="operand must be"):
        qa.quantize_fwd_op(x, 128, 4, operand=torch.zeros(qa.operand_bytes(33, 256), dtype=torch.int16))
    with pytest.raises(ValueError, match="GPU tensor"):
        qa.quantize_fwd_op(x, 128, 4)


def test_fwd_op_rejects_small_or_mistyped_codes_and_mask():
    x = torch.zeros((33, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="codes too small"):
        qa.quantize_fwd_op(x, 128, 4, codes=u8(33 * 128 - 1))
    with pytest.raises(ValueError, match="mask too small"):
        qa.quantize_fwd_op(x, 128, 4, mask=u8(33 * 32 - 1))
    with pytest.raises(TypeError, match="codes must be"):
        qa.quantize_fwd_op(x, 128, 3, codes=torch.zeros(33 * 96, dtype=torch.int8))
    with pytest.raises(ValueError, match="GPU tensor"):
        qa.quantize_fwd_op(x, 128, 4, codes=u8(33 * 128), mask=u8(33 * 32))


def test_fwd_op_group_checks_every_tensors_buffers():
    xs = [torch.zeros((33, 256), dtype=torch.bfloat16), torch.zeros((40, 512), dtype=torch.bfloat16)]
    ok = [dict(operand=u8(qa.operand_bytes(33, 256)), scale=f32(33)),
          dict(operand=u8(qa.operand_bytes(40, 512)), scale=f32(40))]
    with pytest.raises(ValueError, match=r"outs\[1\].operand too small"):
        qa.quantize_fwd_op_group(xs, 128, 4, outs=[ok[0], dict(ok[1], operand=u8(qa.operand_bytes(40, 512) - 1))])
    with pytest.raises(ValueError, match=r"outs\[0\].scale too small"):
        qa.quantize_fwd_op_group(xs, 128, 4, outs=[dict(ok[0], scale=f32(32)), ok[1]])
    with pytest.raises(ValueError, match=r"outs\[1\].codes too small"):
        qa.quantize_fwd_op_group(xs, 128, 4, outs=[ok[0], dict(ok[1], codes=u8(40 * 256 - 1))])
    with pytest.raises(ValueError, match=r"outs\[0\].mask too small"):
        qa.quantize_fwd_op_group(xs, 128, 4, outs=[dict(ok[0], mask=u8(33 * 32 - 1)), ok[1]])
    with pytest.raises(ValueError, match="unknown keys"):
        qa.quantize_fwd_op_group(xs, 128, 4, outs=[dict(ok[0], dq=u8(1)), ok[1]])
    with pytest.raises(ValueError, match="2 tensors but 1 output sets"):
        qa.quantize_fwd_op_group(xs, 128, 4, outs=[ok[0]])
    with pytest.raises(ValueError, match="share the first one's dtype"):
        qa.quantize_fwd_op_group([xs[0], xs[1].float()], 128, 4)
    with pytest.raises(ValueError, match="GPU tensor"):
        qa.quantize_fwd_op_group(xs, 128, 4, outs=ok)


def test_grid_dequantisers_reject_small_inputs():
    with pytest.raises(ValueError, match="codes too small"):
        qa.dequantize_fp4(u8(16 * 256 // 2 - 1), f32(16), 16, 256)
    with pytest.raises(ValueError, match="scale too small"):
        qa.dequantize_fp4(u8(16 * 256 // 2), f32(15), 16, 256)
    lib = qa.load_library()
    nc, ni = int(lib.quest_sparse24_codes_bytes(16, 256, 4)), int(lib.quest_sparse24_index_bytes(16, 256))
    assert nc == 16 * 128 * 4 // 8 and ni == 16 * 256 // 8
    with pytest.raises(ValueError, match="codes too small"):
        qa.dequantize_sparse24(u8(nc - 1), u8(ni), f32(16), 16, 256, 4)
    with pytest.raises(ValueError, match="index too small"):
        qa.dequantize_sparse24(u8(nc), u8(ni - 1), f32(16), 16, 256, 4)
    with pytest.raises(ValueError, match="GPU tensor"):
        qa.dequantize_sparse24(u8(nc), u8(ni), f32(16), 16, 256, 4)
