"""The C ABI of libquest on the CPU: exports, host-side results, argument checks.

No call here launches a kernel: every device call is given arguments that the
library must reject before touching any buffer (the fake pointer values are
never dereferenced), or rows == 0, which is a documented no-op.
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import quantization_aware_amd as qa
from oracle import quest_oracle as qo
from operand_layout import tile_operand

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "quest.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(qa.LIB_PATH):
        pytest.fail("libquest.so is not built; run `python -m quantization_aware_amd.build`")
    return qa.load_library()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(quest_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_binding_symbols():
    assert _declared_functions() == sorted(qa.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_library_exports_nothing_else_named_quest(lib):
    out = os.popen(f"nm -D --defined-only {qa.LIB_PATH}").read()
    exported = sorted(set(re.findall(r"\s[TW]\s+(quest_\w+)$", out, flags=re.M)))
    assert exported == _declared_functions()


@pytest.mark.parametrize("b", range(1, 9))
def test_fit_alpha_matches_oracle(lib, b):
    assert abs(qa.fit_alpha(b) - qo.fit_alpha(b)) <= 1e-12 * qo.fit_alpha(b)


def test_fit_alpha_one_bit_closed_form(lib):
    assert abs(qa.fit_alpha(1) - math.sqrt(2 / math.pi)) <= 1e-15


@pytest.mark.parametrize("b", [-1, 0, 9, 100])
def test_fit_alpha_rejects_bits(lib, b):
    assert math.isnan(qa.fit_alpha(b))


def test_byte_counts(lib):
    assert qa.codes_bytes(16384, 2048, 4) == 16384 * 1024
    assert qa.codes_bytes(3, 128, 3) == 3 * 48
    assert qa.codes_bytes(0, 128, 1) == 0
    assert qa.mask_bytes(16384, 2048) == 16384 * 256
    assert qa.codes_bytes(-1, 128, 4) == 0
    assert qa.codes_bytes(2, 0, 4) == 0
    assert qa.codes_bytes(2, 12, 1) == 0  # 12 bits is not a whole number of bytes
    assert qa.mask_bytes(2, 12) == 0


def test_status_strings(lib):
    names = [lib.quest_status_string(i).decode() for i in range(6)]
    assert names[0] == "ok"
    assert len(set(names[:5])) == 5
    assert names[5] == "unknown status"


# ---------------------------------------------------------------------------
# Argument checks (return codes, nothing launched)
# ---------------------------------------------------------------------------

A = 0x10000  # fake, 16-byte aligned, well-separated addresses (never dereferenced)
B_ = 0x20000000
C_ = 0x40000000
D_ = 0x60000000


def fwd(lib, x=A, dt=qa.QUEST_BF16, rows=4, cols=256, block=128, b=4, codes=B_, scale=C_, mask=D_):
    return lib.quest_quantize_fwd(x, dt, rows, cols, block, b, codes, scale, mask, None)


def bwd(lib, g=A, dt=qa.QUEST_BF16, mask=B_, rows=4, cols=256, block=128, out=C_):
    return lib.quest_trust_bwd(g, dt, mask, rows, cols, block, out, None)


def deq(lib, codes=A, scale=B_, rows=4, cols=256, b=4, out=C_, dt=qa.QUEST_BF16):
    return lib.quest_dequantize(codes, scale, rows, cols, b, out, dt, None)


def test_empty_calls_are_noops(lib):
    assert fwd(lib, x=None, codes=None, scale=None, mask=None, rows=0) == qa.QUEST_OK
    assert bwd(lib, g=None, mask=None, out=None, rows=0) == qa.QUEST_OK
    assert deq(lib, codes=None, scale=None, out=None, rows=0) == qa.QUEST_OK


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(block=32), qa.QUEST_EUNSUPPORTED),
        (dict(block=512), qa.QUEST_EUNSUPPORTED),
        (dict(block=100), qa.QUEST_EUNSUPPORTED),
        (dict(b=0), qa.QUEST_EUNSUPPORTED),
        (dict(b=9), qa.QUEST_EUNSUPPORTED),
        (dict(dt=7), qa.QUEST_EINVAL),
        (dict(rows=-1), qa.QUEST_EINVAL),
        (dict(cols=0), qa.QUEST_EINVAL),
        (dict(cols=320), qa.QUEST_EINVAL),  # not a multiple of 128
        (dict(cols=65536), qa.QUEST_EUNSUPPORTED),
        (dict(rows=1 << 40, cols=1024), qa.QUEST_EUNSUPPORTED),
        (dict(x=None), qa.QUEST_EINVAL),
        (dict(codes=None), qa.QUEST_EINVAL),
        (dict(scale=None), qa.QUEST_EINVAL),
        (dict(mask=None), qa.QUEST_EINVAL),
        (dict(x=A + 8), qa.QUEST_EALIGN),
        (dict(codes=B_ + 4), qa.QUEST_EALIGN),
        (dict(scale=C_ + 2), qa.QUEST_EALIGN),
        (dict(mask=D_ + 1), qa.QUEST_EALIGN),
        (dict(codes=A + 16), qa.QUEST_EINVAL),  # codes inside x
        (dict(mask=A), qa.QUEST_EINVAL),
        (dict(scale=B_ + 16), qa.QUEST_EINVAL),  # scale inside codes
        (dict(mask=C_), qa.QUEST_EINVAL),  # mask == scale
    ],
)
def test_fwd_rejects(lib, kw, status):
    assert fwd(lib, **kw) == status


# A second tensor's buffers, apart from the first one's (fake addresses, never dereferenced).
E_, F_, G_, H_ = 0x70000000, 0x78000000, 0x7C000000, 0x7E000000


def group(lib, items, dt=qa.QUEST_BF16, block=128, b=4, count=None):
    descs = (qa._FwdTensor * max(len(items), 1))()
    for i, it in enumerate(items):
        descs[i] = qa._FwdTensor(it.get("x"), it.get("rows", 4), it.get("cols", 256), it.get("codes"),
                                 it.get("scale"), it.get("mask"))
    return lib.quest_quantize_fwd_group(descs, len(items) if count is None else count, dt, block, b, None)


GOOD = dict(x=E_, codes=F_, scale=G_, mask=H_)


def test_group_empty_calls_are_noops(lib):
    assert group(lib, []) == qa.QUEST_OK
    assert lib.quest_quantize_fwd_group(None, 0, qa.QUEST_BF16, 128, 4, None) == qa.QUEST_OK
    assert group(lib, [dict(rows=0), dict(rows=0, cols=2048)]) == qa.QUEST_OK


@pytest.mark.parametrize("kw,status", [(kw, st) for kw, st in test_fwd_rejects.pytestmark[0].args[1]
                                       if not {"dt", "block", "b"} & set(kw)])
def test_group_rejects_what_fwd_rejects(lib, kw, status):
    """A bad tensor anywhere in a group gives quest_quantize_fwd's status for it; nothing launches."""
    bad = dict(x=A, codes=B_, scale=C_, mask=D_, rows=4, cols=256)
    bad.update(kw)
    assert group(lib, [dict(GOOD), bad]) == status
    assert group(lib, [bad, dict(GOOD)]) == status


@pytest.mark.parametrize("kw,status", [(dict(block=32), qa.QUEST_EUNSUPPORTED), (dict(b=9), qa.QUEST_EUNSUPPORTED),
                                       (dict(dt=7), qa.QUEST_EINVAL)])
def test_group_rejects_bad_common_arguments(lib, kw, status):
    assert group(lib, [dict(GOOD)], **kw) == status


def test_group_rejects_bad_counts(lib):
    assert group(lib, [dict(GOOD)], count=-1) == qa.QUEST_EINVAL
    assert lib.quest_quantize_fwd_group(None, 2, qa.QUEST_BF16, 128, 4, None) == qa.QUEST_EINVAL


@pytest.mark.parametrize("second", [
    dict(x=E_, codes=B_, scale=G_, mask=H_),  # codes of the second on the first's codes
    dict(x=E_, codes=A, scale=G_, mask=H_),  # codes of the second inside the first's input
    dict(x=E_, codes=F_, scale=D_, mask=H_),  # scale of the second on the first's mask
    dict(x=B_, codes=F_, scale=G_, mask=H_),  # input of the second on the first's codes
])
def test_group_rejects_outputs_across_tensors(lib, second):
    first = dict(x=A, codes=B_, scale=C_, mask=D_)
    assert group(lib, [first, dict(second, rows=4, cols=256)]) == qa.QUEST_EINVAL


def test_group_shared_input_and_rows_zero_pointers_unread(lib):
    """Inputs may overlap; a rows == 0 tensor's pointers are not read, so a group whose other
    tensor is invalid still fails on that one (and a misaligned pointer of a skipped tensor does not)."""
    first = dict(x=A, codes=B_, scale=C_, mask=D_)
    assert group(lib, [first, dict(x=A, codes=F_, scale=G_, mask=H_ + 1)]) == qa.QUEST_EALIGN
    assert group(lib, [dict(x=A + 1, rows=0), dict(first, codes=None)]) == qa.QUEST_EINVAL


def test_fwd_outputs_just_past_input_are_accepted_by_checks(lib):
    # x (4 x 256 bf16 = 2048 bytes) ends where codes begin: no overlap.  The call would then
    # launch, so only the overlap predicate is exercised here, through an invalid block size.
    assert fwd(lib, codes=A + 2048, block=96) == qa.QUEST_EUNSUPPORTED


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(block=48), qa.QUEST_EUNSUPPORTED),
        (dict(dt=2), qa.QUEST_EINVAL),
        (dict(rows=-3), qa.QUEST_EINVAL),
        (dict(cols=192), qa.QUEST_EINVAL),
        (dict(cols=1 << 16), qa.QUEST_EUNSUPPORTED),
        (dict(g=None), qa.QUEST_EINVAL),
        (dict(mask=None), qa.QUEST_EINVAL),
        (dict(out=None), qa.QUEST_EINVAL),
        (dict(g=A + 4), qa.QUEST_EALIGN),
        (dict(mask=B_ + 8), qa.QUEST_EALIGN),
        (dict(out=C_ + 12), qa.QUEST_EALIGN),
        (dict(out=A + 16), qa.QUEST_EINVAL),  # partial overlap with grad
        (dict(mask=A + 32), qa.QUEST_EINVAL),  # mask inside grad
        (dict(mask=C_ + 32), qa.QUEST_EINVAL),  # mask inside out
    ],
)
def test_bwd_rejects(lib, kw, status):
    assert bwd(lib, **kw) == status


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(b=0), qa.QUEST_EUNSUPPORTED),
        (dict(b=9), qa.QUEST_EUNSUPPORTED),
        (dict(dt=5), qa.QUEST_EINVAL),
        (dict(cols=96), qa.QUEST_EINVAL),
        (dict(rows=-1), qa.QUEST_EINVAL),
        (dict(codes=None), qa.QUEST_EINVAL),
        (dict(scale=None), qa.QUEST_EINVAL),
        (dict(out=None), qa.QUEST_EINVAL),
        (dict(codes=A + 8), qa.QUEST_EALIGN),
        (dict(out=A), qa.QUEST_EINVAL),
        (dict(out=B_ - 16), qa.QUEST_EINVAL),  # out runs over scale
    ],
)
def test_dequantize_rejects(lib, kw, status):
    assert deq(lib, **kw) == status


E_ = 0x70000000


def fwd_dq(lib, x=A, dt=qa.QUEST_BF16, rows=4, cols=256, block=128, b=4, codes=B_, scale=C_, mask=D_, dq=E_,
           dq_dt=qa.QUEST_BF16):
    return lib.quest_quantize_fwd_dq(x, dt, rows, cols, block, b, codes, scale, mask, dq, dq_dt, None)


def test_fwd_dq_empty_call_is_a_noop(lib):
    assert fwd_dq(lib, x=None, codes=None, scale=None, mask=None, dq=None, rows=0) == qa.QUEST_OK


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(block=32), qa.QUEST_EUNSUPPORTED),
        (dict(b=9), qa.QUEST_EUNSUPPORTED),
        (dict(dt=7), qa.QUEST_EINVAL),
        (dict(dq_dt=3), qa.QUEST_EINVAL),
        (dict(cols=320), qa.QUEST_EINVAL),
        (dict(x=None), qa.QUEST_EINVAL),
        (dict(dq=None), qa.QUEST_EINVAL),
        (dict(scale=None), qa.QUEST_EINVAL),
        (dict(mask=None), qa.QUEST_EINVAL),
        (dict(dq=E_ + 8), qa.QUEST_EALIGN),
        (dict(codes=B_ + 4), qa.QUEST_EALIGN),
        (dict(codes=None, dq=E_ + 4), qa.QUEST_EALIGN),  # codes may be NULL; dq is still checked
        (dict(dq=A + 1024), qa.QUEST_EINVAL),  # dq inside x
        (dict(dq=B_), qa.QUEST_EINVAL),  # dq == codes
        (dict(dq=C_ - 16), qa.QUEST_EINVAL),  # dq runs over scale
        (dict(dq=D_), qa.QUEST_EINVAL),  # dq == mask
        (dict(codes=None, dq=C_ - 16), qa.QUEST_EINVAL),
        (dict(codes=A + 16), qa.QUEST_EINVAL),  # codes inside x
    ],
)
def test_fwd_dq_rejects(lib, kw, status):
    assert fwd_dq(lib, **kw) == status


def fwd_ex(lib, x=A, dt=qa.QUEST_BF16, rows=4, cols=256, block=128, b=4, trust=1.0, codes=B_, scale=C_, mask=D_,
           dq=E_, dq_dt=qa.QUEST_BF16):
    return lib.quest_quantize_fwd_ex(x, dt, rows, cols, block, b, trust, codes, scale, mask, dq, dq_dt, None)


def test_fwd_ex_empty_call_is_a_noop(lib):
    assert fwd_ex(lib, x=None, codes=None, scale=None, mask=None, dq=None, rows=0) == qa.QUEST_OK


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(b=9), qa.QUEST_EUNSUPPORTED),
        (dict(b=0), qa.QUEST_EUNSUPPORTED),
        (dict(trust=-0.5), qa.QUEST_EINVAL),
        (dict(trust=float("nan")), qa.QUEST_EINVAL),
        (dict(trust=float("inf")), qa.QUEST_EINVAL),
        (dict(dq_dt=4), qa.QUEST_EINVAL),
        (dict(x=None), qa.QUEST_EINVAL),
        (dict(mask=None), qa.QUEST_EINVAL),
        (dict(codes=B_ + 2), qa.QUEST_EALIGN),
        (dict(dq=E_ + 2), qa.QUEST_EALIGN),
        (dict(dq=A), qa.QUEST_EINVAL),
        (dict(codes=None, dq=D_), qa.QUEST_EINVAL),  # dq == mask
        (dict(b=8, codes=C_ - 512), qa.QUEST_EINVAL),  # 8-bit codes (1024 B) run over scale
    ],
)
def test_fwd_ex_rejects(lib, kw, status):
    assert fwd_ex(lib, **kw) == status


def test_fwd_ex_unknown_dq_dtype_ignored_without_dq(lib):
    # dq_dtype is only read when dq is given: with no dq an empty call still succeeds,
    # with a dq it is rejected.
    assert fwd_ex(lib, dq=None, dq_dt=9, rows=0) == qa.QUEST_OK
    assert fwd_ex(lib, dq_dt=9, rows=0) == qa.QUEST_EINVAL


def test_fwd_still_requires_codes(lib):
    assert fwd(lib, codes=None) == qa.QUEST_EINVAL


def test_binding_refuses_cpu_tensors(lib):
    import torch

    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        qa.quantize_fwd(x, 128, 4)
    with pytest.raises(ValueError):
        qa.trust_bwd(x, torch.zeros((4, 32), dtype=torch.uint8), 128)


def test_binding_raises_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(qa, "_lib", None)
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        qa.load_library(str(tmp_path / "missing.so"))


# ---------------------------------------------------------------------------
# Matrix-core operand forward and the product of two operands
# ---------------------------------------------------------------------------

def fwd_op(lib, x=A, dt=qa.QUEST_BF16, rows=4, cols=256, block=128, b=4, trust=1.0, codes=None, scale=C_, mask=None,
           op=E_):
    return lib.quest_quantize_fwd_op(x, dt, rows, cols, block, b, trust, codes, scale, mask, op, None)


def gemm(lib, a=A, sa=B_, m=300, ab=4, b=C_, sb=D_, n=200, bb=4, k=256, out=E_, dt=qa.QUEST_BF16):
    return lib.quest_gemm(a, sa, m, ab, b, sb, n, bb, k, out, dt, None)


def test_operand_bytes(lib):
    assert lib.quest_operand_bytes(45, 384) == 64 * 384 * 3 // 4
    assert lib.quest_operand_bytes(32, 128) == 3072
    assert lib.quest_operand_bytes(33, 128) == 2 * 3072
    assert lib.quest_operand_bytes(0, 128) == 0
    assert lib.quest_operand_bytes(4, 192) == 0
    assert lib.quest_operand_bytes(-1, 128) == 0
    rng = np.random.default_rng(0)
    op = rng.integers(0, 256, size=(45, 384 * 3 // 4), dtype=np.uint8)
    assert tile_operand(op, 45, 384).size == lib.quest_operand_bytes(45, 384)


def test_fwd_op_and_gemm_empty_calls_are_noops(lib):
    assert fwd_op(lib, x=None, scale=None, op=None, rows=0) == qa.QUEST_OK
    assert gemm(lib, a=None, sa=None, b=None, sb=None, out=None, m=0) == qa.QUEST_OK
    assert gemm(lib, a=None, sa=None, b=None, sb=None, out=None, n=0) == qa.QUEST_OK


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(b=5), qa.QUEST_EUNSUPPORTED),
        (dict(b=0), qa.QUEST_EUNSUPPORTED),
        (dict(cols=192, block=64), qa.QUEST_EUNSUPPORTED),  # not a multiple of 128
        (dict(block=512), qa.QUEST_EUNSUPPORTED),
        (dict(dt=5), qa.QUEST_EINVAL),
        (dict(trust=-1.0), qa.QUEST_EINVAL),
        (dict(x=None), qa.QUEST_EINVAL),
        (dict(scale=None), qa.QUEST_EINVAL),
        (dict(op=None), qa.QUEST_EINVAL),
        (dict(op=E_ + 8), qa.QUEST_EALIGN),
        (dict(mask=D_ + 4), qa.QUEST_EALIGN),
        (dict(op=A), qa.QUEST_EINVAL),  # overlaps x
        (dict(op=C_ - 1024), qa.QUEST_EINVAL),  # 6144 operand bytes (32 padded rows) run over scale
        (dict(codes=E_ + 64), qa.QUEST_EINVAL),  # codes inside the operand
    ],
)
def test_fwd_op_rejects(lib, kw, status):
    assert fwd_op(lib, **kw) == status


def op_group(lib, items, dt=qa.QUEST_BF16, block=128, b=4, trust=1.0, count=None):
    descs = (qa._FwdOpTensor * max(len(items), 1))()
    for i, it in enumerate(items):
        descs[i] = qa._FwdOpTensor(it.get("x"), it.get("rows", 4), it.get("cols", 256), it.get("codes"),
                                   it.get("scale"), it.get("mask"), it.get("op"))
    return lib.quest_quantize_fwd_op_group(descs, len(items) if count is None else count, dt, block, b, trust, None)


# A second operand tensor's buffers, apart from fwd_op's defaults (fake addresses, never dereferenced).
OP_GOOD = dict(x=F_, scale=G_, op=H_)


def test_op_group_empty_calls_are_noops(lib):
    assert op_group(lib, []) == qa.QUEST_OK
    assert lib.quest_quantize_fwd_op_group(None, 0, qa.QUEST_BF16, 128, 4, 1.0, None) == qa.QUEST_OK
    assert op_group(lib, [dict(rows=0), dict(rows=0, cols=2048)]) == qa.QUEST_OK


@pytest.mark.parametrize("kw,status", [(kw, st) for kw, st in test_fwd_op_rejects.pytestmark[0].args[1]
                                       if not {"dt", "block", "b", "trust"} & set(kw)])
def test_op_group_rejects_what_fwd_op_rejects(lib, kw, status):
    """A bad tensor anywhere in a group gives quest_quantize_fwd_op's status for it; nothing launches."""
    bad = dict(x=A, scale=C_, op=E_, rows=4, cols=256)
    bad.update(kw)
    assert op_group(lib, [dict(OP_GOOD), bad]) == status
    assert op_group(lib, [bad, dict(OP_GOOD)]) == status


@pytest.mark.parametrize("kw,status", [(dict(block=32), qa.QUEST_EUNSUPPORTED), (dict(b=5), qa.QUEST_EUNSUPPORTED),
                                       (dict(dt=7), qa.QUEST_EINVAL), (dict(trust=-0.5), qa.QUEST_EINVAL)])
def test_op_group_rejects_bad_common_arguments(lib, kw, status):
    assert op_group(lib, [dict(OP_GOOD)], **kw) == status


def test_op_group_rejects_bad_counts(lib):
    assert op_group(lib, [dict(OP_GOOD)], count=-1) == qa.QUEST_EINVAL
    assert lib.quest_quantize_fwd_op_group(None, 2, qa.QUEST_BF16, 128, 4, 1.0, None) == qa.QUEST_EINVAL


@pytest.mark.parametrize("second", [
    dict(x=F_, scale=G_, op=E_),  # operand of the second on the first's operand
    dict(x=F_, scale=G_, op=A),  # operand of the second on the first's input
    dict(x=F_, scale=C_, op=H_),  # scale of the second on the first's scale
    dict(x=E_, scale=G_, op=H_),  # input of the second on the first's operand
    dict(x=F_, scale=G_, op=H_, codes=D_),  # codes of the second on the first's mask
])
def test_op_group_rejects_outputs_across_tensors(lib, second):
    first = dict(x=A, scale=C_, mask=D_, op=E_)
    assert op_group(lib, [first, dict(second, rows=4, cols=256)]) == qa.QUEST_EINVAL


def test_op_group_shared_input_and_rows_zero_pointers_unread(lib):
    """Inputs may overlap; a rows == 0 tensor's pointers are not read."""
    first = dict(x=A, scale=C_, op=E_)
    assert op_group(lib, [first, dict(x=A, scale=G_, op=H_ + 8)]) == qa.QUEST_EALIGN
    assert op_group(lib, [dict(x=A + 1, rows=0, op=None), dict(first, op=None)]) == qa.QUEST_EINVAL


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(ab=5), qa.QUEST_EUNSUPPORTED),
        (dict(bb=0), qa.QUEST_EUNSUPPORTED),
        (dict(k=192), qa.QUEST_EUNSUPPORTED),
        (dict(k=65536 + 128), qa.QUEST_EUNSUPPORTED),
        (dict(n=2 ** 20 + 1), qa.QUEST_EUNSUPPORTED),
        (dict(m=2 ** 30 + 1), qa.QUEST_EUNSUPPORTED),
        (dict(m=2 ** 23, n=2 ** 16 + 1), qa.QUEST_EUNSUPPORTED),  # 2^23 tiles: 2^32 work-items
        (dict(m=2 ** 30, n=512), qa.QUEST_EUNSUPPORTED),
        (dict(k=0), qa.QUEST_EINVAL),
        (dict(k=-128), qa.QUEST_EINVAL),
        (dict(m=-1), qa.QUEST_EINVAL),
        (dict(dt=7), qa.QUEST_EINVAL),
        (dict(a=None), qa.QUEST_EINVAL),
        (dict(sb=None), qa.QUEST_EINVAL),
        (dict(out=None), qa.QUEST_EINVAL),
        (dict(a=A + 8), qa.QUEST_EALIGN),
        (dict(sa=B_ + 4), qa.QUEST_EALIGN),
        (dict(out=E_ + 4), qa.QUEST_EALIGN),
        (dict(out=A), qa.QUEST_EINVAL),  # overlaps a
        (dict(out=D_ - 4096), qa.QUEST_EINVAL),  # 120000 output bytes run over b_scale
    ],
)
def test_gemm_rejects(lib, kw, status):
    assert gemm(lib, **kw) == status


# ---------------------------------------------------------------------------
# FP4 and 2:4-sparse grids
# ---------------------------------------------------------------------------

def test_fit_alpha_fp4_matches_oracle(lib):
    assert math.isclose(lib.quest_fit_alpha_fp4(), qo.fit_alpha_fp4(), rel_tol=1e-12)


def test_sparse24_byte_counts(lib):
    assert lib.quest_sparse24_codes_bytes(3, 256, 4) == 3 * 128 // 2
    assert lib.quest_sparse24_codes_bytes(3, 256, 1) == 3 * 128 // 8
    assert lib.quest_sparse24_codes_bytes(3, 256, 5) == 0
    assert lib.quest_sparse24_index_bytes(3, 256) == 3 * 32
    assert lib.quest_sparse24_index_bytes(3, 100) == 0


def fwd_fp4(lib, x=A, dt=qa.QUEST_BF16, rows=4, cols=256, block=128, trust=1.0, codes=B_, scale=C_, mask=D_, dq=None,
            dq_dt=qa.QUEST_BF16):
    return lib.quest_quantize_fwd_fp4(x, dt, rows, cols, block, trust, codes, scale, mask, dq, dq_dt, None)


def fwd_s24(lib, x=A, dt=qa.QUEST_BF16, rows=4, cols=256, block=128, b=4, trust=1.0, codes=B_, index=E_, scale=C_,
            mask=D_, dq=None, dq_dt=qa.QUEST_BF16):
    return lib.quest_quantize_fwd_sparse24(x, dt, rows, cols, block, b, trust, codes, index, scale, mask, dq, dq_dt,
                                           None)


def test_grid_forwards_empty_calls_are_noops(lib):
    assert fwd_fp4(lib, x=None, codes=None, scale=None, mask=None, rows=0) == qa.QUEST_OK
    assert fwd_s24(lib, x=None, codes=None, index=None, scale=None, mask=None, rows=0) == qa.QUEST_OK


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(block=32), qa.QUEST_EUNSUPPORTED),
        (dict(cols=200), qa.QUEST_EINVAL),
        (dict(trust=-1.0), qa.QUEST_EINVAL),
        (dict(dt=3), qa.QUEST_EINVAL),
        (dict(x=None), qa.QUEST_EINVAL),
        (dict(mask=None), qa.QUEST_EINVAL),
        (dict(scale=None), qa.QUEST_EINVAL),
        (dict(codes=B_ + 4), qa.QUEST_EALIGN),
        (dict(dq=E_, dq_dt=7), qa.QUEST_EINVAL),
        (dict(codes=A), qa.QUEST_EINVAL),  # overlaps x
        (dict(codes=C_ - 256), qa.QUEST_EINVAL),  # 512 code bytes run over scale
    ],
)
def test_fwd_fp4_rejects(lib, kw, status):
    assert fwd_fp4(lib, **kw) == status


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(b=5), qa.QUEST_EUNSUPPORTED),
        (dict(b=0), qa.QUEST_EUNSUPPORTED),
        (dict(block=512), qa.QUEST_EUNSUPPORTED),
        (dict(x=None), qa.QUEST_EINVAL),
        (dict(mask=None), qa.QUEST_EINVAL),
        (dict(index=E_ + 8), qa.QUEST_EALIGN),
        (dict(index=D_ + 64), qa.QUEST_EINVAL),  # index inside the mask
        (dict(dq=C_), qa.QUEST_EINVAL),  # dq over scale
    ],
)
def test_fwd_sparse24_rejects(lib, kw, status):
    assert fwd_s24(lib, **kw) == status


def test_grid_dequantize_rejects(lib):
    assert lib.quest_dequantize_fp4(A, B_, 4, 256, C_, 9, None) == qa.QUEST_EINVAL
    assert lib.quest_dequantize_fp4(A, B_, 4, 256, A, qa.QUEST_F32, None) == qa.QUEST_EINVAL
    assert lib.quest_dequantize_fp4(A, B_, 0, 256, None, qa.QUEST_F32, None) == qa.QUEST_OK
    assert lib.quest_dequantize_sparse24(A, D_, B_, 4, 256, 5, C_, qa.QUEST_F32, None) == qa.QUEST_EUNSUPPORTED
    assert lib.quest_dequantize_sparse24(A, None, B_, 4, 256, 4, C_, qa.QUEST_F32, None) == qa.QUEST_EINVAL
    assert lib.quest_dequantize_sparse24(A, D_ + 2, B_, 4, 256, 4, C_, qa.QUEST_F32, None) == qa.QUEST_EALIGN


def c2o(lib, codes=A, rows=4, cols=256, b=4, op=B_):
    return lib.quest_codes_to_operand(codes, rows, cols, b, op, None)


def test_codes_to_operand_checks(lib):
    assert c2o(lib, codes=None, op=None, rows=0) == qa.QUEST_OK
    for kw, status in [(dict(b=0), qa.QUEST_EUNSUPPORTED), (dict(b=5), qa.QUEST_EUNSUPPORTED),
                       (dict(cols=192), qa.QUEST_EINVAL), (dict(cols=0), qa.QUEST_EINVAL),
                       (dict(cols=65536), qa.QUEST_EUNSUPPORTED), (dict(rows=-1), qa.QUEST_EINVAL),
                       (dict(codes=None), qa.QUEST_EINVAL), (dict(op=None), qa.QUEST_EINVAL),
                       (dict(codes=A + 8), qa.QUEST_EALIGN), (dict(op=B_ + 4), qa.QUEST_EALIGN),
                       (dict(op=A + 256), qa.QUEST_EINVAL)]:  # the operand starts inside the codes
        assert c2o(lib, **kw) == status, kw
