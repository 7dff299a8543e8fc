"""The FP4 and 2:4-sparse grids on the GPU, vs the oracle.

* FP4: codes (one code per level, the zero level code 0), mask and scale pass
  the comparison rule of the dense forward, with FP4's own thresholds (the
  midpoints between E2M1 levels and s (1 + t / 6)); dq is the oracle's
  reconstruction to 1e-5 relative (fp32) / 2e-2 (bf16) and equals, bit for
  bit, what the dequantiser makes of the call's own codes.
* 2:4: kept positions, their codes, mask and scale likewise; a group whose
  second and third largest |y| lie within the band of each other may keep
  either pair.  dq as for FP4.
* Both at the 16384 x 2048 activation workload in full, on sampled rows;
  degenerate rows (zeros, constants, spikes) where, at blocks whose
  1/sqrt(block) is a power of two, exact ties must go to the lower index on
  both sides.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import quantization_aware_amd as qa
from oracle import quest_oracle as qo
from parity import TOL_BF16, TOL_F32, check_fwd_fp4, check_fwd_sparse24, check_values
from quest_inputs import WORKLOADS, TensorSpec, make_tensor, to_float64

pytestmark = pytest.mark.gpu


def log(msg: str) -> None:
    print(f"[gpu-grids] {msg}", flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qa.load_library()
    return torch.device("cuda", 0)


def x64_of(x: torch.Tensor) -> np.ndarray:
    return x.cpu().numpy().astype(np.float64) if x.dtype == torch.float32 else to_float64(x)


def np_rows(t: torch.Tensor, rows) -> np.ndarray:
    return t.index_select(0, torch.as_tensor(rows, device=t.device, dtype=torch.long)).cpu().numpy()


CASES = [
    # rows, cols, dtype, block, trust (bf16 rows of 512, 1024 or 2048 columns take the matrix-core 2:4 kernel)
    (77, 2048, "bf16", 128, 1.0),
    (130, 512, "bf16", 64, 1.0),
    (45, 1024, "bf16", 256, 1.3),
    (1, 2048, "bf16", 64, 0.0),
    (33, 1024, "f32", 64, 1.0),
    (21, 5632, "bf16", 128, 1.3),
    (19, 2560, "bf16", 256, 0.0),
    (1, 256, "f32", 256, 1.0),
    (64, 128, "bf16", 128, 1.0),
    (5, 10752, "bf16", 128, 1.0),
]


def make_case(dev, rows, cols, dt, seed):
    spec = TensorSpec("grid.x", rows, cols, dt, "student_t", 4, seed, outlier_cols=max(1, cols // 100),
                      outlier_scale=10.0)
    return make_tensor(spec, dev)


@pytest.mark.parametrize("rows,cols,dt,block,trust", CASES)
def test_fp4_fwd_matches_oracle(dev, rows, cols, dt, block, trust):
    log(f"fp4 {rows}x{cols} {dt} block {block} trust {trust}")
    x = make_case(dev, rows, cols, dt, 9100 + rows + cols)
    codes, scale, mask, dq = qa.quantize_fwd_fp4(x, block, trust, dq_dtype=torch.float32)
    torch.cuda.synchronize()
    x64 = x64_of(x)
    st = check_fwd_fp4(x64, block, codes.cpu().numpy(), scale.cpu().numpy(), mask.cpu().numpy(), trust=trust)
    ref = st["ref"]
    ratio = check_values(dq.cpu().numpy(), ref["q"], TOL_F32, skip=st["bad"])
    # dq is what the dequantiser makes of the same codes, bit for bit
    back = qa.dequantize_fp4(codes, scale, rows, cols, torch.float32)
    assert torch.equal(back, dq)
    # a bf16 dq call writes the same codes, mask and scale
    codes16, scale16, mask16, dq16 = qa.quantize_fwd_fp4(x, block, trust, dq_dtype=torch.bfloat16)
    assert torch.equal(codes16, codes) and torch.equal(scale16, scale) and torch.equal(mask16, mask)
    assert torch.equal(dq16, qa.dequantize_fp4(codes, scale, rows, cols, torch.bfloat16))
    check_values(dq16.float().cpu().numpy(), ref["q"], TOL_BF16, skip=st["bad"])
    # without codes or dq the mask and scale do not change
    none_codes, scale_n, mask_n, none_dq = qa.quantize_fwd_fp4(x, block, trust, with_codes=False)
    assert none_codes is None and none_dq is None
    assert torch.equal(scale_n, scale) and torch.equal(mask_n, mask)
    log(f"fp4 ok: {st['mismatched']} of {st['elements']} differ (all in the band), dq ratio {ratio:.3g}")


@pytest.mark.parametrize("b", [1, 2, 3, 4])
@pytest.mark.parametrize("rows,cols,dt,block,trust", CASES)
def test_sparse24_fwd_matches_oracle(dev, rows, cols, dt, block, trust, b):
    log(f"2:4 b={b} {rows}x{cols} {dt} block {block} trust {trust}")
    x = make_case(dev, rows, cols, dt, 9300 + rows + cols + b)
    codes, index, scale, mask, dq = qa.quantize_fwd_sparse24(x, block, b, trust, dq_dtype=torch.float32)
    torch.cuda.synchronize()
    x64 = x64_of(x)
    st = check_fwd_sparse24(x64, block, b, codes.cpu().numpy(), index.cpu().numpy(), scale.cpu().numpy(),
                            mask.cpu().numpy(), trust=trust)
    ref = st["ref"]
    # entries of exempt slots may reconstruct differently; everything else to the value tolerance
    slot_bad = np.zeros(x64.shape, dtype=bool)
    slot_bad |= st["ex_entry"]
    ratio = check_values(dq.cpu().numpy(), ref["q"], TOL_F32, skip=slot_bad)
    back = qa.dequantize_sparse24(codes, index, scale, rows, cols, b, torch.float32)
    assert torch.equal(back, dq)
    _, _, _, _, dq16 = qa.quantize_fwd_sparse24(x, block, b, trust, dq_dtype=torch.bfloat16)
    assert torch.equal(dq16, qa.dequantize_sparse24(codes, index, scale, rows, cols, b, torch.bfloat16))
    # exactly two nonzeros at most in every group of 4 of the reconstruction
    nz = (dq != 0).reshape(rows, cols // 4, 4).sum(dim=2)
    assert int(nz.max()) <= 2
    log(f"2:4 ok: {st['tie_groups']} tie groups, {st['mismatched_slots']} slots and {st['mismatched_mask']} mask "
        f"entries differ (all exempt), dq ratio {ratio:.3g}")


def test_grids_degenerate_rows(dev):
    rows, cols = 6, 512
    x = np.zeros((rows, cols), dtype=np.float32)
    x[1] = 3.25  # constant row: one nonzero per block, exact zeros elsewhere
    x[2, 77] = -5.0  # a single spike: every Hadamard entry of its block has magnitude 5
    x[3, :128] = 1.0  # one loud block
    x[4] = np.arange(cols, dtype=np.float32) % 7 - 3
    x[5, ::2] = 2.0
    x64 = x.astype(np.float64)
    xt = torch.from_numpy(x).to(dev)
    for block in (64, 128, 256):
        log(f"degenerate fp4 block {block}")
        codes, scale, mask, _ = qa.quantize_fwd_fp4(xt, block)
        torch.cuda.synchronize()
        check_fwd_fp4(x64, block, codes.cpu().numpy(), scale.cpu().numpy(), mask.cpu().numpy(), max_fraction=None)
        assert torch.all(codes[0] == 0) and torch.all(scale[0] == 0) and torch.all(mask[0] == 0xFF)
        for b in (1, 2, 3, 4):
            log(f"degenerate 2:4 b={b} block {block}")
            codes, index, scale, mask, _ = qa.quantize_fwd_sparse24(xt, block, b)
            torch.cuda.synchronize()
            ref = qo.quantize_fwd_sparse24(x64, block, b)
            if block != 128:
                # With 1/sqrt(block) a power of two, the Hadamard entries of these rows are
                # exact on both sides, so ties are exact and go to the lower index: positions
                # agree everywhere.  (At 128 the oracle's fp64 entries of equal magnitude may
                # differ in their last bit; the check below exempts such near ties.)
                assert np.array_equal(index.cpu().numpy(), ref["index"])
            check_fwd_sparse24(x64, block, b, codes.cpu().numpy(), index.cpu().numpy(), scale.cpu().numpy(),
                               mask.cpu().numpy(), max_fraction=None, ref=ref)
            assert torch.all(scale[0] == 0) and torch.all(mask[0] == 0xFF)


@pytest.mark.parametrize("cols", [512, 1024, 2048])
def test_grids_degenerate_rows_bf16(dev, cols):
    """bf16 rows with zeros and exact magnitude ties in the Hadamard domain, at the widths of the
    matrix-core forwards: FP4 (zero row: code 0, scale 0, all trusted) and 2:4 (ties to the lower
    index)."""
    rows = 8
    x = np.zeros((rows, cols), dtype=np.float32)
    x[1] = 3.25
    x[2, 77] = -5.0
    x[3, :128] = 1.0
    x[4] = np.arange(cols, dtype=np.float32) % 7 - 3
    x[5, ::2] = 2.0
    x[6, ::4] = -1.5
    x[7] = np.where(np.arange(cols) % 3 == 0, 0.5, -0.25)
    xt = torch.from_numpy(x).to(dev).to(torch.bfloat16)
    x64 = to_float64(xt)
    for block in (64, 128, 256):
        log(f"fp4 degenerate bf16 {rows}x{cols} block {block}")
        codes, scale, mask, dq = qa.quantize_fwd_fp4(xt, block, dq_dtype=torch.float32)
        torch.cuda.synchronize()
        check_fwd_fp4(x64, block, codes.cpu().numpy(), scale.cpu().numpy(), mask.cpu().numpy(), max_fraction=None)
        assert torch.all(codes[0] == 0) and torch.all(scale[0] == 0) and torch.all(mask[0] == 0xFF)
        assert torch.equal(dq, qa.dequantize_fp4(codes, scale, rows, cols, torch.float32))
        for b in (1, 2, 3, 4):
            log(f"2:4 ties bf16 {rows}x{cols} block {block} b={b}")
            codes, index, scale, mask, dq = qa.quantize_fwd_sparse24(xt, block, b, dq_dtype=torch.float32)
            torch.cuda.synchronize()
            ref = qo.quantize_fwd_sparse24(x64, block, b)
            if block != 128:
                # exact Hadamard entries on both sides: ties are exact, positions agree everywhere
                assert np.array_equal(index.cpu().numpy(), ref["index"])
            check_fwd_sparse24(x64, block, b, codes.cpu().numpy(), index.cpu().numpy(), scale.cpu().numpy(),
                               mask.cpu().numpy(), max_fraction=None, ref=ref)
            assert torch.all(scale[0] == 0) and torch.all(mask[0] == 0xFF) and torch.all(dq[0] == 0)
            assert torch.equal(dq, qa.dequantize_sparse24(codes, index, scale, rows, cols, b, torch.float32))


_VALU_FP4_CHILD = r"""
import sys
import numpy as np
import torch
sys.path[:0] = [sys.argv[1], sys.argv[1] + "/tests"]
import quantization_aware_amd as qa
from quest_inputs import TensorSpec, make_tensor
dev = torch.device("cuda", 0)
x = make_tensor(TensorSpec("valu.fp4", 96, int(sys.argv[2]), "bf16", "student_t", 4, 8600, outlier_cols=20,
                           outlier_scale=20.0), dev)
codes, scale, mask, _ = qa.quantize_fwd_fp4(x, int(sys.argv[3]), float(sys.argv[4]))
torch.cuda.synchronize()
np.savez(sys.argv[5], codes=codes.cpu().numpy(), scale=scale.cpu().numpy(), mask=mask.cpu().numpy())
"""


@pytest.mark.parametrize("cols,block,trust", [(2048, 128, 1.0), (512, 64, 1.3)])
def test_fp4_valu_switch_matches_oracle(dev, tmp_path, cols, block, trust):
    """QUEST_FWD_KERNEL=valu keeps the FP4 forward of these widths on the run-per-lane kernel: it matches
    the oracle, and so does the matrix-core kernel; they agree outside the exempt entries."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = tmp_path / "fp4.npz"
    log(f"vector-ALU FP4 forward in a child process, 96x{cols} block {block} trust {trust}")
    subprocess.run([sys.executable, "-c", _VALU_FP4_CHILD, root, str(cols), str(block), str(trust), str(out)],
                   env=dict(os.environ, QUEST_FWD_KERNEL="valu"), check=True, timeout=300)
    got = np.load(out)
    x = make_tensor(TensorSpec("valu.fp4", 96, cols, "bf16", "student_t", 4, 8600, outlier_cols=20,
                               outlier_scale=20.0), dev)
    x64 = to_float64(x)
    st = check_fwd_fp4(x64, block, got["codes"], got["scale"], got["mask"], trust=trust)
    codes, scale, mask, _ = qa.quantize_fwd_fp4(x, block, trust)
    torch.cuda.synchronize()
    st2 = check_fwd_fp4(x64, block, codes.cpu().numpy(), scale.cpu().numpy(), mask.cpu().numpy(), trust=trust,
                        ref=st["ref"])
    ok = ~(st["bad"] | st2["bad"])
    c_valu = qo.unpack_lsb_first(got["codes"], 4, cols)
    c_mfma = qo.unpack_lsb_first(codes.cpu().numpy(), 4, cols)
    assert np.array_equal(c_valu[ok], c_mfma[ok])


def test_grids_empty(dev):
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=dev)
    codes, scale, mask, dq = qa.quantize_fwd_fp4(x, 128, dq_dtype=torch.float32)
    assert codes.shape == (0, 128) and scale.shape == (0,) and mask.shape == (0, 32) and dq.shape == (0, 256)
    codes, index, scale, mask, dq = qa.quantize_fwd_sparse24(x, 128, 4, dq_dtype=torch.float32)
    assert codes.shape == (0, 64) and index.shape == (0, 32)
    assert qa.dequantize_sparse24(codes, index, scale, 0, 256, 4).shape == (0, 256)


@pytest.mark.parametrize("grid", ["fp4", "sparse24"])
def test_grids_full_size_sampled(dev, grid):
    """16384 x 2048 bf16 activations, the configuration the benchmark times, on sampled rows."""
    wl = WORKLOADS["T"]
    spec = wl.fwd[0]
    block = wl.block
    log(f"{grid} {spec.rows}x{spec.cols} full size")
    x = make_tensor(spec, dev)
    rng = np.random.default_rng(707)
    rows = np.unique(np.concatenate([rng.choice(spec.rows, size=192, replace=False), [0, spec.rows - 1]]))
    x64 = to_float64(x.index_select(0, torch.as_tensor(rows, device=dev)))
    if grid == "fp4":
        codes, scale, mask, dq = qa.quantize_fwd_fp4(x, block, dq_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        st = check_fwd_fp4(x64, block, np_rows(codes, rows), np_rows(scale, rows), np_rows(mask, rows))
        check_values(np_rows(dq.float(), rows), st["ref"]["q"], TOL_BF16, skip=st["bad"])
        log(f"fp4 sampled {len(rows)} rows: {st['mismatched']} differ")
    else:
        codes, index, scale, mask, dq = qa.quantize_fwd_sparse24(x, block, 4, dq_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        st = check_fwd_sparse24(x64, block, 4, np_rows(codes, rows), np_rows(index, rows), np_rows(scale, rows),
                                np_rows(mask, rows))
        check_values(np_rows(dq.float(), rows), st["ref"]["q"], TOL_BF16, skip=st["ex_entry"])
        log(f"2:4 sampled {len(rows)} rows: {st['tie_groups']} tie groups")
