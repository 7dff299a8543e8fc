"""Seeded random sweep of shapes and parameters, every path against the oracle.

Each case draws its own configuration from a fixed seed (rows, columns,
block, bit width, trust factor, input dtype, optional outputs), so the sweep
is reproducible and reaches combinations the hand-picked cases do not: run
counts that are not powers of two, ragged row counts, every kernel family.
The comparison rules are those of the other parity tests.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import quantization_aware_amd as qa
from oracle import quest_oracle as qo
from operand_layout import tile_operand, untile_operand
from parity import (TOL_BF16, TOL_F32, check_fwd, check_fwd_fp4, check_fwd_sparse24, check_grad, check_rate,
                    check_values, exempt_entries)
from quest_inputs import TensorSpec, make_tensor, to_float64

pytestmark = pytest.mark.gpu

N_FWD, N_BWD, N_GRID, N_GEMM = 80, 30, 32, 24


def log(msg: str) -> None:
    print(f"[gpu-sweep] {msg}", flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qa.load_library()
    return torch.device("cuda", 0)


def x64_of(x: torch.Tensor) -> np.ndarray:
    return x.cpu().numpy().astype(np.float64) if x.dtype == torch.float32 else to_float64(x)


def draw_shape(rng, max_blocks: int = 40):
    block = int(rng.choice([64, 128, 256]))
    cols = block * int(rng.integers(1, max_blocks + 1))
    rows = int(rng.integers(1, 258))
    dt = "bf16" if rng.random() < 0.7 else "f32"
    return rows, cols, block, dt


def draw_input(rng, rows, cols, dt, seed, dev):
    spec = TensorSpec("sweep.x", rows, cols, dt, "student_t", float(rng.choice([3.0, 4.0, 8.0])), seed,
                      outlier_cols=int(rng.integers(0, max(2, cols // 64))), outlier_scale=float(rng.choice([5.0, 20.0])))
    return make_tensor(spec, dev)


@pytest.mark.parametrize("case", range(N_FWD))
def test_sweep_forward(dev, case):
    rng = np.random.default_rng(20000 + case)
    rows, cols, block, dt = draw_shape(rng)
    b = int(rng.integers(1, 9))
    trust = float(rng.choice([1.0, 1.3, 0.7, 0.0]))
    dq_dtype = [None, torch.bfloat16, torch.float32][int(rng.integers(0, 3))]
    log(f"fwd case {case}: {rows}x{cols} {dt} block {block} b={b} trust {trust} dq {dq_dtype}")
    x = draw_input(rng, rows, cols, dt, 21000 + case, dev)
    codes, scale, mask, dq = qa.quantize_fwd_ex(x, block, b, trust=trust, with_codes=True, dq_dtype=dq_dtype)
    torch.cuda.synchronize()
    x64 = x64_of(x)
    ref = qo.quantize_fwd(x64, block, b, trust=trust)
    check_fwd(x64, block, b, codes.cpu().numpy(), scale.cpu().numpy(), mask.cpu().numpy(), ref=ref, trust=trust)
    if dq is not None:
        # the call's own codes, dequantised, bit for bit; and the oracle's values outside the band
        assert torch.equal(dq, qa.dequantize(codes, scale, rows, cols, b, out_dtype=dq_dtype))
        u = qo.unpack_lsb_first(codes.cpu().numpy(), b, cols)
        skip = (u != ref["u"]) | exempt_entries(ref["y"], ref["scale"], b, trust=trust)
        expect = qo.dequantize(ref["codes"], ref["scale"], cols, b)
        check_values(dq.float().cpu().numpy(), expect, TOL_F32 if dq_dtype == torch.float32 else TOL_BF16, skip=skip)


@pytest.mark.parametrize("case", range(N_BWD))
def test_sweep_backward(dev, case):
    rng = np.random.default_rng(22000 + case)
    rows, cols, block, dt = draw_shape(rng)
    b = int(rng.integers(1, 5))
    log(f"bwd case {case}: {rows}x{cols} {dt} block {block} (mask of a b={b} forward)")
    x64 = to_float64(draw_input(rng, rows, cols, "bf16", 23000 + case, "cpu"))
    ref = qo.quantize_fwd(x64, block, b)
    g = make_tensor(TensorSpec("sweep.g", rows, cols, dt, "normal", 1e-3, 24000 + case), dev)
    inplace = bool(rng.random() < 0.3)
    g64 = x64_of(g)
    out = qa.trust_bwd(g, torch.from_numpy(ref["mask"]).to(dev), block, out=g if inplace else None)
    torch.cuda.synchronize()
    expect = qo.trust_bwd(g64, ref["mask"], block)
    tol = TOL_BF16 if g.dtype == torch.bfloat16 else TOL_F32
    check_grad(x64_of(out), expect, block, tol)


@pytest.mark.parametrize("case", range(N_GRID))
def test_sweep_grids(dev, case):
    rng = np.random.default_rng(25000 + case)
    rows, cols, block, dt = draw_shape(rng, max_blocks=24)
    trust = float(rng.choice([1.0, 1.3, 0.0]))
    x = draw_input(rng, rows, cols, dt, 26000 + case, dev)
    x64 = x64_of(x)
    if case % 2 == 0:
        log(f"fp4 case {case}: {rows}x{cols} {dt} block {block} trust {trust}")
        codes, scale, mask, dq = qa.quantize_fwd_fp4(x, block, trust, dq_dtype=torch.float32)
        torch.cuda.synchronize()
        st = check_fwd_fp4(x64, block, codes.cpu().numpy(), scale.cpu().numpy(), mask.cpu().numpy(), trust=trust)
        check_values(dq.cpu().numpy(), st["ref"]["q"], TOL_F32, skip=st["bad"])
    else:
        b = int(rng.integers(1, 5))
        log(f"2:4 case {case}: {rows}x{cols} {dt} block {block} b={b} trust {trust}")
        codes, index, scale, mask, dq = qa.quantize_fwd_sparse24(x, block, b, trust, dq_dtype=torch.float32)
        torch.cuda.synchronize()
        st = check_fwd_sparse24(x64, block, b, codes.cpu().numpy(), index.cpu().numpy(), scale.cpu().numpy(),
                                mask.cpu().numpy(), trust=trust)
        check_values(dq.cpu().numpy(), st["ref"]["q"], TOL_F32, skip=st["ex_entry"])


@pytest.mark.parametrize("case", range(N_GEMM))
def test_sweep_gemm(dev, case):
    rng = np.random.default_rng(27000 + case)
    m, n = int(rng.integers(1, 600)), int(rng.integers(1, 600))
    k = 128 * int(rng.integers(1, 9))
    ba, bb = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    log(f"gemm case {case}: {m}x{n}x{k} bits {ba}/{bb}")
    xa = to_float64(make_tensor(TensorSpec("sw.a", m, k, "f32", "student_t", 4, 28000 + case, outlier_cols=2,
                                           outlier_scale=10.0), "cpu"))
    xb = to_float64(make_tensor(TensorSpec("sw.b", n, k, "f32", "normal", 0.02, 29000 + case), "cpu"))
    fa, fb = qo.quantize_fwd(xa, 128, ba), qo.quantize_fwd(xb, 128, bb)
    op_a = tile_operand(qo.operand_e2m3(fa["codes"], k, ba), m, k)
    op_b = tile_operand(qo.operand_e2m3(fb["codes"], k, bb), n, k)
    sa, sb = fa["scale"].astype(np.float32), fb["scale"].astype(np.float32)
    ref = qo.quest_gemm(untile_operand(op_a, m, k), sa.astype(np.float64), ba, untile_operand(op_b, n, k),
                        sb.astype(np.float64), bb, k)
    va = np.abs(qo.e2m3_value(qo.unpack_lsb_first(untile_operand(op_a, m, k), 6, k))) * qo.operand_step(sa, ba)[:, None]
    vb = np.abs(qo.e2m3_value(qo.unpack_lsb_first(untile_operand(op_b, n, k), 6, k))) * qo.operand_step(sb, bb)[:, None]
    slack = 2.0 * k * 2.0 ** -53 * (va @ vb.T)
    out_dtype = torch.float32 if case % 2 == 0 else torch.bfloat16
    y = qa.gemm(torch.from_numpy(op_a).to(dev), torch.from_numpy(sa).to(dev), m, ba, torch.from_numpy(op_b).to(dev),
                torch.from_numpy(sb).to(dev), n, bb, k, out_dtype=out_dtype)
    torch.cuda.synchronize()
    got = y.float().cpu().numpy().astype(np.float64)
    tol = 1e-6 if out_dtype == torch.float32 else 4e-3
    bad = np.abs(got - ref) > tol * np.abs(ref) + slack
    assert not bad.any(), f"{int(bad.sum())} outputs off, first at {np.argwhere(bad)[0]}"


N_GROUP, N_C2O = 16, 16


@pytest.mark.parametrize("case", range(N_GROUP))
def test_sweep_group(dev, case):
    """Random groups (1..12 tensors, mixed widths incl. the grouped ones, ragged rows, empty tensors):
    each tensor equal to its own quest_quantize_fwd bit for bit and checked against the oracle."""
    rng = np.random.default_rng(30000 + case)
    block = int(rng.choice([64, 128, 256]))
    b = int(rng.integers(1, 9))
    dt = "bf16" if rng.random() < 0.8 else "f32"
    widths = [c for c in (512, 1024, 2048, 256, 640, 5632, 1536, 2560, 8192) if c % block == 0]
    count = int(rng.integers(1, 13))
    shapes = [(int(rng.integers(0, 300)) if rng.random() < 0.9 else 0, int(rng.choice(widths))) for _ in range(count)]
    log(f"group case {case}: {count} {dt} tensors, block {block}, b={b}: {shapes}")
    xs = [draw_input(rng, r, c, dt, 31000 + 16 * case + i, dev) if r else
          torch.empty((0, c), dtype=torch.bfloat16 if dt == "bf16" else torch.float32, device=dev)
          for i, (r, c) in enumerate(shapes)]
    got = qa.quantize_fwd_group(xs, block, b)
    for i, x in enumerate(xs):
        if x.shape[0] == 0:
            continue
        ref = qa.quantize_fwd(x, block, b)
        torch.cuda.synchronize()
        assert all(torch.equal(g_, r_) for g_, r_ in zip(got[i], ref)), f"tensor {i} {tuple(x.shape)}"
    # every tensor against the oracle; the in-band rate is taken over the call's entries
    count = entries = 0
    for i, x in enumerate(xs):
        if x.shape[0]:
            c_, s_, m_ = (t.cpu().numpy() for t in got[i])
            st = check_fwd(x64_of(x), block, b, c_, s_, m_, max_fraction=None)
            count, entries = count + st["mismatched"], entries + st["elements"]
    check_rate(count, entries, f"b={b}, block={block}, grouped call of {len(xs)} tensors")


@pytest.mark.parametrize("case", range(N_C2O))
def test_sweep_codes_to_operand(dev, case):
    """Random shapes and widths: the operand of the stored codes equals the operand forward's on every row."""
    rng = np.random.default_rng(32000 + case)
    rows = int(rng.integers(1, 300))
    cols = 128 * int(rng.integers(1, 45))
    b = int(rng.integers(1, 5))
    dt = "bf16" if rng.random() < 0.7 else "f32"
    log(f"codes to operand case {case}: {rows}x{cols} {dt} b={b}")
    x = draw_input(rng, rows, cols, dt, 33000 + case, dev)
    codes, _, _, op = qa.quantize_fwd_op(x, 128, b, with_codes=True)
    op_c = qa.codes_to_operand(codes, rows, cols, b)
    torch.cuda.synchronize()
    n = qa.operand_bytes(rows, cols)
    assert np.array_equal(untile_operand(op_c.cpu().numpy()[:n], rows, cols),
                          untile_operand(op.cpu().numpy()[:n], rows, cols))
