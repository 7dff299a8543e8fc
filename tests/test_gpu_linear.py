"""QuEST linear layer (quest_quantize_fwd_dq + library GEMMs + quest_trust_bwd) vs the oracle.

The oracle composes its pinned quantiser, a float64 matrix product and its
trust backward (oracle.qat_linear_fwd / qat_linear_bwd).  The layer runs in
a compute dtype:

* float32: dequantised operands and GEMMs in fp32, so results agree with the
  oracle to fp32 accumulation error (1e-4 relative);
* bfloat16 (the training default): the dequantised operands are rounded to
  bf16.  Within a row the rounding error of a grid value depends only on its
  code, and with an outlier channel the codes of a block share the sign
  pattern of one Hadamard row, so the errors correlate with that row and the
  inverse transform gathers them onto the outlier's position: a few percent
  of the gradient there.  Element-wise bound 1e-1 of max(|ref|, rms), norm-
  wise 1e-2.

The element-wise scale uses the RMS over the whole tensor for y and over the
entry's row and Hadamard block for the gradients (which leave the kernel
through an inverse transform).

Where the forward product is the FP6 one (int grid, b <= 4, K a multiple of
128) its sums are exact, so y differs from the oracle's only by the fp32
rounding of the two clip scales (at most 2e-6 relative each against the
oracle's float64 scales) and one rounding to the output type: y is held to
1e-5 of |ref| in fp32 and to 2^-8 + 1e-5 of |ref| in bf16 (half a bf16 ulp
is at most 2^-8 of the value), entry by entry, with no RMS floor.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import quantization_aware_amd as qa
from oracle import quest_oracle as qo
from quantization_aware_amd.linear import QuestLinear, QuestLinearFunction, default_trust, quest_linear
from quest_inputs import TensorSpec, make_tensor, to_float64
from parity import exempt_entries, exempt_fp4, sparse24_exempt_entries

pytestmark = pytest.mark.gpu

TOLS = {torch.float32: (1e-4, 1e-4), torch.bfloat16: (1e-1, 1e-2)}  # (element-wise, norm-wise)
Y_TOL_FP6 = {torch.float32: 1e-5, torch.bfloat16: 2.0 ** -8 + 1e-5}  # |y - ref| <= tol |ref|, FP6 product


def log(msg: str) -> None:
    print(f"[gpu-linear] {msg}", flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qa.load_library()
    return torch.device("cuda", 0)


def close(got: torch.Tensor, ref: np.ndarray, what: str, tols, skip=None, block=None) -> None:
    """Element-wise and norm-wise agreement with the oracle, outside `skip`.

    The element-wise scale is max(|ref|, rms), with rms taken over the whole
    tensor, or per row and Hadamard block for the gradients (which leave the
    kernel through an inverse transform: rounding of a large Hadamard-domain
    entry spreads evenly over its block).
    """
    got = got.float().cpu().numpy().astype(np.float64)
    if block is None:
        rms = np.sqrt(np.mean(ref * ref))
    else:
        r, c = ref.shape
        blk = ref.reshape(r, c // block, block)
        rms = np.repeat(np.sqrt(np.mean(blk * blk, axis=2)), block, axis=1)
    tol_elem, tol_norm = tols
    err = np.abs(got - ref)
    bad = err > tol_elem * np.maximum(np.abs(ref), rms)
    if skip is not None:
        bad &= ~skip
    if bad.any():
        r, c = np.argwhere(bad)[0]
        log(f"{what}: relative Frobenius error {np.linalg.norm(got - ref) / np.linalg.norm(ref)!r}")
        ratio = (err / np.maximum(np.abs(ref), rms))[bad]
        raise AssertionError(f"{what}: {int(bad.sum())} entries off, first at ({r},{c}): got {got[r, c]!r} "
                             f"ref {ref[r, c]!r}; worst error / max(|ref|, rms) {ratio.max()!r}")
    keep = np.ones_like(bad) if skip is None else ~skip
    if not keep.any() or not np.any(ref[keep]):
        # at b >= 5 a band entry in every row or Hadamard block can reach the whole tensor
        log(f"{what}: every entry within a band entry's reach; norm-wise check skipped")
        return
    rel = np.linalg.norm((got - ref)[keep]) / np.linalg.norm(ref[keep])
    assert rel <= tol_norm, f"{what}: relative Frobenius error {rel} (outside the band's reach)"


def oracle_slack(f: dict) -> np.ndarray:
    """Bound on the oracle's own rounding in y = Q(x) Q(w)^T (a float64 sum of k products):
    2 k 2^-53 sum |products|."""
    k = f["qx"].shape[1]
    return 2.0 * k * 2.0 ** -53 * (np.abs(f["qx"]) @ np.abs(f["qw"]).T)


def close_relative(got: torch.Tensor, ref: np.ndarray, what: str, tol: float, skip=None, slack=0.0) -> None:
    """|got - ref| <= tol |ref| + slack for every entry outside `skip` (no RMS floor: an exact sum
    that cancels to zero must come back as zero, up to the oracle's own rounding `slack`)."""
    got = got.float().cpu().numpy().astype(np.float64)
    bad = np.abs(got - ref) > tol * np.abs(ref) + slack
    if skip is not None:
        bad &= ~skip
    if bad.any():
        r, c = np.argwhere(bad)[0]
        worst = (np.abs(got - ref) / np.maximum(np.abs(ref), 1e-300))[bad].max()
        raise AssertionError(f"{what}: {int(bad.sum())} entries off, first at ({r},{c}): got {got[r, c]!r} "
                             f"ref {ref[r, c]!r}; worst relative error {worst!r} (bound {tol})")


def close_product_plus_bias(got: torch.Tensor, f: dict, bias: np.ndarray, what: str, skip=None) -> None:
    """bf16 output of an FP6 product (exact sum, scales within 2e-6 each, one bf16 rounding) plus a bias
    (one more bf16 rounding): |got - (prod + bias)| <= 2^-8 |prod| + 2^-8 |prod + bias| + 1e-5 |prod|,
    the second rounding taken of a sum at most 2^-8 |prod| away from prod + bias; plus the oracle's own
    rounding of prod."""
    got = got.float().cpu().numpy().astype(np.float64)
    prod = f["y"]
    ref = prod + bias
    bound = (2.0 ** -8 + 1e-5) * np.abs(prod) + 2.0 ** -8 * (np.abs(ref) + 2.0 ** -8 * np.abs(prod))
    bound += oracle_slack(f)
    bad = np.abs(got - ref) > bound
    if skip is not None:
        bad &= ~skip
    assert not bad.any(), (f"{what}: {int(bad.sum())} entries off; worst error / bound "
                           f"{(np.abs(got - ref) / np.maximum(bound, 1e-300))[bad].max()!r}")


def layer_node(y: torch.Tensor):
    """The QuestLinearFunction node behind y (through reshapes and the bias add)."""
    node = y.grad_fn
    while node is not None and not hasattr(node, "fp6"):
        node = node.next_functions[0][0]
    assert node is not None, "no QuestLinearFunction in y's graph"
    return node


def band_reach(f: dict, bx: int, bw: int, block: int, trust_x: float = 1.0, trust_w: float = 1.0):
    """Entries of y, dx and dw that an operand entry inside the threshold band can move.

    A band entry (within 1e-6 s of a decision or trust threshold) may take the
    neighbouring code or mask bit on the GPU, which is a correct outcome; it
    shifts its row of y, dx or dw and, through the other operand's product,
    the Hadamard block of its column.
    """
    bx_ = exempt_entries(f["fx"]["y"], f["fx"]["scale"], bx, trust=trust_x)
    bw_ = exempt_entries(f["fw"]["y"], f["fw"]["scale"], bw, trust=trust_w)
    return reach_of(bx_, bw_, block)


def reach_of(bx_: np.ndarray, bw_: np.ndarray, block: int):
    """(skip_y, skip_dx, skip_dw) reached from the exempt entries bx_ of x and bw_ of w."""
    rx, rw = bx_.any(axis=1), bw_.any(axis=1)
    k = bx_.shape[1]
    blk_x = np.repeat(bx_.reshape(bx_.shape[0], k // block, block).any(axis=(0, 2)), block)
    blk_w = np.repeat(bw_.reshape(bw_.shape[0], k // block, block).any(axis=(0, 2)), block)
    skip_y = rx[:, None] | rw[None, :]
    skip_dx = rx[:, None] | blk_w[None, :] | blk_x[None, :] & rx[:, None]
    skip_dw = rw[:, None] | blk_x[None, :] | blk_w[None, :] & rw[:, None]
    return skip_y, skip_dx, skip_dw


@pytest.mark.parametrize("compute_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n,k,m,block,bx,bw,fp6", [
    # the FP6 forward product (int grid, b <= 4, K a multiple of 128)
    (256, 1024, 384, 128, 4, 4, True), (96, 2048, 160, 64, 2, 3, True), (130, 512, 64, 256, 4, 1, True),
    (132, 1024, 96, 64, 3, 3, True), (130, 1024, 96, 128, 3, 3, True),
    # the dequantised operands and a library product: K not a multiple of 128, or b > 4
    (96, 192, 160, 64, 2, 3, False), (128, 1024, 96, 128, 5, 4, False), (64, 640, 72, 128, 8, 6, False)])
def test_linear_matches_oracle(dev, n, k, m, block, bx, bw, fp6, compute_dtype):
    log(f"linear {n}x{k} by {m}x{k}, block {block}, bits x{bx} w{bw}, compute {compute_dtype}, fp6 {fp6}")
    tols = TOLS[compute_dtype]
    x = make_tensor(TensorSpec("lin.x", n, k, "bf16", "student_t", 4, 9100 + n, outlier_cols=k // 100,
                               outlier_scale=20.0), dev)
    w = make_tensor(TensorSpec("lin.w", m, k, "bf16", "normal", 0.02, 9200 + m), dev)
    dy = make_tensor(TensorSpec("lin.dy", n, m, "bf16", "normal", 1e-3, 9300 + n), dev)
    # Inputs in the compute dtype (fp32 holds the same values exactly), so the
    # gradients come back in it too.
    xg = x.to(compute_dtype).requires_grad_(True)
    wg = w.to(compute_dtype).requires_grad_(True)
    y = quest_linear(xg, wg, block=block, bits_x=bx, bits_w=bw, compute_dtype=compute_dtype)
    assert layer_node(y).fp6 is fp6
    y.backward(dy.to(compute_dtype))
    torch.cuda.synchronize()
    f = qo.qat_linear_fwd(to_float64(x), to_float64(w), block, bx, bw, default_trust(bx), default_trust(bw))
    dx_ref, dw_ref = qo.qat_linear_bwd(to_float64(dy), f, block)
    skip_y, skip_dx, skip_dw = band_reach(f, bx, bw, block, default_trust(bx), default_trust(bw))
    log(f"band reach: {int(skip_y.sum())} of y, {int(skip_dx.sum())} of dx, {int(skip_dw.sum())} of dw")
    if fp6:
        close_relative(y.detach(), f["y"], "y", Y_TOL_FP6[compute_dtype], skip_y, oracle_slack(f))
    else:
        close(y.detach(), f["y"], "y", tols, skip_y)
    close(xg.grad, dx_ref, "dx", tols, skip_dx, block)
    close(wg.grad, dw_ref, "dw", tols, skip_dw, block)


@pytest.mark.parametrize("trust_x,trust_w", [(1.0, 1.3), (1.3, 1.3)])
def test_linear_fp6_with_outer_trust_factors(dev, trust_x, trust_w):
    """The FP6 layer with one bit width and explicit trust factors: equal ones quantise both operands
    in one grouped launch, different ones in two calls; both against the oracle with those factors."""
    n, k, m, block, bits, compute_dtype = 128, 1024, 96, 128, 3, torch.bfloat16
    log(f"linear {n}x{k} by {m}x{k}, b={bits}, trust x {trust_x} w {trust_w}")
    x = make_tensor(TensorSpec("tr.x", n, k, "bf16", "student_t", 4, 9400, outlier_cols=k // 100,
                               outlier_scale=20.0), dev)
    w = make_tensor(TensorSpec("tr.w", m, k, "bf16", "normal", 0.02, 9401), dev)
    dy = make_tensor(TensorSpec("tr.dy", n, m, "bf16", "normal", 1e-3, 9402), dev)
    xg, wg = x.clone().requires_grad_(True), w.clone().requires_grad_(True)
    y = quest_linear(xg, wg, block=block, bits_x=bits, bits_w=bits, compute_dtype=compute_dtype,
                     trust_x=trust_x, trust_w=trust_w)
    assert layer_node(y).fp6 is True
    y.backward(dy)
    torch.cuda.synchronize()
    f = qo.qat_linear_fwd(to_float64(x), to_float64(w), block, bits, bits, trust_x, trust_w)
    dx_ref, dw_ref = qo.qat_linear_bwd(to_float64(dy), f, block)
    skip_y, skip_dx, skip_dw = band_reach(f, bits, bits, block, trust_x, trust_w)
    tols = TOLS[compute_dtype]
    close_relative(y.detach(), f["y"], "y", Y_TOL_FP6[compute_dtype], skip_y, oracle_slack(f))
    close(xg.grad, dx_ref, "dx", tols, skip_dx, block)
    close(wg.grad, dw_ref, "dw", tols, skip_dw, block)


@pytest.mark.parametrize("compute_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("grid,bx,bw", [("fp4", 4, 4), ("sparse24", 4, 4), ("sparse24", 2, 3)])
def test_linear_grids_match_oracle(dev, grid, bx, bw, compute_dtype):
    """The layer on the FP4 and 2:4-sparse grids against the oracle's composition of the same
    quantiser, a float64 product and the trust backward; exemptions as in the grid parity tests."""
    n, k, m, block = 192, 1024, 256, 128
    log(f"linear on the {grid} grid, {n}x{k} by {m}x{k}, bits x{bx} w{bw}, compute {compute_dtype}")
    tols = TOLS[compute_dtype]
    x = make_tensor(TensorSpec("lin.gx", n, k, "bf16", "student_t", 4, 9600 + bx, outlier_cols=k // 100,
                               outlier_scale=20.0), dev)
    w = make_tensor(TensorSpec("lin.gw", m, k, "bf16", "normal", 0.02, 9700 + bw), dev)
    dy = make_tensor(TensorSpec("lin.gdy", n, m, "bf16", "normal", 1e-3, 9800), dev)
    xg = x.to(compute_dtype).requires_grad_(True)
    wg = w.to(compute_dtype).requires_grad_(True)
    y = quest_linear(xg, wg, block=block, bits_x=bx, bits_w=bw, compute_dtype=compute_dtype, grid=grid)
    y.backward(dy.to(compute_dtype))
    torch.cuda.synchronize()
    f = qo.qat_linear_fwd(to_float64(x), to_float64(w), block, bx, bw, grid=grid)
    dx_ref, dw_ref = qo.qat_linear_bwd(to_float64(dy), f, block)
    if grid == "fp4":
        ex_x, ex_w = exempt_fp4(f["fx"]["y"], f["fx"]["scale"]), exempt_fp4(f["fw"]["y"], f["fw"]["scale"])
    else:
        ex_x, ex_w = sparse24_exempt_entries(f["fx"], bx), sparse24_exempt_entries(f["fw"], bw)
    skip_y, skip_dx, skip_dw = reach_of(ex_x, ex_w, block)
    log(f"band reach: {int(skip_y.sum())} of y, {int(skip_dx.sum())} of dx, {int(skip_dw.sum())} of dw")
    close(y.detach(), f["y"], "y", tols, skip_y)
    close(xg.grad, dx_ref, "dx", tols, skip_dx, block)
    close(wg.grad, dw_ref, "dw", tols, skip_dw, block)


@pytest.mark.parametrize("bits,k,fp6", [(4, 1024, True), (3, 512, True), (5, 1024, False), (4, 192, False)])
def test_linear_training_forward_path(dev, bits, k, fp6):
    """The int-grid training forward takes the FP6 product exactly where its domain allows (b <= 4,
    K a multiple of 128) and then saves the operands' codes, not their dequantised values."""
    block = 64
    x = make_tensor(TensorSpec("path.x", 64, k, "bf16", "normal", 1.0, 9950), dev).requires_grad_(True)
    w = make_tensor(TensorSpec("path.w", 32, k, "bf16", "normal", 0.02, 9951), dev).requires_grad_(True)
    log(f"training forward path: bits {bits}, k {k}")
    y = QuestLinearFunction.apply(x, w, block, bits, bits, torch.bfloat16, 1.0, 1.0, "int")
    saved = y.grad_fn.saved_tensors
    if fp6:
        # one bit width and 64 rows: x's and w's codes, scales and masks as the rows of one tensor each
        assert len(saved) == 3 and saved[0].dtype == torch.uint8 and saved[0].shape == (64 + 32, k * bits // 8)
        assert saved[1].shape == (64 + 32,) and saved[2].shape == (64 + 32, k // 8)
    else:
        assert len(saved) == 4 and saved[0].dtype == torch.bfloat16 and saved[0].shape == (64, k)
    y.float().sum().backward()
    torch.cuda.synchronize()
    assert x.grad is not None and w.grad is not None


def test_linear_module_grid_option(dev):
    layer = QuestLinear(512, 128, grid="sparse24", device=dev, dtype=torch.bfloat16)
    assert layer.grid == "sparse24" and layer.trust_x == 1.0
    with pytest.raises(ValueError):
        layer.freeze()  # the FP6 product holds int-grid levels only
    with pytest.raises(ValueError):
        QuestLinear(512, 128, grid="int8")


def test_linear_module_autograd_3d_input(dev):
    torch.manual_seed(0)
    layer = QuestLinear(1024, 256, bias=True, block=128, device=dev, dtype=torch.bfloat16)
    x = make_tensor(TensorSpec("mod.x", 2 * 64, 1024, "bf16", "student_t", 4, 9400), dev).reshape(2, 64, 1024)
    x.requires_grad_(True)
    log("module forward/backward, input 2x64x1024")
    y = layer(x)
    assert y.shape == (2, 64, 256) and y.dtype == torch.bfloat16
    loss = (y.float() ** 2).mean()
    loss.backward()
    torch.cuda.synchronize()
    # The same through the oracle (bias added after the product).
    f = qo.qat_linear_fwd(to_float64(x.detach().reshape(128, 1024)), to_float64(layer.weight.detach()), 128, 4, 4)
    y_ref = f["y"] + to_float64(layer.bias.detach())[None, :]
    skip_y, skip_dx, skip_dw = band_reach(f, 4, 4, 128)
    tols = TOLS[torch.bfloat16]
    assert layer_node(y).fp6
    close_product_plus_bias(y.detach().reshape(128, 256), f, to_float64(layer.bias.detach())[None, :],
                            "module y", skip_y)
    dy = (2.0 / y.numel()) * y.detach().float().reshape(128, 256).cpu().numpy().astype(np.float64)
    dx_ref, dw_ref = qo.qat_linear_bwd(dy, f, 128)
    close(x.grad.reshape(128, 1024), dx_ref, "module dx", tols, skip_dx, 128)
    close(layer.weight.grad, dw_ref, "module dw", tols, skip_dw, 128)
    assert np.allclose(layer.bias.grad.float().cpu().numpy(), dy.sum(axis=0), rtol=2e-2, atol=1e-6)


@pytest.mark.parametrize("compute_dtype", [torch.float32, torch.bfloat16])
def test_linear_module_frozen_fp6_product(dev, compute_dtype):
    """freeze(): the eval-mode forward runs the FP6 operand path (quest_quantize_fwd_op + quest_gemm) and
    gives the oracle's Q(x) Q(w)^T + bias: the sum is exact, so fp32 output is within 1e-6 relative of
    the oracle, bf16 within one rounding (the tolerance of the product tests); training mode drops the
    operand again."""
    torch.manual_seed(1)
    layer = QuestLinear(2048, 384, bias=True, block=128, compute_dtype=compute_dtype, device=dev,
                        dtype=torch.bfloat16)
    with torch.no_grad():
        layer.bias.copy_(torch.linspace(-1, 1, 384, device=dev).to(torch.bfloat16))
    x = make_tensor(TensorSpec("frz.x", 3 * 40, 2048, "bf16", "student_t", 4, 9500, outlier_cols=20,
                               outlier_scale=20.0), dev).reshape(3, 40, 2048)
    log(f"frozen layer, input 3x40x2048, compute {compute_dtype}")
    layer.freeze()
    assert not layer.training and layer._w_operand is not None
    with torch.no_grad():
        y = layer(x)
    torch.cuda.synchronize()
    assert y.shape == (3, 40, 384)
    f = qo.qat_linear_fwd(to_float64(x.reshape(120, 2048)), to_float64(layer.weight.detach()), 128, 4, 4)
    bias64 = to_float64(layer.bias.detach())[None, :]
    skip_y, _, _ = band_reach(f, 4, 4, 128)
    got = y.reshape(120, 384).float().cpu().numpy().astype(np.float64)
    if compute_dtype == torch.float32:
        # fp32 output: the product exact up to the scale roundings (1e-6 of it), then one fp32
        # rounding of the sum with the bias (2^-24 of |product| + |bias|)
        scale = np.abs(f["y"]) + np.abs(bias64)
        err = np.abs(got - (f["y"] + bias64)) / scale
        assert (err[~skip_y] <= 2e-6).all(), f"max error / (|product| + |bias|) {err[~skip_y].max()}"
    else:
        close_product_plus_bias(y.reshape(120, 384), f, bias64, "frozen y", skip_y)
    layer.train()
    assert layer._w_operand is None


@pytest.mark.parametrize("n", [128, 130])
def test_linear_one_gradient_matches_both(dev, n):
    """The FP6 layer's backward for one gradient (x's or w's alone) against both at once: with one bit
    width and n a multiple of 4 the two operands' state shares one tensor per output and both gradients
    come from one rebuild and one trust backward (n = 128); otherwise (n = 130) each has its own."""
    k, m = 1024, 192
    x = make_tensor(TensorSpec("one.x", n, k, "bf16", "student_t", 4, 9990), dev)
    w = make_tensor(TensorSpec("one.w", m, k, "bf16", "normal", 0.02, 9991), dev)
    dy = make_tensor(TensorSpec("one.dy", n, m, "bf16", "normal", 1e-3, 9992), dev)
    log(f"one gradient against both, {n}x{k} by {m}x{k}")
    xg, wg = x.clone().requires_grad_(True), w.clone().requires_grad_(True)
    dx, dw = torch.autograd.grad(quest_linear(xg, wg, block=128), (xg, wg), dy)
    xg1 = x.clone().requires_grad_(True)
    (dx1,) = torch.autograd.grad(quest_linear(xg1, w, block=128), (xg1,), dy)
    wg1 = w.clone().requires_grad_(True)
    (dw1,) = torch.autograd.grad(quest_linear(x, wg1, block=128), (wg1,), dy)
    torch.cuda.synchronize()
    assert dx.shape == (n, k) and dw.shape == (m, k)
    # the gradient products are library GEMMs: allow their own summation order
    for got, ref, what in ((dx, dx1, "dx"), (dw, dw1, "dw")):
        err = (got.float() - ref.float()).abs().max().item()
        scale = ref.float().abs().max().item()
        assert err <= 1e-3 * scale, f"{what} off by {err} (largest entry {scale})"
