"""Comparison rules between libquest (fp32 on the GPU) and the fp64 oracle.

Codes and mask are integers decided by floating point, and the two sides
decide in different precisions (fp32 kernels, fp64 oracle).  Per the stated
acceptance rule they must agree bit for bit on every entry that is not
within 1e-6 * s_r of a threshold: a decision threshold j * Delta_r
(|j| <= L/2 - 1) or the trust threshold +-s_r L / (L - 1).  Entries inside
that band may differ; the fraction that actually differs must stay at or
below 1e-5, read as a rate: at most ceil(1e-5 * entries) entries, so a
tensor of fewer than 100000 entries may hold one.  Floating-point outputs
(dequantised values, gradients) must be within 1e-5 relative in fp32 and
2e-2 relative in bf16; for the gradient, "relative" is measured against
max(|ref|, RMS of ref over its Hadamard block), since a masked transform can
cancel to almost zero.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import quest_oracle as qo

BAND = 1e-6
MAX_MISMATCH_FRACTION = 1e-5
TOL_F32 = 1e-5
TOL_BF16 = 2e-2


def exempt_entries(y: np.ndarray, s: np.ndarray, b: int, band: float = BAND, trust: float = 1.0) -> np.ndarray:
    """True where y lies within band * s_r of a decision or trust threshold.

    The trust threshold is s_r (1 + trust / (L - 1)) (s_r L / (L - 1) for trust 1).
    """
    big_l = 1 << b
    s = np.asarray(s, dtype=np.float64)[:, None]
    delta = 2.0 * s / (big_l - 1)
    safe = np.where(delta == 0.0, 1.0, delta)
    j = np.clip(np.round(y / safe), -(big_l // 2 - 1), big_l // 2 - 1)
    near_decision = np.abs(y - j * safe) <= band * s
    near_trust = np.abs(np.abs(y) - s * (1.0 + trust / (big_l - 1))) <= band * s
    ex = near_decision | near_trust
    ex[(delta == 0.0)[:, 0], :] = False
    return ex


def check_fwd(x64: np.ndarray, block: int, b: int, codes, scale, mask, ref=None,
              max_fraction: float | None = MAX_MISMATCH_FRACTION, trust: float = 1.0) -> dict:
    """Assert GPU forward outputs (numpy uint8 / float32 arrays) match the oracle on x64.

    max_fraction bounds the share of entries (all inside the band) that differ.  It is a
    property of generic data; hand-built rows that put many entries exactly on a threshold
    (for instance exact zeros, the b = 1 decision threshold) pass None.
    """
    rows, cols = x64.shape
    if ref is None:
        ref = qo.quantize_fwd(x64, block, b, trust=trust)
    codes = np.asarray(codes).reshape(rows, cols * b // 8)
    mask = np.asarray(mask).reshape(rows, cols // 8)
    scale = np.asarray(scale, dtype=np.float64).reshape(rows)
    u = qo.unpack_lsb_first(codes, b, cols)
    m = qo.unpack_lsb_first(mask, 1, cols).astype(bool)
    ex = exempt_entries(ref["y"], ref["scale"], b, trust=trust)
    bad_u = u != ref["u"]
    bad_m = m != ref["m"]
    hard_u = bad_u & ~ex
    hard_m = bad_m & ~ex
    if hard_u.any() or hard_m.any():
        r, c = np.argwhere(hard_u | hard_m)[0]
        raise AssertionError(
            f"non-exempt mismatch at ({r},{c}): gpu u={u[r, c]} m={m[r, c]} oracle u={ref['u'][r, c]} "
            f"m={ref['m'][r, c]} y={ref['y'][r, c]!r} s={ref['scale'][r]!r}; "
            f"{int(hard_u.sum())} code and {int(hard_m.sum())} mask mismatches outside the band"
        )
    frac = float((bad_u | bad_m).mean()) if bad_u.size else 0.0
    if max_fraction is not None:
        # A rate: at most ceil(max_fraction * entries) differing entries, so that
        # a tensor of fewer than 1 / max_fraction entries may hold one.
        allowed = math.ceil(max_fraction * bad_u.size)
        count = int((bad_u | bad_m).sum())
        assert count <= allowed, f"{count} differing entries (fraction {frac}) above {allowed} allowed"
    s_ref = ref["scale"]
    zero = s_ref == 0.0
    assert np.all(scale[zero] == 0.0)
    rel = np.abs(scale[~zero] - s_ref[~zero]) / s_ref[~zero] if (~zero).any() else np.zeros(1)
    assert rel.max(initial=0.0) <= 2e-6, f"scale relative error {rel.max()}"
    return {
        "exempt": int(ex.sum()),
        "mismatched": int((bad_u | bad_m).sum()),
        "mismatch_fraction": frac,
        "scale_max_rel": float(rel.max(initial=0.0)),
        "elements": int(u.size),
    }


def check_values(got: np.ndarray, ref: np.ndarray, tol: float, skip=None) -> float:
    """|got - ref| <= tol * |ref| elementwise (entries in `skip` ignored); returns the max ratio."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    lim = tol * np.abs(ref)
    ok = err <= lim
    if skip is not None:
        ok |= skip
    if not ok.all():
        r, c = np.argwhere(~ok)[0]
        raise AssertionError(f"value mismatch at ({r},{c}): got {got[r, c]!r} ref {ref[r, c]!r}")
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(lim > 0, err / np.where(lim > 0, lim, 1), 0.0)
    if skip is not None:
        ratio = np.where(skip, 0.0, ratio)
    return float(ratio.max(initial=0.0))


def check_grad(got: np.ndarray, ref: np.ndarray, block: int, tol: float) -> float:
    """|got - ref| <= tol * max(|ref|, block RMS of ref); returns the max error ratio."""
    got = np.asarray(got, dtype=np.float64)
    rows, cols = ref.shape
    blk = ref.reshape(rows, cols // block, block)
    rms = np.sqrt(np.mean(blk * blk, axis=2, keepdims=True))
    scale = np.maximum(np.abs(blk), rms).reshape(rows, cols)
    err = np.abs(got - ref)
    ok = err <= tol * scale
    ok |= (err == 0.0)
    if not ok.all():
        r, c = np.argwhere(~ok)[0]
        raise AssertionError(f"gradient mismatch at ({r},{c}): got {got[r, c]!r} ref {ref[r, c]!r}")
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(scale > 0, err / (tol * np.where(scale > 0, scale, 1)), 0.0)
    return float(ratio.max(initial=0.0))
