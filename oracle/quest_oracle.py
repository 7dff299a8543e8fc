"""Plain, slow fp64 CPU oracle of the QuEST quantiser hot path.

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The
product library (libquest, HIP) never calls it and shares no code with it:
no kernels, headers, helpers, tables or constant generators.

What it computes (sources are the web pages about QuEST, arXiv 2502.05003;
each function names the page and section it follows):

* Forward: each row of x is cut into blocks of n entries and every block is
  multiplied by the orthonormal Hadamard matrix; the row is RMS-normalised;
  the result is projected onto a b-bit symmetric uniform grid whose clip
  scale alpha_b * RMS minimises the expected squared error for a standard
  Gaussian; the trust mask marks entries whose quantisation error is at most
  half a grid step.
* Backward: the Hadamard-domain gradient is multiplied by the stored mask and
  transformed back by the inverse Hadamard matrix.
* Product of two quantised operands (b <= 4): each grid value over its row's
  step is a half-integer, held as an FP6 E2M3 element; the product is the
  float64 matrix product of the decoded, rescaled operands.
* Other grids: FP4 (E2M1) levels with a Gaussian-MSE-optimal scale, and
  2:4-sparse b-bit codes (2 of every 4 Hadamard-domain entries kept).

Everything is float64 NumPy.  The Hadamard product is the dense O(n^2)
definition (a matrix product against the explicit n x n matrix), the clip
scale alpha_b is found by numerical minimisation, and rounding, masking and
bit packing are written elementwise.  ``quantize_rows_loop`` repeats the
quantiser as a literal per-element Python loop for small inputs.

Readings taken where the pages are silent (each listed with its reason in the
design notes of this repository):

* grid: 2^b levels, outermost levels at +-s with s = alpha_b * RMS, step
  Delta = 2 s / (L - 1), values beyond +-s clip to the outer level;
* RMS over the whole row, in the Hadamard domain;
* a zero row gives s = 0, the middle code L/2, q = 0 and mask 1;
* codes are offset-binary u = clamp(floor(y / Delta) + L/2, 0, L-1); an exact
  tie y = j * Delta goes to the larger code;
* mask = [|q - y| <= Delta / 2], inclusive;
* Sylvester natural order, orthonormal scaling 1/sqrt(n), no random signs;
* codes and mask are packed as LSB-first bit streams per row;
* the backward pass treats the scale as a constant: dX = H (M * G).

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (closed forms, a published table, brute force,
invariants and hand-packed bytes).  End-to-end values on real tensors are
not printed on the pages, so beyond those pins the oracle is the reference.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "sylvester_hadamard",
    "normalized_hadamard",
    "blockwise_hadamard",
    "grid_levels",
    "grid_thresholds",
    "gaussian_mse",
    "gaussian_mse_derivative",
    "fit_alpha",
    "quantize_rows",
    "quantize_rows_loop",
    "pack_lsb_first",
    "unpack_lsb_first",
    "quantize_fwd",
    "dequantize",
    "trust_bwd",
    "qat_linear_fwd",
    "qat_linear_bwd",
    "e2m3_value",
    "e2m3_encode",
    "operand_e2m3",
    "operand_step",
    "quest_gemm",
    "gaussian_mse_levels",
    "gaussian_mse_levels_derivative",
    "fit_alpha_levels",
    "e2m1_value",
    "e2m1_round",
    "fit_alpha_fp4",
    "quantize_rows_fp4",
    "quantize_fwd_fp4",
    "dequantize_fp4",
    "sparse24_keep",
    "quantize_rows_sparse24",
    "quantize_fwd_sparse24",
    "dequantize_sparse24",
]


# ---------------------------------------------------------------------------
# Hadamard transform
# pith.science review of QuEST, "Assumptions & free parameters" (the
# standard-math item: Hadamard matrices are orthogonal and fast transforms
# exist) and "What carries the argument" (the forward step applies a Hadamard
# transform to weights and activations).
# ---------------------------------------------------------------------------

def sylvester_hadamard(n: int) -> np.ndarray:
    """Unnormalised Sylvester Hadamard matrix H_n (entries +-1).

    Built by the doubling recursion H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]],
    which puts it in natural (Sylvester) order.
    """
    if n < 1 or (n & (n - 1)) != 0:
        raise ValueError(f"Hadamard size must be a power of two, got {n}")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def normalized_hadamard(n: int) -> np.ndarray:
    """Orthonormal Hadamard matrix H_n / sqrt(n); symmetric and its own inverse."""
    return sylvester_hadamard(n) / math.sqrt(n)


def blockwise_hadamard(x: np.ndarray, n: int) -> np.ndarray:
    """Apply the orthonormal Hadamard matrix to every length-n block of every row.

    y[r, k*n:(k+1)*n] = (H_n / sqrt(n)) @ x[r, k*n:(k+1)*n], computed as a
    dense matrix product against the explicit +-1 matrix H_n, divided by
    sqrt(n) afterwards.  The +-1 sums of bf16 inputs (and of fp32 inputs of
    moderate dynamic range) are exact in float64, and one division per entry
    maps equal sums to equal outputs, so entries that are equal in magnitude
    by the definition stay equal: the 2:4 rule breaks such ties by index, not
    by rounding noise of the product.
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("x must be 2-D (rows x cols)")
    rows, cols = x.shape
    if cols % n != 0:
        raise ValueError(f"cols={cols} is not a multiple of the block size {n}")
    h = sylvester_hadamard(n)
    blocks = x.reshape(rows, cols // n, n)
    # For each block vector v (a row of `blocks`), v @ h.T == (h @ v) as a row.
    y = (blocks @ h.T) / math.sqrt(n)
    return y.reshape(rows, cols)


# ---------------------------------------------------------------------------
# The Gaussian-optimal clip scale alpha_b
# pith.science review of QuEST, "What carries the argument" (the grid scale
# minimises the L2 error against a standard Gaussian) and "Assumptions & free
# parameters" (alpha* comes from a fixed N(0,1) target, not from data);
# atlas.scime.ai summary of QuEST, "Approach" (MSE-optimal clipping fitted to
# a Gaussian).
# ---------------------------------------------------------------------------

_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def _std_normal_cdf(t: float) -> float:
    if t == math.inf:
        return 1.0
    if t == -math.inf:
        return 0.0
    return 0.5 * math.erfc(-t / math.sqrt(2.0))


def _std_normal_pdf(t: float) -> float:
    if math.isinf(t):
        return 0.0
    return _INV_SQRT_2PI * math.exp(-0.5 * t * t)


def _t_times_pdf(t: float) -> float:
    if math.isinf(t):
        return 0.0
    return t * _std_normal_pdf(t)


def grid_levels(alpha: float, b: int) -> list[float]:
    """The L = 2^b reconstruction levels (2k - L + 1) * alpha / (L - 1), k = 0..L-1.

    The outermost levels sit at +-alpha and neighbours are 2 alpha / (L - 1) apart.
    """
    big_l = 1 << b
    return [(2 * k - big_l + 1) * alpha / (big_l - 1) for k in range(big_l)]


def grid_thresholds(alpha: float, b: int) -> list[float]:
    """Decision thresholds t_0 = -inf < t_1 < ... < t_{L-1} < t_L = +inf.

    Interior thresholds are the midpoints of neighbouring levels, so cell k
    is [t_k, t_{k+1}) and maps to level k (nearest-level rounding).
    """
    lv = grid_levels(alpha, b)
    inner = [0.5 * (lv[k - 1] + lv[k]) for k in range(1, len(lv))]
    return [-math.inf] + inner + [math.inf]


def gaussian_mse(alpha: float, b: int) -> float:
    """E[(Q_{alpha,b}(X) - X)^2] for X ~ N(0, 1), in closed form.

    Over a cell [a, c] mapped to level l:
      int (x - l)^2 phi(x) dx
        = (1 + l^2) (Phi(c) - Phi(a)) - (c phi(c) - a phi(a)) + 2 l (phi(c) - phi(a)),
    using int phi = Phi, int x phi = -phi and int x^2 phi = Phi - x phi.
    """
    lv = grid_levels(alpha, b)
    th = grid_thresholds(alpha, b)
    total = 0.0
    for k, level in enumerate(lv):
        a, c = th[k], th[k + 1]
        mass = _std_normal_cdf(c) - _std_normal_cdf(a)
        total += (1.0 + level * level) * mass
        total -= _t_times_pdf(c) - _t_times_pdf(a)
        total += 2.0 * level * (_std_normal_pdf(c) - _std_normal_pdf(a))
    return total


def gaussian_mse_derivative(alpha: float, b: int) -> float:
    """d/d alpha of ``gaussian_mse``.

    With level k = c_k alpha, c_k = (2k - L + 1)/(L - 1), the moving cell
    edges contribute nothing (the integrand is continuous across a midpoint),
    so  dMSE/d alpha = -2 sum_k c_k [ (phi(t_k) - phi(t_{k+1}))
                                      - c_k alpha (Phi(t_{k+1}) - Phi(t_k)) ].
    """
    big_l = 1 << b
    th = grid_thresholds(alpha, b)
    total = 0.0
    for k in range(big_l):
        ck = (2 * k - big_l + 1) / (big_l - 1)
        a, c = th[k], th[k + 1]
        first_moment = _std_normal_pdf(a) - _std_normal_pdf(c)
        mass = _std_normal_cdf(c) - _std_normal_cdf(a)
        total += ck * (first_moment - ck * alpha * mass)
    return -2.0 * total


def _golden_section_min(f, lo: float, hi: float, tol: float) -> float:
    inv_phi = (math.sqrt(5.0) - 1.0) / 2.0
    a, b = lo, hi
    c = b - inv_phi * (b - a)
    d = a + inv_phi * (b - a)
    fc, fd = f(c), f(d)
    while (b - a) > tol:
        if fc < fd:
            b, d, fd = d, c, fc
            c = b - inv_phi * (b - a)
            fc = f(c)
        else:
            a, c, fc = c, d, fd
            d = a + inv_phi * (b - a)
            fd = f(d)
    return 0.5 * (a + b)


def fit_alpha(b: int) -> float:
    """alpha_b = argmin_alpha E[(Q_{alpha,b}(X) - X)^2], X ~ N(0, 1).

    Golden-section search of ``gaussian_mse`` on [0.05, 8], then bisection on
    the sign of ``gaussian_mse_derivative`` around that point.  The minimum is
    flat (the MSE is quadratic there), so the golden-section result alone is
    good to only about 1e-8 relative; the derivative has a clean sign change
    and bisection takes it to the last bit.
    """
    if not 1 <= b <= 16:
        raise ValueError(f"b must be in [1, 16], got {b}")
    guess = _golden_section_min(lambda a: gaussian_mse(a, b), 0.05, 8.0, 1e-9)
    lo, hi = guess * (1.0 - 1e-4), guess * (1.0 + 1e-4)
    while gaussian_mse_derivative(lo, b) > 0.0:
        lo *= 0.9
    while gaussian_mse_derivative(hi, b) < 0.0:
        hi *= 1.1
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if mid <= lo or mid >= hi:
            break
        if gaussian_mse_derivative(mid, b) < 0.0:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


# ---------------------------------------------------------------------------
# RMS scale, grid projection and trust mask
# atlas.scime.ai summary of QuEST, "Approach" (Hadamard transform followed by
# RMS normalisation and MSE-optimal clipping; gradients are masked for
# entries whose quantisation error exceeds a trust threshold); pith.science
# review, "What carries the argument" (projection onto the uniform grid; the
# mask zeroes entries whose error exceeds half a quantisation interval) and
# Figure 7 caption (the mask M_alpha*).
# ---------------------------------------------------------------------------

def quantize_rows(y: np.ndarray, b: int, alpha: float, trust: float = 1.0):
    """Quantise Hadamard-domain rows y (R x C).

    Returns (u, s, m, q):
      s[r]    = alpha * RMS_r with RMS_r = sqrt(mean_c y[r, c]^2)   (clip scale)
      u[r, c] = clamp(floor(y / Delta_r) + L/2, 0, L - 1), Delta_r = 2 s_r / (L - 1)
      q[r, c] = (2 u - L + 1) * Delta_r / 2                      (the grid value)
      m[r, c] = |q - y| <= Delta_r / 2             for |y| <= s_r  (trust mask)
              = |q - y| <= trust * Delta_r / 2     for |y| >  s_r  (outer trust region)
    A row of zeros has s = 0; it takes the middle code L/2 and q = 0, m = 1.

    The outer trust factor scales the trust region beyond the outermost
    levels (pith.science review of QuEST, "Assumptions & free parameters":
    the outer trust scaling factor, s* = 1.30 for 1-bit runs; atlas.scime.ai
    summary, "Approach" and "Limitations").  Inside the grid the rounding
    error never exceeds Delta / 2, so only clipped entries are affected; with
    trust = 1 the mask is the plain |q - y| <= Delta / 2.
    """
    y = np.asarray(y, dtype=np.float64)
    big_l = 1 << b
    rms = np.sqrt(np.mean(y * y, axis=1))
    s = alpha * rms
    delta = 2.0 * s / (big_l - 1)
    zero_row = delta == 0.0
    safe_delta = np.where(zero_row, 1.0, delta)
    u = np.floor(y / safe_delta[:, None]) + big_l // 2
    u = np.clip(u, 0, big_l - 1)
    u[zero_row, :] = big_l // 2
    u = u.astype(np.int64)
    q = (2 * u - big_l + 1) * delta[:, None] / 2.0
    err = np.abs(q - y)
    inside = np.abs(y) <= s[:, None]
    m = np.where(inside, err <= delta[:, None] / 2.0, err <= trust * delta[:, None] / 2.0)
    return u, s, m, q


def quantize_rows_loop(y, b: int, alpha: float, trust: float = 1.0):
    """The same quantiser as ``quantize_rows`` written as a scalar Python loop.

    Used on small inputs to cross-check the vectorised form.
    """
    big_l = 1 << b
    rows = len(y)
    cols = len(y[0])
    u = np.zeros((rows, cols), dtype=np.int64)
    m = np.zeros((rows, cols), dtype=bool)
    q = np.zeros((rows, cols), dtype=np.float64)
    s = np.zeros(rows, dtype=np.float64)
    for r in range(rows):
        acc = 0.0
        for c in range(cols):
            acc += float(y[r][c]) * float(y[r][c])
        s_r = alpha * math.sqrt(acc / cols)
        d_r = 2.0 * s_r / (big_l - 1)
        s[r] = s_r
        for c in range(cols):
            v = float(y[r][c])
            if d_r == 0.0:
                code = big_l // 2
            else:
                code = math.floor(v / d_r) + big_l // 2
                code = min(max(code, 0), big_l - 1)
            level = (2 * code - big_l + 1) * d_r / 2.0
            u[r, c] = code
            q[r, c] = level
            if abs(v) <= s_r:
                m[r, c] = abs(level - v) <= d_r / 2.0
            else:
                m[r, c] = abs(level - v) <= trust * d_r / 2.0
    return u, s, m, q


# ---------------------------------------------------------------------------
# Bit packing (a storage layout; the pages only say that INT4 codes are
# stored and that the mask is kept from the forward pass for the backward).
# ---------------------------------------------------------------------------

def pack_lsb_first(values: np.ndarray, width: int) -> np.ndarray:
    """Pack each row of unsigned ints (< 2^width) into an LSB-first byte stream.

    Element c occupies stream bits [c*width, (c+1)*width), low bit first;
    stream bit 8j + i is bit i of byte j.  Returns R x (C*width/8) uint8.
    """
    values = np.asarray(values, dtype=np.int64)
    rows, cols = values.shape
    nbits = cols * width
    if nbits % 8 != 0:
        raise ValueError("cols * width must be a multiple of 8")
    if values.size and (values.min() < 0 or values.max() >= (1 << width)):
        raise ValueError("value out of range for the bit width")
    bits = (values[:, :, None] >> np.arange(width)[None, None, :]) & 1
    stream = bits.reshape(rows, nbits)
    byte_bits = stream.reshape(rows, nbits // 8, 8)
    packed = (byte_bits << np.arange(8)[None, None, :]).sum(axis=2)
    return packed.astype(np.uint8)


def unpack_lsb_first(packed: np.ndarray, width: int, cols: int) -> np.ndarray:
    """Inverse of ``pack_lsb_first``: R x (C*width/8) uint8 -> R x C int64."""
    packed = np.asarray(packed, dtype=np.uint8)
    rows = packed.shape[0]
    if packed.shape[1] * 8 != cols * width:
        raise ValueError("packed width does not match cols * width / 8")
    stream = (packed[:, :, None].astype(np.int64) >> np.arange(8)[None, None, :]) & 1
    stream = stream.reshape(rows, cols, width)
    return (stream << np.arange(width)[None, None, :]).sum(axis=2)


# ---------------------------------------------------------------------------
# The three calls of the path
# ---------------------------------------------------------------------------

def quantize_fwd(x: np.ndarray, block: int, b: int, alpha: float | None = None, trust: float = 1.0) -> dict:
    """Forward QuEST quantisation of x (R x C): Hadamard -> RMS -> clip/round -> mask.

    QuEST abstract (codewithpapers.app record; Hadamard normalisation and
    MSE-optimal fitting), atlas.scime.ai summary "Approach", pith.science
    review "What carries the argument".
    Returns packed codes (R x C*b/8 uint8), the clip scale s (R, float64),
    the packed mask (R x C/8 uint8) and the unpacked intermediates.
    """
    if alpha is None:
        alpha = fit_alpha(b)
    y = blockwise_hadamard(x, block)
    u, s, m, q = quantize_rows(y, b, alpha, trust)
    return {
        "codes": pack_lsb_first(u, b),
        "scale": s,
        "mask": pack_lsb_first(m.astype(np.int64), 1),
        "y": y,
        "u": u,
        "m": m,
        "q": q,
        "alpha": alpha,
    }


def dequantize(codes: np.ndarray, scale: np.ndarray, cols: int, b: int) -> np.ndarray:
    """Grid values (2u - L + 1) * s / (L - 1), in the Hadamard domain.

    The conceptual twin of the official repository's ``dequantize_dense``
    entry (named in the codewithpapers.app record).  Quantised operands stay
    in the Hadamard domain because the transform is orthogonal and is applied
    to both operands of a product (pith.science review, "Assumptions & free
    parameters").
    """
    big_l = 1 << b
    u = unpack_lsb_first(codes, b, cols)
    s = np.asarray(scale, dtype=np.float64)
    return (2 * u - big_l + 1) * s[:, None] / (big_l - 1)


def trust_bwd(grad: np.ndarray, mask: np.ndarray, block: int) -> np.ndarray:
    """Trust-gradient backward: dX = H (M * G) per block.

    pith.science review, "What carries the argument" (the Hadamard-domain
    gradient is multiplied by the binary trust mask) and Figure 2 caption
    (inverse Hadamard transforms on the backward pass).  H is symmetric and
    orthonormal, so the inverse transform is the same block product.
    """
    grad = np.asarray(grad, dtype=np.float64)
    m = unpack_lsb_first(mask, 1, grad.shape[1]).astype(np.float64)
    return blockwise_hadamard(m * grad, block)


# ---------------------------------------------------------------------------
# A quantisation-aware linear layer built from the pieces above.
# pith.science review of QuEST, "Assumptions & free parameters" (the
# orthogonal transform is applied to both operands of a product, so their
# product can be taken in the transformed domain), "What carries the
# argument" and the Figure 2 caption (the backward pass masks the
# Hadamard-domain gradient with the trust mask and transforms it back).
# ---------------------------------------------------------------------------
def qat_linear_fwd(x: np.ndarray, w: np.ndarray, block: int, bits_x: int, bits_w: int, trust_x: float = 1.0,
                   trust_w: float = 1.0, grid: str = "int") -> dict:
    """y = Q(x) Q(w)^T with both operands quantised along their last axis.

    x is N x K (activations), w is M x K (weights); the Hadamard blocks run
    along K, the contraction axis.  Q(.) is the dequantised grid value in the
    Hadamard domain, so y = (x~ H)(w~ H)^T = x~ w~^T, where x~ and w~ are the
    original-domain reconstructions.  grid: "int" (b-bit midrise levels),
    "fp4" (E2M1 levels; the bit widths are unused) or "sparse24" (2:4-sparse
    b-bit levels): the formats the pages train with, each through its own
    quantiser above.
    """
    def quantise(t, bits, trust):
        t = np.asarray(t, dtype=np.float64)
        if grid == "int":
            return quantize_fwd(t, block, bits, trust=trust)
        if grid == "fp4":
            return quantize_fwd_fp4(t, block, trust=trust)
        if grid == "sparse24":
            return quantize_fwd_sparse24(t, block, bits, trust=trust)
        raise ValueError(f"unknown grid {grid!r}")

    fx = quantise(x, bits_x, trust_x)
    fw = quantise(w, bits_w, trust_w)
    qx = fx["q"]
    qw = fw["q"]
    return {"y": qx @ qw.T, "qx": qx, "qw": qw, "mask_x": fx["mask"], "mask_w": fw["mask"], "fx": fx, "fw": fw}


def qat_linear_bwd(dy: np.ndarray, fwd: dict, block: int) -> tuple:
    """Gradients of the layer with the trust estimator on both operands.

    The gradient reaching Q(x) is dy Q(w), the one reaching Q(w) is
    dy^T Q(x); each is masked by its operand's trust mask and transformed
    back (trust_bwd).  Returns (dx, dw).
    """
    dy = np.asarray(dy, dtype=np.float64)
    dx = trust_bwd(dy @ fwd["qw"], fwd["mask_x"], block)
    dw = trust_bwd(dy.T @ fwd["qx"], fwd["mask_w"], block)
    return dx, dw


# ---------------------------------------------------------------------------
# Low-precision product of two quantised operands.
# The pages time QuEST's 4-bit matrix products against BF16 ones, with the
# quantisation, dequantisation and Hadamard costs included (pith.science
# review of QuEST, Figure 5 caption; atlas.scime.ai summary, "Key results").
# On the midrise grid every level is a half-integer multiple of the step,
# q = (u - (L - 1)/2) * Delta, so for b <= 4 the half-integer fits the FP6
# E2M3 element format exactly and the product of two operands is
# Delta_a Delta_b times a sum of products of half-integers.
# E2M3 is the FP6 element type of the OCP Microscaling (MX) Formats
# specification v1.0: one sign bit, two exponent bits with bias 1, three
# mantissa bits, subnormals at exponent 0, no infinities and no NaN.
# ---------------------------------------------------------------------------

def e2m3_value(code) -> np.ndarray:
    """Decode 6-bit E2M3 codes (sign bit 5, exponent bits 4..3, mantissa bits 2..0)."""
    code = np.asarray(code, dtype=np.int64)
    if code.size and (code.min() < 0 or code.max() > 63):
        raise ValueError("E2M3 codes are 6-bit")
    sign = np.where((code >> 5) & 1, -1.0, 1.0)
    exp = (code >> 3) & 3
    man = (code & 7).astype(np.float64)
    mag = np.where(exp == 0, man / 8.0, (1.0 + man / 8.0) * np.exp2(exp - 1.0))
    return sign * mag


def e2m3_encode(v) -> np.ndarray:
    """Encode values that E2M3 holds exactly; anything else is an error.

    |v| < 1 is a subnormal (exponent field 0, mantissa |v| * 8); otherwise the
    exponent field is floor(log2 |v|) + 1 and the mantissa (|v| / 2^(e-1) - 1) * 8.
    Zero encodes as +0.
    """
    v = np.asarray(v, dtype=np.float64)
    mag = np.abs(v)
    out = np.zeros(v.shape, dtype=np.int64)
    sub = mag < 1.0
    man_sub = mag * 8.0
    e = np.where(sub, 0, np.floor(np.log2(np.where(sub, 1.0, mag))).astype(np.int64) + 1)
    man_norm = (mag / np.exp2(np.maximum(e, 1) - 1.0) - 1.0) * 8.0
    man = np.where(sub, man_sub, man_norm)
    if np.any(e > 3) or np.any(man != np.round(man)) or np.any(man < 0) or np.any(man > 7):
        raise ValueError("value not exactly representable in E2M3")
    out = (np.where(v < 0, 1, 0) << 5) | (e << 3) | man.astype(np.int64)
    return out


def operand_e2m3(codes: np.ndarray, cols: int, b: int) -> np.ndarray:
    """Matrix-core operand of packed b-bit codes: u - (L - 1)/2 as E2M3, 6 bits per element.

    Returns R x (C * 6 / 8) uint8, an LSB-first 6-bit stream per row (the
    same stream layout as the codes).  Defined for b <= 4, where the largest
    half-integer (L - 1)/2 = 7.5 is E2M3's largest value.
    """
    if not 1 <= b <= 4:
        raise ValueError("the E2M3 operand holds b <= 4 bit grids")
    big_l = 1 << b
    u = unpack_lsb_first(codes, b, cols)
    return pack_lsb_first(e2m3_encode(u - (big_l - 1) / 2.0), 6)


def operand_step(scale: np.ndarray, b: int) -> np.ndarray:
    """Grid step Delta = 2 s / (L - 1) of each row, from its clip scale s."""
    return 2.0 * np.asarray(scale, dtype=np.float64) / ((1 << b) - 1)


def quest_gemm(a_op: np.ndarray, a_scale: np.ndarray, bits_a: int, b_op: np.ndarray, b_scale: np.ndarray,
               bits_b: int, k: int) -> np.ndarray:
    """y = Q(a) Q(b)^T from two E2M3 operands (M x K and N x K) and their clip scales.

    Q(.)[r, c] = e2m3_value(field c of row r) * Delta_r; the product is a
    float64 matrix product of the decoded operands.  With Hadamard-domain
    operands this is the layer output of ``qat_linear_fwd``.
    """
    va = e2m3_value(unpack_lsb_first(a_op, 6, k)) * operand_step(a_scale, bits_a)[:, None]
    vb = e2m3_value(unpack_lsb_first(b_op, 6, k)) * operand_step(b_scale, bits_b)[:, None]
    return va @ vb.T


# ---------------------------------------------------------------------------
# Other grids: FP4 levels and 2:4-sparse integer codes.
# The pages extend the method to an FP4 format and to 2:4-sparse INT4
# (pith.science review of QuEST, the list of contributions and the captions
# of Figures 3 and 4; atlas.scime.ai summary, "Key results": FP4 fits a
# slightly worse scaling law than INT4, which the authors attribute to a
# higher Gaussian MSE once clipping is allowed; the ablation table: 2:4
# sparsity added to INT4).  FP4 is the E2M1 element type of the OCP MX
# specification v1.0: sign bit 3, exponent bits 2..1 with bias 1, mantissa
# bit 0, subnormals at exponent 0, no infinities or NaN; magnitudes
# 0, 0.5, 1, 1.5, 2, 3, 4, 6.
# ---------------------------------------------------------------------------

def gaussian_mse_levels(levels) -> float:
    """E[(Q(X) - X)^2], X ~ N(0, 1), for nearest-level rounding onto `levels` (sorted).

    Cells run between midpoints of neighbouring levels; the outer cells are
    unbounded (clipping).  Same per-cell closed form as ``gaussian_mse``.
    """
    lv = [float(v) for v in levels]
    th = [-math.inf] + [0.5 * (lv[k - 1] + lv[k]) for k in range(1, len(lv))] + [math.inf]
    total = 0.0
    for k, level in enumerate(lv):
        a, c = th[k], th[k + 1]
        total += (1.0 + level * level) * (_std_normal_cdf(c) - _std_normal_cdf(a))
        total -= _t_times_pdf(c) - _t_times_pdf(a)
        total += 2.0 * level * (_std_normal_pdf(c) - _std_normal_pdf(a))
    return total


def gaussian_mse_levels_derivative(unit_levels, alpha: float) -> float:
    """d/d alpha of gaussian_mse_levels(alpha * unit_levels) (cell edges contribute nothing)."""
    lv = [alpha * float(v) for v in unit_levels]
    th = [-math.inf] + [0.5 * (lv[k - 1] + lv[k]) for k in range(1, len(lv))] + [math.inf]
    total = 0.0
    for k, unit in enumerate(unit_levels):
        a, c = th[k], th[k + 1]
        first_moment = _std_normal_pdf(a) - _std_normal_pdf(c)
        mass = _std_normal_cdf(c) - _std_normal_cdf(a)
        total += float(unit) * (first_moment - float(unit) * alpha * mass)
    return -2.0 * total


def fit_alpha_levels(unit_levels) -> float:
    """alpha minimising the Gaussian MSE of the grid alpha * unit_levels (largest level 1).

    Golden-section search on [0.05, 8], then bisection on the derivative, as
    ``fit_alpha``.
    """
    f = lambda a: gaussian_mse_levels([a * v for v in unit_levels])
    guess = _golden_section_min(f, 0.05, 8.0, 1e-9)
    lo, hi = guess * (1.0 - 1e-4), guess * (1.0 + 1e-4)
    while gaussian_mse_levels_derivative(unit_levels, lo) > 0.0:
        lo *= 0.9
    while gaussian_mse_levels_derivative(unit_levels, hi) < 0.0:
        hi *= 1.1
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if mid <= lo or mid >= hi:
            break
        if gaussian_mse_levels_derivative(unit_levels, mid) < 0.0:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def e2m1_value(code) -> np.ndarray:
    """Decode 4-bit E2M1 codes (sign bit 3, exponent bits 2..1, mantissa bit 0)."""
    code = np.asarray(code, dtype=np.int64)
    if code.size and (code.min() < 0 or code.max() > 15):
        raise ValueError("E2M1 codes are 4-bit")
    sign = np.where((code >> 3) & 1, -1.0, 1.0)
    exp = (code >> 1) & 3
    man = (code & 1).astype(np.float64)
    mag = np.where(exp == 0, man * 0.5, (1.0 + man * 0.5) * np.exp2(exp - 1.0))
    return sign * mag


FP4_MAGNITUDES = e2m1_value(np.arange(8))  # 0, 0.5, 1, 1.5, 2, 3, 4, 6
FP4_UNIT_LEVELS = np.concatenate([-FP4_MAGNITUDES[:0:-1], FP4_MAGNITUDES]) / 6.0  # 15 levels, largest 1


def e2m1_round(z) -> np.ndarray:
    """E2M1 code of the level nearest to z; a tie goes to the code with mantissa bit 0;
    beyond 6 in magnitude the code saturates at +-6.  The sign bit is that of z, except on
    the zero level, which is always code 0: one code per level of the grid, so that codes
    compare as levels do."""
    z = np.asarray(z, dtype=np.float64)
    mag = np.abs(z)
    dist = np.abs(mag[..., None] - FP4_MAGNITUDES)  # to each magnitude level
    best = dist.min(axis=-1, keepdims=True)
    cand = dist == best  # nearest levels (two on a tie)
    # among the nearest, prefer an even code (mantissa bit 0), then the smaller code
    score = np.where(cand, (np.arange(8) & 1) * 16 + np.arange(8), 1000)
    code = np.argmin(score, axis=-1)
    code = np.where(mag > 6.0, 7, code)
    return np.where(np.signbit(z) & (code != 0), code | 8, code).astype(np.int64)


def fit_alpha_fp4() -> float:
    """alpha of the FP4 grid: its largest level sits at alpha * RMS."""
    return fit_alpha_levels(FP4_UNIT_LEVELS)


def quantize_rows_fp4(y: np.ndarray, alpha: float, trust: float = 1.0):
    """FP4 quantiser of Hadamard-domain rows y (R x C).

    s = alpha * RMS (the largest level), q = e2m1(code) * s / 6 with
    code = e2m1_round(6 y / s).  Trust (the pages' rule of at most half a
    quantisation interval, read for an uneven grid): inside [-s, s] the error
    must not exceed half the interval between the two levels around y;
    beyond it, t times half the outermost interval, (6 - 4)/2 * s/6.  A zero
    row gives s = 0, code 0, q = 0, mask 1.
    Returns (codes, s, m, q).
    """
    y = np.asarray(y, dtype=np.float64)
    rms = np.sqrt(np.mean(y * y, axis=1))
    s = alpha * rms
    zero_row = s == 0.0
    safe_s = np.where(zero_row, 1.0, s)
    code = e2m1_round(6.0 * y / safe_s[:, None])
    code[zero_row, :] = 0
    unit = s[:, None] / 6.0
    q = e2m1_value(code) * unit
    err = np.abs(q - y)
    a = np.abs(y) / np.where(zero_row, 1.0, unit[:, 0])[:, None]  # |y| in units of s/6
    idx = np.clip(np.searchsorted(FP4_MAGNITUDES, a, side="right") - 1, 0, 6)
    half_local = 0.5 * (FP4_MAGNITUDES[idx + 1] - FP4_MAGNITUDES[idx]) * unit
    half_outer = 0.5 * (FP4_MAGNITUDES[7] - FP4_MAGNITUDES[6]) * unit
    inside = np.abs(y) <= s[:, None]
    m = np.where(inside, err <= half_local, err <= trust * half_outer)
    m[zero_row, :] = True
    return code, s, m, q


def quantize_fwd_fp4(x: np.ndarray, block: int, alpha: float | None = None, trust: float = 1.0) -> dict:
    """Hadamard -> RMS -> FP4 levels -> trust mask; codes packed 4 bits per element LSB-first."""
    if alpha is None:
        alpha = fit_alpha_fp4()
    y = blockwise_hadamard(x, block)
    code, s, m, q = quantize_rows_fp4(y, alpha, trust)
    return {"codes": pack_lsb_first(code, 4), "scale": s, "mask": pack_lsb_first(m.astype(np.int64), 1), "y": y,
            "u": code, "m": m, "q": q, "alpha": alpha}


def dequantize_fp4(codes: np.ndarray, scale: np.ndarray, cols: int) -> np.ndarray:
    """FP4 grid values e2m1(code) * s / 6."""
    code = unpack_lsb_first(codes, 4, cols)
    return e2m1_value(code) * np.asarray(scale, dtype=np.float64)[:, None] / 6.0


def sparse24_keep(y: np.ndarray) -> np.ndarray:
    """2:4 pattern: in each group of 4 consecutive entries of a row the 2 largest |y| stay
    (on equal magnitudes the lower index wins)."""
    y = np.asarray(y, dtype=np.float64)
    rows, cols = y.shape
    g = np.abs(y).reshape(rows, cols // 4, 4)
    keep = np.zeros(g.shape, dtype=bool)
    for r in range(rows):
        for k in range(cols // 4):
            order = sorted(range(4), key=lambda i: (-g[r, k, i], i))
            keep[r, k, order[0]] = True
            keep[r, k, order[1]] = True
    return keep.reshape(rows, cols)


def quantize_rows_sparse24(y: np.ndarray, b: int, alpha: float, trust: float = 1.0):
    """2:4-sparse b-bit quantiser of Hadamard-domain rows y (R x C, C a multiple of 4).

    The pattern keeps 2 of every 4 entries (``sparse24_keep``); the clip
    scale is s = alpha_b * RMS of the kept entries; kept entries take the
    b-bit code and level of ``quantize_rows`` (with that s); pruned entries
    reconstruct as 0.  The mask is the literal trust rule on the sparse
    reconstruction: kept entries as in ``quantize_rows``, pruned ones trusted
    iff |0 - y| <= Delta / 2.
    Returns (keep, u_kept (R x C/2, in index order), s, m, q).
    """
    y = np.asarray(y, dtype=np.float64)
    rows, cols = y.shape
    keep = sparse24_keep(y)
    kept = y[keep].reshape(rows, cols // 2)
    u, s, m_kept, q_kept = quantize_rows(kept, b, alpha, trust)
    big_l = 1 << b
    delta = 2.0 * s / (big_l - 1)
    q = np.zeros_like(y)
    q[keep] = q_kept.reshape(-1)
    m = np.abs(y) <= delta[:, None] / 2.0
    m[keep] = m_kept.reshape(-1)
    return keep, u, s, m, q


def quantize_fwd_sparse24(x: np.ndarray, block: int, b: int, alpha: float | None = None, trust: float = 1.0) -> dict:
    """Hadamard -> 2:4 pattern -> RMS of the kept entries -> b-bit codes -> trust mask.

    Packed per row: the kept entries' codes (C/2 codes of b bits, LSB-first,
    in index order) and their positions inside their group of 4 (C/2
    2-bit fields, LSB-first); the mask as for the dense quantiser.
    """
    if alpha is None:
        alpha = fit_alpha(b)
    y = blockwise_hadamard(x, block)
    keep, u, s, m, q = quantize_rows_sparse24(y, b, alpha, trust)
    rows, cols = y.shape
    pos = np.nonzero(keep.reshape(rows, cols // 4, 4))[2].reshape(rows, cols // 2)
    return {"codes": pack_lsb_first(u, b), "index": pack_lsb_first(pos, 2), "scale": s,
            "mask": pack_lsb_first(m.astype(np.int64), 1), "y": y, "u": u, "keep": keep, "m": m, "q": q,
            "alpha": alpha}


def dequantize_sparse24(codes: np.ndarray, index: np.ndarray, scale: np.ndarray, cols: int, b: int) -> np.ndarray:
    """Dense Hadamard-domain values of a 2:4-sparse code stream (pruned entries 0)."""
    big_l = 1 << b
    u = unpack_lsb_first(codes, b, cols // 2)
    pos = unpack_lsb_first(index, 2, cols // 2)
    rows = u.shape[0]
    s = np.asarray(scale, dtype=np.float64)
    vals = (2 * u - big_l + 1) * s[:, None] / (big_l - 1)
    out = np.zeros((rows, cols), dtype=np.float64)
    grp = np.arange(cols // 2) // 2
    for r in range(rows):
        out[r, 4 * grp + pos[r]] = vals[r]
    return out
