"""QuEST quantisation-aware linear layer on libquest.

y = Q(x) Q(w)^T + bias, where Q(.) quantises each operand along the
contraction axis (blockwise Hadamard transform, RMS clip scale, b-bit grid)
and returns the grid values in the Hadamard domain.  The transform is
orthogonal and applied to both operands, so the product of the transformed
operands equals the product of their original-domain reconstructions
(pith.science review of QuEST, "Assumptions & free parameters").  The
backward pass uses the trust estimator on both operands: the gradient
reaching Q(x) is dy Q(w), the one reaching Q(w) is dy^T Q(x); each is masked
by its operand's trust mask and transformed back (pith.science review,
"What carries the argument" and the Figure 2 caption).

Quantisation, masking and both transforms run in libquest's kernels
(quest_quantize_fwd_ex, or the FP4 and 2:4-sparse forwards, and
quest_trust_bwd).  On the int grid with b <= 4 and K a multiple of 128 the
forward product is libquest's FP6 product of the two operands
(quest_quantize_fwd_op with codes and mask, both operands in one
quest_quantize_fwd_op_group launch when they share dtype and trust factor,
then quest_gemm: exact sums, one rounding to the compute dtype), and the backward rebuilds Q(x) and Q(w) from
the saved codes (quest_dequantize, the same values as the dequantised
forward output).  The two gradient products, and the forward product of the
other configurations, are plain library GEMMs through torch.  ``grid`` picks the format the operands are quantised to: "int"
(b-bit midrise levels), "fp4" (E2M1 levels, 4 bits whatever bits_x and
bits_w say) or "sparse24" (2:4-sparse b-bit levels), the formats the pages
train with (pith.science review of QuEST, the list of contributions and the
captions of Figures 3 and 4); all three share the transform, the RMS scale
and the trust rule.

Inference (``QuestLinear.freeze``, then eval mode): the weight is quantised
once into the FP6 matrix-core operand, each activation by
quest_quantize_fwd_op, and the product is libquest's FP6 GEMM (quest_gemm):
the 4-bit layer product whose speed the pages compare with BF16 (pith.science
review, Figure 5 caption).
"""
from __future__ import annotations

import torch

from . import (dequantize, gemm, quantize_fwd_ex, quantize_fwd_fp4, quantize_fwd_op, quantize_fwd_op_group,
               quantize_fwd_sparse24, trust_bwd)

__all__ = ["QuestLinearFunction", "quest_linear", "quest_linear_operand", "QuestLinear", "default_trust",
           "ONE_BIT_OUTER_TRUST", "GRIDS"]


ONE_BIT_OUTER_TRUST = 1.30  # pith.science review of QuEST, "Assumptions & free parameters" (s*)
GRIDS = ("int", "fp4", "sparse24")


def _check_grid(grid: str) -> None:
    if grid not in GRIDS:
        raise ValueError(f"grid must be one of {GRIDS}, not {grid!r}")


def _quantise(t: torch.Tensor, block: int, bits: int, trust: float, grid: str, dtype):
    """(trust mask, dequantised Hadamard-domain values in dtype) of t on the chosen grid."""
    if grid == "int":
        _, _, mask, q = quantize_fwd_ex(t, block, bits, trust=trust, with_codes=False, dq_dtype=dtype)
    elif grid == "fp4":
        _, _, mask, q = quantize_fwd_fp4(t, block, trust, with_codes=False, dq_dtype=dtype)
    else:
        _, _, _, mask, q = quantize_fwd_sparse24(t, block, bits, trust, with_codes=False, dq_dtype=dtype)
    return mask, q


def default_trust(bits: int) -> float:
    """Outer trust factor used when none is given: 1.30 at 1 bit, 1 otherwise."""
    return ONE_BIT_OUTER_TRUST if bits == 1 else 1.0


class QuestLinearFunction(torch.autograd.Function):
    """y = Q(x) Q(w)^T for 2-D x (N x K) and w (M x K), K a multiple of `block`."""

    @staticmethod
    def forward(ctx, x, w, block, bits_x, bits_w, compute_dtype, trust_x=1.0, trust_w=1.0, grid="int"):
        ctx.block = block
        ctx.x_dtype, ctx.w_dtype = x.dtype, w.dtype
        # the FP6 product's domain: midrise levels of at most 4 bits, k a multiple of 128 up to 65536
        # (exact fp32 sums), at most 2^20 output features
        ctx.fp6 = (grid == "int" and max(bits_x, bits_w) <= 4 and x.shape[1] % 128 == 0 and x.shape[1] <= 65536
                   and 0 < w.shape[0] <= 2 ** 20 and 0 < x.shape[0] <= 2 ** 30)
        if ctx.fp6:
            n, k = x.shape
            m = w.shape[0]
            # With one bit width and n a multiple of 4 (every buffer 16-byte
            # aligned), the codes, scales and masks of x and w are the rows of
            # one (n + m)-row tensor each, so that the backward rebuilds both
            # operands in one quest_dequantize launch and masks both gradients
            # in one quest_trust_bwd launch.
            ctx.joint = bits_x == bits_w and n % 4 == 0
            if ctx.joint:
                dev = x.device
                codes = torch.empty((n + m, k * bits_x // 8), dtype=torch.uint8, device=dev)
                scale = torch.empty((n + m,), dtype=torch.float32, device=dev)
                mask = torch.empty((n + m, k // 8), dtype=torch.uint8, device=dev)
                outs = [dict(codes=codes[:n], scale=scale[:n], mask=mask[:n]),
                        dict(codes=codes[n:], scale=scale[n:], mask=mask[n:])]
                if trust_x == trust_w and x.dtype == w.dtype:
                    # one launch for both operands (quest_quantize_fwd_op_group)
                    (cx, sx, mask_x, ox), (cw, sw, mask_w, ow) = quantize_fwd_op_group([x, w], block, bits_x,
                                                                                      trust=trust_x, outs=outs)
                else:
                    cx, sx, mask_x, ox = quantize_fwd_op(x, block, bits_x, trust=trust_x, **outs[0])
                    cw, sw, mask_w, ow = quantize_fwd_op(w, block, bits_w, trust=trust_w, **outs[1])
            else:
                cx, sx, mask_x, ox = quantize_fwd_op(x, block, bits_x, trust=trust_x, with_codes=True,
                                                     with_mask=True)
                cw, sw, mask_w, ow = quantize_fwd_op(w, block, bits_w, trust=trust_w, with_codes=True,
                                                     with_mask=True)
            out_dtype = torch.float32 if compute_dtype == torch.float32 else torch.bfloat16
            y = gemm(ox, sx, n, bits_x, ow, sw, m, bits_w, k, out_dtype=out_dtype)
            y = y.to(compute_dtype)
            if ctx.joint:
                ctx.save_for_backward(codes, scale, mask)
            else:
                ctx.save_for_backward(cx, sx, cw, sw, mask_x, mask_w)
            ctx.dims = (n, m, k, bits_x, bits_w, compute_dtype)
            return y
        mask_x, qx = _quantise(x, block, bits_x, trust_x, grid, compute_dtype)
        mask_w, qw = _quantise(w, block, bits_w, trust_w, grid, compute_dtype)
        y = torch.nn.functional.linear(qx, qw)
        ctx.save_for_backward(qx, qw, mask_x, mask_w)
        return y

    @staticmethod
    def backward(ctx, dy):
        if ctx.fp6 and ctx.joint and ctx.needs_input_grad[0] and ctx.needs_input_grad[1]:
            return QuestLinearFunction._backward_joint(ctx, dy)
        if ctx.fp6:
            if ctx.joint:
                codes, scale, mask = ctx.saved_tensors
                n = ctx.dims[0]
                cx, sx, mask_x, cw, sw, mask_w = codes[:n], scale[:n], mask[:n], codes[n:], scale[n:], mask[n:]
            else:
                cx, sx, cw, sw, mask_x, mask_w = ctx.saved_tensors
            n, m, k, bits_x, bits_w, compute_dtype = ctx.dims
            # Q(x) for the weight gradient and Q(w) for the input gradient,
            # rebuilt from the codes (both first: the rebuilds keep the GPU
            # busy while the host sets up the products)
            qx = dequantize(cx, sx, n, k, bits_x, out_dtype=compute_dtype) if ctx.needs_input_grad[1] else None
            qw = dequantize(cw, sw, m, k, bits_w, out_dtype=compute_dtype) if ctx.needs_input_grad[0] else None
        else:
            qx, qw, mask_x, mask_w = ctx.saved_tensors
            compute_dtype = qx.dtype
        dy = dy.to(compute_dtype).contiguous()
        dx = dw = None
        # The weight gradient first: its product reads Q(x) just after the
        # rebuild wrote it, while it is still in the last-level cache.
        if ctx.needs_input_grad[1]:
            # gradient reaching Q(w), Hadamard domain (a 2-D product with a
            # transposed left operand, as torch's own linear backward computes it)
            g = torch.mm(dy.t(), qx)
            dw = trust_bwd(g, mask_w, ctx.block, out=g).to(ctx.w_dtype)
        if ctx.needs_input_grad[0]:
            g = torch.mm(dy, qw)  # gradient reaching Q(x), Hadamard domain
            dx = trust_bwd(g, mask_x, ctx.block, out=g).to(ctx.x_dtype)
        return dx, dw, None, None, None, None, None, None, None

    @staticmethod
    def _backward_joint(ctx, dy):
        """Both gradients of the FP6 path, x's and w's state held as the rows of one tensor each.

        One rebuild launch gives [Q(x); Q(w)], the two products write
        [dy Q(w); dy^T Q(x)] (the weight gradient first, while Q(x) is still in
        the last-level cache), and one trust backward masks and transforms
        both back in place.
        """
        codes, scale, mask = ctx.saved_tensors
        n, m, k, bits, _, compute_dtype = ctx.dims
        q = dequantize(codes, scale, n + m, k, bits, out_dtype=compute_dtype)
        qx, qw = q[:n], q[n:]
        dy = dy.to(compute_dtype).contiguous()
        g = torch.empty((n + m, k), dtype=compute_dtype, device=dy.device)
        # gradients reaching Q(w) and Q(x), Hadamard domain (the weight's as a
        # 2-D product with a transposed left operand, as torch's own linear
        # backward computes it)
        torch.mm(dy.t(), qx, out=g[n:])
        torch.mm(dy, qw, out=g[:n])
        trust_bwd(g, mask, ctx.block, out=g)
        return g[:n].to(ctx.x_dtype), g[n:].to(ctx.w_dtype), None, None, None, None, None, None, None


def quest_linear(x: torch.Tensor, w: torch.Tensor, bias: torch.Tensor | None = None, block: int = 128,
                 bits_x: int = 4, bits_w: int = 4, compute_dtype=torch.bfloat16, trust_x: float | None = None,
                 trust_w: float | None = None, grid: str = "int") -> torch.Tensor:
    """QuEST linear map of x (..., K) by w (M, K); leading axes of x are flattened.

    trust_x / trust_w: outer trust factors; by default 1.30 for 1-bit operands
    of the "int" grid (the factor the pages tune for their 1-bit runs) and 1
    otherwise.  grid: "int", "fp4" or "sparse24".
    """
    _check_grid(grid)
    trust_x = (default_trust(bits_x) if grid == "int" else 1.0) if trust_x is None else trust_x
    trust_w = (default_trust(bits_w) if grid == "int" else 1.0) if trust_w is None else trust_w
    lead = x.shape[:-1]
    x2 = x.reshape(-1, x.shape[-1]).contiguous()
    y = QuestLinearFunction.apply(x2, w.contiguous(), block, bits_x, bits_w, compute_dtype, trust_x, trust_w, grid)
    if bias is not None:
        y = y + bias.to(y.dtype)
    return y.reshape(*lead, w.shape[0])


def quest_linear_operand(x: torch.Tensor, w_operand: torch.Tensor, w_scale: torch.Tensor, out_features: int,
                         bits_w: int, bias: torch.Tensor | None = None, block: int = 128, bits_x: int = 4,
                         out_dtype=torch.bfloat16) -> torch.Tensor:
    """Inference product Q(x) Q(w)^T (+ bias) with w already in operand form.

    x (..., K) bf16 or fp32 with K a multiple of 128; w_operand / w_scale as
    returned by quantize_fwd_op for the (out_features x K) weight at bits_w.
    The activation is quantised (b = bits_x <= 4) straight into its operand
    and multiplied on the matrix cores; no gradient flows.
    """
    lead = x.shape[:-1]
    k = x.shape[-1]
    x2 = x.reshape(-1, k).contiguous()
    _, x_scale, _, x_op = quantize_fwd_op(x2, block, bits_x)
    y = gemm(x_op, x_scale, x2.shape[0], bits_x, w_operand, w_scale, out_features, bits_w, k, out_dtype=out_dtype)
    if bias is not None:
        y = y + bias.to(y.dtype)
    return y.reshape(*lead, out_features)


class QuestLinear(torch.nn.Module):
    """Drop-in linear layer trained with QuEST quantisation of weights and activations."""

    def __init__(self, in_features: int, out_features: int, bias: bool = True, block: int = 128, bits_x: int = 4,
                 bits_w: int = 4, compute_dtype=torch.bfloat16, trust_x: float | None = None,
                 trust_w: float | None = None, grid: str = "int", device=None, dtype=None):
        super().__init__()
        if in_features % block:
            raise ValueError(f"in_features ({in_features}) must be a multiple of the Hadamard block ({block})")
        _check_grid(grid)
        self.block, self.bits_x, self.bits_w, self.compute_dtype = block, bits_x, bits_w, compute_dtype
        self.grid = grid
        self.trust_x = (default_trust(bits_x) if grid == "int" else 1.0) if trust_x is None else trust_x
        self.trust_w = (default_trust(bits_w) if grid == "int" else 1.0) if trust_w is None else trust_w
        self.weight = torch.nn.Parameter(torch.empty(out_features, in_features, device=device, dtype=dtype))
        self.bias = torch.nn.Parameter(torch.zeros(out_features, device=device, dtype=dtype)) if bias else None
        torch.nn.init.kaiming_uniform_(self.weight, a=5 ** 0.5)
        self._w_operand = self._w_scale = None

    def freeze(self) -> "QuestLinear":
        """Quantise the weight once into the FP6 operand and switch to eval mode; eval-mode
        forwards then run the matrix-core product.  Needs bits_x, bits_w <= 4 and
        in_features a multiple of 128, on the "int" grid; training mode (``train()``) drops the operand."""
        if self.grid != "int" or max(self.bits_x, self.bits_w) > 4 or self.weight.shape[1] % 128:
            raise ValueError("the FP6 product needs the int grid, bits <= 4 and in_features a multiple of 128")
        with torch.no_grad():
            _, self._w_scale, _, self._w_operand = quantize_fwd_op(self.weight.detach().contiguous(), self.block,
                                                                   self.bits_w)
        return self.eval()

    def train(self, mode: bool = True) -> "QuestLinear":
        if mode:
            self._w_operand = self._w_scale = None
        return super().train(mode)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if not self.training and self._w_operand is not None:
            out_dtype = torch.float32 if self.compute_dtype == torch.float32 else torch.bfloat16
            return quest_linear_operand(x, self._w_operand, self._w_scale, self.weight.shape[0], self.bits_w,
                                        self.bias, self.block, self.bits_x, out_dtype)
        return quest_linear(x, self.weight, self.bias, self.block, self.bits_x, self.bits_w, self.compute_dtype,
                            self.trust_x, self.trust_w, self.grid)
