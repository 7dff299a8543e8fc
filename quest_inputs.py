"""Seeded synthetic inputs for the QuEST quantiser workloads.

This module only draws random tensors; it holds none of the method's
arithmetic (no Hadamard transform, no scale, no rounding, no masking).  Both
sides of a parity check take their inputs from here: the GPU path receives
the tensor as generated, the CPU oracle receives the same bits copied to the
host and widened exactly to float64.

Recipe (the pages train Llama-style models on C4, which is not available
here; these tensors stand in for those activations, weights and gradients
with the shapes the pages use: hidden size 2048, MLP width 5632 = 8/3 * 2048
rounded up to a multiple of 256, token counts in multiples of 512-token
sequences):

* entries are drawn in float32 with ``torch.randn`` from a
  ``torch.Generator`` seeded per 4096-row chunk (seed, chunk) on the target
  device, so a chunk can be regenerated alone;
* Student-t(nu) for integer nu is Z / sqrt(chi2_nu / nu) with
  chi2_nu = sum of nu squared standard normals (standard t, not rescaled);
* outlier channels: k columns drawn without replacement by a CPU generator
  seeded with the workload seed, the same for every row, multiplied by the
  outlier factor before the cast;
* bfloat16 tensors are the float32 draw rounded to nearest even
  (``Tensor.to(torch.bfloat16)``).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

CHUNK_ROWS = 4096


@dataclass(frozen=True)
class TensorSpec:
    """One synthetic tensor: shape, element distribution, outliers, dtype, seed."""

    name: str
    rows: int
    cols: int
    dtype: str  # "bf16" or "f32"
    dist: str  # "normal" or "student_t"
    param: float  # sigma for "normal", nu for "student_t"
    seed: int
    outlier_cols: int = 0
    outlier_scale: float = 1.0

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def elements(self) -> int:
        return self.rows * self.cols


def _chunk_generator(device: torch.device, seed: int, chunk: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + chunk * 7_919) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def _draw_chunk(spec: TensorSpec, rows: int, gen: torch.Generator, device) -> torch.Tensor:
    shape = (rows, spec.cols)
    if spec.dist == "normal":
        return torch.randn(shape, generator=gen, device=device) * float(spec.param)
    if spec.dist == "student_t":
        nu = int(spec.param)
        if nu != spec.param or nu < 1:
            raise ValueError("student_t needs an integer nu >= 1")
        z = torch.randn(shape, generator=gen, device=device)
        chi2 = torch.zeros(shape, device=device)
        for _ in range(nu):
            w = torch.randn(shape, generator=gen, device=device)
            chi2.addcmul_(w, w)
        return z / torch.sqrt(chi2 / nu)
    raise ValueError(f"unknown distribution {spec.dist!r}")


def outlier_columns(spec: TensorSpec) -> torch.Tensor:
    """Sorted indices of the outlier channels (CPU generator, workload seed)."""
    if spec.outlier_cols == 0:
        return torch.zeros(0, dtype=torch.long)
    g = torch.Generator().manual_seed(spec.seed)
    return torch.sort(torch.randperm(spec.cols, generator=g)[: spec.outlier_cols]).values


def make_tensor(spec: TensorSpec, device="cpu", row_start: int = 0, row_count: int | None = None) -> torch.Tensor:
    """Rows [row_start, row_start + row_count) of the tensor, contiguous, on `device`.

    Rows are generated a 4096-row chunk at a time, so any row range of a
    tensor comes out the same on a given device type whether or not the
    rest of the tensor is generated.
    """
    device = torch.device(device)
    if row_count is None:
        row_count = spec.rows - row_start
    if row_start < 0 or row_count < 0 or row_start + row_count > spec.rows:
        raise ValueError("row range outside the tensor")
    out = torch.empty((row_count, spec.cols), dtype=spec.torch_dtype, device=device)
    cols_out = outlier_columns(spec).to(device)
    first = row_start // CHUNK_ROWS
    last = (row_start + row_count - 1) // CHUNK_ROWS if row_count else first - 1
    for chunk in range(first, last + 1):
        c0 = chunk * CHUNK_ROWS
        c_rows = min(CHUNK_ROWS, spec.rows - c0)
        vals = _draw_chunk(spec, c_rows, _chunk_generator(device, spec.seed, chunk), device)
        if spec.outlier_cols:
            vals[:, cols_out] *= float(spec.outlier_scale)
        lo = max(row_start, c0)
        hi = min(row_start + row_count, c0 + c_rows)
        out[lo - row_start : hi - row_start] = vals[lo - c0 : hi - c0].to(spec.torch_dtype)
    return out


# ---------------------------------------------------------------------------
# The workloads: one small parity case, four full-size cases and the
# 16384 x 2048 headline tensor.
# ---------------------------------------------------------------------------

def _weights_c3() -> list[TensorSpec]:
    shapes = [
        ("q", 2048, 2048),
        ("k", 2048, 2048),
        ("v", 2048, 2048),
        ("o", 2048, 2048),
        ("gate", 5632, 2048),
        ("up", 5632, 2048),
        ("down", 2048, 5632),
    ]
    return [
        TensorSpec(f"C3.{nm}", r, c, "bf16", "normal", 0.02, 3000 + i)
        for i, (nm, r, c) in enumerate(shapes)
    ]


@dataclass(frozen=True)
class Workload:
    """A named workload: the tensors it quantises and how (block, bits, passes)."""

    name: str
    description: str
    fwd: tuple  # TensorSpecs quantised forward
    grad: tuple  # gradient TensorSpecs for the backward pass (same shapes), or ()
    block: int
    bits: tuple  # bit widths run
    passes: str  # "fwd", "bwd", "fwd+bwd"


WORKLOADS = {
    "C1": Workload(
        "C1",
        "256x512 fp32 N(0,1), 4 columns x10; block 128, b=4; fwd + dequantise",
        (TensorSpec("C1.x", 256, 512, "f32", "normal", 1.0, 1, outlier_cols=4, outlier_scale=10.0),),
        (),
        128,
        (4,),
        "fwd",
    ),
    "C2": Workload(
        "C2",
        "activations 16384x512 bf16 Student-t(4), 5 channels x20; block 128, b=1..4; fwd",
        (TensorSpec("C2.x", 16384, 512, "bf16", "student_t", 4, 2, outlier_cols=5, outlier_scale=20.0),),
        (),
        128,
        (1, 2, 3, 4),
        "fwd",
    ),
    "C3": Workload(
        "C3",
        "seven weight tensors of a 1.6B-scale Llama block, bf16 N(0,0.02^2); block 128, b=4; fwd",
        tuple(_weights_c3()),
        (),
        128,
        (4,),
        "fwd",
    ),
    "C4": Workload(
        "C4",
        "gradient 65536x2048 bf16 N(0,1e-3^2); mask from fwd(b=4) of a Student-t(4) activation; bwd",
        (TensorSpec("C4.act", 65536, 2048, "bf16", "student_t", 4, 4),),
        (TensorSpec("C4.grad", 65536, 2048, "bf16", "normal", 1e-3, 40),),
        128,
        (4,),
        "bwd",
    ),
    "C5": Workload(
        "C5",
        "MLP activation 131072x5632 bf16 Student-t(3), 28 channels x50; b=1; fwd then bwd",
        (TensorSpec("C5.act", 131072, 5632, "bf16", "student_t", 3, 5, outlier_cols=28, outlier_scale=50.0),),
        (TensorSpec("C5.grad", 131072, 5632, "bf16", "normal", 1e-3, 50),),
        128,
        (1,),
        "fwd+bwd",
    ),
    "T": Workload(
        "T",
        "activation 16384x2048 bf16 Student-t(4), 20 channels x20; block 128, b=4; fwd then bwd",
        (TensorSpec("T.act", 16384, 2048, "bf16", "student_t", 4, 6, outlier_cols=20, outlier_scale=20.0),),
        (TensorSpec("T.grad", 16384, 2048, "bf16", "normal", 1e-3, 60),),
        128,
        (4,),
        "fwd+bwd",
    ),
}


# The seven products of one 1.6B-scale Llama block at 16384 tokens: the
# activations (16384 x 2048 into q, k, v, o, gate and up; the 16384 x 5632
# MLP intermediate into down) times the C3 weights, both quantised to 4 bits
# along the contraction axis (block 128).
LAYER_TOKENS = 16384
LAYER_ACT_2048 = TensorSpec("L.x2048", LAYER_TOKENS, 2048, "bf16", "student_t", 4, 7, outlier_cols=20,
                            outlier_scale=20.0)
LAYER_ACT_5632 = TensorSpec("L.x5632", LAYER_TOKENS, 5632, "bf16", "student_t", 4, 8, outlier_cols=56,
                            outlier_scale=20.0)


def layer_products() -> list[tuple[str, TensorSpec, TensorSpec]]:
    """(name, activation spec, weight spec) of the block's seven matrix products."""
    out = []
    for w in WORKLOADS["C3"].fwd:
        act = LAYER_ACT_5632 if w.cols == 5632 else LAYER_ACT_2048
        out.append((w.name.split(".", 1)[1], act, w))
    return out


def to_float64(t: torch.Tensor):
    """Exact float64 NumPy copy of a float32 / bfloat16 tensor (for the oracle)."""
    return t.detach().to("cpu").to(torch.float64).numpy()
