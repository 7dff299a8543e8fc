"""Python binding of libquest (the QuEST quantiser hot path on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libquest.so, reached through its C ABI (include/quest.h).  torch
supplies device memory and the stream; the functions here check tensors,
allocate outputs when none are given and pass raw pointers.  If libquest.so
is missing the calls raise: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "QuestError",
    "LIB_PATH",
    "load_library",
    "fit_alpha",
    "codes_bytes",
    "mask_bytes",
    "quantize_fwd",
    "quantize_fwd_group",
    "quantize_fwd_dq",
    "quantize_fwd_ex",
    "quantize_fwd_op",
    "operand_bytes",
    "codes_to_operand",
    "gemm",
    "quantize_fwd_op_group",
    "quantize_fwd_fp4",
    "quantize_fwd_sparse24",
    "dequantize_fp4",
    "dequantize_sparse24",
    "dequantize",
    "trust_bwd",
    "EXPORTED_SYMBOLS",
]

# The library next to this file; QUEST_LIBRARY names another build of it (the
# sanitizer build the CPU tests make, for instance).
LIB_PATH = os.environ.get("QUEST_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libquest.so")

QUEST_OK, QUEST_EINVAL, QUEST_EUNSUPPORTED, QUEST_EALIGN, QUEST_EHIP = range(5)
QUEST_F32, QUEST_BF16 = 0, 1

EXPORTED_SYMBOLS = (
    "quest_fit_alpha",
    "quest_quantize_fwd",
    "quest_quantize_fwd_group",
    "quest_quantize_fwd_dq",
    "quest_quantize_fwd_ex",
    "quest_quantize_fwd_op",
    "quest_quantize_fwd_op_group",
    "quest_gemm",
    "quest_operand_bytes",
    "quest_codes_to_operand",
    "quest_fit_alpha_fp4",
    "quest_quantize_fwd_fp4",
    "quest_quantize_fwd_sparse24",
    "quest_dequantize_fp4",
    "quest_dequantize_sparse24",
    "quest_sparse24_codes_bytes",
    "quest_sparse24_index_bytes",
    "quest_dequantize",
    "quest_trust_bwd",
    "quest_codes_bytes",
    "quest_mask_bytes",
    "quest_status_string",
)


class QuestError(RuntimeError):
    """A libquest call returned a status other than QUEST_OK."""

    def __init__(self, call: str, status: int, message: str):
        super().__init__(f"{call}: {message} (status {status})")
        self.status = status


_lib = None


class _FwdTensor(ctypes.Structure):
    """quest_fwd_tensor of include/quest.h."""

    _fields_ = [("x", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("mask", ctypes.c_void_p)]


class _FwdOpTensor(ctypes.Structure):
    """quest_fwd_op_tensor of include/quest.h."""

    _fields_ = [("x", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("mask", ctypes.c_void_p),
                ("operand", ctypes.c_void_p)]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libquest.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"libquest.so not found at {path}; build it with `python -m quantization_aware_amd.build` "
            "(there is no CPU fallback)"
        )
    lib = ctypes.CDLL(path)
    i64, vp, c_int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.quest_fit_alpha.argtypes = [c_int]
    lib.quest_fit_alpha.restype = ctypes.c_double
    lib.quest_quantize_fwd.argtypes = [vp, c_int, i64, i64, c_int, c_int, vp, vp, vp, vp]
    lib.quest_quantize_fwd.restype = c_int
    lib.quest_quantize_fwd_group.argtypes = [ctypes.POINTER(_FwdTensor), c_int, c_int, c_int, c_int, vp]
    lib.quest_quantize_fwd_group.restype = c_int
    lib.quest_quantize_fwd_dq.argtypes = [vp, c_int, i64, i64, c_int, c_int, vp, vp, vp, vp, c_int, vp]
    lib.quest_quantize_fwd_dq.restype = c_int
    lib.quest_quantize_fwd_ex.argtypes = [vp, c_int, i64, i64, c_int, c_int, ctypes.c_double, vp, vp, vp, vp, c_int, vp]
    lib.quest_quantize_fwd_ex.restype = c_int
    lib.quest_quantize_fwd_op.argtypes = [vp, c_int, i64, i64, c_int, c_int, ctypes.c_double, vp, vp, vp, vp, vp]
    lib.quest_quantize_fwd_op.restype = c_int
    lib.quest_quantize_fwd_op_group.argtypes = [ctypes.POINTER(_FwdOpTensor), c_int, c_int, c_int, c_int,
                                                ctypes.c_double, vp]
    lib.quest_quantize_fwd_op_group.restype = c_int
    lib.quest_gemm.argtypes = [vp, vp, i64, c_int, vp, vp, i64, c_int, i64, vp, c_int, vp]
    lib.quest_gemm.restype = c_int
    lib.quest_codes_to_operand.argtypes = [vp, i64, i64, c_int, vp, vp]
    lib.quest_codes_to_operand.restype = c_int
    lib.quest_operand_bytes.argtypes = [i64, i64]
    lib.quest_operand_bytes.restype = ctypes.c_size_t
    lib.quest_fit_alpha_fp4.argtypes = []
    lib.quest_fit_alpha_fp4.restype = ctypes.c_double
    lib.quest_quantize_fwd_fp4.argtypes = [vp, c_int, i64, i64, c_int, ctypes.c_double, vp, vp, vp, vp, c_int, vp]
    lib.quest_quantize_fwd_fp4.restype = c_int
    lib.quest_quantize_fwd_sparse24.argtypes = [vp, c_int, i64, i64, c_int, c_int, ctypes.c_double, vp, vp, vp, vp,
                                                vp, c_int, vp]
    lib.quest_quantize_fwd_sparse24.restype = c_int
    lib.quest_dequantize_fp4.argtypes = [vp, vp, i64, i64, vp, c_int, vp]
    lib.quest_dequantize_fp4.restype = c_int
    lib.quest_dequantize_sparse24.argtypes = [vp, vp, vp, i64, i64, c_int, vp, c_int, vp]
    lib.quest_dequantize_sparse24.restype = c_int
    lib.quest_sparse24_codes_bytes.argtypes = [i64, i64, c_int]
    lib.quest_sparse24_codes_bytes.restype = ctypes.c_size_t
    lib.quest_sparse24_index_bytes.argtypes = [i64, i64]
    lib.quest_sparse24_index_bytes.restype = ctypes.c_size_t
    lib.quest_dequantize.argtypes = [vp, vp, i64, i64, c_int, vp, c_int, vp]
    lib.quest_dequantize.restype = c_int
    lib.quest_trust_bwd.argtypes = [vp, c_int, vp, i64, i64, c_int, vp, vp]
    lib.quest_trust_bwd.restype = c_int
    lib.quest_codes_bytes.argtypes = [i64, i64, c_int]
    lib.quest_codes_bytes.restype = ctypes.c_size_t
    lib.quest_mask_bytes.argtypes = [i64, i64]
    lib.quest_mask_bytes.restype = ctypes.c_size_t
    lib.quest_status_string.argtypes = [c_int]
    lib.quest_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(call: str, status: int) -> None:
    if status != QUEST_OK:
        msg = load_library().quest_status_string(status).decode()
        raise QuestError(call, status, msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return QUEST_BF16
    if t.dtype == torch.float32:
        return QUEST_F32
    raise TypeError(f"libquest takes float32 or bfloat16 tensors, got {t.dtype}")


def _device_tensor(name: str, t: torch.Tensor) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got device {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _buffer(name: str, t, dtype, need: int) -> None:
    """A caller-supplied buffer: a tensor of `dtype` holding at least `need` elements.  The C ABI takes raw
    pointers and cannot see sizes, so a short buffer would be read or written past its end; it is rejected
    here instead.  (Device and contiguity are checked by _on_device once every size has been.)"""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() < need:
        raise ValueError(f"{name} too small: {t.numel()} elements, the call needs {need}")


def _on_device(device, **tensors) -> None:
    """Every tensor contiguous on the GPU, on `device`."""
    for name, t in tensors.items():
        _device_tensor(name, t)
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, the call runs on {device}")


def _stream_handle(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


def fit_alpha(b: int) -> float:
    """Clip scale alpha_b of the b-bit Gaussian-MSE-optimal grid (host, float64)."""
    return float(load_library().quest_fit_alpha(int(b)))


def codes_bytes(rows: int, cols: int, b: int) -> int:
    return int(load_library().quest_codes_bytes(int(rows), int(cols), int(b)))


def mask_bytes(rows: int, cols: int) -> int:
    return int(load_library().quest_mask_bytes(int(rows), int(cols)))


def quantize_fwd(x: torch.Tensor, block: int, b: int, codes=None, scale=None, mask=None, stream=None):
    """Forward QuEST quantisation of a 2-D tensor; returns (codes, scale, mask).

    codes: uint8 (rows, cols*b/8); scale: float32 (rows,); mask: uint8 (rows, cols/8).
    Outputs are allocated on x's device unless given.
    """
    lib = load_library()
    _device_tensor("x", x)
    if x.dim() != 2:
        raise ValueError("x must be 2-D (rows x cols)")
    rows, cols = x.shape
    dev = x.device
    if codes is None:
        codes = torch.empty((rows, cols * b // 8), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty((rows,), dtype=torch.float32, device=dev)
    if mask is None:
        mask = torch.empty((rows, cols // 8), dtype=torch.uint8, device=dev)
    for name, t, dt in (("codes", codes, torch.uint8), ("scale", scale, torch.float32), ("mask", mask, torch.uint8)):
        _device_tensor(name, t)
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}")
    if codes.numel() < codes_bytes(rows, cols, b) or scale.numel() < rows or mask.numel() < mask_bytes(rows, cols):
        raise ValueError("output buffer too small")
    st = lib.quest_quantize_fwd(
        x.data_ptr(), _dtype_code(x), rows, cols, int(block), int(b),
        codes.data_ptr(), scale.data_ptr(), mask.data_ptr(), _stream_handle(dev, stream),
    )
    _check("quest_quantize_fwd", st)
    return codes, scale, mask


def quantize_fwd_group(xs, block: int, b: int, stream=None):
    """quantize_fwd of several 2-D tensors of one dtype and device in one call (quest_quantize_fwd_group).

    Returns a list of (codes, scale, mask), one per tensor, equal to what
    quantize_fwd returns for each.  bf16 tensors (b <= 4) of 512, 1024 or 2048
    columns, and of 2560 to 8192 columns (a multiple of 512), share launches.
    """
    lib = load_library()
    xs = list(xs)
    if not xs:
        return []
    outs, descs = [], (_FwdTensor * len(xs))()
    for i, x in enumerate(xs):
        _device_tensor(f"xs[{i}]", x)
        if x.dim() != 2:
            raise ValueError(f"xs[{i}] must be 2-D (rows x cols)")
        if x.dtype != xs[0].dtype or x.device != xs[0].device:
            raise ValueError("every tensor of a group must share the first one's dtype and device")
        rows, cols = x.shape
        codes = torch.empty((rows, cols * b // 8), dtype=torch.uint8, device=x.device)
        scale = torch.empty((rows,), dtype=torch.float32, device=x.device)
        mask = torch.empty((rows, cols // 8), dtype=torch.uint8, device=x.device)
        outs.append((codes, scale, mask))
        descs[i] = _FwdTensor(x.data_ptr(), rows, cols, codes.data_ptr(), scale.data_ptr(), mask.data_ptr())
    st = lib.quest_quantize_fwd_group(descs, len(xs), _dtype_code(xs[0]), int(block), int(b),
                                      _stream_handle(xs[0].device, stream))
    _check("quest_quantize_fwd_group", st)
    return outs


def quantize_fwd_dq(x: torch.Tensor, block: int, b: int, dq_dtype=torch.bfloat16, with_codes: bool = True,
                    codes=None, scale=None, mask=None, dq=None, stream=None):
    """Forward quantisation that also returns the dequantised tensor, in one pass.

    Returns (codes, scale, mask, dq); codes is None when with_codes is False
    (they are then not written).  dq holds the grid value of every entry's
    code in the Hadamard domain, rows x cols of dq_dtype (bfloat16 or float32).
    """
    lib = load_library()
    _device_tensor("x", x)
    if x.dim() != 2:
        raise ValueError("x must be 2-D (rows x cols)")
    rows, cols = x.shape
    dev = x.device
    if with_codes and codes is None:
        codes = torch.empty((rows, cols * b // 8), dtype=torch.uint8, device=dev)
    if not with_codes:
        codes = None
    if scale is None:
        scale = torch.empty((rows,), dtype=torch.float32, device=dev)
    if mask is None:
        mask = torch.empty((rows, cols // 8), dtype=torch.uint8, device=dev)
    if dq is None:
        dq = torch.empty((rows, cols), dtype=dq_dtype, device=dev)
    checks = [("scale", scale, torch.float32), ("mask", mask, torch.uint8)]
    if codes is not None:
        checks.append(("codes", codes, torch.uint8))
    for name, t, dt in checks:
        _device_tensor(name, t)
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}")
    _device_tensor("dq", dq)
    if (codes is not None and codes.numel() < codes_bytes(rows, cols, b)) or scale.numel() < rows \
            or mask.numel() < mask_bytes(rows, cols) or dq.numel() < rows * cols:
        raise ValueError("output buffer too small")
    st = lib.quest_quantize_fwd_dq(
        x.data_ptr(), _dtype_code(x), rows, cols, int(block), int(b),
        codes.data_ptr() if codes is not None else None, scale.data_ptr(), mask.data_ptr(),
        dq.data_ptr(), _dtype_code(dq), _stream_handle(dev, stream),
    )
    _check("quest_quantize_fwd_dq", st)
    return codes, scale, mask, dq


def quantize_fwd_ex(x: torch.Tensor, block: int, b: int, trust: float = 1.0, with_codes: bool = True,
                    dq_dtype=None, stream=None):
    """The general forward (quest_quantize_fwd_ex): outer trust factor, optional codes and dq.

    Returns (codes or None, scale, mask, dq or None); dq_dtype None means no
    dequantised output.
    """
    lib = load_library()
    _device_tensor("x", x)
    if x.dim() != 2:
        raise ValueError("x must be 2-D (rows x cols)")
    rows, cols = x.shape
    dev = x.device
    codes = torch.empty((rows, cols * b // 8), dtype=torch.uint8, device=dev) if with_codes else None
    scale = torch.empty((rows,), dtype=torch.float32, device=dev)
    mask = torch.empty((rows, cols // 8), dtype=torch.uint8, device=dev)
    dq = torch.empty((rows, cols), dtype=dq_dtype, device=dev) if dq_dtype is not None else None
    st = lib.quest_quantize_fwd_ex(
        x.data_ptr(), _dtype_code(x), rows, cols, int(block), int(b), float(trust),
        codes.data_ptr() if codes is not None else None, scale.data_ptr(), mask.data_ptr(),
        dq.data_ptr() if dq is not None else None, _dtype_code(dq) if dq is not None else QUEST_BF16,
        _stream_handle(dev, stream),
    )
    _check("quest_quantize_fwd_ex", st)
    return codes, scale, mask, dq


def operand_bytes(rows: int, cols: int) -> int:
    """Bytes of the tiled FP6 operand of a rows x cols tensor (quest_operand_bytes)."""
    return int(load_library().quest_operand_bytes(rows, cols))


def quantize_fwd_op(x: torch.Tensor, block: int, b: int, trust: float = 1.0, with_codes: bool = False,
                    with_mask: bool = False, operand=None, scale=None, stream=None, codes=None, mask=None):
    """Forward writing the matrix-core operand (quest_quantize_fwd_op).

    Returns (codes or None, scale, mask or None, operand); the operand is a
    flat uint8 tensor of operand_bytes(rows, cols) bytes.  codes / mask, when
    given, are caller buffers for those outputs (uint8, contiguous, at least
    codes_bytes / mask_bytes long) and imply with_codes / with_mask.
    """
    lib = load_library()
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor (rows x cols)")
    rows, cols = x.shape
    dev = x.device
    if codes is None and with_codes:
        codes = torch.empty((rows, cols * b // 8), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty((rows,), dtype=torch.float32, device=dev)
    if mask is None and with_mask:
        mask = torch.empty((rows, cols // 8), dtype=torch.uint8, device=dev)
    if operand is None:
        operand = torch.empty((max(operand_bytes(rows, cols), 1),), dtype=torch.uint8, device=dev)
    _buffer("scale", scale, torch.float32, rows)
    _buffer("operand", operand, torch.uint8, operand_bytes(rows, cols))
    outs = {}
    if codes is not None:
        _buffer("codes", codes, torch.uint8, codes_bytes(rows, cols, b))
        outs["codes"] = codes
    if mask is not None:
        _buffer("mask", mask, torch.uint8, mask_bytes(rows, cols))
        outs["mask"] = mask
    _on_device(dev, x=x, scale=scale, operand=operand, **outs)
    st = lib.quest_quantize_fwd_op(
        x.data_ptr(), _dtype_code(x), rows, cols, int(block), int(b), float(trust),
        codes.data_ptr() if codes is not None else None, scale.data_ptr(),
        mask.data_ptr() if mask is not None else None, operand.data_ptr(), _stream_handle(dev, stream),
    )
    _check("quest_quantize_fwd_op", st)
    return codes, scale, mask, operand


def quantize_fwd_op_group(xs, block: int, b: int, trust: float = 1.0, outs=None, stream=None):
    """quantize_fwd_op of several 2-D tensors of one dtype and device in one call (quest_quantize_fwd_op_group).

    outs: None, or one dict per tensor of caller buffers with the keyword
    names of quantize_fwd_op (operand, scale, and optionally codes and mask;
    operand and scale are allocated when missing).  Returns a list of
    (codes or None, scale, mask or None, operand), equal to what
    quantize_fwd_op returns for each tensor.  bf16 tensors of 512, 1024 or
    2048 columns share launches.
    """
    lib = load_library()
    xs = list(xs)
    if not xs:
        return []
    if outs is None:
        outs = [{} for _ in xs]
    if len(outs) != len(xs):
        raise ValueError(f"{len(xs)} tensors but {len(outs)} output sets")
    dev = xs[0].device
    res, checked, descs = [], [], (_FwdOpTensor * len(xs))()
    for i, (x, o) in enumerate(zip(xs, outs)):
        if not isinstance(x, torch.Tensor) or x.dim() != 2:
            raise ValueError(f"xs[{i}] must be a 2-D tensor (rows x cols)")
        if x.dtype != xs[0].dtype or x.device != dev:
            raise ValueError("every tensor of a group must share the first one's dtype and device")
        unknown = set(o) - {"codes", "scale", "mask", "operand"}
        if unknown:
            raise ValueError(f"outs[{i}] has unknown keys {sorted(unknown)}")
        rows, cols = x.shape
        scale = o.get("scale")
        if scale is None:
            scale = torch.empty((rows,), dtype=torch.float32, device=dev)
        operand = o.get("operand")
        if operand is None:
            operand = torch.empty((max(operand_bytes(rows, cols), 1),), dtype=torch.uint8, device=dev)
        codes, mask = o.get("codes"), o.get("mask")
        _buffer(f"outs[{i}].scale", scale, torch.float32, rows)
        _buffer(f"outs[{i}].operand", operand, torch.uint8, operand_bytes(rows, cols))
        bufs = {}
        if codes is not None:
            _buffer(f"outs[{i}].codes", codes, torch.uint8, codes_bytes(rows, cols, b))
            bufs[f"outs[{i}].codes"] = codes
        if mask is not None:
            _buffer(f"outs[{i}].mask", mask, torch.uint8, mask_bytes(rows, cols))
            bufs[f"outs[{i}].mask"] = mask
        bufs.update({f"xs[{i}]": x, f"outs[{i}].scale": scale, f"outs[{i}].operand": operand})
        checked.append(bufs)
        res.append((codes, scale, mask, operand))
        descs[i] = _FwdOpTensor(x.data_ptr(), rows, cols, codes.data_ptr() if codes is not None else None,
                                scale.data_ptr(), mask.data_ptr() if mask is not None else None, operand.data_ptr())
    for bufs in checked:  # every size first, then the devices
        _on_device(dev, **bufs)
    st = lib.quest_quantize_fwd_op_group(descs, len(xs), _dtype_code(xs[0]), int(block), int(b), float(trust),
                                         _stream_handle(dev, stream))
    _check("quest_quantize_fwd_op_group", st)
    return res


def codes_to_operand(codes: torch.Tensor, rows: int, cols: int, b: int, operand=None, stream=None) -> torch.Tensor:
    """The matrix-core operand of packed b-bit codes (quest_codes_to_operand), b <= 4."""
    lib = load_library()
    rows, cols, b = int(rows), int(cols), int(b)
    _buffer("codes", codes, torch.uint8, codes_bytes(rows, cols, b))
    if operand is None:
        operand = torch.empty((max(operand_bytes(rows, cols), 1),), dtype=torch.uint8, device=codes.device)
    _buffer("operand", operand, torch.uint8, operand_bytes(rows, cols))
    _on_device(codes.device, codes=codes, operand=operand)
    st = lib.quest_codes_to_operand(codes.data_ptr(), rows, cols, b, operand.data_ptr(),
                                    _stream_handle(codes.device, stream))
    _check("quest_codes_to_operand", st)
    return operand


def gemm(a: torch.Tensor, a_scale: torch.Tensor, m: int, a_bits: int, b: torch.Tensor, b_scale: torch.Tensor,
         n: int, b_bits: int, k: int, out_dtype=torch.bfloat16, out=None, stream=None) -> torch.Tensor:
    """Product of two matrix-core operands (quest_gemm): an m x n tensor of out_dtype."""
    lib = load_library()
    m, n, k = int(m), int(n), int(k)
    _buffer("a", a, torch.uint8, operand_bytes(m, k))
    _buffer("a_scale", a_scale, torch.float32, m)
    _buffer("b", b, torch.uint8, operand_bytes(n, k))
    _buffer("b_scale", b_scale, torch.float32, n)
    dev = a.device
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=dev)
    if not isinstance(out, torch.Tensor) or out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"out must be a float32 or bfloat16 tensor, got {getattr(out, 'dtype', type(out))}")
    _buffer("out", out, out.dtype, m * n)
    _on_device(dev, a=a, a_scale=a_scale, b=b, b_scale=b_scale, out=out)
    st = lib.quest_gemm(a.data_ptr(), a_scale.data_ptr(), m, int(a_bits), b.data_ptr(), b_scale.data_ptr(), n,
                        int(b_bits), k, out.data_ptr(), _dtype_code(out), _stream_handle(dev, stream))
    _check("quest_gemm", st)
    return out


def quantize_fwd_fp4(x: torch.Tensor, block: int, trust: float = 1.0, with_codes: bool = True, dq_dtype=None,
                     stream=None):
    """Forward onto the FP4 grid (quest_quantize_fwd_fp4): (codes or None, scale, mask, dq or None)."""
    lib = load_library()
    _device_tensor("x", x)
    if x.dim() != 2:
        raise ValueError("x must be 2-D (rows x cols)")
    rows, cols = x.shape
    dev = x.device
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev) if with_codes else None
    scale = torch.empty((rows,), dtype=torch.float32, device=dev)
    mask = torch.empty((rows, cols // 8), dtype=torch.uint8, device=dev)
    dq = torch.empty((rows, cols), dtype=dq_dtype, device=dev) if dq_dtype is not None else None
    st = lib.quest_quantize_fwd_fp4(
        x.data_ptr(), _dtype_code(x), rows, cols, int(block), float(trust),
        codes.data_ptr() if codes is not None else None, scale.data_ptr(), mask.data_ptr(),
        dq.data_ptr() if dq is not None else None, _dtype_code(dq) if dq is not None else QUEST_BF16,
        _stream_handle(dev, stream),
    )
    _check("quest_quantize_fwd_fp4", st)
    return codes, scale, mask, dq


def quantize_fwd_sparse24(x: torch.Tensor, block: int, b: int, trust: float = 1.0, with_codes: bool = True,
                          dq_dtype=None, stream=None):
    """Forward onto the 2:4-sparse b-bit grid (quest_quantize_fwd_sparse24).

    Returns (codes or None, index or None, scale, mask, dq or None).
    """
    lib = load_library()
    _device_tensor("x", x)
    if x.dim() != 2:
        raise ValueError("x must be 2-D (rows x cols)")
    rows, cols = x.shape
    dev = x.device
    codes = torch.empty((rows, cols // 2 * b // 8), dtype=torch.uint8, device=dev) if with_codes else None
    index = torch.empty((rows, cols // 8), dtype=torch.uint8, device=dev) if with_codes else None
    scale = torch.empty((rows,), dtype=torch.float32, device=dev)
    mask = torch.empty((rows, cols // 8), dtype=torch.uint8, device=dev)
    dq = torch.empty((rows, cols), dtype=dq_dtype, device=dev) if dq_dtype is not None else None
    st = lib.quest_quantize_fwd_sparse24(
        x.data_ptr(), _dtype_code(x), rows, cols, int(block), int(b), float(trust),
        codes.data_ptr() if codes is not None else None, index.data_ptr() if index is not None else None,
        scale.data_ptr(), mask.data_ptr(), dq.data_ptr() if dq is not None else None,
        _dtype_code(dq) if dq is not None else QUEST_BF16, _stream_handle(dev, stream),
    )
    _check("quest_quantize_fwd_sparse24", st)
    return codes, index, scale, mask, dq


def dequantize_fp4(codes: torch.Tensor, scale: torch.Tensor, rows: int, cols: int, out_dtype=torch.float32,
                   stream=None) -> torch.Tensor:
    """FP4 codes back to their levels (quest_dequantize_fp4)."""
    lib = load_library()
    rows, cols = int(rows), int(cols)
    _buffer("codes", codes, torch.uint8, max(rows, 0) * max(cols, 0) // 2)
    _buffer("scale", scale, torch.float32, rows)
    _on_device(codes.device, codes=codes, scale=scale)
    out = torch.empty((rows, cols), dtype=out_dtype, device=codes.device)
    st = lib.quest_dequantize_fp4(codes.data_ptr(), scale.data_ptr(), rows, cols, out.data_ptr(), _dtype_code(out),
                                  _stream_handle(codes.device, stream))
    _check("quest_dequantize_fp4", st)
    return out


def dequantize_sparse24(codes: torch.Tensor, index: torch.Tensor, scale: torch.Tensor, rows: int, cols: int, b: int,
                        out_dtype=torch.float32, stream=None) -> torch.Tensor:
    """2:4-sparse codes back to the dense reconstruction (quest_dequantize_sparse24)."""
    lib = load_library()
    rows, cols, b = int(rows), int(cols), int(b)
    _buffer("codes", codes, torch.uint8, int(lib.quest_sparse24_codes_bytes(rows, cols, b)))
    _buffer("index", index, torch.uint8, int(lib.quest_sparse24_index_bytes(rows, cols)))
    _buffer("scale", scale, torch.float32, rows)
    _on_device(codes.device, codes=codes, index=index, scale=scale)
    out = torch.empty((rows, cols), dtype=out_dtype, device=codes.device)
    st = lib.quest_dequantize_sparse24(codes.data_ptr(), index.data_ptr(), scale.data_ptr(), rows, cols, int(b),
                                       out.data_ptr(), _dtype_code(out), _stream_handle(codes.device, stream))
    _check("quest_dequantize_sparse24", st)
    return out


def dequantize(codes: torch.Tensor, scale: torch.Tensor, rows: int, cols: int, b: int,
               out_dtype=torch.bfloat16, out=None, stream=None) -> torch.Tensor:
    """Grid values (2u - L + 1) s / (L - 1) of packed codes, in the Hadamard domain."""
    lib = load_library()
    _device_tensor("codes", codes)
    _device_tensor("scale", scale)
    if codes.dtype != torch.uint8 or scale.dtype != torch.float32:
        raise TypeError("codes must be uint8 and scale float32")
    if codes.numel() < codes_bytes(rows, cols, b) or scale.numel() < rows:
        raise ValueError("codes or scale smaller than rows x cols needs")
    if out is None:
        out = torch.empty((rows, cols), dtype=out_dtype, device=codes.device)
    _device_tensor("out", out)
    if out.numel() < rows * cols:
        raise ValueError("out smaller than rows x cols")
    st = lib.quest_dequantize(
        codes.data_ptr(), scale.data_ptr(), int(rows), int(cols), int(b),
        out.data_ptr(), _dtype_code(out), _stream_handle(codes.device, stream),
    )
    _check("quest_dequantize", st)
    return out


def trust_bwd(grad: torch.Tensor, mask: torch.Tensor, block: int, out=None, stream=None) -> torch.Tensor:
    """Trust-gradient backward H (M * G) per block; out may be grad itself (in place)."""
    lib = load_library()
    _device_tensor("grad", grad)
    _device_tensor("mask", mask)
    if grad.dim() != 2:
        raise ValueError("grad must be 2-D (rows x cols)")
    if mask.dtype != torch.uint8:
        raise TypeError("mask must be uint8")
    rows, cols = grad.shape
    if mask.numel() < mask_bytes(rows, cols):
        raise ValueError("mask smaller than rows x cols / 8 bytes")
    if out is None:
        out = torch.empty_like(grad)
    _device_tensor("out", out)
    if out.dtype != grad.dtype or out.shape != grad.shape:
        raise ValueError("out must match grad in dtype and shape")
    st = lib.quest_trust_bwd(
        grad.data_ptr(), _dtype_code(grad), mask.data_ptr(), rows, cols, int(block),
        out.data_ptr(), _stream_handle(grad.device, stream),
    )
    _check("quest_trust_bwd", st)
    return out
