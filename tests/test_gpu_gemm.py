"""The matrix-core operand forward and the product of two operands, vs the oracle.

* quest_quantize_fwd_op: codes, mask and scale must pass the same checks as
  the plain forward, and the operand must hold, bit for bit, the E2M3 fields
  of the call's own codes (h = u - (L - 1)/2) in the tiled layout.  Since the
  codes match the oracle's outside the threshold band, so do the fields.
* quest_gemm on operands built by the oracle (no GPU output is an oracle
  input): the sum of half-integer products is exact in fp32, so each output
  is the oracle's float64 product up to the roundings of Delta_a Delta_b, the
  product and the output type -- relative 1e-6 in fp32, 4e-3 in bf16 (one
  bf16 rounding, 2^-9, on top), elementwise, including outputs that cancel
  to small values.
* The layer end to end (forward on both operands, then the product) against
  the oracle's Q(x) Q(w)^T, outside the reach of band entries.
* The seven products of a 1.6B-scale block at 16384 tokens, in the launch
  configuration the benchmark times, on a seeded sample of output rows and
  columns recomputed by the oracle (every row is quantised independently).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import quantization_aware_amd as qa
from oracle import quest_oracle as qo
from operand_layout import tile_operand, untile_operand
from parity import check_fwd, exempt_entries
from quest_inputs import TensorSpec, layer_products, make_tensor, to_float64

pytestmark = pytest.mark.gpu


def log(msg: str) -> None:
    print(f"[gpu-gemm] {msg}", flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qa.load_library()
    return torch.device("cuda", 0)


def halves_e2m3(u: np.ndarray, b: int) -> np.ndarray:
    """E2M3 fields of the half-integers u - (L - 1)/2 (oracle encoder)."""
    return qo.e2m3_encode(u - ((1 << b) - 1) / 2.0)


def gpu_fields(op: torch.Tensor, rows: int, cols: int) -> np.ndarray:
    """6-bit fields of a GPU operand, rows x cols, read back through the layout's definition."""
    flat = op.cpu().numpy()[: qa.operand_bytes(rows, cols)]
    return qo.unpack_lsb_first(untile_operand(flat, rows, cols), 6, cols)


# ---------------------------------------------------------------------------
# The operand forward, every kernel family: matrix-core tiles (16, 32, 64
# runs per row), matrix-core wide rows (one row per wave up to 8192 columns,
# the row kernel beyond), run-per-lane tiles and rows (fp32, and run counts
# that are not powers of two); ragged row counts.
# ---------------------------------------------------------------------------
FWD_OP_CASES = [
    # rows, cols, dtype, block, b, trust
    (77, 2048, "bf16", 128, 4, 1.0),
    (45, 512, "bf16", 128, 2, 1.0),
    (33, 1024, "bf16", 64, 3, 1.0),
    (21, 5632, "bf16", 128, 4, 1.0),
    (19, 2560, "bf16", 256, 1, 1.3),
    (50, 2048, "f32", 128, 4, 1.0),
    (37, 384, "bf16", 128, 4, 1.0),
    (29, 640, "f32", 128, 3, 1.0),
    (64, 128, "bf16", 128, 4, 1.0),
    (1, 256, "f32", 256, 1, 1.3),
    (7, 10752, "bf16", 128, 4, 1.0),  # rows wider than 8192 columns: the row kernel, 3 rows per workgroup
    (130, 4096, "bf16", 128, 2, 1.0),  # one row per wave, 2 chunks of 64 runs
    (9, 8192, "bf16", 128, 3, 1.0),  # one row per wave, 4 full chunks
    (33, 7168, "bf16", 64, 4, 1.3),  # one row per wave, 4 chunks, the last one half empty
]


@pytest.mark.parametrize("rows,cols,dt,block,b,trust", FWD_OP_CASES)
def test_fwd_op_matches_oracle(dev, rows, cols, dt, block, b, trust):
    log(f"fwd_op {rows}x{cols} {dt} block {block} b={b} trust {trust}")
    spec = TensorSpec("op.x", rows, cols, dt, "student_t", 4, 7000 + rows + cols, outlier_cols=max(1, cols // 100),
                      outlier_scale=20.0)
    x = make_tensor(spec, dev)
    codes, scale, mask, op = qa.quantize_fwd_op(x, block, b, trust=trust, with_codes=True, with_mask=True)
    torch.cuda.synchronize()
    st = check_fwd(to_float64(x), block, b, codes.cpu().numpy(), scale.cpu().numpy(), mask.cpu().numpy(),
                   trust=trust)
    u = qo.unpack_lsb_first(codes.cpu().numpy(), b, cols)
    fields = gpu_fields(op, rows, cols)
    want = halves_e2m3(u, b)
    bad = fields != want
    assert not bad.any(), f"{int(bad.sum())} operand fields differ from the call's own codes, first at {np.argwhere(bad)[0]}"
    # The same call without codes or mask writes the same operand and scale.
    _, scale2, _, op2 = qa.quantize_fwd_op(x, block, b, trust=trust)
    torch.cuda.synchronize()
    n = qa.operand_bytes(rows, cols)
    assert torch.equal(scale2, scale)
    assert np.array_equal(gpu_fields(op2, rows, cols), fields)
    assert op2.numel() == n
    log(f"fwd_op ok {st}")


def test_fwd_op_matches_plain_forward_bitwise(dev):
    # Codes, mask and scale of the operand forward are those of quest_quantize_fwd_ex.
    x = make_tensor(TensorSpec("op.same", 300, 2048, "bf16", "student_t", 4, 7100, outlier_cols=20,
                               outlier_scale=20.0), dev)
    c1, s1, m1, _ = qa.quantize_fwd_ex(x, 128, 4)
    c2, s2, m2, _ = qa.quantize_fwd_op(x, 128, 4, with_codes=True, with_mask=True)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(s1, s2) and torch.equal(m1, m2)


def test_fwd_op_leaves_bytes_outside_the_operand_alone(dev):
    rows, cols = 40, 256
    x = make_tensor(TensorSpec("op.guard", rows, cols, "bf16", "normal", 1.0, 7200), dev)
    n = qa.operand_bytes(rows, cols)
    buf = torch.full((n + 512,), 0xA5, dtype=torch.uint8, device=dev)
    op = buf[256:256 + n]
    qa.quantize_fwd_op(x, 128, 4, operand=op)
    torch.cuda.synchronize()
    assert bool((buf[:256] == 0xA5).all()) and bool((buf[256 + n:] == 0xA5).all())


# ---------------------------------------------------------------------------
# Grouped operand forward (quest_quantize_fwd_op_group): every output equal,
# bit for bit, to one quest_quantize_fwd_op call per tensor.  Operands start
# zeroed on both sides, so the padding rows the launches leave alone compare
# too; guard bytes around each operand must stay untouched.
# ---------------------------------------------------------------------------
OP_GROUP_CASES = [
    # (rows, cols, with codes and mask) per tensor, block, b, trust
    ([(77, 2048, True), (130, 2048, True), (1, 2048, False), (64, 2048, True), (33, 2048, False),
      (200, 2048, True)], 128, 4, 1.0),  # six tensors of one width: two launches
    ([(45, 512, True), (33, 1024, False), (0, 2048, True), (96, 2048, True), (21, 5632, True),
      (37, 384, False)], 64, 2, 1.0),  # three widths, an empty tensor, two tensors outside the grouped widths
    ([(300, 1024, True), (129, 512, True)], 256, 3, 1.3),
    ([(31, 2048, False), (2, 512, False)], 128, 1, 1.0),  # neither codes nor mask
]


@pytest.mark.parametrize("specs,block,b,trust", OP_GROUP_CASES)
def test_fwd_op_group_equals_single_calls(dev, specs, block, b, trust):
    log(f"fwd_op_group {specs} block {block} b={b} trust {trust}")
    xs = [make_tensor(TensorSpec(f"opg.x{i}", r, c, "bf16", "student_t", 4, 7300 + 13 * i + r, outlier_cols=max(1, c // 100),
                                 outlier_scale=20.0), dev) for i, (r, c, _) in enumerate(specs)]
    guard = 256

    def buffers():
        outs, bufs = [], []
        for (r, c, q) in specs:
            n = qa.operand_bytes(r, c)
            buf = torch.full((n + 2 * guard,), 0xA5, dtype=torch.uint8, device=dev)
            buf[guard:guard + n].zero_()
            o = dict(operand=buf[guard:guard + n], scale=torch.zeros((r,), dtype=torch.float32, device=dev))
            if q:
                o["codes"] = torch.zeros((r, c * b // 8), dtype=torch.uint8, device=dev)
                o["mask"] = torch.zeros((r, c // 8), dtype=torch.uint8, device=dev)
            outs.append(o)
            bufs.append(buf)
        return outs, bufs

    single, single_bufs = buffers()
    for x, o in zip(xs, single):
        qa.quantize_fwd_op(x, block, b, trust=trust, **o)
    grouped, grouped_bufs = buffers()
    res = qa.quantize_fwd_op_group(xs, block, b, trust=trust, outs=grouped)
    torch.cuda.synchronize()
    for i, ((r, c, q), o1, o2, b1, b2) in enumerate(zip(specs, single, grouped, single_bufs, grouped_bufs)):
        assert res[i][3].data_ptr() == o2["operand"].data_ptr()
        n = qa.operand_bytes(r, c)
        assert bool((b2[:guard] == 0xA5).all()) and bool((b2[guard + n:] == 0xA5).all()), f"tensor {i}: guard bytes"
        for key in o1:
            assert torch.equal(o1[key], o2[key]), f"tensor {i} ({r}x{c}): {key} differs from the single call"
    # the first ragged tensor against the oracle as well (the single calls are checked in the tests above)
    i = next((j for j, (r, c, q) in enumerate(specs) if q and r > 0), None)
    if i is None:
        log("fwd_op_group ok (no tensor with codes)")
        return
    r, c, _ = specs[i]
    st = check_fwd(to_float64(xs[i]), block, b, grouped[i]["codes"].cpu().numpy(), grouped[i]["scale"].cpu().numpy(),
                   grouped[i]["mask"].cpu().numpy(), trust=trust)
    log(f"fwd_op_group ok, tensor {i} {r}x{c} {st}")


def test_fwd_op_group_fp32_tensors_equal_single_calls(dev):
    """fp32 tensors take one quest_quantize_fwd_op launch each inside the group call."""
    shapes = [(50, 2048), (37, 384), (29, 640)]
    log(f"fwd_op_group fp32 {shapes}")
    xs = [make_tensor(TensorSpec(f"opg.f{i}", r, c, "f32", "student_t", 4, 7500 + i, outlier_cols=max(1, c // 100),
                                 outlier_scale=20.0), dev) for i, (r, c) in enumerate(shapes)]
    singles = [qa.quantize_fwd_op(x, 128, 3, trust=1.3, with_codes=True, with_mask=True) for x in xs]
    outs = [dict(codes=torch.empty_like(s[0]), mask=torch.empty_like(s[2]),
                 operand=torch.zeros_like(s[3])) for s in singles]
    for s in singles:
        s[3].zero_()
    singles = [qa.quantize_fwd_op(x, 128, 3, trust=1.3, with_codes=True, with_mask=True, operand=s[3])
               for x, s in zip(xs, singles)]
    res = qa.quantize_fwd_op_group(xs, 128, 3, trust=1.3, outs=outs)
    torch.cuda.synchronize()
    for i, (s, r) in enumerate(zip(singles, res)):
        for a, b, what in zip(s, r, ("codes", "scale", "mask", "operand")):
            assert torch.equal(a, b), f"tensor {i}: {what} differs from the single call"


def test_fwd_op_group_at_the_layer_shapes(dev):
    """The two operand forwards of a 2048-feature layer at 16384 tokens, as the layer launches them."""
    shapes = [(16384, 2048), (2048, 2048)]
    log(f"fwd_op_group at {shapes}")
    xs = [make_tensor(TensorSpec("opg.act", 16384, 2048, "bf16", "student_t", 4, 7400, outlier_cols=20,
                                 outlier_scale=20.0), dev),
          make_tensor(TensorSpec("opg.wt", 2048, 2048, "bf16", "normal", 0.02, 7401), dev)]
    singles = [qa.quantize_fwd_op(x, 128, 4, with_codes=True, with_mask=True) for x in xs]
    outs = [dict(codes=torch.empty_like(s[0]), scale=torch.empty_like(s[1]), mask=torch.empty_like(s[2]),
                 operand=torch.empty_like(s[3])) for s in singles]
    qa.quantize_fwd_op_group(xs, 128, 4, outs=outs)
    torch.cuda.synchronize()
    for (r, c), s, o in zip(shapes, singles, outs):
        assert torch.equal(s[0], o["codes"]) and torch.equal(s[1], o["scale"]) and torch.equal(s[2], o["mask"])
        assert torch.equal(s[3], o["operand"])  # rows are whole 32-row blocks: no padding


# ---------------------------------------------------------------------------
# The product on oracle-built operands.
# ---------------------------------------------------------------------------

def oracle_operand(x64: np.ndarray, block: int, b: int):
    rows, cols = x64.shape
    f = qo.quantize_fwd(x64, block, b)
    tiled = tile_operand(qo.operand_e2m3(f["codes"], cols, b), rows, cols)
    return f, tiled, f["scale"].astype(np.float32)


def gemm_reference(op_a, sa32, ba, op_b, sb32, bb, m, n, k):
    """The oracle's product and the float64 sum of |products| (which bounds its own rounding)."""
    a_rows = untile_operand(op_a, m, k)
    b_rows = untile_operand(op_b, n, k)
    ref = qo.quest_gemm(a_rows, sa32.astype(np.float64), ba, b_rows, sb32.astype(np.float64), bb, k)
    va = np.abs(qo.e2m3_value(qo.unpack_lsb_first(a_rows, 6, k))) * qo.operand_step(sa32, ba)[:, None]
    vb = np.abs(qo.e2m3_value(qo.unpack_lsb_first(b_rows, 6, k))) * qo.operand_step(sb32, bb)[:, None]
    return ref, va @ vb.T


def check_product(got: torch.Tensor, ref: np.ndarray, tol: float, skip=None, abs_sum=None, k: int = 0) -> float:
    """|got - ref| <= tol |ref| + 2 k 2^-53 abs_sum: the GPU's sum of half-integer products
    is exact, the float64 reference carries summation error up to the second term."""
    got = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    slack = 0.0 if abs_sum is None else 2.0 * k * 2.0 ** -53 * abs_sum
    ok = err <= tol * np.abs(ref) + slack
    if skip is not None:
        ok |= skip
    if not ok.all():
        r, c = np.argwhere(~ok)[0]
        raise AssertionError(f"{int((~ok).sum())} outputs off, first ({r},{c}): got {got[r, c]!r} ref {ref[r, c]!r}")
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(ref != 0, err / np.abs(ref), 0.0)
    if skip is not None:
        ratio = np.where(skip, 0.0, ratio)
    return float(ratio.max(initial=0.0))


GEMM_CASES = [
    # m, n, k, bits_a, bits_b
    (300, 200, 256, 4, 4),
    (513, 260, 384, 2, 3),  # bf16 rows of 260: element stores
    (256, 256, 128, 4, 1),  # one stage
    (97, 45, 640, 3, 4),  # odd n: element stores in both types; 5 stages
    (1024, 512, 2048, 4, 4),  # 8 tiles, 16 stages
    (40, 700, 1152, 1, 2),  # 9 stages
    (33280, 300, 128, 4, 4),  # 260 tiles: the last round's 4 tiles run as 8 half tiles, 2 of them past n
]


@pytest.mark.parametrize("m,n,k,ba,bb", GEMM_CASES)
def test_gemm_matches_oracle(dev, m, n, k, ba, bb):
    log(f"gemm {m}x{n}x{k} bits {ba}/{bb}")
    xa = to_float64(make_tensor(TensorSpec("g.a", m, k, "f32", "student_t", 4, 8000 + m, outlier_cols=3,
                                           outlier_scale=10.0), "cpu"))
    xb = to_float64(make_tensor(TensorSpec("g.b", n, k, "f32", "normal", 0.02, 8100 + n), "cpu"))
    xa[min(5, m - 1)] = 0.0  # a zero row: scale 0, outputs exactly 0
    _, op_a, sa = oracle_operand(xa, 128, ba)
    _, op_b, sb = oracle_operand(xb, 128, bb)
    ref, abs_sum = gemm_reference(op_a, sa, ba, op_b, sb, bb, m, n, k)
    ta, tb = torch.from_numpy(op_a).to(dev), torch.from_numpy(op_b).to(dev)
    tsa, tsb = torch.from_numpy(sa).to(dev), torch.from_numpy(sb).to(dev)
    side = torch.cuda.Stream()  # the stream argument is honoured
    with torch.cuda.stream(side):
        y32 = qa.gemm(ta, tsa, m, ba, tb, tsb, n, bb, k, out_dtype=torch.float32)
        y16 = qa.gemm(ta, tsa, m, ba, tb, tsb, n, bb, k, out_dtype=torch.bfloat16)
    side.synchronize()
    r32 = check_product(y32, ref, 1e-6, abs_sum=abs_sum, k=k)
    r16 = check_product(y16, ref, 4e-3, abs_sum=abs_sum, k=k)
    assert bool((y32[min(5, m - 1)] == 0).all())
    # deterministic: a second call gives the same bits
    y32b = qa.gemm(ta, tsa, m, ba, tb, tsb, n, bb, k, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y32, y32b)
    log(f"gemm ok: max relative error fp32 {r32:.3g}, bf16 {r16:.3g}")


def test_gemm_exact_at_the_largest_k(dev):
    """k = 65536, the largest accepted, with every level at +-7.5 (the largest magnitude):
    sums reach 65536 * 56.25 = 3686400 in quarter steps, which fp32 still holds exactly.
    With clip scales 7.5 the steps are 1, so every fp32 output is the exact sum."""
    m, n, k, b = 32, 24, 65536, 4
    log(f"gemm {m}x{n}x{k}, every level +-7.5")
    rng = np.random.default_rng(8400)
    ua = np.where(rng.random((m, k)) < 0.5, 0, 15)
    ub = np.where(rng.random((n, k)) < 0.5, 0, 15)
    ua[0] = 15  # rows of one sign: the largest sums, +3686400 and -3686400
    ub[0] = 15
    ub[1] = 0
    op_a = tile_operand(qo.operand_e2m3(qo.pack_lsb_first(ua, b), k, b), m, k)
    op_b = tile_operand(qo.operand_e2m3(qo.pack_lsb_first(ub, b), k, b), n, k)
    sa = np.full(m, 7.5, dtype=np.float32)
    sb = np.full(n, 7.5, dtype=np.float32)
    ref = qo.quest_gemm(untile_operand(op_a, m, k), sa.astype(np.float64), b, untile_operand(op_b, n, k),
                        sb.astype(np.float64), b, k)
    assert ref[0, 0] == 3686400.0 and ref[0, 1] == -3686400.0
    y = qa.gemm(torch.from_numpy(op_a).to(dev), torch.from_numpy(sa).to(dev), m, b, torch.from_numpy(op_b).to(dev),
                torch.from_numpy(sb).to(dev), n, b, k, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} outputs differ from the exact sums"


def test_gemm_writes_nothing_outside_the_output(dev):
    m, n, k = 70, 36, 256
    xa = to_float64(make_tensor(TensorSpec("g.ga", m, k, "f32", "normal", 1.0, 8200), "cpu"))
    xb = to_float64(make_tensor(TensorSpec("g.gb", n, k, "f32", "normal", 1.0, 8201), "cpu"))
    _, op_a, sa = oracle_operand(xa, 128, 4)
    _, op_b, sb = oracle_operand(xb, 128, 4)
    buf = torch.full((m * n + 256,), -7.0, dtype=torch.float32, device=dev)
    out = buf[128:128 + m * n].view(m, n)
    qa.gemm(torch.from_numpy(op_a).to(dev), torch.from_numpy(sa).to(dev), m, 4, torch.from_numpy(op_b).to(dev),
            torch.from_numpy(sb).to(dev), n, 4, k, out=out)
    torch.cuda.synchronize()
    assert bool((buf[:128] == -7.0).all()) and bool((buf[128 + m * n:] == -7.0).all())
    ref, abs_sum = gemm_reference(op_a, sa, 4, op_b, sb, 4, m, n, k)
    check_product(out, ref, 1e-6, abs_sum=abs_sum, k=k)


# ---------------------------------------------------------------------------
# The layer end to end: forward on both operands, then the product.
# ---------------------------------------------------------------------------

def band_rows(f: dict, b: int) -> np.ndarray:
    """Rows holding an entry within the threshold band (its code may differ, correctly)."""
    return exempt_entries(f["y"], f["scale"], b).any(axis=1)


@pytest.mark.parametrize("m,n,k,bx,bw", [(200, 96, 2048, 4, 4), (64, 160, 5632, 4, 4), (130, 64, 512, 2, 3)])
def test_layer_end_to_end(dev, m, n, k, bx, bw):
    log(f"layer {m}x{k} by {n}x{k}, bits {bx}/{bw}")
    x = make_tensor(TensorSpec("e.x", m, k, "bf16", "student_t", 4, 8300 + m, outlier_cols=k // 100,
                               outlier_scale=20.0), dev)
    w = make_tensor(TensorSpec("e.w", n, k, "bf16", "normal", 0.02, 8400 + n), dev)
    _, sx, _, ox = qa.quantize_fwd_op(x, 128, bx)
    _, sw, _, ow = qa.quantize_fwd_op(w, 128, bw)
    y = qa.gemm(ox, sx, m, bx, ow, sw, n, bw, k, out_dtype=torch.float32)
    torch.cuda.synchronize()
    f = qo.qat_linear_fwd(to_float64(x), to_float64(w), 128, bx, bw)
    skip = band_rows(f["fx"], bx)[:, None] | band_rows(f["fw"], bw)[None, :]
    # GPU scales are within 2e-6 of the oracle's (checked by check_fwd): 1e-5 covers both Deltas.
    ratio = check_product(y, f["y"], 1e-5, skip, abs_sum=np.abs(f["qx"]) @ np.abs(f["qw"]).T, k=k)
    log(f"layer ok: {int(skip.sum())} outputs in band reach, max relative error {ratio:.3g}")


# ---------------------------------------------------------------------------
# The 1.6B block's seven products at full size, sampled.
# ---------------------------------------------------------------------------

def sample(n: int, k: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([rng.choice(n, size=min(k, n), replace=False), [0, n - 1]]))


@pytest.mark.parametrize("name,act,wt", layer_products(), ids=[p[0] for p in layer_products()])
def test_block_products_full_size_sampled(dev, name, act, wt):
    m, k, n = act.rows, act.cols, wt.rows
    log(f"block product {name}: {m}x{k} by {n}x{k}")
    x = make_tensor(act, dev)
    w = make_tensor(wt, dev)
    _, sx, _, ox = qa.quantize_fwd_op(x, 128, 4)
    _, sw, _, ow = qa.quantize_fwd_op(w, 128, 4)
    y = qa.gemm(ox, sx, m, 4, ow, sw, n, 4, k, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ri = sample(m, 24, 9000 + k)
    rj = sample(n, 24, 9100 + n)
    # the sampled rows of the seeded inputs (generated on the GPU), widened exactly
    xs = to_float64(x.index_select(0, torch.as_tensor(ri, device=dev)))
    ws = to_float64(w.index_select(0, torch.as_tensor(rj, device=dev)))
    f = qo.qat_linear_fwd(xs, ws, 128, 4, 4)
    skip = band_rows(f["fx"], 4)[:, None] | band_rows(f["fw"], 4)[None, :]
    got = y.index_select(0, torch.as_tensor(ri, device=dev)).index_select(1, torch.as_tensor(rj, device=dev))
    ratio = check_product(got, f["y"], 4e-3 + 1e-5, skip, abs_sum=np.abs(f["qx"]) @ np.abs(f["qw"]).T, k=k)
    log(f"{name} ok: {len(ri)}x{len(rj)} sampled outputs, {int(skip.sum())} in band reach, max rel {ratio:.3g}")


# ---------------------------------------------------------------------------
# Products of more full tiles than compute units, whose workgroups each walk
# several tiles (bf16 output): ragged m and n, a short last round split into
# half tiles, sampled outputs against the oracle and a guard band around the
# output.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("m,n,k", [(10000, 3000, 1024), (16484, 2048, 2048), (16384, 5632, 384)])
def test_product_tile_walk_sampled(dev, m, n, k):
    log(f"tile-walk product {m}x{k} by {n}x{k}")
    x = make_tensor(TensorSpec("w.x", m, k, "bf16", "student_t", 4, 9300 + m, outlier_cols=k // 100,
                               outlier_scale=20.0), dev)
    w = make_tensor(TensorSpec("w.w", n, k, "bf16", "normal", 0.02, 9400 + n), dev)
    _, sx, _, ox = qa.quantize_fwd_op(x, 128, 4)
    _, sw, _, ow = qa.quantize_fwd_op(w, 128, 4)
    guard = 4096
    buf = torch.full((m * n + 2 * guard,), -7.0, dtype=torch.bfloat16, device=dev)
    y = buf[guard:guard + m * n].view(m, n)
    qa.gemm(ox, sx, m, 4, ow, sw, n, 4, k, out=y)
    torch.cuda.synchronize()
    assert bool((buf[:guard] == -7.0).all()) and bool((buf[guard + m * n:] == -7.0).all())
    ri = sample(m, 24, 9500 + m)
    rj = sample(n, 24, 9600 + n)
    xs = to_float64(x.index_select(0, torch.as_tensor(ri, device=dev)))
    ws = to_float64(w.index_select(0, torch.as_tensor(rj, device=dev)))
    f = qo.qat_linear_fwd(xs, ws, 128, 4, 4)
    skip = band_rows(f["fx"], 4)[:, None] | band_rows(f["fw"], 4)[None, :]
    got = y.index_select(0, torch.as_tensor(ri, device=dev)).index_select(1, torch.as_tensor(rj, device=dev))
    ratio = check_product(got, f["y"], 4e-3 + 1e-5, skip, abs_sum=np.abs(f["qx"]) @ np.abs(f["qw"]).T, k=k)
    assert not bool(torch.isnan(y).any())
    log(f"tile walk ok: {len(ri)}x{len(rj)} sampled outputs, max rel {ratio:.3g}")


# ---------------------------------------------------------------------------
# Stored codes to the operand (quest_codes_to_operand): the same bytes as the
# operand quest_quantize_fwd_op writes with those codes on every row of the
# tensor (the padding rows of the last 32-row block are left alone by the
# conversion, while the forward's spare waves may write them), and the same
# product.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("rows,cols,b", [(45, 384, 4), (64, 2048, 1), (64, 2048, 2), (33, 2048, 3), (33, 5632, 4),
                                         (1000, 640, 2), (7, 128, 4), (96, 1152, 3)])
def test_codes_to_operand_equals_forward_operand(dev, rows, cols, b):
    log(f"codes to operand {rows}x{cols} b={b}")
    x = make_tensor(TensorSpec("c2o.x", rows, cols, "bf16", "student_t", 4, 8700 + cols + b, outlier_cols=2,
                               outlier_scale=20.0), dev)
    nbytes = qa.operand_bytes(rows, cols)
    op_fwd = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=dev)
    codes, scale, _, _ = qa.quantize_fwd_op(x, 128, b, with_codes=True, operand=op_fwd)
    op_c = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=dev)
    qa.codes_to_operand(codes, rows, cols, b, operand=op_c)
    torch.cuda.synchronize()
    rows_c = untile_operand(op_c.cpu().numpy()[:nbytes], rows, cols)
    rows_f = untile_operand(op_fwd.cpu().numpy()[:nbytes], rows, cols)
    assert np.array_equal(rows_c, rows_f), f"{int((rows_c != rows_f).sum())} operand bytes differ"
    # the conversion writes no padding row
    pad = op_c.cpu().numpy()[:nbytes].copy()
    pad_rows = untile_operand(pad, ((rows + 31) // 32) * 32, cols)[rows:]
    assert (pad_rows == 0xA5).all()
    # the fields decode to the codes' levels (read back through the layout helper)
    u = qo.unpack_lsb_first(codes.cpu().numpy(), b, cols)
    fields = gpu_fields(op_c, rows, cols)
    assert np.array_equal(fields, halves_e2m3(u, b))


def test_product_from_stored_codes(dev):
    """A weight kept as 4-bit codes feeds the product through quest_codes_to_operand and gives the
    product of the operand forward exactly."""
    m, n, k = 300, 256, 2048
    x = make_tensor(TensorSpec("c2o.a", m, k, "bf16", "student_t", 4, 8800, outlier_cols=20, outlier_scale=20.0), dev)
    w = make_tensor(TensorSpec("c2o.w", n, k, "bf16", "normal", 0.02, 8801), dev)
    _, sx, _, ox = qa.quantize_fwd_op(x, 128, 4)
    cw, sw, _, ow = qa.quantize_fwd_op(w, 128, 4, with_codes=True)
    ow_c = qa.codes_to_operand(cw, n, k, 4)
    y_fwd = qa.gemm(ox, sx, m, 4, ow, sw, n, 4, k, out_dtype=torch.float32)
    y_codes = qa.gemm(ox, sx, m, 4, ow_c, sw, n, 4, k, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y_fwd, y_codes)
