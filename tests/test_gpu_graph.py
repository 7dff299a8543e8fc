"""The library's launches recorded in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Every entry point launches kernels on the caller's stream and calls no
allocator, copy, fill or synchronisation, so a step of the hot path can be
captured once and replayed.  Each graph here is replayed several times, with
eager work (refilling its output buffers) and device synchronisations between
the replays, and every replay is compared bit for bit with the eager calls on
the same inputs.
"""
from __future__ import annotations

import pytest
import torch

import quantization_aware_amd as qa
from quest_inputs import TensorSpec, make_tensor

pytestmark = pytest.mark.gpu


def log(msg: str) -> None:
    print(f"[gpu-graph] {msg}", flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qa.load_library()
    return torch.device("cuda", 0)


def capture(fn):
    """fn() recorded in a graph, after one warm call on a side stream (torch's capture recipe)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def replay_and_check(graph, outs, refs, what, replays=3):
    for r in range(replays):
        for o in outs:
            o.fill_(7 if o.dtype in (torch.uint8,) else 3.0)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, ref) in enumerate(zip(outs, refs)):
            assert torch.equal(o, ref), f"{what}: replay {r}, output {i} differs from the eager call"


@pytest.mark.parametrize("rows,cols,block,b", [(2048, 2048, 128, 4), (1000, 512, 64, 2), (96, 5632, 128, 1)])
def test_forward_backward_step_in_a_graph(dev, rows, cols, block, b):
    log(f"graph of forward + trust backward, {rows}x{cols}, block {block}, b={b}")
    x = make_tensor(TensorSpec("graph.x", rows, cols, "bf16", "student_t", 4, 9500 + rows, outlier_cols=cols // 100,
                               outlier_scale=20.0), dev)
    g = make_tensor(TensorSpec("graph.g", rows, cols, "bf16", "normal", 1e-3, 9600 + rows), dev)
    codes_e, scale_e, mask_e = qa.quantize_fwd(x, block, b)
    dx_e = qa.trust_bwd(g, mask_e, block)
    torch.cuda.synchronize()
    codes, scale, mask = torch.empty_like(codes_e), torch.empty_like(scale_e), torch.empty_like(mask_e)
    dx = torch.empty_like(dx_e)

    def step():
        qa.quantize_fwd(x, block, b, codes=codes, scale=scale, mask=mask)
        qa.trust_bwd(g, mask, block, out=dx)

    replay_and_check(capture(step), [codes, scale, mask, dx], [codes_e, scale_e, mask_e, dx_e], "fwd + bwd")


def test_grouped_forward_in_a_graph(dev):
    shapes = [(256, 2048), (128, 1024), (64, 5632), (96, 2048)]
    log(f"graph of one grouped forward over {shapes}")
    xs = [make_tensor(TensorSpec(f"graph.gx{i}", r, c, "bf16", "normal", 0.02, 9700 + i), dev)
          for i, (r, c) in enumerate(shapes)]
    refs = [t for out in qa.quantize_fwd_group(xs, 128, 4) for t in out]
    torch.cuda.synchronize()
    held = []

    def step():
        held.clear()
        held.extend(t for out in qa.quantize_fwd_group(xs, 128, 4) for t in out)

    graph = capture(step)
    replay_and_check(graph, list(held), refs, "grouped forward")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_operand_forward_and_product_in_a_graph(dev, out_dtype):
    m, n, k = 16384, 2048, 2048
    log(f"graph of two operand forwards and the FP6 product {m}x{n}x{k}, {out_dtype}")
    a = make_tensor(TensorSpec("graph.a", m, k, "bf16", "student_t", 4, 9800), dev)
    w = make_tensor(TensorSpec("graph.w", n, k, "bf16", "normal", 0.02, 9801), dev)
    _, sa_e, _, oa_e = qa.quantize_fwd_op(a, 128, 4)
    _, sw_e, _, ow_e = qa.quantize_fwd_op(w, 128, 4)
    y_e = qa.gemm(oa_e, sa_e, m, 4, ow_e, sw_e, n, 4, k, out_dtype=out_dtype)
    torch.cuda.synchronize()
    sa, oa, sw, ow = (torch.empty_like(t) for t in (sa_e, oa_e, sw_e, ow_e))
    y = torch.empty_like(y_e)

    def step():
        qa.quantize_fwd_op(a, 128, 4, operand=oa, scale=sa)
        qa.quantize_fwd_op(w, 128, 4, operand=ow, scale=sw)
        qa.gemm(oa, sa, m, 4, ow, sw, n, 4, k, out=y)

    replay_and_check(capture(step), [sa, oa, sw, ow, y], [sa_e, oa_e, sw_e, ow_e, y_e], "operand forwards + product")


def test_grouped_operand_forwards_in_a_graph(dev):
    shapes = [(1024, 2048), (512, 2048), (96, 512)]
    log(f"graph of one grouped operand forward over {shapes}")
    xs = [make_tensor(TensorSpec(f"graph.ox{i}", r, c, "bf16", "student_t", 4, 9900 + i), dev)
          for i, (r, c) in enumerate(shapes)]
    refs = qa.quantize_fwd_op_group(xs, 128, 4, outs=[
        dict(codes=torch.empty((r, c // 2), dtype=torch.uint8, device=dev),
             mask=torch.empty((r, c // 8), dtype=torch.uint8, device=dev)) for r, c in shapes])
    torch.cuda.synchronize()
    outs = [{k: torch.empty_like(t) for k, t in zip(("codes", "scale", "mask", "operand"), ref)} for ref in refs]

    def step():
        qa.quantize_fwd_op_group(xs, 128, 4, outs=outs)

    graph = capture(step)
    keys = ("codes", "scale", "mask", "operand")
    replay_and_check(graph, [o[k] for o in outs for k in keys], [t for ref in refs for t in ref],
                     "grouped operand forward")
