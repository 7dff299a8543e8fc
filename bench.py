"""Throughput of the QuEST quantiser hot path on one MI355X.

One step = the whole path over one batch: forward quantisation (Hadamard,
RMS scale, codes, trust mask) of a 16384 x 2048 bf16 activation at b = 4,
block 128, then the trust-masked inverse-Hadamard backward of a 16384 x 2048
bf16 gradient with that step's mask.  Inputs are synthetic (seeded
Student-t(4) activations with 20 outlier channels x20, N(0, 1e-3^2)
gradients) and resident in HBM before timing starts.  Steps rotate over
several buffer sets so that no step finds its data in the 256 MB last-level
cache.

Timing, all with HIP events on the stream the kernels are launched on:
  * the step: K steps bracketed by device synchronisation.  Steps are
    independent batches on two streams, step i on stream i % 2 with its
    backward after its forward in that stream's order, so consecutive steps
    overlap (the one-stream time is reported too).  Each stream records a
    start and an end event; the event time is the span from the earlier
    start to the later end, and ms_per_step is the larger of that and the
    wall clock between the two synchronisations, over K;
  * each kernel: K back-to-back launches of that kernel alone between two
    events (events between every kernel would add their own gaps);
  * a plain copy kernel (elementwise negation) moving as many bytes as the
    backward, as the practical bandwidth reference of this GPU.

Prints one JSON line: throughput in quantised elements/s, the roofline of
the dominant kernel (algorithmic bytes per launch over its mean duration),
and the CPU oracle's rate on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantised elements/s and % HBM roofline for fused Hadamard-quantize fwd+bwd"
HBM_PEAK_GBPS = 8000.0
ROWS, COLS, BLOCK, BITS = 16384, 2048, 128, 4
N_SETS = 8
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_16384x2048.txt")
KERNEL_SOURCES = ["quest_device.h", "quest_kernels.h", "quest_grids.hip"]


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-block-products", action="store_true",
                   help="skip the 4-bit products of a 1.6B-scale block (FP6 matrix cores vs BF16)")
    p.add_argument("--product-reps", type=int, default=50, help="back-to-back launches per product timing")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain elementwise copy of known size (for counter calibration)")
    p.add_argument("--configs", default="C2,C3,C4,C5",
                   help="comma-separated full-size configurations to time beside the headline ('none': skip)")
    p.add_argument("--only-configs", action="store_true",
                   help="time only the --configs (no headline step, products or CPU baseline; for profiling)")
    return p.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "quantization_aware_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_tag: str):
    """HBM bytes per launch from the committed counter summary, if it matches the current kernels."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    key = f"{kernel_tag}_hbm_bytes_per_launch"
    return float(vals[key]) if key in vals else None


def alg_bytes_fwd(rows, cols, in_bytes, bits):
    return rows * cols * in_bytes + rows * cols * bits // 8 + rows * cols // 8 + 4 * rows


def alg_bytes_bwd(rows, cols, g_bytes):
    return 2 * rows * cols * g_bytes + rows * cols // 8


def cpu_baseline(x_dev, g_dev, target_seconds):
    """Time the fp64 oracle (fwd then bwd) on a bounded sample of the same tensors.

    Rows are taken in order in chunks, wrapping round to row 0, until the
    oracle has run for target_seconds; the rate counts every element it
    processed.  Widening to fp64 happens outside the timed part.
    """
    import numpy as np

    from oracle import quest_oracle as qo
    from quest_inputs import to_float64

    try:
        from threadpoolctl import threadpool_info

        threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = 1
    qo.fit_alpha(BITS)  # the fit is a one-off per bit width, outside the per-tensor work
    chunk = 1024
    elapsed = 0.0
    done = 0
    start = 0
    while elapsed < target_seconds:
        x64 = to_float64(x_dev[start : start + chunk])
        g64 = to_float64(g_dev[start : start + chunk])
        t0 = time.perf_counter()
        ref = qo.quantize_fwd(x64, BLOCK, BITS)
        qo.trust_bwd(g64, ref["mask"], BLOCK)
        elapsed += time.perf_counter() - t0
        done += x64.shape[0]
        start = (start + chunk) % ROWS
    return {
        "value": done * COLS / elapsed,
        "unit": "elements/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} rows ({done * COLS} elements; {done / ROWS:.2f} passes over the 16384x2048 workload, "
        f"in {chunk}-row chunks), fwd then bwd, {elapsed:.1f} s of oracle time",
        "cpu_count": os.cpu_count(),
        "cpu_model": cpu_model(),
        "blas_threads": int(threads),
    }


def cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


CONFIG_TARGET_FRAC = 0.70  # the bar: 70% of the HBM roofline
COLD_BYTES = 640 << 20  # buffer sets rotate until this much lies between two uses of one set


def config_runs(lib, qa, torch, dev, reps, names):
    """Full-size configurations C2-C5, each pass timed cache-cold against 70% of the HBM roofline.

    Every timing is `reps` back-to-back repetitions between HIP events on the
    launch stream, rotating over enough copies of the inputs and outputs that
    more than 512 MiB is touched between two uses of one copy (the 256 MB
    last-level cache then serves no repetition from an earlier one).
    C2: 16384x512 bf16 Student-t(4) activation, forward at b = 1..4;
    C3: the seven weight tensors of a 1.6B-scale block, forward at b = 4, one
        repetition quantising all seven;
    C4: trust backward of a 65536x2048 bf16 gradient with the mask of a
        Student-t(4) activation's forward;
    C5: 131072x5632 bf16 Student-t(3) activation, forward at b = 1 then the
        backward of a gradient of that shape, one step.
    """
    from quest_inputs import WORKLOADS, make_tensor

    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    vp = ctypes.c_void_p
    f_fwd, f_bwd = lib.quest_quantize_fwd, lib.quest_trust_bwd

    def check(name, st):
        if st:
            raise qa.QuestError(name, st, lib.quest_status_string(st).decode())

    def timed(launch, nsets):
        for i in range(min(nsets, 3)):
            launch(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(reps):
            launch(i % nsets)
        b.record(stream)
        torch.cuda.synchronize()
        return 1000.0 * a.elapsed_time(b) / reps

    def sets_for(set_bytes):
        return max(2, -(-COLD_BYTES // set_bytes) + 1)

    def entry(us, alg_bytes, elements):
        gbps = alg_bytes / (us * 1e3)
        return {"us": round(us, 3), "alg_bytes": alg_bytes, "gbps": round(gbps, 1),
                "frac": round(gbps / HBM_PEAK_GBPS, 4), "elements_per_s": elements / (us * 1e-6),
                "target_us_at_70pct": round(alg_bytes / (CONFIG_TARGET_FRAC * HBM_PEAK_GBPS * 1e3), 3)}

    def fwd_set(x, bits):
        r, c = x.shape
        return (x, torch.empty((r, c * bits // 8), dtype=torch.uint8, device=dev),
                torch.empty((r,), dtype=torch.float32, device=dev),
                torch.empty((r, c // 8), dtype=torch.uint8, device=dev))

    def fwd_call(st_, block, bits):
        x, cd, sc, mk = st_
        return lambda: check("quest_quantize_fwd", f_fwd(vp(x.data_ptr()), qa.QUEST_BF16, x.shape[0], x.shape[1],
                                                         block, bits, vp(cd.data_ptr()), vp(sc.data_ptr()),
                                                         vp(mk.data_ptr()), sh))

    def bwd_call(g, mk, out, block):
        return lambda: check("quest_trust_bwd", f_bwd(vp(g.data_ptr()), qa.QUEST_BF16, vp(mk.data_ptr()), g.shape[0],
                                                      g.shape[1], block, vp(out.data_ptr()), sh))

    res = {}
    if "C2" in names:
        wl = WORKLOADS["C2"]
        spec = wl.fwd[0]
        x0 = make_tensor(spec, dev)
        rec = {"workload": wl.description}
        for bits in wl.bits:
            alg = alg_bytes_fwd(spec.rows, spec.cols, 2, bits)
            n = sets_for(alg)
            sets = [fwd_set(x0 if i == 0 else x0.clone(), bits) for i in range(n)]
            calls = [fwd_call(st_, wl.block, bits) for st_ in sets]
            rec[f"b{bits}"] = entry(timed(lambda i: calls[i](), n), alg, spec.elements)
            rec[f"b{bits}"]["buffer_sets"] = n
            del sets, calls
        res["C2"] = rec
        del x0
    if "C3" in names:
        wl = WORKLOADS["C3"]
        ws = [make_tensor(spec, dev) for spec in wl.fwd]
        alg = sum(alg_bytes_fwd(w.shape[0], w.shape[1], 2, 4) for w in ws)
        n = sets_for(alg)
        sets = [[fwd_set(w if i == 0 else w.clone(), 4) for w in ws] for i in range(n)]
        calls = [[fwd_call(st_, wl.block, 4) for st_ in one] for one in sets]

        def all_seven(i):
            for c in calls[i]:
                c()

        descs = []
        for one in sets:
            d = (qa._FwdTensor * len(one))()
            for j, (x, cd, sc, mk) in enumerate(one):
                d[j] = qa._FwdTensor(x.data_ptr(), x.shape[0], x.shape[1], cd.data_ptr(), sc.data_ptr(), mk.data_ptr())
            descs.append(d)
        f_group = lib.quest_quantize_fwd_group

        def grouped(i):
            check("quest_quantize_fwd_group", f_group(descs[i], len(ws), qa.QUEST_BF16, wl.block, 4, sh))

        elements = sum(w.numel() for w in ws)
        rec = {"workload": wl.description,
               "grouped": entry(timed(grouped, n), alg, elements),
               "all_seven": entry(timed(all_seven, n), alg, elements),
               "note": "grouped: one quest_quantize_fwd_group call (one launch: the tiles of q, k, v, o, gate, up, "
                       "then down's rows); all_seven: seven quest_quantize_fwd calls",
               "buffer_sets": n, "per_tensor_us": {}}
        for j, spec in enumerate(wl.fwd):
            rec["per_tensor_us"][spec.name.split(".")[1]] = round(timed(lambda i: calls[i][j](), n), 3)
        res["C3"] = rec
        del ws, sets, calls
    if "C4" in names:
        wl = WORKLOADS["C4"]
        act, gspec = wl.fwd[0], wl.grad[0]
        _, _, mask = qa.quantize_fwd(make_tensor(act, dev), wl.block, 4)
        g0 = make_tensor(gspec, dev)
        alg = alg_bytes_bwd(gspec.rows, gspec.cols, 2)
        n = sets_for(alg)
        sets = [(g0 if i == 0 else g0.clone(), mask if i == 0 else mask.clone(), torch.empty_like(g0))
                for i in range(n)]
        calls = [bwd_call(g, mk, o, wl.block) for g, mk, o in sets]
        res["C4"] = {"workload": wl.description, "bwd": entry(timed(lambda i: calls[i](), n), alg, gspec.elements),
                     "buffer_sets": n}
        del sets, calls, g0, mask
    if "C5" in names:
        wl = WORKLOADS["C5"]
        act, gspec = wl.fwd[0], wl.grad[0]
        x0, g0 = make_tensor(act, dev), make_tensor(gspec, dev)
        fwd_b = alg_bytes_fwd(act.rows, act.cols, 2, 1)
        bwd_b = alg_bytes_bwd(gspec.rows, gspec.cols, 2)
        sets = []
        for i in range(2):
            fs = fwd_set(x0 if i == 0 else x0.clone(), 1)
            sets.append((fs, g0 if i == 0 else g0.clone(), torch.empty_like(g0)))
        fcalls = [fwd_call(fs, wl.block, 1) for fs, _, _ in sets]
        bcalls = [bwd_call(g, fs[3], o, wl.block) for fs, g, o in sets]

        def step(i):
            fcalls[i]()
            bcalls[i]()

        res["C5"] = {"workload": wl.description,
                     "step": entry(timed(step, 2), fwd_b + bwd_b, act.elements),
                     "fwd": entry(timed(lambda i: fcalls[i](), 2), fwd_b, act.elements),
                     "bwd": entry(timed(lambda i: bcalls[i](), 2), bwd_b, gspec.elements),
                     "buffer_sets": 2, "schedule": "forward then backward on one stream, back to back"}
        del sets, fcalls, bcalls, x0, g0
    torch.cuda.synchronize()
    return res


FP6_PEAK_TFLOPS = 10100.0  # MI355X dense FP6/FP4 matrix peak
BF16_PEAK_TFLOPS = 2500.0


def block_products(lib, qa, torch, dev, reps):
    """The seven 4-bit products of a 1.6B-scale Llama block at 16384 tokens.

    Per product: the activation's forward into the matrix-core operand
    (Hadamard, RMS scale, codes as FP6 levels), the FP6 product with the
    pre-quantised weight (bf16 output), and torch's BF16 product of the same
    bf16 tensors (hipBLASLt) -- each timed as `reps` back-to-back launches
    between HIP events on the launch stream.  The quantisation rotates
    copies of its input and outputs (cache-cold, like the headline); the two
    products, bound by their matrix cores, reuse one set each.  The block total quantises each
    distinct activation once (attention input for q, k, v; attention output
    for o; MLP input for gate and up; MLP intermediate for down).
    """
    from quest_inputs import LAYER_ACT_2048, LAYER_ACT_5632, layer_products, make_tensor

    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)

    def timed(launch):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(3):
            launch()
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            launch()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def check(name, st):
        if st:
            raise qa.QuestError(name, st, lib.quest_status_string(st).decode())

    acts = {}
    for spec in (LAYER_ACT_2048, LAYER_ACT_5632):
        x = make_tensor(spec, dev)
        op = torch.empty((qa.operand_bytes(spec.rows, spec.cols),), dtype=torch.uint8, device=dev)
        sc = torch.empty((spec.rows,), dtype=torch.float32, device=dev)
        # The activation's quantisation is timed cache-cold: copies of the input
        # and outputs rotate so that more than 640 MiB lies between two uses.
        set_bytes = x.numel() * 2 + op.numel() + sc.numel() * 4
        n_sets = max(2, -(-COLD_BYTES // set_bytes) + 1)
        sets = [(x, op, sc)] + [(x.clone(), torch.empty_like(op), torch.empty_like(sc)) for _ in range(n_sets - 1)]
        args = [(ctypes.c_void_p(xi.data_ptr()), qa.QUEST_BF16, spec.rows, spec.cols, BLOCK, 4, ctypes.c_double(1.0),
                 None, ctypes.c_void_p(sci.data_ptr()), None, ctypes.c_void_p(opi.data_ptr()), sh)
                for xi, opi, sci in sets]
        turn = [0]

        def quantise():
            a = args[turn[0] % n_sets]
            turn[0] += 1
            check("quest_quantize_fwd_op", lib.quest_quantize_fwd_op(*a))

        t_q = timed(quantise)
        del sets, args
        acts[spec.cols] = {"x": x, "op": op, "scale": sc, "quant_ms": t_q, "quant_sets": n_sets}
    rows = []
    for name, act, wt in layer_products():
        a = acts[act.cols]
        m, k, n = act.rows, act.cols, wt.rows
        w = make_tensor(wt, dev)
        _, w_scale, _, w_op = qa.quantize_fwd_op(w, BLOCK, 4)
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        gargs = (ctypes.c_void_p(a["op"].data_ptr()), ctypes.c_void_p(a["scale"].data_ptr()), m, 4,
                 ctypes.c_void_p(w_op.data_ptr()), ctypes.c_void_p(w_scale.data_ptr()), n, 4, k,
                 ctypes.c_void_p(out.data_ptr()), qa.QUEST_BF16, sh)
        t_g = timed(lambda: check("quest_gemm", lib.quest_gemm(*gargs)))
        x = a["x"]
        t_b = timed(lambda: torch.nn.functional.linear(x, w))
        flops = 2.0 * m * n * k
        rows.append({
            "product": name, "m": m, "n": n, "k": k,
            "quest_gemm_us": 1000 * t_g, "quantise_activation_us": 1000 * a["quant_ms"],
            "quantise_activation_buffer_sets": a["quant_sets"],
            "bf16_us": 1000 * t_b,
            "fp6_tflops": flops / (t_g * 1e9), "bf16_tflops": flops / (t_b * 1e9),
            "speedup_product": t_b / t_g,
            "speedup_with_quantisation": t_b / (t_g + a["quant_ms"]),
        })
        del w, w_op, w_scale, out
    t_fp6 = sum(r["quest_gemm_us"] for r in rows) + 3 * acts[2048]["quant_ms"] * 1000 + acts[5632]["quant_ms"] * 1000
    t_bf16 = sum(r["bf16_us"] for r in rows)
    flops = sum(2.0 * r["m"] * r["n"] * r["k"] for r in rows)
    big = max(rows, key=lambda r: r["m"] * r["n"] * r["k"] / r["quest_gemm_us"])
    return {
        "workload": "the q, k, v, o, gate, up, down products of a 1.6B-scale Llama block at 16384 tokens, "
                    "activations and weights quantised to 4 bits (block 128) vs the same bf16 products",
        "products": rows,
        "block_fp6_us": t_fp6,
        "block_bf16_us": t_bf16,
        "block_speedup": t_bf16 / t_fp6,
        "block_tflops_fp6_incl_quantisation": flops / (t_fp6 * 1e6),
        "roofline": {"bound": "mfma", "kernel": "quest_gemm_e2m3_kernel<bf16>", "product": big["product"],
                     "achieved": round(big["fp6_tflops"], 1), "peak": FP6_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(big["fp6_tflops"] / FP6_PEAK_TFLOPS, 4)},
        "reps": reps,
    }


def qat_linear_step(torch, dev, reps):
    """One training step (forward and backward) of the QuEST linear layer against BF16.

    The q projection of the block (16384 tokens x 2048 by 2048 x 2048), b = 4
    for both operands, block 128, bf16 compute: quest_linear (both operand
    forwards with codes and mask in one grouped launch, the FP6 product; in
    the backward both
    operands rebuilt from their codes in one launch, the two BF16 gradient
    products, and both gradients masked and transformed back in one launch)
    against torch's BF16 linear, each as
    `reps` back-to-back forward + backward passes (torch.autograd.grad, so no
    gradient accumulation) between events on the launch stream, over rotating
    copies of the inputs; three interleaved rounds of the two, medians.
    """
    from quantization_aware_amd.linear import quest_linear
    from quest_inputs import LAYER_ACT_2048, TensorSpec, layer_products, make_tensor

    wt = [w for name, _, w in layer_products() if name == "q"][0]
    x0 = make_tensor(LAYER_ACT_2048, dev)
    w0 = make_tensor(wt, dev)
    dy0 = make_tensor(TensorSpec("bench.qat.dy", x0.shape[0], w0.shape[0], "bf16", "normal", 1e-3, 9900), dev)
    # Copies of x, w and dy (136 MiB a set) rotate, so that more than 512 MiB is
    # touched between two uses of one set and no step finds its inputs in the
    # 256 MB last-level cache.
    sets = 4
    xs = [x0.clone().requires_grad_(True) for _ in range(sets)]
    ws = [w0.clone().requires_grad_(True) for _ in range(sets)]
    dys = [dy0.clone() for _ in range(sets)]
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        for i in range(3):
            fn(i % sets)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(reps):
            fn(i % sets)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def quest(i):
        y = quest_linear(xs[i], ws[i], block=BLOCK, bits_x=4, bits_w=4, compute_dtype=torch.bfloat16)
        torch.autograd.grad(y, (xs[i], ws[i]), dys[i])

    def bf16(i):
        y = torch.nn.functional.linear(xs[i], ws[i])
        torch.autograd.grad(y, (xs[i], ws[i]), dys[i])

    # Interleaved rounds, medians: the two layers see the same clock and power
    # history instead of one always running after the other.
    rounds_q, rounds_b = [], []
    for _ in range(3):
        rounds_q.append(timed(quest))
        rounds_b.append(timed(bf16))
    t_q, t_b = sorted(rounds_q)[1], sorted(rounds_b)[1]
    return {"layer": "q projection", "tokens": x0.shape[0], "in_features": x0.shape[1], "out_features": w0.shape[0],
            "bits": 4, "block": BLOCK, "compute_dtype": "bf16", "quest_step_us": 1000 * t_q,
            "bf16_step_us": 1000 * t_b, "quest_over_bf16": t_q / t_b, "input_sets": sets,
            "rounds_us": {"quest": [round(1000 * t, 1) for t in rounds_q], "bf16": [round(1000 * t, 1) for t in rounds_b]},
            "note": "training step of the QuEST layer (quantisers, FP6 forward product, BF16 gradient products, "
                    "trust backwards) vs a plain BF16 linear layer"}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(
            f"bench.py runs on one GPU: this path shards by rows with no communication, and only the "
            f"single-GPU measurement is made here (asked for --gpus {args.gpus}).",
            file=sys.stderr,
        )
        sys.exit(2)

    import torch

    import quantization_aware_amd as qa
    from quest_inputs import WORKLOADS, make_tensor

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    lib = qa.load_library()
    dev = torch.device("cuda", 0)
    config_names = [] if args.configs.strip().lower() == "none" else [c.strip() for c in args.configs.split(",")]
    unknown = [c for c in config_names if c not in ("C2", "C3", "C4", "C5")]
    if unknown:
        sys.exit(f"unknown --configs {unknown}; the full-size configurations are C2, C3, C4, C5")
    if args.only_configs:
        print(json.dumps({"configs": config_runs(lib, qa, torch, dev, args.product_reps, config_names)}), flush=True)
        return
    wl = WORKLOADS["T"]
    x0 = make_tensor(wl.fwd[0], dev)
    g0 = make_tensor(wl.grad[0], dev)
    xs = [x0] + [x0.clone() for _ in range(N_SETS - 1)]
    gs = [g0] + [g0.clone() for _ in range(N_SETS - 1)]
    codes = [torch.empty((ROWS, COLS * BITS // 8), dtype=torch.uint8, device=dev) for _ in range(N_SETS)]
    scales = [torch.empty((ROWS,), dtype=torch.float32, device=dev) for _ in range(N_SETS)]
    masks = [torch.empty((ROWS, COLS // 8), dtype=torch.uint8, device=dev) for _ in range(N_SETS)]
    dxs = [torch.empty_like(g0) for _ in range(N_SETS)]
    dqs = [torch.empty_like(x0) for _ in range(N_SETS)]  # fake-quantised outputs of the fused forward
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    # Two streams created here with hipStreamCreate (default priority): the
    # null stream would synchronise with the other stream and serialise the
    # two.
    def hip_stream():
        st = ctypes.c_void_p()
        if lib.hipStreamCreate(ctypes.byref(st)):
            raise RuntimeError("hipStreamCreate failed")
        return st

    sh_a = hip_stream()
    sh_b = hip_stream()
    # The timed loop calls the C ABI directly with prepared arguments.
    fwd_args = [
        (ctypes.c_void_p(xs[i].data_ptr()), qa.QUEST_BF16, ROWS, COLS, BLOCK, BITS, ctypes.c_void_p(codes[i].data_ptr()),
         ctypes.c_void_p(scales[i].data_ptr()), ctypes.c_void_p(masks[i].data_ptr()), sh)
        for i in range(N_SETS)
    ]
    bwd_args = [
        (ctypes.c_void_p(gs[i].data_ptr()), qa.QUEST_BF16, ctypes.c_void_p(masks[i].data_ptr()), ROWS, COLS, BLOCK,
         ctypes.c_void_p(dxs[i].data_ptr()), sh)
        for i in range(N_SETS)
    ]
    f_fwd, f_bwd = lib.quest_quantize_fwd, lib.quest_trust_bwd
    # Events of the HIP runtime that libquest (and torch) use, called
    # directly: they bracket the timed region on both streams.
    hip_record = lib.hipEventRecord
    hip_record.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    # Steps are independent batches.  Step i runs on stream i % 2, its
    # backward after its forward in that stream's order; steps on the two
    # streams overlap.  Step i + N_SETS reuses step i's buffers and, N_SETS
    # being even, runs on the same stream after it.
    streams = (sh_a, sh_b)

    def check(name, st):
        if st:
            raise qa.QuestError(name, st, lib.quest_status_string(st).decode())

    def run_steps(first, count):
        for i in range(first, first + count):
            s = i % N_SETS
            st = streams[i % 2]
            check("quest_quantize_fwd", f_fwd(*fwd_args[s][:-1], st))
            check("quest_trust_bwd", f_bwd(*bwd_args[s][:-1], st))

    def step_one_stream(i):
        s = i % N_SETS
        check("quest_quantize_fwd", f_fwd(*fwd_args[s]))
        check("quest_trust_bwd", f_bwd(*bwd_args[s]))

    if args.copy_calibration:
        src = torch.empty((256 << 20) // 2, dtype=torch.bfloat16, device=dev).normal_()
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)  # reads 256 MiB, writes 256 MiB
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: 3 x elementwise neg of {src.numel() * 2} bytes", file=sys.stderr, flush=True)

    run_steps(0, args.warmup)
    torch.cuda.synchronize()

    # Timed region: exactly K steps between two device synchronisations.  A
    # start and an end event on each stream (no stream waits on the other:
    # a cross-stream wait costs microseconds at both ends of a short region);
    # the event time is the span from the earlier start to the later end.
    K = args.steps

    def timing_event():
        e = ctypes.c_void_p()
        if lib.hipEventCreate(ctypes.byref(e)):
            raise RuntimeError("hipEventCreate failed")
        return e

    def elapsed_ms(a, b):
        t = ctypes.c_float()
        if lib.hipEventElapsedTime(ctypes.byref(t), a, b):
            raise RuntimeError("hipEventElapsedTime failed")
        return t.value

    starts = [timing_event() for _ in streams]
    ends = [timing_event() for _ in streams]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e, st in zip(starts, streams):
        hip_record(e, st)
    run_steps(args.warmup, K)
    for e, st in zip(ends, streams):
        hip_record(e, st)
    enqueue = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = max(elapsed_ms(a, b) for a in starts for b in ends)
    ms_per_step = max(step_ms, 1000.0 * wall) / K
    elements = ROWS * COLS
    value = elements / (ms_per_step / 1000.0)

    # The same K steps with forward and backward on one stream, for reference.
    torch.cuda.synchronize()
    e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t2 = time.perf_counter()
    e2.record(stream)
    for i in range(K):
        step_one_stream(i)
    e3.record(stream)
    enqueue_one = time.perf_counter() - t2
    torch.cuda.synchronize()
    one_stream_ms = e2.elapsed_time(e3) / K

    def timed_launches(launch):
        """Mean duration of K back-to-back launches, HIP events on the launch stream."""
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(2):  # first launches load the kernel's code object
            launch(i % N_SETS)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(K):
            launch(i % N_SETS)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / K

    fwd_avg = timed_launches(lambda s_: f_fwd(*fwd_args[s_]))
    bwd_avg = timed_launches(lambda s_: f_bwd(*bwd_args[s_]))
    copy_avg = timed_launches(lambda s_: torch.neg(gs[s_], out=dxs[s_]))
    f_fwd_dq = lib.quest_quantize_fwd_dq
    fwd_dq_args = [
        (ctypes.c_void_p(xs[i].data_ptr()), qa.QUEST_BF16, ROWS, COLS, BLOCK, BITS, None,
         ctypes.c_void_p(scales[i].data_ptr()), ctypes.c_void_p(masks[i].data_ptr()),
         ctypes.c_void_p(dqs[i].data_ptr()), qa.QUEST_BF16, sh)
        for i in range(N_SETS)
    ]
    fwd_dq_avg = timed_launches(lambda s_: check("quest_quantize_fwd_dq", f_fwd_dq(*fwd_dq_args[s_])))
    fwd_dq_bytes = ROWS * COLS * 2 + ROWS * COLS * 2 + ROWS * COLS // 8 + 4 * ROWS
    # The other grids at the same workload: FP4 codes, and 2:4-sparse 4-bit codes with their positions.
    fp4_codes = [torch.empty((ROWS, COLS // 2), dtype=torch.uint8, device=dev) for _ in range(N_SETS)]
    s24_codes = [torch.empty((ROWS, COLS // 4), dtype=torch.uint8, device=dev) for _ in range(N_SETS)]
    s24_index = [torch.empty((ROWS, COLS // 8), dtype=torch.uint8, device=dev) for _ in range(N_SETS)]
    f_fp4, f_s24 = lib.quest_quantize_fwd_fp4, lib.quest_quantize_fwd_sparse24
    fp4_args = [
        (ctypes.c_void_p(xs[i].data_ptr()), qa.QUEST_BF16, ROWS, COLS, BLOCK, 1.0,
         ctypes.c_void_p(fp4_codes[i].data_ptr()), ctypes.c_void_p(scales[i].data_ptr()),
         ctypes.c_void_p(masks[i].data_ptr()), None, qa.QUEST_BF16, sh)
        for i in range(N_SETS)
    ]
    s24_args = [
        (ctypes.c_void_p(xs[i].data_ptr()), qa.QUEST_BF16, ROWS, COLS, BLOCK, 4, 1.0,
         ctypes.c_void_p(s24_codes[i].data_ptr()), ctypes.c_void_p(s24_index[i].data_ptr()),
         ctypes.c_void_p(scales[i].data_ptr()), ctypes.c_void_p(masks[i].data_ptr()), None, qa.QUEST_BF16, sh)
        for i in range(N_SETS)
    ]
    fp4_avg = timed_launches(lambda s_: check("quest_quantize_fwd_fp4", f_fp4(*fp4_args[s_])))
    s24_avg = timed_launches(lambda s_: check("quest_quantize_fwd_sparse24", f_s24(*s24_args[s_])))
    fp4_bytes = ROWS * COLS * 2 + ROWS * COLS // 2 + ROWS * COLS // 8 + 4 * ROWS
    s24_bytes = ROWS * COLS * 2 + ROWS * COLS // 4 + ROWS * COLS // 8 + ROWS * COLS // 8 + 4 * ROWS
    fwd_bytes = alg_bytes_fwd(ROWS, COLS, 2, BITS)
    bwd_bytes = alg_bytes_bwd(ROWS, COLS, 2)
    copy_bytes = 2 * ROWS * COLS * 2
    copy_gbps = copy_bytes / (copy_avg * 1e6)
    kernels = {
        "quest_fwd_mfma_kernel<7,4,6>": {"avg_us": 1000 * fwd_avg, "alg_bytes": fwd_bytes,
                                         "gbps": fwd_bytes / (fwd_avg * 1e6)},
        "quest_bwd_mfma_kernel<7>": {"avg_us": 1000 * bwd_avg, "alg_bytes": bwd_bytes,
                                     "gbps": bwd_bytes / (bwd_avg * 1e6)},
    }
    for v in kernels.values():
        v["frac_of_copy"] = round(v["gbps"] / copy_gbps, 4)
    dom_name = max(kernels, key=lambda k: kernels[k]["avg_us"])
    dom = kernels[dom_name]
    traffic = read_traffic("fwd" if dom_name.startswith("quest_fwd") else "bwd")
    roofline = {
        "bound": "hbm",
        "achieved": round(dom["gbps"], 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(dom["gbps"] / HBM_PEAK_GBPS, 4),
        "traffic": traffic,
        "kernel": dom_name,
        "scope": "the dominant kernel alone, K back-to-back launches; the whole step's fraction is step_frac",
    }
    step_bytes = fwd_bytes + bwd_bytes
    roofline["step_frac"] = round(step_bytes / (ms_per_step * 1e6) / HBM_PEAK_GBPS, 4)
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "16384x2048 bf16 activation (Student-t(4), 20 channels x20) quantised at b=4, block 128, "
            "then trust-masked backward of a 16384x2048 bf16 gradient",
            "rows": ROWS,
            "cols": COLS,
            "block": BLOCK,
            "bits": BITS,
            "input_dtype": "bf16",
            "buffer_sets": N_SETS,
        },
        "roofline": roofline,
        "step_hbm_gbps": step_bytes / (ms_per_step * 1e6),
        "step_roofline_frac": step_bytes / (ms_per_step * 1e6) / HBM_PEAK_GBPS,
        "kernels": kernels,
        "other_kernels": {
            "quest_quantize_fwd_dq (no codes, bf16 dequantised output; fake-quant training forward)": {
                "avg_us": 1000 * fwd_dq_avg, "alg_bytes": fwd_dq_bytes,
                "gbps": fwd_dq_bytes / (fwd_dq_avg * 1e6),
                "frac_of_peak": round(fwd_dq_bytes / (fwd_dq_avg * 1e6) / HBM_PEAK_GBPS, 4),
                "traffic": read_traffic("fwd_dq")},
            "quest_quantize_fwd_fp4 (FP4 codes, mask, scale)": {
                "avg_us": 1000 * fp4_avg, "alg_bytes": fp4_bytes, "gbps": fp4_bytes / (fp4_avg * 1e6),
                "frac_of_peak": round(fp4_bytes / (fp4_avg * 1e6) / HBM_PEAK_GBPS, 4),
                "traffic": read_traffic("fp4")},
            "quest_quantize_fwd_sparse24 (b=4: kept codes, positions, mask, scale)": {
                "avg_us": 1000 * s24_avg, "alg_bytes": s24_bytes, "gbps": s24_bytes / (s24_avg * 1e6),
                "frac_of_peak": round(s24_bytes / (s24_avg * 1e6) / HBM_PEAK_GBPS, 4),
                "traffic": read_traffic("sparse24")},
        },
        "copy_reference": {"kernel": "torch.neg, 16384x2048 bf16", "bytes": copy_bytes, "avg_us": 1000 * copy_avg,
                           "gbps": copy_gbps, "frac_of_peak": round(copy_gbps / HBM_PEAK_GBPS, 4)},
        "timing": {"step_events_ms": step_ms, "step_wall_s": wall,
                   "schedule": "step i on stream i % 2 (forward then backward in stream order); "
                               "consecutive steps overlap; start and end events on both streams",
                   "one_stream_ms_per_step": one_stream_ms,
                   "host_enqueue_s": enqueue, "one_stream_host_enqueue_s": enqueue_one},
    }
    if config_names:
        out["configs"] = config_runs(lib, qa, torch, dev, args.product_reps, config_names)
    if not args.no_block_products:
        out["block_products"] = block_products(lib, qa, torch, dev, args.product_reps)
        out["qat_linear_step"] = qat_linear_step(torch, dev, args.product_reps)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x0, g0, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
