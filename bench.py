#!/usr/bin/env python3
"""Benchmark of the LLM.int8() decomposed int8 matmul on one MI355X.

A step is one forward of the whole per-layer path on one batch of synthetic
input already resident in HBM: outlier-column detection, row-wise
quantisation with the outlier gather, and the int8 MFMA product with the
fused dequantise + fp16 outlier epilogue. Weights are converted once at load
time (timed separately, not part of a step).

Prints ONE JSON line. `value` is the effective throughput 2*s*h*o / t_step
(TOPS) on the largest layer, the 175B-style fused QKV projection prefill
(X [4096, 12288], W [12288, 36864], 7 outlier columns in 75% of rows).
`roofline` is the product kernel on that layer against the MI355X dense int8
MFMA peak; `decode` reports the weight-streaming GB/s of the 175B-style FFN
expansion decode layer (X [8, 12288], W [12288, 49152]) against 8 TB/s HBM;
`all_configs` times every other workload (tiny, the OPT-6.7B-style FFN
prefill and the nine outlier-density sweep points), each with its own CPU
oracle baseline; `cpu_baseline` times the CPU oracle on host cores on a
bounded sample of the headline layer; `clocks` are the GPU clocks and socket
power read from the GPU's metrics table (amdsmi) over a clock window of the same
step (the table is refreshed every few hundred ms).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time


ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective int8-mixed matmul TOPS (prefill) + weight GB/s (decode), % roofline"
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, 5.0 POP/s
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
FP16_PEAK_TFLOPS = 2500.0    # dense fp16 MFMA


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def product_kernel_ms(i8, torch, n, launch):
    """Average duration of the product kernel: n back-to-back launches on the
    launch stream between one pair of HIP events (its inputs are the step's
    intermediates, already in place)."""
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    e0.record()
    for _ in range(n):
        launch()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def settle(torch, fn, window=20, tol=0.01, max_ms=300.0):
    """Untimed back-to-back calls of fn until the GPU runs them at a steady
    rate: windows of `window` calls are timed until two in a row agree
    within `tol` (at most ~max_ms of GPU time). After an idle spell the
    GPU's clocks take a while to come back up (the first ~10 ms of steps
    run ~10 % slower), so this runs before the warm-up steps and the timed
    region measures steady state."""
    prev, spent = None, 0.0
    while spent < max_ms:
        e0, e1 = _events(torch)
        e0.record()
        for _ in range(window):
            fn()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1)
        spent += t
        if prev is not None and abs(t - prev) <= tol * prev:
            break
        prev = t


def timed_ms(torch, n, fn, warmup=3):
    """Average of n back-to-back calls of fn between one pair of HIP events."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def step_percentiles(torch, n, fn):
    """p10 / p50 / p90 of n individually timed calls (an event pair per call)."""
    evs = [_events(torch) for _ in range(n)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    q = lambda f: ts[min(n - 1, int(round(f * (n - 1))))]
    return {"p10": round(q(0.1), 5), "p50": round(q(0.5), 5), "p90": round(q(0.9), 5)}


def table5_set(i8, torch, X, W, Wq, c_w, alpha, n, ws=None):
    """The pages' Table 5 comparison set on one layer (raw matmul time, inputs
    resident): the FP16 GEMM of the vendor library (torch.matmul -> hipBLASLt)
    and the library's own dense fp16 kernel (i8mm_fp16_gemm, weights packed at
    load time), the vendor library's int8 GEMM with int32 output
    (torch._int_mm, for scale: no scales, no outliers),
    the int8 product alone ("Int8 without overhead": the same main loop with an
    int32 store, and the fused product with no outlier columns), vector-wise
    quantisation only (forward at alpha = inf: no decomposition) and the full
    LLM.int8() forward. Speed-ups are FP16 time / variant time."""
    s, h = X.shape
    o = W.shape[1]
    dev = X.device
    if ws is None:
        ws = i8.forward_workspace(s, h, dev)
    v = i8.forward_workspace_views(ws, s, h)
    C = torch.empty((s, o), dtype=torch.float16, device=dev)
    Cf = torch.empty((s, o), dtype=torch.float16, device=dev)
    Ci = torch.empty((s, o), dtype=torch.int32, device=dev)
    t_fp16 = timed_ms(torch, n, lambda: torch.matmul(X, W, out=Cf))
    Wp = i8.pack_fp16_weights(W)          # load time for the library's own fp16 baseline
    t_fp16_own = timed_ms(torch, n, lambda: i8.fp16_gemm(X, Wp, C=Cf))
    del Wp
    t_llm = timed_ms(torch, n, lambda: i8.forward(X, Wq, c_w, W, alpha, workspace=ws, C=C))
    t_vec = timed_ms(torch, n, lambda: i8.forward(X, Wq, c_w, W, float("inf"), workspace=ws, C=C))
    # the forward at alpha = inf left Xq / c_x for the no-outlier product in the workspace
    zero = torch.zeros((1,), dtype=torch.int32, device=dev)
    t_i32 = timed_ms(torch, n, lambda: i8.int8_gemm_i32(v["Xq"], Wq, C=Ci))
    t_fused0 = timed_ms(torch, n, lambda: i8.int8_mixed_matmul(v["Xq"], v["c_x"], v["X_O"], v["idx"], zero,
                                                                Wq, c_w, W, C))
    # for scale: the vendor library's int8 GEMM (torch._int_mm -> hipBLASLt,
    # int32 out) on the same codes, its fast layout (weights [o, h], K-major)
    vendor = {}
    try:
        Wt = i8.panels_to_rows(Wq).contiguous()
        Cv = torch._int_mm(v["Xq"], Wt.t())
        i8.int8_gemm_i32(v["Xq"], Wq, C=Ci)
        torch.cuda.synchronize()
        vendor = {"int8_library_ms": round(timed_ms(torch, n, lambda: torch._int_mm(v["Xq"], Wt.t())), 5),
                  "int8_library_equals_int8_gemm_i32": bool(torch.equal(Cv, Ci))}
        del Wt, Cv
    except Exception as e:   # the op missing or refusing the shape
        vendor = {"int8_library_error": repr(e)[:200]}
    r = lambda t: round(t_fp16 / t, 3)
    return {
        "fp16_library_ms": round(t_fp16, 5),
        "fp16_own_ms": round(t_fp16_own, 5),
        "fp16_own_tflops": round(2.0 * s * h * o / (t_fp16_own * 1e-3) / 1e12, 1),
        "int8_gemm_i32_ms": round(t_i32, 5),
        **vendor,
        "int8_product_no_outliers_ms": round(t_fused0, 5),
        "vectorwise_only_ms": round(t_vec, 5),
        "llm_int8_ms": round(t_llm, 5),
        "speedup_vs_fp16": {"int8_without_overhead": r(min(t_i32, t_fused0)), "vectorwise_only": r(t_vec),
                            "llm_int8": r(t_llm)},
        "speedup_vs_own_fp16": {"int8_without_overhead": round(t_fp16_own / min(t_i32, t_fused0), 3),
                                "vectorwise_only": round(t_fp16_own / t_vec, 3),
                                "llm_int8": round(t_fp16_own / t_llm, 3)},
    }


def run_prefill(i8, torch, w, steps, warmup, dev, clocks=None, extras=True):
    from workloads import make_inputs
    inp = make_inputs(w)
    X = torch.from_numpy(inp["X"]).to(dev)
    W = torch.from_numpy(inp["W"]).to(dev)
    s, h, o = w.s, w.h, w.o
    torch.cuda.synchronize()

    # load-time conversion (timed on its own)
    Wq, c_w = i8.quantize_colwise_weights(W)
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    e0.record()
    for _ in range(3):
        i8.quantize_colwise_weights(W, Wq, c_w)
    e1.record()
    torch.cuda.synchronize()
    conv_ms = e0.elapsed_time(e1) / 3

    ws = i8.forward_workspace(s, h, dev)
    v = i8.forward_workspace_views(ws, s, h)
    C = torch.empty((s, o), dtype=torch.float16, device=dev)

    def step():
        # one forward: detect -> quantise rows -> decomposed product (one C-ABI call)
        i8.forward(X, Wq, c_w, W, w.alpha, workspace=ws, C=C)

    settle(torch, step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = _events(torch)
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = t0.elapsed_time(t1) / steps
    gemm_ms = product_kernel_ms(i8, torch, steps, lambda: i8.int8_mixed_matmul(
        v["Xq"], v["c_x"], v["X_O"], v["idx"], v["n_out"], Wq, c_w, W, C))
    clk = clock_window(torch, step, step_ms, clocks) if clocks is not None else None

    n_out = int(v["n_out"].cpu()[0])
    pct = step_percentiles(torch, steps, step)
    # the same forward with the int8 codes of X made inside the product
    # (i8mm_forward_inline_quant, no Xq round trip), interleaved with the
    # two-pass step, best of three windows each
    inline = two = float("inf")
    for _ in range(3):
        two = min(two, timed_ms(torch, steps, step))
        inline = min(inline, timed_ms(torch, steps, lambda: i8.forward_inline_quant(X, Wq, c_w, W, w.alpha,
                                                                                    workspace=ws, C=C)))
    iq = dict(inline=inline, two=two)
    step()
    if not extras:
        return dict(step_ms=step_ms, gemm_ms=gemm_ms, conv_ms=conv_ms, wall_s=wall, n_out=n_out, inputs=inp,
                    pct=pct, clk=clk, iq=iq)
    table5 = table5_set(i8, torch, X, W, Wq, c_w, w.alpha, steps)
    # MALL-cold steps: rotate over weight copies whose total exceeds the
    # 256 MB Infinity Cache, so every step streams its weights from HBM
    copies = max(2, -(-512 * 2**20 // (3 * h * o)))
    sets = [(Wq, c_w, W)] + [(Wq.clone(), c_w.clone(), W.clone()) for _ in range(copies - 1)]
    it = [0]

    def cold_step():
        a, b, c = sets[it[0] % copies]
        it[0] += 1
        i8.forward(X, a, b, c, w.alpha, workspace=ws, C=C)

    cold_ms = timed_ms(torch, steps, cold_step, warmup=copies)
    del sets
    # without a resident fp16 W (outlier rows rebuilt from the int8 codes),
    # timed the same way as the step with W right beside it
    w8 = variant_ms(i8, torch, steps, X, Wq, c_w, W, w.alpha, ws, C)
    quant = quantiser_variants(i8, torch, steps, X, W, w.alpha, w8["base"])
    # the step's intermediates again for anything that reads them later
    step()
    torch.cuda.synchronize()
    return dict(step_ms=step_ms, gemm_ms=gemm_ms, conv_ms=conv_ms, wall_s=wall, n_out=n_out,
                inputs=inp, pct=pct, table5=table5, cold_ms=cold_ms, copies=copies, w8=w8, quant=quant, clk=clk,
                iq=iq)


def run_decode(i8, torch, w, steps, warmup, dev, extras=True, clocks=None):
    from workloads import make_inputs
    inp = make_inputs(w)
    X = torch.from_numpy(inp["X"]).to(dev)
    W = torch.from_numpy(inp["W"]).to(dev)
    s, h, o = w.s, w.h, w.o
    Wq, c_w = i8.quantize_colwise_weights(W)
    ws = i8.forward_workspace(s, h, dev)
    v = i8.forward_workspace_views(ws, s, h)
    C = torch.empty((s, o), dtype=torch.float16, device=dev)
    settle(torch, lambda: i8.forward(X, Wq, c_w, W, w.alpha, workspace=ws, C=C))
    for _ in range(warmup):
        i8.forward(X, Wq, c_w, W, w.alpha, workspace=ws, C=C)
    torch.cuda.synchronize()
    t0, t1 = _events(torch)
    t0.record()
    for _ in range(steps):
        i8.forward(X, Wq, c_w, W, w.alpha, workspace=ws, C=C)
    t1.record()
    torch.cuda.synchronize()
    step_ms = t0.elapsed_time(t1) / steps
    gemm_ms = product_kernel_ms(i8, torch, steps, lambda: i8.int8_mixed_matmul(
        v["Xq"], v["c_x"], v["X_O"], v["idx"], v["n_out"], Wq, c_w, W, C))
    clk = None
    if clocks is not None:
        clk = clock_window(torch, lambda: i8.forward(X, Wq, c_w, W, w.alpha, workspace=ws, C=C), step_ms, clocks)
    n_out = int(v["n_out"].cpu()[0])
    weight_bytes = h * o + 2 * n_out * o + 4 * o
    # the same forward as one launch (i8mm_forward_decode), interleaved with
    # the three-launch step, best of three windows each
    single = three = float("inf")
    for _ in range(3):
        three = min(three, timed_ms(torch, steps, lambda: i8.forward(X, Wq, c_w, W, w.alpha, workspace=ws, C=C)))
        single = min(single, timed_ms(torch, steps, lambda: i8.forward_decode(X, Wq, c_w, W, w.alpha,
                                                                              workspace=ws, C=C)))
    # batched decode on the same weights: 32 and 48 rows of X drawn with the
    # same recipe (the weight-streaming product with 2 and 3 row groups)
    import dataclasses
    from workloads import make_inputs as _mk
    batched = []
    for sb in (32, 48):
        Xb = torch.from_numpy(_mk(dataclasses.replace(w, name=f"{w.name}_s{sb}", s=sb), with_W=False)["X"]).to(dev)
        wsb = i8.forward_workspace(sb, h, dev)
        Cb = torch.empty((sb, o), dtype=torch.float16, device=dev)
        tb = timed_ms(torch, steps, lambda: i8.forward(Xb, Wq, c_w, W, w.alpha, workspace=wsb, C=Cb))
        batched.append({"s": sb, "ms_per_step": round(tb, 5),
                        "weight_GB_per_s": round((h * o + 4 * o) / (tb * 1e-3) / 1e9, 1)})
        del Xb, wsb, Cb
    if not extras:
        return dict(step_ms=step_ms, gemm_ms=gemm_ms, n_out=n_out, weight_bytes=weight_bytes, inputs=inp,
                    single=single, three=three, clk=clk, batched=batched)
    w8 = variant_ms(i8, torch, steps, X, Wq, c_w, W, w.alpha, ws, C)
    del Wq, c_w
    quant = quantiser_variants(i8, torch, steps, X, W, w.alpha, w8["base"])
    return dict(step_ms=step_ms, gemm_ms=gemm_ms, n_out=n_out, weight_bytes=weight_bytes, w8=w8, quant=quant,
                inputs=inp, single=single, three=three, clk=clk, batched=batched)


def quantiser_variants(i8, torch, steps, X, W, alpha, fused_ms):
    """Table 1's quantiser schemes on the same layer ([DIGEST] "Quantization
    Primitives", "Vector-wise Quantization"): one forward of each, as the
    sequence of C-ABI calls variant_forward makes (detection, the scheme's
    row quantiser, its product; weights converted beforehand) and as the
    scheme's one-call forward, average ms of `steps` back-to-back forwards,
    with the bench's own vector-wise step for reference."""
    out = {}
    s, h = X.shape
    ws = i8.forward_workspace(s, h, X.device, zeropoint=True)
    C = torch.empty((s, W.shape[1]), dtype=torch.float16, device=X.device)
    one_call = {}
    for scheme in i8.SCHEMES:
        qw = i8.quantize_weights(W, scheme)
        out[scheme + "_ms"] = round(timed_ms(torch, steps, lambda: i8.variant_forward(X, qw, W, scheme, alpha)), 5)
        # the same scheme through its one-call forward (row- and vector-wise
        # share i8mm_forward; they differ in the weights' constants)
        if scheme == "tensor":
            fn = lambda: i8.forward_tensorwise(X, qw[0], qw[1], W, alpha, workspace=ws, C=C)
        elif scheme == "zeropoint":
            fn = lambda: i8.forward_zeropoint(X, qw, W, alpha, workspace=ws, C=C)
        else:
            fn = lambda: i8.forward(X, qw[0], qw[1], W, alpha, workspace=ws, C=C)
        one_call[scheme + "_ms"] = round(timed_ms(torch, steps, fn), 5)
        del qw
    out["one_call"] = one_call
    out["vector_fused_forward_ms"] = round(fused_ms, 5)
    out["zeropoint_vs_vector"] = round(out["zeropoint_ms"] / out["vector_ms"], 3)
    out["one_call_zeropoint_vs_vector"] = round(one_call["zeropoint_ms"] / one_call["vector_ms"], 3)
    return out


def variant_ms(i8, torch, steps, X, Wq, c_w, W, alpha, ws, C):
    """Step variants timed the same way one after the other (each the average
    of `steps` back-to-back forwards): the plain step, the step without a
    resident fp16 W, and the step with an fp16 layer bias."""
    o = Wq.shape[1]
    bias = (torch.arange(o, device=X.device, dtype=torch.float32) % 7 - 3).to(torch.float16) * 0.125
    fns = {"base": lambda: i8.forward(X, Wq, c_w, W, alpha, workspace=ws, C=C),
           "no_w": lambda: i8.forward(X, Wq, c_w, None, alpha, workspace=ws, C=C),
           "bias": lambda: i8.forward(X, Wq, c_w, W, alpha, workspace=ws, C=C, bias=bias)}
    # three interleaved rounds, the best of each variant
    best = {k: float("inf") for k in fns}
    for _ in range(3):
        for k, fn in fns.items():
            best[k] = min(best[k], timed_ms(torch, steps, fn))
    return best


# The pages' Table 5 (raw matmul of the first FFN layer of GPT-3 models, X [s, d]
# times W [d, 4d], speed-up over FP16): widths and their printed ratios.
TABLE5_WIDTHS = [768, 2560, 4096, 5120, 12288]
TABLE5_PAGES = {"llm_int8": {"768": 0.14, "2560": 0.64, "4096": 0.86, "5120": 1.22, "12288": 1.81},
                "vectorwise_only": {"5120": 1.59, "12288": 2.00},
                "int8_without_overhead": {"768": 0.99, "12288": 2.29}}


def run_table5(i8, torch, dev, s, n):
    """The Table 5 comparison set at each width on inputs drawn on the GPU from
    a seeded generator: X ~ N(0,1) clipped to |x| < 5.5 with 6 (7 at 12288)
    one-sided outlier columns of magnitude U(6, 20) in 75 % of the rows,
    W ~ 0.02 N(0,1). (The pages give 5140 for the 13B width; 5120 is used, as
    the library takes widths that are multiples of 64.)"""
    rows = []
    for d in TABLE5_WIDTHS:
        g = torch.Generator(device=dev)
        g.manual_seed(d)
        o = 4 * d
        X = torch.randn((s, d), generator=g, device=dev).clamp_(-5.49, 5.49)
        n_out = 7 if d >= 12288 else 6
        cols = torch.randperm(d, generator=g, device=dev)[:n_out]
        for c in cols.tolist():
            sel = torch.randperm(s, generator=g, device=dev)[: round(0.75 * s)]
            sign = 1.0 if torch.rand((), generator=g, device=dev).item() < 0.5 else -1.0
            X[sel, c] = sign * (6.0 + 14.0 * torch.rand((sel.numel(),), generator=g, device=dev))
        X = X.half()
        W = (0.02 * torch.randn((d, o), generator=g, device=dev)).half()
        Wq, c_w = i8.quantize_colwise_weights(W)
        res = table5_set(i8, torch, X, W, Wq, c_w, 6.0, n)
        res.update({"d": d, "s": s, "o": o, "planted_outliers": n_out})
        rows.append(res)
        _log(f"[table5] d={d}: {res['speedup_vs_fp16']}")
        del X, W, Wq, c_w
        torch.cuda.empty_cache()
    return rows


def config_row(w, n_out, step_ms, gemm_ms):
    """One workload's step and product-kernel figures in the metric's units:
    effective TOPS (2 s h o / step) for prefill shapes, weight bytes per
    second for the weight-streaming one."""
    s, h, o = w.s, w.h, w.o
    row = {"workload": w.name, "s": s, "h": h, "o": o, "n_outliers": n_out, "outlier_row_frac": w.row_frac,
           "step_ms": round(step_ms, 5), "product_kernel_ms": round(gemm_ms, 5)}
    if w.decode:
        wb = h * o + 2 * n_out * o + 4 * o
        row["weight_GB_per_s"] = round(wb / (step_ms * 1e-3) / 1e9, 1)
        row["pct_hbm_peak"] = round(100 * wb / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)
        row["product_kernel_weight_GB_per_s"] = round(wb / (gemm_ms * 1e-3) / 1e9, 1)
    else:
        tops = 2.0 * s * h * o / (step_ms * 1e-3) / 1e12
        gemm_tops = 2.0 * s * (h - n_out) * o / (gemm_ms * 1e-3) / 1e12
        row["effective_TOPS"] = round(tops, 1)
        row["pct_int8_peak"] = round(100 * tops / INT8_PEAK_TOPS, 2)
        row["product_kernel_TOPS"] = round(gemm_tops, 1)
        row["product_kernel_pct_peak"] = round(100 * gemm_tops / INT8_PEAK_TOPS, 2)
    return row


def run_all_configs(i8, torch, dev, steps, names, host=None, cpu_budget=0.0):
    """The one-call forward step and the product kernel alone on each named
    configuration's seeded inputs (the parity tests' inputs), weights
    converted beforehand, each with a CPU oracle baseline on a bounded
    sample when cpu_budget > 0. The next configuration's inputs are drawn in
    a background thread while the current one is timed, except beside the
    small layers, whose timing is bound by the host's launch rate."""
    from concurrent.futures import ThreadPoolExecutor
    from workloads import get_config, make_inputs
    rows = []
    with ThreadPoolExecutor(1) as pool:
        pending = pool.submit(make_inputs, get_config(names[0])) if names else None
        for k, name in enumerate(names):
            w = get_config(name)
            inp = pending.result()
            pending = pool.submit(make_inputs, get_config(names[k + 1])) if k + 1 < len(names) else None
            X = torch.from_numpy(inp["X"]).to(dev)
            W = torch.from_numpy(inp["W"]).to(dev)
            s, h, o = w.s, w.h, w.o
            if pending is not None and 2 * s * h * o < (1 << 34):
                pending.result()   # launch-bound: no input generation beside its timing
            Wq, c_w = i8.quantize_colwise_weights(W)
            ws = i8.forward_workspace(s, h, dev)
            v = i8.forward_workspace_views(ws, s, h)
            C = torch.empty((s, o), dtype=torch.float16, device=dev)

            def step():
                i8.forward(X, Wq, c_w, W, w.alpha, workspace=ws, C=C)

            settle(torch, step)
            step_ms = timed_ms(torch, steps, step)
            gemm_ms = product_kernel_ms(i8, torch, steps, lambda: i8.int8_mixed_matmul(
                v["Xq"], v["c_x"], v["X_O"], v["idx"], v["n_out"], Wq, c_w, W, C))
            row = config_row(w, int(v["n_out"].cpu()[0]), step_ms, gemm_ms)
            del X, W, Wq, c_w, ws, v, C
            torch.cuda.empty_cache()
            if cpu_budget > 0:
                row["cpu_baseline"] = cpu_baseline(w, inp, cpu_budget, host, rows=512)
            _log(f"[configs] {row}")
            rows.append(row)
            del inp
    return rows


def host_info():
    """The host the CPU baseline runs on: the cores this process may use,
    the CPU model, and numpy's BLAS (vendor, version, threads)."""
    import numpy as np  # noqa: F401  (loads the BLAS so that threadpoolctl sees it)
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", int(os.environ.get("OMP_NUM_THREADS", "1"))
    try:
        from threadpoolctl import threadpool_info
        libs = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        if libs:
            d = libs[0]
            blas = f"{d.get('internal_api')} {d.get('version')} ({d.get('threading_layer')}, {d.get('architecture')})"
            threads = max(int(x.get("num_threads", 1)) for x in libs)
    except Exception:  # threadpoolctl missing or unreadable
        pass
    return {"affinity_cores": affinity, "cpu_model": model, "blas": blas, "blas_threads": threads}


def _sample_work(w, rows, cols, n_out):
    """The metric's amount of work in an oracle sample of rows x cols."""
    if w.decode:
        return (w.h * cols + 2 * n_out * cols + 4 * cols) / 1e9, "GB/s"   # weight bytes
    return 2.0 * rows * w.h * cols / 1e12, "TOPS"


def cpu_baseline(w, inputs, budget_s, host, rows=None, reps=3):
    """Time the CPU oracle (as it stands) on a bounded sample of one workload.

    The sample is the first R rows of X (all rows, or `rows`) against the
    first Q = min(o, 2048) columns of W (columns are independent: each
    output column needs only its own weight column and constant); their
    load-time weight conversion is done first and not timed. One untimed
    warm-up forward, then at least `reps` timed repetitions of
    oracle.forward, more while they fit in budget_s. A fixed sample per
    workload keeps the oracle's per-call costs (weight-side conversions
    that do not depend on R) the same share of every figure. The result is
    scaled to the metric's unit: effective TOPS 2 R h Q / t (prefill), or
    weight bytes (h Q + 2 |O| Q + 4 Q) / t in GB/s (decode).
    """
    import oracle
    X, W = inputs["X"], inputs["W"]
    n_out = int(oracle.outlier_columns(X, w.alpha)[2])
    cols = min(w.o, 2048)
    rows = min(w.s, rows or w.s)
    Wq_t, c_w = oracle.quantize_colwise_weights(W[:, :cols])     # load time, not timed
    Xs, Ws = X[:rows], W[:, :cols]
    t = time.perf_counter()
    oracle.forward(Xs, Ws, w.alpha, Wq_t=Wq_t, c_w=c_w)              # warm-up
    warm = max(time.perf_counter() - t, 1e-6)
    reps = max(reps, int(budget_s / warm))
    t = time.perf_counter()
    for _ in range(reps):
        oracle.forward(Xs, Ws, w.alpha, Wq_t=Wq_t, c_w=c_w)
    el = time.perf_counter() - t
    work, unit = _sample_work(w, rows, cols, n_out)
    return {
        "value": round(work * reps / el, 6),
        "unit": unit,
        "cores": host["blas_threads"],
        "kind": "oracle",
        "sample": (f"oracle.forward on the first {rows} of {w.s} rows of X and the first {cols} of {w.o} "
                   f"columns of W [{w.h}x{w.o}] (weights converted beforehand), 1 warm-up + {reps} timed "
                   f"rep(s) in {el:.2f} s; numpy BLAS ({host['blas']}) with {host['blas_threads']} "
                   f"thread(s) for the products, elementwise steps on one thread"),
        "affinity_cores": host["affinity_cores"],
        "cpu_model": host["cpu_model"],
    }


class ClockSampler:
    """Samples the GPU's graphics clock (per XCD), memory clock and socket
    power from the GPU's metrics table (amdsmi) in a background thread.
    The table is refreshed by the power-management firmware only every few
    hundred ms, so the sampler is run over a clock window of >= 1 s of the
    same step back to back, and the distinct snapshots are reported.
    Reading the table touches no GPU queue."""

    def __init__(self, torch, period_s=0.01):
        self.period = period_s
        self.samples = []
        self.error = None
        self.handle = None
        self._amdsmi = None
        try:
            import amdsmi
            amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
            handles = amdsmi.amdsmi_get_processor_handles()
            self.handle = handles[0] if handles else None
            try:   # the handle of the GPU torch uses, by PCI bus
                want = int(getattr(torch.cuda.get_device_properties(0), "pci_bus_id"))
                for hd in handles:
                    if int(amdsmi.amdsmi_get_gpu_device_bdf(hd).split(":")[1], 16) == want:
                        self.handle = hd
                        break
            except Exception:
                pass
            self._amdsmi = amdsmi
            if self.handle is None:
                self.error = "no GPU handle"
        except Exception as e:  # amdsmi missing or the metrics table unreadable
            self.error = repr(e)

    def read(self):
        m = self._amdsmi.amdsmi_get_gpu_metrics_info(self.handle)

        def nums(v):
            vals = v if isinstance(v, (list, tuple)) else [v]
            return [float(x) for x in vals if isinstance(x, (int, float)) and 0 < x < 0xFFFF]

        gfx = nums(m.get("current_gfxclks", [])) or nums(m.get("current_gfxclk"))
        return (tuple(gfx), (nums(m.get("current_uclk")) or [None])[0],
                (nums(m.get("current_socket_power")) or [None])[0])

    def __enter__(self):
        import threading
        self._stop = threading.Event()
        self._thread = None
        if self.error is None:
            def loop():
                while not self._stop.is_set():
                    try:
                        self.samples.append(self.read())
                    except Exception as e:
                        self.error = repr(e)
                        return
                    self._stop.wait(self.period)
            self._thread = threading.Thread(target=loop, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
        return False

    def summary(self, window_s=None, steps=None):
        if self.error is not None and not self.samples:
            return {"error": self.error}
        # the table holds each snapshot for a while: keep the distinct ones,
        # and drop the first (it may predate the window) and idle ones
        snaps = []
        for smp in self.samples:
            if not snaps or smp != snaps[-1]:
                snaps.append(smp)
        if len(snaps) > 1:
            snaps = snaps[1:]
        busy = [x for x in snaps if x[0] and sum(x[0]) / len(x[0]) > 500.0] or snaps

        def med(vals):
            vals = sorted(v for v in vals if v is not None)
            return vals[len(vals) // 2] if vals else None

        return {"sclk_MHz_median": med(sum(x[0]) / len(x[0]) for x in busy if x[0]),
                "sclk_MHz_per_xcd_last": list(busy[-1][0]) if busy and busy[-1][0] else None,
                "mclk_MHz_median": med(x[1] for x in busy),
                "socket_power_W_median": med(x[2] for x in busy),
                "snapshots": len(busy), "polls": len(self.samples),
                "window_s": window_s, "window_steps": steps,
                "source": "amdsmi gpu_metrics current_gfxclks / current_uclk / current_socket_power, polled every "
                          f"{self.period * 1e3:.0f} ms over a window of the same step run back to back right after "
                          "the timed steps (the firmware refreshes the table every few hundred ms, longer than the "
                          "timed steps)"}


def clock_window(torch, fn, step_ms, clocks, seconds=1.5):
    """Runs fn back to back for about `seconds` under the clock sampler."""
    n = max(50, int(seconds * 1e3 / max(step_ms, 1e-3)))
    clocks.samples.clear()   # a window of its own
    with clocks:
        t0 = time.perf_counter()
        done = 0
        while done < n:
            k = min(200, n - done)
            for _ in range(k):
                fn()
            torch.cuda.synchronize()
            done += k
        el = time.perf_counter() - t0
    return clocks.summary(round(el, 3), n)


def mfma_stream_ceiling(i8, torch, dev, clocks, seconds=3.0):
    """The int8 matrix-core rate the chip sustains under load: one block of
    four wavefronts per compute unit issuing v_mfma_i32_32x32x32_i8 back to
    back on register-resident random codes (i8mm_calib_mfma_i8), timed with
    HIP events, then run back to back for a clock window. The published
    peak assumes the 2.4 GHz clock; this is what the clock and power limits
    leave of it, the practical ceiling for the prefill product."""
    blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 40000
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    codes = torch.randint(-127, 128, (blocks * 65536,), generator=g, dtype=torch.int8, device=dev)
    out = torch.empty((blocks * 256,), dtype=torch.int32, device=dev)
    fn = lambda: i8.calib_mfma_i8(codes, iters, out)
    ops = fn()
    torch.cuda.synchronize()
    ms = timed_ms(torch, 4, fn, warmup=1)
    clk = clock_window(torch, fn, ms, clocks, seconds) if clocks is not None else None
    tops = ops / (ms * 1e-3) / 1e12
    return {"kernel": "k_calib_mfma_i8", "blocks": blocks, "mfma_per_wavefront": 32 * iters,
            "ms_per_launch": round(ms, 4), "TOP/s": round(tops, 1), "frac_of_peak": round(tops / INT8_PEAK_TOPS, 4),
            "clocks": clk}


CONFIG_NAMES = ["tiny", "opt67b_ffn1_prefill", "sweep_o0"] + \
    [f"sweep_o{n}_r{r}" for n in (7, 64) for r in (6, 28, 75, 100)]


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="b175_qkv_prefill")
    ap.add_argument("--decode-workload", default="b175_ffn1_decode")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="headline step and product kernel only: no Table 5 set, weight-copy rotation, "
                         "storage, bias or quantiser variants")
    ap.add_argument("--no-all-configs", action="store_true", help="skip the per-configuration rows")
    ap.add_argument("--config-steps", type=int, default=30, help="timed steps per configuration row")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of timed oracle work for the headline cpu_baseline")
    ap.add_argument("--config-cpu-budget", type=float, default=1.5,
                    help="seconds of timed oracle work for each configuration's cpu_baseline")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM traffic of the product kernel measured with rocprofv3 counters")
    ap.add_argument("--table5", action="store_true",
                    help="only run the pages' Table 5 comparison set over the GPT-3 FFN widths "
                         "and print it as one JSON line")
    ap.add_argument("--table5-rows", type=int, default=2048, help="rows of X (tokens) for --table5")
    ap.add_argument("--all-configs", action="store_true",
                    help="only time the one-call forward and the product kernel on every configuration "
                         "(no CPU baselines) and print one JSON line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB",
                    help="only run a plain device copy of this many MiB (5 times) and exit; its "
                         "FETCH_SIZE/WRITE_SIZE counters calibrate the HBM traffic figures")
    ap.add_argument("--calibration", action="store_true",
                    help="only run the sustained int8 MFMA stream (the prefill product's practical ceiling) "
                         "and print it as one JSON line")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(no sharding, no collectives). Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import int8_quantized_matmul_amd as i8
    from workloads import CONFIGS, get_config

    dev = torch.device("cuda:0")
    if args.calibration:
        print(json.dumps({"sustained_mfma_stream": mfma_stream_ceiling(i8, torch, dev, ClockSampler(torch)),
                          "peak_TOPS": INT8_PEAK_TOPS}), flush=True)
        return 0
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.bitwise_not(src, out=dst)   # elementwise: reads n bytes, writes n bytes
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 5}), flush=True)
        return 0
    if args.table5:
        rows = run_table5(i8, torch, dev, args.table5_rows, args.steps)
        print(json.dumps({"table5": rows, "pages_table5": TABLE5_PAGES,
                          "note": "raw matmul of X [s, d] x W [d, 4d], inputs resident; "
                                  "speed-up = FP16 library GEMM time / variant time"}), flush=True)
        return 0
    if args.all_configs:
        print(json.dumps({"all_configs": run_all_configs(i8, torch, dev, args.steps, list(CONFIGS)),
                          "note": "one-call forward step (detect + quantise + product) and the product "
                                  "kernel alone, weights converted beforehand, inputs resident"}), flush=True)
        return 0
    host = host_info()
    w = get_config(args.workload)
    _log(f"[bench] prefill workload {w.name}: s={w.s} h={w.h} o={w.o}")
    clocks = ClockSampler(torch)
    pre = run_prefill(i8, torch, w, args.steps, args.warmup, dev, clocks=clocks, extras=not args.no_extras)
    s, h, o, n_out = w.s, w.h, w.o, pre["n_out"]
    tops = 2.0 * s * h * o / (pre["step_ms"] * 1e-3) / 1e12
    alg_ops = 2.0 * s * (h - n_out) * o                  # int8 ops one product launch performs
    gemm_tops = alg_ops / (pre["gemm_ms"] * 1e-3) / 1e12

    traffic = None
    if os.path.exists(args.traffic):
        try:
            with open(args.traffic) as f:
                tr = json.load(f)
            if tr.get("workload") == w.name and tr.get("kernel_source_sha") == _kernel_sha():
                traffic = tr.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None

    out = {
        "metric": METRIC,
        "value": round(tops, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": w.name, "s": s, "h": h, "o": o, "n_outliers": n_out,
                   "outlier_row_frac": w.row_frac, "alpha": w.alpha, "parallelism": "none"},
        "roofline": {
            "bound": "mfma",
            "kernel": "k_gemm_prefill (int8 MFMA + fused dequant/outlier epilogue)",
            "achieved": round(gemm_tops, 3),
            "peak": INT8_PEAK_TOPS,
            "unit": "TOP/s",
            "frac": round(gemm_tops / INT8_PEAK_TOPS, 4),
            "traffic": traffic,
            "algorithmic_ops_per_launch": alg_ops,
            "avg_launch_ms": round(pre["gemm_ms"], 5),
        },
        "pct_int8_peak_effective": round(100 * tops / INT8_PEAK_TOPS, 2),
        "prologue_ms": round(pre["step_ms"] - pre["gemm_ms"], 5),
        "step_ms_percentiles": pre["pct"],
        "clocks": pre["clk"],
        "inline_quant": {"ms_per_step": round(pre["iq"]["inline"], 5),
                         "two_pass_ms_per_step": round(pre["iq"]["two"], 5),
                         "vs_two_pass": round(pre["iq"]["inline"] / pre["iq"]["two"], 3)},
        "weight_conversion": {"ms": round(pre["conv_ms"], 4),
                              "GB_per_s_3ho": round(3.0 * h * o / (pre["conv_ms"] * 1e-3) / 1e9, 1),
                              "GB_per_s_5ho_moved": round(5.0 * h * o / (pre["conv_ms"] * 1e-3) / 1e9, 1),
                              "pct_hbm_peak_5ho": round(100 * 5.0 * h * o / (pre["conv_ms"] * 1e-3) / 1e9
                                                        / HBM_PEAK_GBS, 2)},
    }
    if not args.no_extras:
        _log("[bench] sustained int8 MFMA stream (practical ceiling)")
        ceil = mfma_stream_ceiling(i8, torch, dev, clocks)
        ceil["product_kernel_over_stream"] = round(gemm_tops / ceil["TOP/s"], 4)
        out["roofline"]["sustained_mfma_stream"] = ceil
        out.update({
            "step_ms_weights_from_hbm": {"ms": round(pre["cold_ms"], 5), "weight_copies_rotated": pre["copies"]},
            "table5_comparison": pre["table5"],
            "without_fp16_weights": _w8_entry(pre["w8"], h, o),
            "with_bias": _bias_entry(pre["w8"]),
            "quantiser_variants": pre["quant"],
        })
    inputs = pre.pop("inputs")
    rows = [config_row(w, n_out, pre["step_ms"], pre["gemm_ms"])]
    if not args.no_cpu_baseline:
        _log("[bench] timing the CPU oracle (headline)")
        out["cpu_baseline"] = cpu_baseline(w, inputs, args.cpu_budget, host)
        rows[0]["cpu_baseline"] = out["cpu_baseline"]
    del inputs

    if not args.no_decode:
        wd = get_config(args.decode_workload)
        _log(f"[bench] decode workload {wd.name}: s={wd.s} h={wd.h} o={wd.o}")
        dec = run_decode(i8, torch, wd, args.steps, args.warmup, dev, extras=not args.no_extras, clocks=clocks)
        gbs = dec["weight_bytes"] / (dec["step_ms"] * 1e-3) / 1e9
        gbs_gemm = dec["weight_bytes"] / (dec["gemm_ms"] * 1e-3) / 1e9
        out["decode"] = {
            "workload": wd.name, "s": wd.s, "h": wd.h, "o": wd.o, "n_outliers": dec["n_out"],
            "ms_per_step": round(dec["step_ms"], 5),
            "weight_GB_per_s": round(gbs, 1),
            "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "product_kernel_ms": round(dec["gemm_ms"], 5),
            "product_kernel_weight_GB_per_s": round(gbs_gemm, 1),
            "prologue_ms": round(dec["step_ms"] - dec["gemm_ms"], 5),
            "clocks": dec["clk"],
            "single_launch": {"ms_per_step": round(dec["single"], 5), "three_launch_ms_per_step": round(dec["three"], 5),
                              "vs_three_launch": round(dec["single"] / dec["three"], 3)},
            "batched": dec["batched"],
        }
        if not args.no_extras:
            out["decode"].update({
                "without_fp16_weights": _w8_entry(dec["w8"], wd.h, wd.o),
                "with_bias": _bias_entry(dec["w8"]),
                "quantiser_variants": dec["quant"],
            })
        drow = config_row(wd, dec["n_out"], dec["step_ms"], dec["gemm_ms"])
        if not args.no_cpu_baseline:
            _log("[bench] timing the CPU oracle (decode)")
            out["decode"]["cpu_baseline"] = cpu_baseline(wd, dec.pop("inputs"), args.config_cpu_budget * 2, host)
            drow["cpu_baseline"] = out["decode"]["cpu_baseline"]
        dec.pop("inputs", None)
        rows.append(drow)
        del dec
        torch.cuda.empty_cache()

    if not args.no_all_configs:
        _log("[bench] every other configuration")
        rows += run_all_configs(i8, torch, dev, args.config_steps, CONFIG_NAMES, host,
                                0.0 if args.no_cpu_baseline else args.config_cpu_budget)
        out["all_configs"] = rows
    out["host"] = host
    print(json.dumps(out), flush=True)
    return 0


def _bias_entry(v):
    """The step with an fp16 layer bias added in the product's epilogue."""
    return {"ms_per_step": round(v["bias"], 5), "vs_without_bias": round(v["bias"] / v["base"], 3)}


def _w8_entry(v, h, o):
    """The step with no resident fp16 W (outlier rows rebuilt from Wq / c_w)
    next to the step with it, and the weight bytes each storage keeps resident."""
    with_w, ms = v["base"], v["no_w"]
    return {"ms_per_step": round(ms, 5), "ms_per_step_with_fp16_W": round(with_w, 5),
            "vs_with_fp16_weights": round(ms / with_w, 3),
            "resident_weight_bytes": h * o + 4 * o,
            "resident_weight_bytes_with_fp16_W": 3 * h * o + 4 * o,
            "memory_reduction_vs_fp16_weights": round(2 * h * o / (h * o + 4 * o), 3)}


def _kernel_sha():
    import hashlib
    hsh = hashlib.sha256()
    src = os.path.join(ROOT, "int8_quantized_matmul_amd", "csrc", "gemm_kernels.hip")
    with open(src, "rb") as f:
        hsh.update(f.read())
    return hsh.hexdigest()[:16]


if __name__ == "__main__":
    sys.exit(main())
