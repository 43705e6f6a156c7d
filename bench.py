#!/usr/bin/env python3
"""Benchmark of the importance-weighted row quantizer on one MI355X.

Headline workload: Q4_K quantization of an 11008 x 4096 fp32 FFN weight matrix
(x = s_r * 0.015*N(0,1), per-row scale s_r ~ LogNormal(0, 0.3), per-column
importance LogNormal(0, 1.5); synthetic, seeded). One step = one call of
qr_quantize_rows over the whole matrix: load, row statistic, importances,
trial scales, least squares, flips, super-block scales, packing.

Protocol: W untimed warm-up steps, then K timed steps. Before every step a
1 GiB buffer is read (outside the timed interval) so that neither L2 nor the
256 MB Infinity Cache holds the input. It is read rather than written so
that no dirty lines of the flush buffer are left to be written back to HBM
inside the timed interval (a written flush slows streaming kernels by up to
a third that way). Each step is bracketed by HIP
events recorded on the stream the kernel is launched on; ms_per_step is
their mean. The whole loop is bracketed by torch.cuda.synchronize().

Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz: VALU lane-operations per second
# (packed fp32 instructions are not used, so one instruction = one op/lane)
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# Operations of the method per Q4_K weight (3 trial scales, 1 flip pass),
# counted from the oracle's loops: row statistic 2, importance + zero test 4,
# range 2, w*x etc. 4, trials 24, block solves 2.5, winner codes 4, flip
# setup 2, flip pass 19, refit sums 2, Q4_K re-round and scales 5.5.
ALG_OPS_PER_WEIGHT_Q4K = 71.0
# MI355X dense int8 matrix-core peak (no sparsity), Tera-ops per second
INT8_PEAK_TOPS = 5000.0
METRIC = "Gweights/s quantized (Q4_0, Q4_K) + achieved HBM GB/s fraction"
COUNTERS = os.path.join(ROOT, "profiles", "q4_k_11008x4096_counters.json")
KERNEL_SRC = os.path.join(ROOT, "post_weight_quantization_row_amd", "csrc", "qrow.hip")


def measured_traffic():
    """HBM bytes per launch of the Q4_K kernel from the committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    import hashlib
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
        with open(KERNEL_SRC, "rb") as f:
            h = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha256") != h:
        return None
    return int(c["hbm_bytes_per_launch"])


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def evict(flush):
    """Reads the whole flush buffer (1 GiB), evicting L2 and Infinity Cache."""
    import torch
    torch.sum(flush[0], dim=0, out=flush[1])


def timed_steps(fn, steps, warmup, flush):
    import torch
    for _ in range(warmup):
        evict(flush)
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        evict(flush)
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return sum(ms) / len(ms), min(ms), wall


def _setup(name, dev):
    """Returns (step function, algorithmic bytes per launch, elements)."""
    import numpy as np
    import torch
    from post_weight_quantization_row_amd import qrow, synth
    if name == "q4_k_11008x4096":
        x, q = synth.torch_q4_k_matrix(dev)
        out = torch.empty((11008, qrow.qr_row_bytes("q4_k", 4096)), dtype=torch.uint8, device=dev)
        return (lambda: qrow.qr_quantize_rows("q4_k", x, q, out=out),
                x.numel() * 4 + q.numel() * 4 + out.numel(), x.numel())
    if name in ("q6_k_11008x4096", "q5_k_11008x4096"):
        # the same matrix in the 6-bit or 5-bit K-quant
        t = name[:4]
        x, q = synth.torch_q4_k_matrix(dev)
        out = torch.empty((11008, qrow.qr_row_bytes(t, 4096)), dtype=torch.uint8, device=dev)
        return (lambda: qrow.qr_quantize_rows(t, x, q, out=out),
                x.numel() * 4 + q.numel() * 4 + out.numel(), x.numel())
    if name == "q4_k_fit_11008x4096":
        # the same matrix with the weighted fit of the 6-bit sub-scales
        x, q = synth.torch_q4_k_matrix(dev)
        out = torch.empty((11008, qrow.qr_row_bytes("q4_k", 4096)), dtype=torch.uint8, device=dev)
        return (lambda: qrow.qr_quantize_rows_ex("q4_k", x, q, subscale_fit="weighted", out=out),
                x.numel() * 4 + q.numel() * 4 + out.numel(), x.numel())
    if name == "q4_0_2048x2048":
        x, q = synth.q4_0_matrix()
        xd, qd = torch.from_numpy(x).to(dev), torch.from_numpy(q).to(dev)
        out = torch.empty((2048, qrow.qr_row_bytes("q4_0", 2048)), dtype=torch.uint8, device=dev)
        return (lambda: qrow.qr_quantize_rows("q4_0", xd, qd, out=out),
                x.nbytes + q.nbytes + out.numel(), x.size)
    if name == "q8_k128_8192x7168":
        x, _ = synth.q8_k128_activations()
        xd = torch.from_numpy(x).to(dev)
        out = torch.empty((8192, qrow.qr_row_bytes("q8_k128", 7168)), dtype=torch.uint8, device=dev)
        return (lambda: qrow.qr_quantize_activations_q8k128(xd, out=out),
                x.nbytes + out.numel(), x.size)
    if name in ("q8_k64_8192x7168", "q8_k16_8192x7168"):
        act = name.split("_8192")[0]
        x, _ = synth.q8_k128_activations()
        xd = torch.from_numpy(x).to(dev)
        out = torch.empty((8192, qrow.qr_row_bytes(act, 7168)), dtype=torch.uint8, device=dev)
        return (lambda: qrow.qr_quantize_activations_q8k(act, xd, out=out),
                x.nbytes + out.numel(), x.size)
    if name == "dequantize_q4_k_11008x4096":
        x, q = synth.torch_q4_k_matrix(dev)
        packed = qrow.qr_quantize_rows("q4_k", x, q)
        y = torch.empty_like(x)
        return (lambda: qrow.qr_dequantize_rows("q4_k", packed, 11008, 4096, out=y),
                packed.numel() + y.numel() * 4, y.numel())
    if name == "stack_7b_layer0_bf16":
        mats = [synth.torch_stack_matrix(0, w, dev) for w in range(7)]
        outs = [torch.empty((x.shape[0], qrow.qr_row_bytes(t, x.shape[1])), dtype=torch.uint8, device=dev)
                for t, x, q in mats]

        def step():
            for (t, x, q), o in zip(mats, outs):
                qrow.qr_quantize_rows(t, x, q, out=o)
        nb = sum(x.numel() * 2 + q.numel() * 4 + o.numel() for (t, x, q), o in zip(mats, outs))
        return step, nb, sum(x.numel() for _, x, _ in mats)
    if name == "moe_256x2048x7168":
        x, q = synth.torch_moe_stack(dev)
        out = torch.empty((x.shape[0], qrow.qr_row_bytes("q4_k", 7168)), dtype=torch.uint8, device=dev)
        return (lambda: qrow.qr_quantize_rows_grouped("q4_k", x, q, 2048, out=out),
                x.numel() * 2 + q.numel() * 4 + out.numel(), x.numel())
    if name.startswith("imatrix_"):
        a, ids, E = synth.imatrix_inputs(name)
        w = synth.WORKLOADS[name]
        bits = synth.f32_to_bf16_bits(a)
        ad = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
        idd = None if ids is None else torch.from_numpy(ids).to(dev)
        sums, counts = qrow.imatrix_state(E, w["n_cols"], dev)
        need = qrow.qr_imatrix_workspace_bytes(w["n_tokens"], w["top_k"], E, w["n_cols"])
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        # unique activation bytes, routing ids, state read and written
        nb = ad.numel() * 2 + (0 if ids is None else ids.nbytes) + 2 * (sums.numel() * 8 + counts.numel() * 8)
        return (lambda: qrow.qr_imatrix_accumulate(ad, sums, counts, idd, workspace=ws),
                nb, ad.numel())
    if name.startswith("mmq_"):
        # weights and activations quantized by the library, then the product
        # (activations Q8_K_128 unless the name ends in another Q8_K format)
        act = "q8_k128"
        for a_t in ("q8_k64", "q8_k16"):
            if name.endswith("_" + a_t):
                act, name = a_t, name[:-len(a_t) - 1]
        t, x, q, a = synth.matmul_sources(name)
        xd, qd, ad = (torch.from_numpy(v).to(dev) for v in (x, q, a))
        w = qrow.qr_quantize_rows(t, xd, qd)
        xa = qrow.qr_quantize_activations_q8k(act, ad)
        n_in = x.shape[1]
        y = torch.empty((a.shape[0], x.shape[0]), dtype=torch.float32, device=dev)
        del xd
        return (lambda: qrow.qr_matmul_q8k(t, act, w, xa, n_in, out=y),
                w.numel() + xa.numel() + y.numel() * 4, x.size)
    if name == "stats_q4_k_11008x4096":
        # error statistics of the Q4_K matrix against its source
        x, q = synth.torch_q4_k_matrix(dev)
        packed = qrow.qr_quantize_rows("q4_k", x, q)
        ws = torch.empty(qrow.qr_stats_workspace_bytes(*x.shape), dtype=torch.uint8, device=dev)
        # one read of the source and the packed rows (the kernels make three)
        return (lambda: qrow.qr_quantize_stats("q4_k", x, packed, q, workspace=ws),
                x.numel() * 4 + packed.numel() + q.numel() * 4, x.numel())
    if name == "mix_q4_k_m_stack_7b":
        plan, mats, outs = _mix_stack(dev)

        def step():
            for t, (x, q), o in zip(plan.tensors, mats, outs):
                qrow.qr_quantize_rows(t.type, x, q, out=o)
        nb = sum(x.numel() * 2 + q.numel() * 4 + o.numel() for (x, q), o in zip(mats, outs))
        return step, nb, plan.weights
    if name == "copy_1gib":
        # plain device copy of a known size: calibrates the HBM byte counters
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        return (lambda: b.copy_(a)), 2 * a.numel() * 4, a.numel()
    raise ValueError(name)


def _mix_stack(dev):
    """The 32-layer 7B-shaped stack (bf16, resident) with its Q4_K_M-style
    plan: Q4_K everywhere, Q6_K for attn_v and ffn_down in the layers that
    fit a +10% size budget."""
    import torch
    from post_weight_quantization_row_amd import mix, qrow, synth
    plan = mix.plan_stack()
    mats = [synth.torch_stack_matrix(t.layer, t.which, dev)[1:] for t in plan.tensors]
    outs = [torch.empty((t.n_rows, qrow.qr_row_bytes(t.type, t.n_per_row)), dtype=torch.uint8, device=dev)
            for t in plan.tensors]
    return plan, mats, outs


def mix_stack_entry(dev, flush):
    """Time to quantize the whole stack with the plan, and the stack's error
    against the same stack at plain Q4_K."""
    from post_weight_quantization_row_amd import mix, qrow
    plan, mats, outs = _mix_stack(dev)

    def step():
        for t, (x, q), o in zip(plan.tensors, mats, outs):
            qrow.qr_quantize_rows(t.type, x, q, out=o)
    nb = sum(x.numel() * 2 + q.numel() * 4 + o.numel() for (x, q), o in zip(mats, outs))
    ms, _, _ = timed_steps(step, 3, 1, flush)
    by_name = {t.name: m for t, m in zip(plan.tensors, mats)}
    ev = mix.evaluate(plan, lambda t: by_name[t.name])
    return {"ms": round(ms, 4), "tensors": len(plan.tensors), "launches": len(plan.tensors),
            "Gweights/s": round(plan.weights / ms / 1e6, 3), "alg_bytes": nb,
            "hbm_frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "promoted_layers": len(plan.promoted_layers),
            "bytes": ev["bytes"], "base_bytes": ev["base_bytes"], "bpw": round(ev["bpw"], 4),
            "rel_rmse": round(ev["rel_rmse"], 6), "base_rel_rmse": round(ev["base_rel_rmse"], 6),
            "weighted_rel_rmse": round(ev["weighted_rel_rmse"], 6),
            "base_weighted_rel_rmse": round(ev["base_weighted_rel_rmse"], 6)}


IMATRIX_WORKLOADS = ("imatrix_moe_256x8_4096x7168", "imatrix_moe_slots_256x8_4096x2048",
                     "imatrix_dense_4096x4096")
MATMUL_WORKLOADS = ("mmq_q4_k_11008x4096_t1", "mmq_q4_0_4096x4096_t8",
                    "mmq_q4_k_11008x4096_t1_q8_k16", "mmq_q4_0_4096x4096_t8_q8_k16",
                    "mmq_q4_k_11008x4096_t512")
ACT_WORKLOADS = ("q8_k64_8192x7168", "q8_k16_8192x7168")
STATS_WORKLOADS = ("stats_q4_k_11008x4096",)
ONLY_WORKLOADS = ("q4_k_11008x4096", "q4_0_2048x2048", "q8_k128_8192x7168",
                  "dequantize_q4_k_11008x4096", "stack_7b_layer0_bf16",
                  "moe_256x2048x7168", "copy_1gib", "mix_q4_k_m_stack_7b", "q4_k_fit_11008x4096", "q6_k_11008x4096", "q5_k_11008x4096") + ACT_WORKLOADS + IMATRIX_WORKLOADS + MATMUL_WORKLOADS + STATS_WORKLOADS


def run_only(args, dev, flush):
    step, nbytes, n_el = _setup(args.only, dev)
    log(f"{args.only}: warmup {args.warmup}, steps {args.steps}")
    ms, ms_min, wall = timed_steps(step, args.steps, args.warmup, flush)
    print(json.dumps({"workload": args.only, "ms_per_step": round(ms, 5),
                      "ms_min": round(ms_min, 5),
                      "G_elements_per_s": round(n_el / ms / 1e6, 3),
                      "algorithmic_bytes": nbytes,
                      "GB/s": round(nbytes / ms / 1e6, 1),
                      "hbm_frac": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}),
          flush=True)


def activation_block_ablation(dev, flush):
    """Each Q8_K block size on calibration-like activations (8192 x 7168,
    per-channel LogNormal scales, 0.1% outlier channels at 20x): the
    quantization time of the 8192x7168 matrix, bytes per value, relative
    RMSE of the activations, and the relative error of the product of 8 such
    tokens with the Q4_0 4096x4096 weights against the product of the
    decoded weights with the unquantized activations (float64)."""
    import torch
    from post_weight_quantization_row_amd import qrow, synth
    x = synth.calib_activations(8192, 7168, seed=1012, bf16=False)
    xd = torch.from_numpy(x).to(dev)
    t, wx, wq, a = synth.matmul_sources("mmq_q4_0_4096x4096_t8")
    w = qrow.qr_quantize_rows(t, torch.from_numpy(wx).to(dev), torch.from_numpy(wq).to(dev))
    W = qrow.qr_dequantize_rows(t, w, wx.shape[0], wx.shape[1]).double()
    ad = torch.from_numpy(a).to(dev)
    exact = ad.double() @ W.T
    rows = {}
    for act in qrow.ACT_TYPES:
        out = qrow.qr_quantize_activations_q8k(act, xd)
        ms, _, _ = timed_steps(lambda: qrow.qr_quantize_activations_q8k(act, xd, out=out), 5, 1, flush)
        st = qrow.qr_quantize_stats(act, xd, out)
        y = qrow.qr_matmul_q8k(t, act, w, qrow.qr_quantize_activations_q8k(act, ad), wx.shape[1]).double()
        rows[act] = {"ms": round(ms, 5), "bytes_per_value": round(out.numel() / x.size, 4),
                     "rel_rmse": round(st["rel_rmse"], 6),
                     "product_rel_err": round(float(torch.linalg.norm(y - exact) / torch.linalg.norm(exact)), 6)}
    return rows


def subscale_fit_comparison(x, q, flush):
    """The two choices of the Q4_K 6-bit sub-scales on the Q4_K matrix:
    quantization time and the error statistics of each output."""
    from post_weight_quantization_row_amd import qrow
    rows = {}
    for fit in qrow.FITS:
        out = qrow.qr_quantize_rows_ex("q4_k", x, q, subscale_fit=fit)
        ms, _, _ = timed_steps(lambda: qrow.qr_quantize_rows_ex("q4_k", x, q, subscale_fit=fit, out=out), 5, 1,
                               flush)
        st = qrow.qr_quantize_stats("q4_k", x, out, q)
        rows[fit] = {"ms": round(ms, 5), "rel_rmse": round(st["rel_rmse"], 6),
                     "weighted_rel_rmse": round(st["weighted_rel_rmse"], 6),
                     "max_abs_err": st["max_abs_err"], "p95_abs_err": st["p95_abs_err"]}
    return rows


def weighting_ablation(x, q, flush):
    """Each element-importance weighting on the Q4_K matrix: quantization
    time and the error statistics of its output (relative RMSE, imatrix-
    weighted relative RMSE, max and p95 of |e|)."""
    from post_weight_quantization_row_amd import qrow
    rows = {}
    for mode in qrow.WEIGHTINGS:
        out = qrow.qr_quantize_rows_weighted("q4_k", x, q, mode)
        ms, _, _ = timed_steps(lambda: qrow.qr_quantize_rows_weighted("q4_k", x, q, mode, out=out), 5, 1, flush)
        st = qrow.qr_quantize_stats("q4_k", x, out, q)
        rows[mode] = {"ms": round(ms, 5), "rel_rmse": round(st["rel_rmse"], 6),
                      "weighted_rel_rmse": round(st["weighted_rel_rmse"], 6),
                      "max_abs_err": st["max_abs_err"], "p95_abs_err": st["p95_abs_err"]}
    return rows


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the secondary workloads")
    ap.add_argument("--only", default=None,
                    choices=sorted(ONLY_WORKLOADS),
                    help="time one workload alone (for profiler runs) and "
                         "print its own JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} "
              "is not supported (rows and experts are independent: several GPUs "
              "would each quantize their own share with the same kernel)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from post_weight_quantization_row_amd import qrow, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    qrow.load_library()
    dev = torch.device("cuda:0")
    flush = (torch.ones(1 << 28, dtype=torch.float32, device=dev),   # 1 GiB
             torch.zeros((), dtype=torch.float32, device=dev))
    if args.only:
        run_only(args, dev, flush)
        return

    # ---- headline: Q4_K, 11008 x 4096 fp32
    n_rows, n = 11008, 4096
    x, q = synth.torch_q4_k_matrix(dev, n_rows, n)
    rb = qrow.qr_row_bytes("q4_k", n)
    out = torch.empty((n_rows, rb), dtype=torch.uint8, device=dev)
    step = lambda: qrow.qr_quantize_rows("q4_k", x, q, out=out)
    log(f"q4_k {n_rows}x{n}: warmup {args.warmup}, steps {args.steps}")
    ms, ms_min, wall = timed_steps(step, args.steps, args.warmup, flush)
    weights = n_rows * n
    alg_bytes = weights * 4 + n * 4 + n_rows * rb
    gws = weights / (ms * 1e-3) / 1e9
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    tops = ALG_OPS_PER_WEIGHT_Q4K * weights / (ms * 1e-3) / 1e12
    torch.cuda.synchronize()
    # back-to-back (input may stay in the Infinity Cache), for context only
    t = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_b2b = (time.perf_counter() - t) * 1e3 / args.steps

    result = {
        "metric": METRIC,
        "value": round(gws, 3),
        "unit": "Gweights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "q4_k_11008x4096", "type": "q4_k",
                   "n_rows": n_rows, "n_per_row": n, "src": "f32",
                   "imatrix": "LogNormal(0,1.5) per column",
                   "cache_flush_between_steps": "1 GiB read"},
        "roofline": {"bound": "alu", "achieved": round(tops, 3),
                     "peak": round(VALU_PEAK_TOPS, 2), "unit": "Tops/s",
                     "frac": round(tops / VALU_PEAK_TOPS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "k_quantize_rows<Q4_K,f32>",
                     "alg_ops_per_weight": ALG_OPS_PER_WEIGHT_Q4K,
                     "alg_bytes_per_launch": alg_bytes},
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "hbm_GB/s": round(gbs, 1),
        "ms_per_step_min": round(ms_min, 5),
        "ms_per_step_back_to_back": round(ms_b2b, 5),
        "wall_s_timed_loop": round(wall, 4),
    }

    # ---- CPU baseline: the oracle on the same matrix (it also checks parity)
    if not args.no_cpu_baseline:
        import oracle
        xh = x.cpu().numpy()
        qh = q.cpu().numpy()
        threads = min(16, os.cpu_count() or 1)
        # whole passes over the full matrix until about 10 s of CPU work
        # (wall time x threads), at least one and at most 32
        log(f"cpu baseline: oracle on the full matrix, {threads} threads")
        passes, dt = 0, 0.0
        while passes < 32 and (passes == 0 or dt * threads < 10.0):
            t = time.perf_counter()
            ref = oracle.quantize_rows("q4_k", xh, qh, threads=threads)
            dt += time.perf_counter() - t
            passes += 1
        same = np.array_equal(ref, out.cpu().numpy())
        result["cpu_baseline"] = {
            "value": round(passes * weights / dt / 1e9, 5), "unit": "Gweights/s",
            "cores": threads, "kind": "oracle",
            "sample": f"the full 11008x4096 matrix, {passes} passes (about 10 s of CPU time)",
            "seconds": round(dt, 3)}
        result["parity_vs_oracle"] = "bit-identical" if same else "DIFFERS"

    # ---- secondary workloads (one line of numbers each)
    if not args.no_extra:
        extra = {}
        x0, q0 = synth.q4_0_matrix()
        x0d, q0d = torch.from_numpy(x0).to(dev), torch.from_numpy(q0).to(dev)
        o0 = torch.empty((2048, qrow.qr_row_bytes("q4_0", 2048)), dtype=torch.uint8, device=dev)
        m0, _, _ = timed_steps(lambda: qrow.qr_quantize_rows("q4_0", x0d, q0d, out=o0), 10, 2, flush)
        b0 = 2048 * 2048 * 4 + 2048 * 4 + o0.numel()
        extra["q4_0_2048x2048"] = {"ms": round(m0, 5), "Gweights/s": round(2048 * 2048 / m0 / 1e6, 3),
                                   "hbm_frac": round(b0 / (m0 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        xa, _ = synth.q8_k128_activations()
        xad = torch.from_numpy(xa).to(dev)
        oa = torch.empty((8192, qrow.qr_row_bytes("q8_k128", 7168)), dtype=torch.uint8, device=dev)
        ma, _, _ = timed_steps(lambda: qrow.qr_quantize_activations_q8k128(xad, out=oa), 10, 2, flush)
        ba = xa.nbytes + oa.numel()
        extra["q8_k128_8192x7168"] = {"ms": round(ma, 5), "Gvalues/s": round(xa.size / ma / 1e6, 3),
                                      "hbm_frac": round(ba / (ma * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        y = torch.empty((n_rows, n), dtype=torch.float32, device=dev)
        md, _, _ = timed_steps(lambda: qrow.qr_dequantize_rows("q4_k", out, n_rows, n, out=y), 10, 2, flush)
        bd = out.numel() + y.numel() * 4
        extra["dequantize_q4_k_11008x4096"] = {"ms": round(md, 5),
                                               "hbm_frac": round(bd / (md * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        # importance-matrix accumulation (the step that produces the imatrix)
        # and the product with Q8_K_128 activations (the step that consumes both)
        for name in ("q6_k_11008x4096", "q5_k_11008x4096") + ACT_WORKLOADS + IMATRIX_WORKLOADS + MATMUL_WORKLOADS + STATS_WORKLOADS:
            fn, nb, n_el = _setup(name, dev)
            mi, _, _ = timed_steps(fn, 10, 2, flush)
            extra[name] = {"ms": round(mi, 5), "alg_bytes": nb, "G_elements_per_s": round(n_el / mi / 1e6, 3),
                           "GB/s": round(nb / (mi * 1e-3) / 1e9, 1),
                           "hbm_frac": round(nb / (mi * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            if name.startswith("mmq_"):
                # integer multiply-adds against the dense int8 matrix-core peak
                base = name
                for suffix in ("_q8_k64", "_q8_k16"):
                    if base.endswith(suffix):
                        base = base[:-len(suffix)]
                wl = synth.WORKLOADS[base]
                tops = 2.0 * wl["n_out"] * wl["n_tok"] * wl["n_in"] / (mi * 1e-3) / 1e12
                extra[name]["int8_Tops"] = round(tops, 2)
                extra[name]["int8_mfma_frac"] = round(tops / INT8_PEAK_TOPS, 4)
        extra["weighting_ablation_q4_k_11008x4096"] = weighting_ablation(x, q, flush)
        extra["subscale_fit_q4_k_11008x4096"] = subscale_fit_comparison(x, q, flush)
        extra["mix_q4_k_m_stack_7b"] = mix_stack_entry(dev, flush)
        extra["activation_block_ablation_calib_8192x7168"] = activation_block_ablation(dev, flush)
        result["extra"] = extra

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
