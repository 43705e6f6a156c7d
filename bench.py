#!/usr/bin/env python3
"""Benchmark of the importance-weighted row quantizer on one MI355X.

Headline workload: Q4_K quantization of an 11008 x 4096 fp32 FFN weight matrix
(x = s_r * 0.015*N(0,1), per-row scale s_r ~ LogNormal(0, 0.3), per-column
importance LogNormal(0, 1.5); synthetic, seeded). One step = one call of
qr_quantize_rows over the whole matrix: load, row statistic, importances,
trial scales, least squares, flips, super-block scales, packing.

The same run times all five workloads the method is measured on
("configs": Q4_0 2048x2048 fp32; the headline; the 32-layer 7B-shaped bf16
stack of 224 matrices, Q4_0 attention and Q5_1 FFN, one launch per matrix
(on one stream, and spread over four) and, the same matrices in the same
buffers, one grouped launch per group of same-shape matrices; Q8_K_128
activations 8192x7168 fp32; the 256-expert bf16 MoE stack in one
grouped launch), each against the HBM roofline, and times the CPU oracle on
a bounded sample of each (cpu_baseline), checking the GPU bytes against it.

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
# MI355X dense int8 matrix-core peak (no sparsity), Tera-ops per second
INT8_PEAK_TOPS = 5000.0
METRIC = "Gweights/s quantized (Q4_0, Q4_K) + achieved HBM GB/s fraction"
COUNTERS = os.path.join(ROOT, "profiles", "q4_k_11008x4096_counters.json")
VALU_COUNTERS = os.path.join(ROOT, "profiles", "q4_k_11008x4096_valu_counters.json")
KERNEL_SRC = os.path.join(ROOT, "post_weight_quantization_row_amd", "csrc", "qrow.hip")
# Host threads for the oracle: the host share of one GPU's job (the box runs
# one GPU's work on 16 cores, whatever the machine's total).
HOST_SHARE = 16


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


def measured_valu():
    """Per-weight VALU figures of the Q4_K kernel (instruction counts by
    class, dual issue, issue cycles) from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source."""
    import hashlib
    try:
        with open(VALU_COUNTERS) as f:
            c = json.load(f)
        with open(KERNEL_SRC, "rb") as f:
            h = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha256") != h:
        return None
    return c.get("summary")


VALU_CLASSES = ("fma_f32", "add_f32", "xor_b32", "rndne_f32", "med3_f32", "cmp_cndmask",
                "fma_rndne_mix", "fma_f64", "sqrt_f32", "fma_f32_one_chain")


def valu_rates(waves_per_simd=8):
    """SIMD cycles per wave64 instruction (at 2.4 GHz) of the instruction
    classes of the row kernels, measured now by libqrow_probe.so (register-
    only kernels, eight independent chains per lane unless named)."""
    import ctypes as C
    import torch
    path = os.path.join(ROOT, "post_weight_quantization_row_amd", "libqrow_probe.so")
    if not os.path.exists(path):
        return None
    L = C.CDLL(path)
    L.qrp_valu_rates.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_void_p]
    L.qrp_valu_classes.restype = C.c_int
    n = L.qrp_valu_classes()
    if n != len(VALU_CLASSES):
        return None
    n_simds = 4 * torch.cuda.get_device_properties(0).multi_processor_count
    inp = torch.tensor([1.0000001, 1e-7], dtype=torch.float32, device="cuda")
    sink = torch.empty(n_simds * waves_per_simd // 4, dtype=torch.float32, device="cuda")
    out = (C.c_float * n)()
    torch.cuda.synchronize()
    if L.qrp_valu_rates(C.c_void_p(inp.data_ptr()), C.c_void_p(sink.data_ptr()), waves_per_simd, n_simds, out) != 0:
        return None
    return {k: round(float(v), 2) for k, v in zip(VALU_CLASSES, out)}


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
    if name in ("stack_7b_32x7", "stack_7b_32x7_grouped", "stack_7b_32x7_streams"):
        # the whole 32-layer stack: 224 launches per step, or one grouped
        # launch per group of same-shape matrices (3 per step)
        groups, outs_g, mats, outs = _stack(dev)
        if name == "stack_7b_32x7":
            def step():
                for (t, x, q), o in zip(mats, outs):
                    qrow.qr_quantize_rows(t, x, q, out=o)
        elif name == "stack_7b_32x7_streams":
            streams = [torch.cuda.Stream() for _ in range(4)]

            def step():
                main = torch.cuda.current_stream()
                start = torch.cuda.Event()
                start.record(main)
                for st in streams:
                    st.wait_event(start)
                for k, ((t, x, q), o) in enumerate(zip(mats, outs)):
                    with torch.cuda.stream(streams[k % 4]):
                        qrow.qr_quantize_rows(t, x, q, out=o)
                for st in streams:
                    done = torch.cuda.Event()
                    done.record(st)
                    main.wait_event(done)
        else:
            def step():
                for (t, x, q, r), o in zip(groups, outs_g):
                    qrow.qr_quantize_rows_grouped(t, x, q, r, out=o)
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


def _stack(dev):
    """The 32-layer stack, drawn on the GPU in its three same-shape groups:
    (groups, their outputs, the 224 matrices as views, their outputs as
    views of the same buffers)."""
    import torch
    from post_weight_quantization_row_amd import qrow, synth
    groups, members = synth.torch_stack_grouped(dev)
    outs_g = [torch.empty((x.shape[0], qrow.qr_row_bytes(t, x.shape[1])), dtype=torch.uint8, device=dev)
              for t, x, _, _ in groups]
    mats = synth.torch_stack_views(groups, members)
    outs = []
    for layer in range(32):
        for which in range(7):
            gi, i = members[(layer, which)]
            r = groups[gi][3]
            outs.append(outs_g[gi][i * r:(i + 1) * r])
    return groups, outs_g, mats, outs


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
                  "moe_256x2048x7168", "stack_7b_32x7", "stack_7b_32x7_grouped", "stack_7b_32x7_streams", "copy_1gib", "valu_rates", "q4_k_row_scan", "mix_q4_k_m_stack_7b", "q4_k_fit_11008x4096", "q6_k_11008x4096", "q5_k_11008x4096") + ACT_WORKLOADS + IMATRIX_WORKLOADS + MATMUL_WORKLOADS + STATS_WORKLOADS


def run_only(args, dev, flush):
    if args.only == "valu_rates":
        # issue cycles per wave64 instruction of each class at 1, 2, 4, 8
        # waves per SIMD (the calibration of the VALU figures)
        print(json.dumps({"workload": "valu_rates", "unit": "SIMD cycles per wave64 instruction at 2.4 GHz",
                          "by_waves_per_simd": {w: valu_rates(w) for w in (1, 2, 4, 8)}}), flush=True)
        return
    if args.only == "q4_k_row_scan":
        # the Q4_K row kernel on 4096-value fp32 rows at several row counts:
        # time against rows separates the per-row rate from the per-launch cost
        import torch
        from post_weight_quantization_row_amd import qrow
        g = torch.Generator(device=dev).manual_seed(5)
        q = torch.exp(1.5 * torch.randn(4096, generator=g, device=dev))
        scan = {}
        for rows in (1024, 2048, 4096, 6144, 8192, 10240, 11008, 12288, 16384, 20480):
            x = 0.015 * torch.randn(rows, 4096, generator=g, device=dev)
            out = torch.empty((rows, qrow.qr_row_bytes("q4_k", 4096)), dtype=torch.uint8, device=dev)
            ms, _, _ = timed_steps(lambda: qrow.qr_quantize_rows("q4_k", x, q, out=out), args.steps,
                                   args.warmup, flush)
            scan[rows] = round(ms * 1e3, 2)
            log(f"q4_k_row_scan: {rows} rows {ms * 1e3:.2f} us")
        print(json.dumps({"workload": "q4_k_row_scan", "unit": "us per launch", "rows_of_4096": scan}), flush=True)
        return
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


def host_threads() -> int:
    """Threads for the oracle: the visible CPUs, within OMP_NUM_THREADS when
    set and within the host share of one GPU's job."""
    n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, min(n, HOST_SHARE))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def hbm_frac(nbytes, ms):
    return round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)


def timed_oracle(fn, min_wall):
    """Runs fn() until at least min_wall seconds have passed (at least
    once); returns (last result, passes, seconds)."""
    passes, dt, out = 0, 0.0, None
    while passes == 0 or dt < min_wall:
        t = time.perf_counter()
        out = fn()
        dt += time.perf_counter() - t
        passes += 1
    return out, passes, dt


def rows_differing(a, b) -> int:
    """Rows (of packed bytes) that differ between two lists of 2-D arrays."""
    import numpy as np
    return int(sum((np.asarray(x) != np.asarray(y)).any(axis=1).sum() for x, y in zip(a, b)))


def stack_step_times(mats, outs, steps, warmup, flush):
    """The 224-launch stack: (end-to-end ms per step, sum of the launches'
    own times per step). Two passes: one with events only around the whole
    stack, one with events around every launch."""
    import torch
    from post_weight_quantization_row_amd import qrow

    def launch_all():
        for (t, x, q), o in zip(mats, outs):
            qrow.qr_quantize_rows(t, x, q, out=o)
    e2e, _, _ = timed_steps(launch_all, steps, warmup, flush)
    sums = []
    for _ in range(steps):
        evict(flush)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in mats]
        for ((t, x, q), o), (a, b) in zip(zip(mats, outs), ev):
            a.record()
            qrow.qr_quantize_rows(t, x, q, out=o)
            b.record()
        torch.cuda.synchronize()
        sums.append(sum(a.elapsed_time(b) for a, b in ev))
    return e2e, sum(sums) / len(sums)


def stack_streams_ms(mats, outs, n_streams, steps, warmup, flush):
    """The 224 launches spread round-robin over n_streams streams (default
    priority), so that one matrix's launch fills the chip while another's
    drains: mean ms per step between events on the current stream, which
    waits for every stream at the end of the step."""
    import torch
    from post_weight_quantization_row_amd import qrow
    streams = [torch.cuda.Stream() for _ in range(n_streams)]

    def launch_all():
        main = torch.cuda.current_stream()
        start = torch.cuda.Event()
        start.record(main)
        for st in streams:
            st.wait_event(start)
        for k, ((t, x, q), o) in enumerate(zip(mats, outs)):
            with torch.cuda.stream(streams[k % n_streams]):
                qrow.qr_quantize_rows(t, x, q, out=o)
        for st in streams:
            done = torch.cuda.Event()
            done.record(st)
            main.wait_event(done)
    ms, _, _ = timed_steps(launch_all, steps, warmup, flush)
    return ms


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
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not "
              "supported (rows and experts are independent: several GPUs "
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
    cpu = not args.no_cpu_baseline
    if cpu:
        import oracle
        threads = host_threads()
    host = {}   # per workload: (oracle timing function, GPU bytes, sample) for the CPU leg

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
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "k_quantize_rows<Q4_K,f32>",
                     "alg_bytes_per_launch": alg_bytes},
        "ms_per_step_min": round(ms_min, 5),
        "ms_per_step_back_to_back": round(ms_b2b, 5),
        "wall_s_timed_loop": round(wall, 4),
    }
    # VALU figures beside the HBM roofline (secondary): issue cycles of the
    # instruction classes, measured in this run, and the kernel's own
    # instruction counts from the committed counters (if taken on this source)
    valu = {"issue_cycles_per_wave64_instr_at_2.4GHz": valu_rates()}
    counted = measured_valu()
    if counted is not None:
        valu.update(counted)
    result["valu"] = valu
    configs = {"q4_k_11008x4096": {"ms": round(ms, 5), "Gweights/s": round(gws, 3),
                                   "alg_bytes": alg_bytes, "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}}
    if cpu:
        xh, qh, gh = x.cpu().numpy(), q.cpu().numpy(), out.cpu().numpy()
        host["q4_k_11008x4096"] = (lambda: [oracle.quantize_rows("q4_k", xh, qh, threads=threads)], [gh],
                                   weights, "the full 11008x4096 matrix")
    del x, out

    # ---- Q4_0, 2048 x 2048 fp32
    x0, q0 = synth.q4_0_matrix()
    x0d, q0d = torch.from_numpy(x0).to(dev), torch.from_numpy(q0).to(dev)
    o0 = torch.empty((2048, qrow.qr_row_bytes("q4_0", 2048)), dtype=torch.uint8, device=dev)
    log("q4_0 2048x2048")
    m0, _, _ = timed_steps(lambda: qrow.qr_quantize_rows("q4_0", x0d, q0d, out=o0), args.steps, args.warmup, flush)
    b0 = x0.nbytes + q0.nbytes + o0.numel()
    configs["q4_0_2048x2048"] = {"ms": round(m0, 5), "Gweights/s": round(x0.size / m0 / 1e6, 3),
                                 "alg_bytes": b0, "hbm_frac": hbm_frac(b0, m0)}
    if cpu:
        g0 = o0.cpu().numpy()
        host["q4_0_2048x2048"] = (lambda: [oracle.quantize_rows("q4_0", x0, q0, threads=threads)], [g0], x0.size,
                                  "the full 2048x2048 matrix")

    # ---- Q8_K_128 activations, 8192 x 7168 fp32
    xa, _ = synth.q8_k128_activations()
    xad = torch.from_numpy(xa).to(dev)
    oa = torch.empty((8192, qrow.qr_row_bytes("q8_k128", 7168)), dtype=torch.uint8, device=dev)
    log("q8_k128 8192x7168")
    ma, _, _ = timed_steps(lambda: qrow.qr_quantize_activations_q8k128(xad, out=oa), args.steps, args.warmup, flush)
    ba = xa.nbytes + oa.numel()
    configs["q8_k128_8192x7168"] = {"ms": round(ma, 5), "Gvalues/s": round(xa.size / ma / 1e6, 3),
                                    "alg_bytes": ba, "hbm_frac": hbm_frac(ba, ma)}
    if cpu:
        ga = oa.cpu().numpy()
        host["q8_k128_8192x7168"] = (lambda: [oracle.quantize_q8k128(xa, threads=threads)], [ga], xa.size,
                                     "the full 8192x7168 matrix")
    del xad, oa

    # ---- the 7B-shaped stack: 32 layers x 7 bf16 matrices, one launch per
    # matrix (224) and one grouped launch per group of same-shape matrices (3)
    log("stack_7b_32x7: drawing 224 bf16 matrices in 3 same-shape groups")
    groups, outs_g, mats, outs = _stack(dev)
    st_steps = max(1, min(args.steps, 5))
    log(f"stack_7b_32x7: warmup 1, steps {st_steps}")
    e2e, ksum = stack_step_times(mats, outs, st_steps, 1, flush)
    mg, _, _ = timed_steps(lambda: [qrow.qr_quantize_rows_grouped(t, x, q, r, out=o)
                                    for (t, x, q, r), o in zip(groups, outs_g)], st_steps, 1, flush)
    m4 = stack_streams_ms(mats, outs, 4, st_steps, 1, flush)
    w_att = sum(x.numel() for t, x, _ in mats if t == "q4_0")
    w_ffn = sum(x.numel() for t, x, _ in mats if t == "q5_1")
    b_st = sum(x.numel() * 2 + q.numel() * 4 + o.numel() for (t, x, q), o in zip(mats, outs))
    configs["stack_7b_32x7"] = {
        "launches": len(mats), "ms_end_to_end": round(e2e, 4), "ms_kernel_sum": round(ksum, 4),
        "Gweights/s": round((w_att + w_ffn) / e2e / 1e6, 3), "alg_bytes": b_st,
        "hbm_frac": hbm_frac(b_st, e2e), "hbm_frac_kernel_sum": hbm_frac(b_st, ksum),
        "grouped": {"launches": len(groups), "ms": round(mg, 4),
                    "Gweights/s": round((w_att + w_ffn) / mg / 1e6, 3), "hbm_frac": hbm_frac(b_st, mg)},
        "four_streams": {"launches": len(mats), "ms": round(m4, 4),
                         "Gweights/s": round((w_att + w_ffn) / m4 / 1e6, 3), "hbm_frac": hbm_frac(b_st, m4)}}
    # the attention (Q4_0) part alone, from one layer's launches
    att = [(m, o) for m, o in zip(mats[:7], outs[:7]) if m[0] == "q4_0"]
    ma0, _, _ = timed_steps(lambda: [qrow.qr_quantize_rows(t, x, q, out=o) for (t, x, q), o in att], 10, 2, flush)
    b_a0 = sum(x.numel() * 2 + q.numel() * 4 + o.numel() for (t, x, q), o in att)
    configs["stack_7b_32x7"]["q4_0_attention_layer"] = {"ms": round(ma0, 4), "hbm_frac": hbm_frac(b_a0, ma0)}
    if cpu:
        smp = [(t, x.float().cpu().numpy(), q.cpu().numpy(), o.cpu().numpy()) for (t, x, q), o in
               zip(mats[:7], outs[:7])]

        def stack_oracle(smp=smp):
            return [oracle.quantize_rows(t, xs, qs, threads=threads) for t, xs, qs, _ in smp]
        host["stack_7b_32x7"] = (stack_oracle, [g for *_, g in smp], sum(v[1].size for v in smp),
                                 "layer 0 of the stack: its 7 matrices, every row")
    del mats, outs, groups, outs_g
    torch.cuda.empty_cache()

    # ---- the 256-expert MoE stack, bf16, one grouped launch
    log("moe_256x2048x7168: drawing the stack")
    xm, qm = synth.torch_moe_stack(dev)
    om = torch.empty((xm.shape[0], qrow.qr_row_bytes("q4_k", 7168)), dtype=torch.uint8, device=dev)
    mo_steps = max(1, min(args.steps, 5))
    log(f"moe_256x2048x7168: warmup 1, steps {mo_steps}")
    mm, _, _ = timed_steps(lambda: qrow.qr_quantize_rows_grouped("q4_k", xm, qm, 2048, out=om), mo_steps, 1, flush)
    bm = xm.numel() * 2 + qm.numel() * 4 + om.numel()
    configs["moe_256x2048x7168"] = {"ms": round(mm, 4), "Gweights/s": round(xm.numel() / mm / 1e6, 3),
                                    "alg_bytes": bm, "hbm_frac": hbm_frac(bm, mm)}
    if cpu:
        experts = [0, 37, 74, 111, 148, 185, 222, 255]
        zero = synth.moe_zero_experts()
        experts[1] = int(zero[0])                      # one expert with importances 1e-6
        qmh = qm.cpu().numpy()
        smp = [(e, xm[2048 * e:2048 * (e + 1)].float().cpu().numpy(),
                om[2048 * e:2048 * (e + 1)].cpu().numpy()) for e in experts]

        def moe_oracle(smp=smp):
            return [oracle.quantize_rows("q4_k", xs, qmh[e], threads=threads) for e, xs, _ in smp]
        host["moe_256x2048x7168"] = (moe_oracle, [g for _, _, g in smp], sum(v[1].size for v in smp),
                                     f"experts {experts}, every row")
    del xm, om
    torch.cuda.empty_cache()
    result["configs"] = configs

    # ---- CPU baseline: the oracle on bounded samples of every workload, on
    # the host share of cores; each sample's bytes are compared with the GPU's
    if cpu:
        log(f"cpu baseline: oracle on {threads} threads")
        per = {}
        for name, (fn, gpu_bytes, n_el, what) in host.items():
            ref, passes, dt = timed_oracle(fn, 1.0 if name == "q4_k_11008x4096" else 0.5)
            per[name] = {"G_elements_per_s": round(passes * n_el / dt / 1e9, 5), "seconds": round(dt, 3),
                         "passes": passes, "sample": what,
                         "rows_differing_from_gpu": rows_differing(ref, gpu_bytes)}
        # one thread on the Q4_0 matrix
        x1, q1 = synth.q4_0_matrix()
        _, p1, d1 = timed_oracle(lambda: oracle.quantize_rows("q4_0", x1, q1, threads=1), 1.0)
        head = per["q4_k_11008x4096"]
        result["cpu_baseline"] = {
            "value": head["G_elements_per_s"], "unit": "Gweights/s", "cores": threads, "kind": "oracle",
            "sample": f"{head['sample']}, {head['passes']} passes",
            "seconds": head["seconds"], "cpu_model": cpu_model(), "host_cpus_visible": os.cpu_count(),
            "q4_0_2048x2048_one_thread_Gweights/s": round(p1 * x1.size / d1 / 1e9, 5),
            "per_workload": per}
        result["parity_vs_oracle"] = ("bit-identical" if all(v["rows_differing_from_gpu"] == 0 for v in per.values())
                                      else "rows differ: see cpu_baseline.per_workload")

    # ---- secondary workloads (one line of numbers each)
    if not args.no_extra:
        extra = {}
        x, q = synth.torch_q4_k_matrix(dev, n_rows, n)
        out = qrow.qr_quantize_rows("q4_k", x, q)
        y = torch.empty((n_rows, n), dtype=torch.float32, device=dev)
        md, _, _ = timed_steps(lambda: qrow.qr_dequantize_rows("q4_k", out, n_rows, n, out=y), 10, 2, flush)
        bd = out.numel() + y.numel() * 4
        extra["dequantize_q4_k_11008x4096"] = {"ms": round(md, 5), "hbm_frac": hbm_frac(bd, md)}
        del y
        # importance-matrix accumulation (the step that produces the imatrix)
        # and the product with Q8_K_128 activations (the step that consumes both)
        for name in ("q6_k_11008x4096", "q5_k_11008x4096") + ACT_WORKLOADS + IMATRIX_WORKLOADS + MATMUL_WORKLOADS + STATS_WORKLOADS:
            fn, nb, n_el = _setup(name, dev)
            mi, _, _ = timed_steps(fn, 10, 2, flush)
            extra[name] = {"ms": round(mi, 5), "alg_bytes": nb, "G_elements_per_s": round(n_el / mi / 1e6, 3),
                           "GB/s": round(nb / (mi * 1e-3) / 1e9, 1), "hbm_frac": hbm_frac(nb, mi)}
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
        del x, q, out
        torch.cuda.empty_cache()
        extra["mix_q4_k_m_stack_7b"] = mix_stack_entry(dev, flush)
        extra["activation_block_ablation_calib_8192x7168"] = activation_block_ablation(dev, flush)
        result["extra"] = extra

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
