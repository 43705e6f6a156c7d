"""Seeded synthetic inputs for the quantizers.

This module holds no arithmetic of the quantization method: it only draws the
weight matrices, activations and importance vectors that the GPU library and
the CPU oracle both consume, so that the two sides see identical bytes.

The workloads stand in for real LLM weights and calibration data (none are
available here). Their shapes and value distributions are:

* ``q4_0_2048x2048``: one fp32 matrix, x = 0.02*N(0,1); round(0.1%) distinct
  entries multiplied by 10; per-column importance LogNormal(0, 1).
* ``q4_k_11008x4096``: one fp32 FFN matrix, x = s_r * 0.015*N(0,1) with a
  per-row scale s_r ~ LogNormal(0, 0.3); importance LogNormal(0, 1.5).
* ``stack_7b_32x7``: 32 layers of 4 attention matrices [4096, 4096] (Q4_0)
  and 3 FFN matrices [11008, 4096], [11008, 4096], [4096, 11008] (Q5_1), bf16
  values 0.02*StudentT(5); per-matrix importance LogNormal(0, 1).
* ``q8_k128_8192x7168``: fp32 activations N(0,1) with one channel (0.01% of
  7168, rounded up to one) whose magnitudes are replaced by U(1e4, 2e5),
  keeping their signs.
* ``moe_256x2048x7168``: 256 experts of bf16 [2048, 7168], x = 0.01*N(0,1) *
  s_{e,r} with s ~ LogNormal(0, 0.5) per expert row; per-expert importance
  LogNormal(0, 2), with 26 experts (10%) set to 1e-6.
* ``imatrix_moe_256x8_4096x7168``: importance accumulation for a stacked
  expert tensor: 4096 tokens of bf16 hidden states [4096, 7168] (one row per
  token, seen by each of its experts), a[t, c] = s_c * N(0,1) with channel
  scales s_c ~ LogNormal(0, 1) and 0.1% of the channels (at least one)
  multiplied by 20; each token routed to 8 distinct experts out of 256 by
  Gumbel top-k over log-popularities N(0, 0.5), with 3 experts that are never
  routed (partial coverage).
* ``imatrix_moe_slots_256x8_4096x2048``: as the expert case above for the
  down projection: one bf16 row of 2048 values per routed slot,
  [4096, 8, 2048], each seen only by the expert of its slot.
* ``imatrix_dense_4096x4096``: importance accumulation for a dense tensor:
  4096 tokens of bf16 activations [4096, 4096] drawn as above.
* ``mmq_q4_k_11008x4096_t1``: product of the Q4_K-quantized
  ``q4_k_11008x4096`` matrix (with its importances) with one token of fp32
  activations drawn as the calibration activations above, quantized to
  Q8_K_128 (a decode step).
* ``mmq_q4_0_4096x4096_t8``: product of the Q4_0-quantized first attention
  matrix of ``stack_7b_32x7`` with 8 such tokens.
* ``mmq_q4_k_11008x4096_t512``: the Q4_K matrix of ``mmq_q4_k_11008x4096_t1``
  with 512 such tokens (a prompt processed at once).

Two back-ends draw the same recipes: numpy (CPU, used by the CPU tests and by
small GPU tests) and torch on the GPU (used for the multi-GB stacks). The two
back-ends draw different numbers; each run names the back-end it used.
"""
from __future__ import annotations

import hashlib

import numpy as np

# workload name -> shape/type description
WORKLOADS = {
    "q4_0_2048x2048": dict(type="q4_0", dtype="f32", n_rows=2048,
                           n_per_row=2048, seed=1001),
    "q4_k_11008x4096": dict(type="q4_k", dtype="f32", n_rows=11008,
                            n_per_row=4096, seed=1002),
    "stack_7b_32x7": dict(type="mixed", dtype="bf16", n_layers=32, seed=1003),
    "q8_k128_8192x7168": dict(type="q8_k128", dtype="f32", n_rows=8192,
                              n_per_row=7168, seed=1004),
    "moe_256x2048x7168": dict(type="q4_k", dtype="bf16", n_experts=256,
                              n_rows=2048, n_per_row=7168, seed=1005,
                              n_zero_experts=26),
    "imatrix_moe_256x8_4096x7168": dict(type="imatrix", dtype="bf16",
                                        n_tokens=4096, n_cols=7168,
                                        n_experts=256, top_k=8, n_slots=1,
                                        n_dead=3, seed=1006),
    "imatrix_moe_slots_256x8_4096x2048": dict(type="imatrix", dtype="bf16",
                                              n_tokens=4096, n_cols=2048,
                                              n_experts=256, top_k=8,
                                              n_slots=8, n_dead=3, seed=1008),
    "mmq_q4_k_11008x4096_t1": dict(type="matmul", wtype="q4_k", n_out=11008,
                                   n_in=4096, n_tok=1, weights="q4_k_11008x4096",
                                   seed=1009),
    "mmq_q4_0_4096x4096_t8": dict(type="matmul", wtype="q4_0", n_out=4096,
                                  n_in=4096, n_tok=8, weights="stack_7b_32x7",
                                  seed=1010),
    "mmq_q4_k_11008x4096_t512": dict(type="matmul", wtype="q4_k", n_out=11008,
                                     n_in=4096, n_tok=512, weights="q4_k_11008x4096",
                                     seed=1013),
    "imatrix_dense_4096x4096": dict(type="imatrix", dtype="bf16",
                                    n_tokens=4096, n_cols=4096, n_experts=1,
                                    top_k=0, n_slots=1, n_dead=0, seed=1007),
}

# The seven matrices of one 7B-shaped layer: (name, type, n_rows, n_per_row).
STACK_LAYER = [
    ("attn_q", "q4_0", 4096, 4096),
    ("attn_k", "q4_0", 4096, 4096),
    ("attn_v", "q4_0", 4096, 4096),
    ("attn_o", "q4_0", 4096, 4096),
    ("ffn_gate", "q5_1", 11008, 4096),
    ("ffn_up", "q5_1", 11008, 4096),
    ("ffn_down", "q5_1", 4096, 11008),
]


def stream_seed(seed: int, *keys) -> int:
    """A 63-bit seed derived from (seed, keys) by SHA-256."""
    h = hashlib.sha256(repr((int(seed),) + tuple(keys)).encode()).digest()
    return int.from_bytes(h[:8], "little") >> 1


def rng(seed: int, *keys) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(stream_seed(seed, *keys)))


# --------------------------------------------------------------------------
# bfloat16 helpers (round to nearest-even, as torch's .to(torch.bfloat16))

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << 16).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values that are exactly representable in bfloat16."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# --------------------------------------------------------------------------
# numpy back-end

def q4_0_matrix(n_rows=2048, n_per_row=2048, seed=1001, outlier_frac=1e-3):
    g = rng(seed, "x")
    x = (0.02 * g.standard_normal((n_rows, n_per_row))).astype(np.float32)
    k = int(round(outlier_frac * n_rows * n_per_row))
    if k:
        idx = g.choice(n_rows * n_per_row, size=k, replace=False)
        x.reshape(-1)[idx] *= np.float32(10.0)
    q = np.exp(rng(seed, "imatrix").standard_normal(n_per_row)).astype(np.float32)
    return x, q


def q4_k_matrix(n_rows=11008, n_per_row=4096, seed=1002):
    g = rng(seed, "x")
    z = 0.015 * g.standard_normal((n_rows, n_per_row))
    s = np.exp(0.3 * rng(seed, "rowscale").standard_normal((n_rows, 1)))
    x = (s * z).astype(np.float32)
    q = np.exp(1.5 * rng(seed, "imatrix").standard_normal(n_per_row)).astype(np.float32)
    return x, q


def stack_matrix(layer: int, which: int, seed=1003, rows=None):
    """One matrix of the 7B-shaped stack: returns (type, x_f32 (bf16 values),
    importance). ``rows`` limits the number of rows drawn (a prefix)."""
    name, typ, n_rows, n = STACK_LAYER[which]
    r = n_rows if rows is None else min(rows, n_rows)
    g = rng(seed, "x", layer, which)
    x = round_to_bf16((0.02 * g.standard_t(5, size=(r, n))).astype(np.float32))
    q = np.exp(rng(seed, "imatrix", layer, which).standard_normal(n)).astype(np.float32)
    return typ, x, q


def q8_k128_activations(n_rows=8192, n_per_row=7168, seed=1004):
    g = rng(seed, "x")
    x = g.standard_normal((n_rows, n_per_row)).astype(np.float32)
    n_out = max(1, int(round(1e-4 * n_per_row)))
    ch = rng(seed, "channels").choice(n_per_row, size=n_out, replace=False)
    mags = rng(seed, "magnitudes").uniform(1e4, 2e5, size=(n_rows, n_out))
    sgn = np.where(x[:, ch] < 0, -1.0, 1.0)
    x[:, ch] = (sgn * mags).astype(np.float32)
    return x, ch


def moe_zero_experts(n_experts=256, n_zero=26, seed=1005):
    return np.sort(rng(seed, "zero-experts").choice(n_experts, size=n_zero,
                                                    replace=False))


def moe_imatrix(n_experts=256, n_per_row=7168, seed=1005, n_zero=26):
    q = np.exp(2.0 * rng(seed, "imatrix").standard_normal((n_experts, n_per_row)))
    q = q.astype(np.float32)
    q[moe_zero_experts(n_experts, n_zero, seed)] = np.float32(1e-6)
    return q


def moe_expert(e: int, n_rows=2048, n_per_row=7168, seed=1005, rows=None):
    r = n_rows if rows is None else min(rows, n_rows)
    z = 0.01 * rng(seed, "x", e).standard_normal((n_rows, n_per_row))[:r]
    s = np.exp(0.5 * rng(seed, "rowscale", e).standard_normal((n_rows, 1)))[:r]
    return round_to_bf16((z * s).astype(np.float32))


def calib_activations(n_tokens, n_cols, seed, n_slots=1, outlier_frac=1e-3,
                      outlier_gain=20.0, bf16=True):
    """Calibration-like activations [n_tokens, n_slots, n_cols] (n_slots == 1
    gives [n_tokens, n_cols]): per-channel scales LogNormal(0, 1), a few
    outlier channels; float32 holding bf16 values when ``bf16``."""
    g = rng(seed, "act")
    s = np.exp(rng(seed, "channel-scale").standard_normal(n_cols))
    k = max(1, int(round(outlier_frac * n_cols)))
    s[rng(seed, "outlier-channels").choice(n_cols, size=k, replace=False)] *= outlier_gain
    shape = (n_tokens, n_cols) if n_slots == 1 else (n_tokens, n_slots, n_cols)
    a = (g.standard_normal(shape) * s).astype(np.float32)
    return round_to_bf16(a) if bf16 else a


def routing_ids(n_tokens, n_experts, top_k, seed, n_dead=0, spread=0.5):
    """[n_tokens, top_k] int32: top_k distinct experts per token, drawn by
    Gumbel top-k over log-popularities N(0, spread); ``n_dead`` experts are
    never chosen. Each row lists its experts in decreasing score order."""
    if n_experts - n_dead < top_k:
        raise ValueError("not enough live experts for top_k")
    logp = spread * rng(seed, "popularity").standard_normal(n_experts)
    if n_dead:
        logp[rng(seed, "dead").choice(n_experts, size=n_dead, replace=False)] = -np.inf
    score = logp + rng(seed, "gumbel").gumbel(size=(n_tokens, n_experts))
    top = np.argpartition(-score, top_k - 1, axis=1)[:, :top_k]
    order = np.argsort(-np.take_along_axis(score, top, axis=1), axis=1, kind="stable")
    return np.take_along_axis(top, order, axis=1).astype(np.int32)


def matmul_sources(name):
    """(weight type, fp32 weights, importances, fp32 activations) of a
    matmul workload; the caller quantizes both."""
    w = WORKLOADS[name]
    if w["weights"] == "q4_k_11008x4096":
        x, q = q4_k_matrix()
    else:
        _, x, q = stack_matrix(0, 0)
    a = calib_activations(w["n_tok"], w["n_in"], w["seed"], bf16=False)
    return w["wtype"], x, q, a


def imatrix_inputs(name):
    """(activations, ids or None, n_experts) of an imatrix workload."""
    w = WORKLOADS[name]
    a = calib_activations(w["n_tokens"], w["n_cols"], w["seed"], w["n_slots"],
                          bf16=w["dtype"] == "bf16")
    if w["top_k"] == 0:
        return a, None, 1
    ids = routing_ids(w["n_tokens"], w["n_experts"], w["top_k"], w["seed"],
                      n_dead=w["n_dead"])
    return a, ids, w["n_experts"]


# --------------------------------------------------------------------------
# torch back-end (on the GPU; used for multi-GB stacks)

def _tgen(device, seed, *keys):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(stream_seed(seed, "torch", *keys))
    return g


def torch_stack_matrix(layer, which, device, seed=1003):
    """(type, bf16 tensor [n_rows, n], fp32 importance) on ``device``."""
    import torch
    name, typ, n_rows, n = STACK_LAYER[which]
    g = _tgen(device, seed, "x", layer, which)
    # Student-t(5) = N(0,1) / sqrt(chi2_5 / 5), chi2_5 = 2 * Gamma(5/2)
    z = torch.randn((n_rows, n), generator=g, device=device)
    alpha = torch.full((n_rows, n), 2.5, device=device)
    chi = 2.0 * torch._standard_gamma(alpha, generator=g)
    del alpha
    x = (0.02 * z / torch.sqrt(chi / 5.0)).to(torch.bfloat16)
    gq = _tgen(device, seed, "imatrix", layer, which)
    q = torch.exp(torch.randn(n, generator=gq, device=device)).float()
    return typ, x, q


# The stack's matrices in three groups of one shape and type each: the four
# attention matrices of every layer, the gate and up matrices, the down
# matrices. Member i of a group is rows i*n_rows .. (i+1)*n_rows - 1 of one
# contiguous tensor, so a group is quantized by one grouped launch.
STACK_GROUPS = [(0, 1, 2, 3), (4, 5), (6,)]


def torch_stack_grouped(device, seed=1003, n_layers=32):
    """(groups, members) for the stack with the values of torch_stack_matrix.
    groups: [(type, bf16 [n_members * n_rows, n], fp32 [n_members, n],
    n_rows)]; members[(layer, which)] = (group index, member index)."""
    import torch
    groups, members = [], {}
    for gi, whichs in enumerate(STACK_GROUPS):
        _, typ, n_rows, n = STACK_LAYER[whichs[0]]
        keys = [(layer, which) for layer in range(n_layers) for which in whichs]
        x = torch.empty((len(keys) * n_rows, n), dtype=torch.bfloat16, device=device)
        q = torch.empty((len(keys), n), dtype=torch.float32, device=device)
        for i, (layer, which) in enumerate(keys):
            _, xi, qi = torch_stack_matrix(layer, which, device, seed)
            x[i * n_rows:(i + 1) * n_rows] = xi
            q[i] = qi
            members[(layer, which)] = (gi, i)
            del xi
        groups.append((typ, x, q, n_rows))
    return groups, members


def torch_stack_views(groups, members, n_layers=32):
    """The stack as (type, x, q) per matrix, layer by layer, as views of the
    grouped tensors."""
    out = []
    for layer in range(n_layers):
        for which in range(len(STACK_LAYER)):
            gi, i = members[(layer, which)]
            typ, x, q, n_rows = groups[gi]
            out.append((typ, x[i * n_rows:(i + 1) * n_rows], q[i]))
    return out


def torch_moe_stack(device, n_experts=256, n_rows=2048, n_per_row=7168,
                    seed=1005, n_zero=26):
    """bf16 [n_experts*n_rows, n_per_row] and fp32 [n_experts, n_per_row]."""
    import torch
    x = torch.empty((n_experts * n_rows, n_per_row), dtype=torch.bfloat16,
                    device=device)
    for e in range(n_experts):
        g = _tgen(device, seed, "x", e)
        z = torch.randn((n_rows, n_per_row), generator=g, device=device)
        s = torch.exp(0.5 * torch.randn((n_rows, 1), generator=g, device=device))
        x[e * n_rows:(e + 1) * n_rows] = (0.01 * z * s).to(torch.bfloat16)
    gq = _tgen(device, seed, "imatrix")
    q = torch.exp(2.0 * torch.randn((n_experts, n_per_row), generator=gq,
                                    device=device)).float()
    zero = torch.as_tensor(moe_zero_experts(n_experts, n_zero, seed),
                           device=device)
    q[zero] = 1e-6
    return x, q


def torch_q4_k_matrix(device, n_rows=11008, n_per_row=4096, seed=1002):
    import torch
    g = _tgen(device, seed, "x")
    z = 0.015 * torch.randn((n_rows, n_per_row), generator=g, device=device)
    s = torch.exp(0.3 * torch.randn((n_rows, 1), generator=g, device=device))
    gq = _tgen(device, seed, "imatrix")
    q = torch.exp(1.5 * torch.randn(n_per_row, generator=gq, device=device))
    return (s * z).float().contiguous(), q.float().contiguous()
