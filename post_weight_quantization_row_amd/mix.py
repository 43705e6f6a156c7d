"""Per-tensor type plans for a layer stack ("3.2 K-quants 与重要性矩阵：量化兵器谱",
section 一, the second step: precision allocated by layer).

The page describes Q4_K_M: the attention projection tensors and the FFN
down-projection tensors, the two kinds most sensitive to quantization, are
raised to 6 bits in proportion, the rest stay at 4 bits, and the file grows
by only about a tenth over plain 4 bits; its FAQ adds that the list of
sensitive tensors differs by architecture. Readings taken here:

* the sensitive roles are the attention value projection (attn_v) and the
  FFN down projection (ffn_down) -- both configurable;
* the share promoted is set by a size budget: the promoted tensors are those roles in
  as many layers as fit in the budget (default +10% over the all-base
  plan), the layers spread evenly over the depth;
* the base type is Q4_K and the 6-bit type this library's Q6_K, the same
  two-level K-quant scaling at 6 bits (Q6_0, the 32-weight 6-bit block,
  can be chosen instead); ``base="q5_k"`` gives the Q5_K_M-shaped plan the
  page names beside Q4_K_M.

``plan_stack`` builds a plan (pure host arithmetic on row sizes),
``describe`` prints it (the dry run), and ``run`` quantizes every tensor on
the GPU with its type and reports the error statistics of each. Command
line: ``python -m post_weight_quantization_row_amd.mix --dry-run``.
"""
from __future__ import annotations

import argparse
import json
import sys
from dataclasses import dataclass, field

from . import qrow, synth


@dataclass
class TensorPlan:
    layer: int
    which: int        # index into synth.STACK_LAYER
    name: str
    n_rows: int
    n_per_row: int
    type: str

    @property
    def weights(self) -> int:
        return self.n_rows * self.n_per_row

    @property
    def bytes(self) -> int:
        return self.n_rows * qrow.qr_row_bytes(self.type, self.n_per_row)


@dataclass
class Plan:
    base: str
    high: str
    roles: tuple
    budget: float
    promoted_layers: list
    tensors: list = field(default_factory=list)

    @property
    def weights(self) -> int:
        return sum(t.weights for t in self.tensors)

    @property
    def bytes(self) -> int:
        return sum(t.bytes for t in self.tensors)

    def base_bytes(self) -> int:
        return sum(t.n_rows * qrow.qr_row_bytes(self.base, t.n_per_row) for t in self.tensors)


def _spread(k: int, n: int) -> list:
    """k layer indices out of n, evenly spread (first and last included)."""
    if k <= 0:
        return []
    if k >= n:
        return list(range(n))
    if k == 1:
        return [n // 2]
    return sorted({round(i * (n - 1) / (k - 1)) for i in range(k)})


def plan_stack(n_layers: int = 32, base: str = "q4_k", high: str = "q6_k",
               roles=("attn_v", "ffn_down"), budget: float = 0.10) -> Plan:
    """A type for every tensor of the 7B-shaped stack (synth.STACK_LAYER per
    layer): `roles` get `high` in the largest evenly spread set of layers
    whose extra size stays within `budget` of the all-`base` size."""
    layer = synth.STACK_LAYER
    unknown = set(roles) - {name for name, *_ in layer}
    if unknown:
        raise ValueError(f"unknown roles {sorted(unknown)}")
    for t in (base, high):
        if qrow.qr_row_bytes(t, 256) == 0 or t == "q8_k128":
            raise ValueError(f"{t} is not a weight type")
    per_layer_base = sum(r * qrow.qr_row_bytes(base, n) for _, _, r, n in layer)
    per_layer_extra = sum(r * (qrow.qr_row_bytes(high, n) - qrow.qr_row_bytes(base, n))
                          for name, _, r, n in layer if name in roles)
    allowed = budget * per_layer_base * n_layers
    k = n_layers if per_layer_extra <= 0 else min(n_layers, int(allowed // per_layer_extra))
    promoted = _spread(k, n_layers)
    plan = Plan(base, high, tuple(roles), budget, promoted)
    for li in range(n_layers):
        for wi, (name, _, r, n) in enumerate(layer):
            t = high if (li in promoted and name in roles) else base
            plan.tensors.append(TensorPlan(li, wi, f"blk.{li}.{name}", r, n, t))
    return plan


def describe(plan: Plan) -> str:
    """The dry run: one line per role and type, then the totals."""
    lines = [f"plan: base {plan.base}, {plan.high} for {', '.join(plan.roles)} in "
             f"{len(plan.promoted_layers)} of {1 + max(t.layer for t in plan.tensors)} layers "
             f"(budget +{100 * plan.budget:.0f}%)",
             f"promoted layers: {plan.promoted_layers}", "",
             f"{'role':10s} {'type':6s} {'tensors':>7s} {'weights':>14s} {'bytes':>14s} {'bpw':>6s}"]
    groups = {}
    for t in plan.tensors:
        role = t.name.split(".", 2)[2]
        g = groups.setdefault((role, t.type), [0, 0, 0])
        g[0] += 1
        g[1] += t.weights
        g[2] += t.bytes
    for (role, ty), (c, w, b) in sorted(groups.items()):
        lines.append(f"{role:10s} {ty:6s} {c:7d} {w:14d} {b:14d} {8 * b / w:6.3f}")
    bb = plan.base_bytes()
    lines += ["", f"total: {plan.weights} weights, {plan.bytes} bytes, {8 * plan.bytes / plan.weights:.3f} bpw; "
                  f"all-{plan.base}: {bb} bytes; +{100 * (plan.bytes / bb - 1):.2f}%"]
    return "\n".join(lines)


def run(plan: Plan, tensor_fn, stats: bool = True):
    """Quantizes every tensor of the plan on the GPU. tensor_fn(t) returns
    (x, imatrix) as CUDA tensors for TensorPlan t. Yields, per tensor, the
    plan entry, the packed rows and (with stats) qr_quantize_stats."""
    for t in plan.tensors:
        x, q = tensor_fn(t)
        packed = qrow.qr_quantize_rows(t.type, x, q)
        st = qrow.qr_quantize_stats(t.type, x, packed, q) if stats else None
        yield t, packed, st


def _main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--dry-run", action="store_true", help="print the plan only")
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--base", default="q4_k")
    ap.add_argument("--high", default="q6_k")
    ap.add_argument("--roles", default="attn_v,ffn_down")
    ap.add_argument("--budget", type=float, default=0.10)
    args = ap.parse_args(argv)
    plan = plan_stack(args.layers, args.base, args.high, tuple(args.roles.split(",")), args.budget)
    print(describe(plan))
    if args.dry_run:
        return 0
    import torch
    dev = torch.device("cuda:0")

    def tensor_fn(t):
        _, x, q = synth.torch_stack_matrix(t.layer, t.which, dev)
        return x, q

    def show(t, st, sb):
        print(json.dumps({"tensor": t.name, "type": t.type, "rel_rmse": round(st["rel_rmse"], 6),
                          "weighted_rel_rmse": round(st["weighted_rel_rmse"], 6),
                          "max_abs_err": st["max_abs_err"], "p95_abs_err": st["p95_abs_err"],
                          "base_rel_rmse": round(sb["rel_rmse"], 6)}), flush=True)
    print(json.dumps(evaluate(plan, tensor_fn, show)))
    return 0


def evaluate(plan: Plan, tensor_fn, on_tensor=None) -> dict:
    """Quantizes the stack with the plan and, for every promoted tensor, also
    with the base type; returns summary() of both. on_tensor(t, stats,
    base_stats) is called per tensor."""
    keys = ("sum_err2", "sum_x2", "sum_werr2", "sum_wx2")
    tot = dict.fromkeys(keys, 0.0)
    tot_base = dict.fromkeys(keys, 0.0)      # the same stack, every tensor at the base type
    for t in plan.tensors:
        x, q = tensor_fn(t)
        st = qrow.qr_quantize_stats(t.type, x, qrow.qr_quantize_rows(t.type, x, q), q)
        sb = st
        if t.type != plan.base:
            sb = qrow.qr_quantize_stats(plan.base, x, qrow.qr_quantize_rows(plan.base, x, q), q)
        for k in keys:
            tot[k] += st[k]
            tot_base[k] += sb[k]
        if on_tensor is not None:
            on_tensor(t, st, sb)
    return summary(plan, tot, tot_base)


def summary(plan: Plan, tot: dict, tot_base: dict) -> dict:
    """Stack-wide relative errors of the plan and of the all-base stack,
    from per-tensor sums of squared errors and squared values (report
    arithmetic over the library's per-tensor sums; the per-tensor ratios
    come from the library itself)."""
    def rel(d, e, x):
        return (d[e] / d[x]) ** 0.5 if d[x] > 0 else 0.0
    return {"stack": "total", "bytes": plan.bytes, "base_bytes": plan.base_bytes(),
            "bpw": 8 * plan.bytes / plan.weights,
            "rel_rmse": rel(tot, "sum_err2", "sum_x2"),
            "weighted_rel_rmse": rel(tot, "sum_werr2", "sum_wx2"),
            "base_rel_rmse": rel(tot_base, "sum_err2", "sum_x2"),
            "base_weighted_rel_rmse": rel(tot_base, "sum_werr2", "sum_wx2")}


if __name__ == "__main__":
    sys.exit(_main())
