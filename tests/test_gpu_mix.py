"""A mixed-type plan quantized on the GPU: every tensor with the type the plan
gives it, checked against the oracle on sampled rows (bit for bit), and the
error statistics of one promoted tensor against the oracle's in full."""
import numpy as np
import pytest

import oracle
from post_weight_quantization_row_amd import mix, synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from post_weight_quantization_row_amd import qrow
    qrow.load_library()
    return qrow


def test_two_layer_plan(qr):
    plan = mix.plan_stack(2)
    assert plan.promoted_layers == [1]
    dev = torch.device("cuda:0")

    def tensor_fn(t):
        _, x, q = synth.torch_stack_matrix(t.layer, t.which, dev)
        return x, q

    seen = set()
    errs = {}
    for t, packed, st in mix.run(plan, tensor_fn):
        print(f"mix {t.name} {t.type}", flush=True)
        x, q = tensor_fn(t)
        assert packed.shape == (t.n_rows, qr.qr_row_bytes(t.type, t.n_per_row))
        rows = [0, t.n_rows // 2, t.n_rows - 1]
        xs = x[rows].float().cpu().numpy()
        want = oracle.quantize_rows(t.type, xs, q.cpu().numpy())
        assert np.array_equal(packed[rows].cpu().numpy(), want), t.name
        assert st["n"] == t.weights
        errs[t.name] = st["rel_rmse"]
        seen.add(t.type)
        if t.name == "blk.1.attn_v":
            o = oracle.quantize_stats(t.type, x.float().cpu().numpy(), packed.cpu().numpy(),
                                      q.cpu().numpy())
            assert np.float32(st["max_abs_err"]) == o["max_abs_err"]
            assert np.float32(st["p95_abs_err"]) == o["p95_abs_err"]
            for k in ("sum_err2", "sum_x2", "sum_werr2", "sum_wx2"):
                assert abs(st[k] - o[k]) <= 2.0 * o["n"] * 2.0 ** -53 * o[k], k
    assert seen == {"q4_k", "q6_k"}
    # six bits cut the error of the promoted tensors well below their 4-bit neighbours
    assert errs["blk.1.attn_v"] < 0.5 * errs["blk.0.attn_v"]
    assert errs["blk.1.ffn_down"] < 0.5 * errs["blk.0.ffn_down"]
