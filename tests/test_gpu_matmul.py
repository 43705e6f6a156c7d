"""GPU parity of the product of quantized weight rows with Q8_K_128
activations, against the CPU oracle, through the C-ABI.

Bar (derived from the arithmetic): per 32 weights the integer part
sum(u*q) and its offset fold are exact int32 on both sides; the GPU then
applies the scales in fp32 (a product or fused multiply-add per term, at
most three roundings) and adds the terms in a fixed order, at most n_in/1024
per lane in sequence (32 or 64 lanes per row) and then a butterfly of at
most 6 levels. Standard error analysis bounds the deviation from the exact
sum by (n_in/1024 + 9) * 2^-24 * S (n_in/512 for Q6_K, two terms per 32
weights), where S = sum_i (|scale part_i| + |offset
part_i|) * |a_i| is what the oracle returns with the exact product (in
double). That bound is asserted on every output. Outputs are also
reproducible bit for bit.
"""
import numpy as np
import pytest

import oracle
from post_weight_quantization_row_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TYPES = ["q4_0", "q4_1", "q5_0", "q5_1", "q4_k", "q6_0", "q6_k"]


@pytest.fixture(scope="module")
def qr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from post_weight_quantization_row_amd import qrow
    qrow.load_library()
    return qrow


def say(*a):
    print(*a, flush=True)


def inputs(t, n_out, n_tok, n_in, seed, outliers=False):
    x, q = synth.q4_0_matrix(n_out, n_in, seed=seed)
    w = oracle.quantize_rows(t, x, q)
    if outliers:
        a = synth.q8_k128_activations(n_tok, n_in, seed=seed + 1)[0]
    else:
        a = synth.calib_activations(n_tok, n_in, seed=seed + 1, bf16=False)
    xa = oracle.quantize_q8k128(a)
    return w, xa


def check(qr, t, w, xa, n_in):
    n_out, n_tok = w.shape[0], xa.shape[0]
    y = qr.qr_matmul_q8k128(t, torch.from_numpy(w).cuda(), torch.from_numpy(xa).cuda(), n_in)
    torch.cuda.synchronize()
    yg = y.cpu().numpy().astype(np.float64)
    yo, S = oracle.matmul_q8k128(t, w, xa, n_out, n_tok, n_in, with_magnitude=True)
    # Q6_K adds two fp32 terms per 32 weights (one per 16-weight half)
    bound = (n_in / (512 if t == "q6_k" else 1024) + 9) * 2.0 ** -24 * S
    err = np.abs(yg - yo)
    assert np.all(np.isfinite(yg))
    assert np.all(err <= bound), f"{np.sum(err > bound)} outputs outside the bound; worst {np.max(err / np.maximum(bound, 1e-300)):.3f}x"
    return y


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("n_out,n_tok,n_in", [(37, 1, 256), (16, 3, 768), (100, 8, 1024), (33, 13, 2048),
                                              (5, 2, 8192)])
def test_types_and_shapes(qr, t, n_out, n_tok, n_in):
    say(f"{t} n_out={n_out} n_tok={n_tok} n_in={n_in}")
    w, xa = inputs(t, n_out, n_tok, n_in, seed=n_out + n_in)
    check(qr, t, w, xa, n_in)


@pytest.mark.parametrize("t", ["q4_1", "q4_k"])
def test_outlier_activations_stay_finite(qr, t):
    # activations above the fp16 range: the int16 sums keep the offset fold
    # exact, so every output is finite and within the bound
    say(f"outliers {t}")
    w, xa = inputs(t, 24, 8, 4096, seed=91, outliers=True)
    check(qr, t, w, xa, 4096)


def test_long_rows_use_smaller_token_tiles(qr):
    # 16384-wide rows: a tile of 8 tokens would exceed the activation budget
    say("long rows")
    w, xa = inputs("q4_0", 20, 9, 16384, seed=92)
    check(qr, "q4_0", w, xa, 16384)


@pytest.mark.parametrize("t", ["q4_k", "q6_k", "q5_1"])
@pytest.mark.parametrize("n_tok", [1, 8])
def test_longest_rows(qr, t, n_tok):
    # n_in = QR_MATMUL_MAX_IN: one token per tile (the staged tile would not
    # fit the activation budget), several groups per lane
    say(f"longest rows {t} n_tok={n_tok}")
    w, xa = inputs(t, 24, n_tok, 32768, seed=95 + n_tok)
    check(qr, t, w, xa, 32768)


def test_reproducible(qr):
    w, xa = inputs("q4_k", 64, 8, 4096, seed=93)
    wd, xd = torch.from_numpy(w).cuda(), torch.from_numpy(xa).cuda()
    y1 = qr.qr_matmul_q8k128("q4_k", wd, xd, 4096)
    y2 = qr.qr_matmul_q8k128("q4_k", wd, xd, 4096)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_empty_is_a_no_op(qr):
    w = torch.zeros((0, qr.qr_row_bytes("q4_0", 256)), dtype=torch.uint8, device="cuda")
    x = torch.zeros((3, qr.qr_row_bytes("q8_k128", 256)), dtype=torch.uint8, device="cuda")
    y = qr.qr_matmul_q8k128("q4_0", w, x, 256)
    assert y.shape == (3, 0)


@pytest.mark.parametrize("name", ["mmq_q4_k_11008x4096_t1", "mmq_q4_0_4096x4096_t8"])
def test_full_size_workloads(qr, name):
    say(f"full size {name}")
    t, x, q, a = synth.matmul_sources(name)
    w = oracle.quantize_rows(t, x, q, threads=8)
    xa = oracle.quantize_q8k128(a)
    check(qr, t, w, xa, x.shape[1])
