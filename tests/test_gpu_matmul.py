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

TYPES = ["q4_0", "q4_1", "q5_0", "q5_1", "q4_k", "q6_0", "q6_k", "q5_k"]


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


@pytest.mark.parametrize("t", ["q4_k", "q6_k", "q5_1", "q5_k"])
@pytest.mark.parametrize("n_tok", [1, 8])
def test_longest_rows(qr, t, n_tok):
    # n_in = QR_MATMUL_MAX_IN: one token per tile (the staged tile would not
    # fit the activation budget), several groups per lane
    say(f"longest rows {t} n_tok={n_tok}")
    w, xa = inputs(t, 24, n_tok, 32768, seed=95 + n_tok)
    check(qr, t, w, xa, 32768)


# ---------------------------------------------------------------------------
# 17 tokens or more with Q8_K_128 or Q8_K64 activations: the int8 matrix-core kernel
# (tiles of 64 tokens x 64 rows; block sums in fp32, accumulation in double)

@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("n_out,n_tok,n_in", [(64, 64, 256), (100, 33, 768), (37, 130, 1024),
                                              (130, 64, 2048), (16, 257, 512), (20, 17, 512), (1, 40, 256)])
def test_many_tokens(qr, t, n_out, n_tok, n_in):
    say(f"many tokens {t} n_out={n_out} n_tok={n_tok} n_in={n_in}")
    w, xa = inputs(t, n_out, n_tok, n_in, seed=3 * n_out + n_tok + n_in)
    y = check(qr, t, w, xa, n_in).cpu().numpy().astype(np.float64)
    # the integer products are exact; the (at most eight) scaled terms of an
    # activation block are summed with fp32 fused multiply-adds, the blocks
    # in double, and the result rounded once to fp32: within
    # 2^-24 |y| + 8 * 2^-24 S of the exact product whatever n_in, plus the
    # double roundings of both sides (the oracle sums n_in terms)
    yo, S = oracle.matmul_q8k128(t, w, xa, n_out, n_tok, n_in, with_magnitude=True)
    tight = 2.0 ** -24 * np.abs(yo) + 8 * 2.0 ** -24 * S + (2 * n_in + 64) * 2.0 ** -52 * S
    assert np.all(np.abs(y - yo) <= tight)


@pytest.mark.parametrize("t", ["q4_0", "q4_k", "q6_k", "q5_k"])
@pytest.mark.parametrize("n_out,n_tok", [(4096, 512), (4033, 449)])
def test_many_tokens_large_tiles(qr, t, n_out, n_tok):
    # enough 64 x 64 tiles (512) for the kernel's 64-row tiles; the smaller
    # cases above take its 32-row tiles
    say(f"many tokens, 64-row tiles {t} n_out={n_out} n_tok={n_tok}")
    w, xa = inputs(t, n_out, n_tok, 256, seed=n_out + n_tok)
    check(qr, t, w, xa, 256)


@pytest.mark.parametrize("t", ["q4_1", "q4_k", "q6_k"])
def test_many_tokens_outlier_activations(qr, t):
    say(f"many tokens, outliers {t}")
    w, xa = inputs(t, 40, 70, 4096, seed=97, outliers=True)
    check(qr, t, w, xa, 4096)


def test_many_tokens_longest_rows(qr):
    say("many tokens, longest rows")
    w, xa = inputs("q5_1", 20, 40, 32768, seed=98)
    check(qr, "q5_1", w, xa, 32768)


def test_many_tokens_reproducible_and_independent_of_the_tiling(qr):
    # the same rows and tokens give the same outputs whatever the tile they
    # fall in: tokens 0..39 alone, and as part of 100 tokens
    w, xa = inputs("q4_k", 70, 100, 2048, seed=99)
    wd, xd = torch.from_numpy(w).cuda(), torch.from_numpy(xa).cuda()
    y1 = qr.qr_matmul_q8k128("q4_k", wd, xd, 2048)
    y2 = qr.qr_matmul_q8k128("q4_k", wd, xd, 2048)
    y3 = qr.qr_matmul_q8k128("q4_k", wd, xd[:40].contiguous(), 2048)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(y1[:40], y3)


def k64_inputs(t, n_out, n_tok, n_in, seed):
    x, q = synth.q4_0_matrix(n_out, n_in, seed=seed)
    w = oracle.quantize_rows(t, x, q)
    a = synth.calib_activations(n_tok, n_in, seed=seed + 1, bf16=False)
    return w, oracle.quantize_q8k("q8_k64", a)


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("n_out,n_tok,n_in", [(100, 33, 768), (37, 130, 1024), (20, 17, 512), (4033, 449, 256)])
def test_many_tokens_q8_k64(qr, t, n_out, n_tok, n_in):
    # Q8_K64 activations on the matrix cores: a 128-value step holds two
    # blocks, each scaling its two groups (32- and 64-row tiles)
    say(f"many tokens q8_k64 {t} n_out={n_out} n_tok={n_tok} n_in={n_in}")
    w, xa = k64_inputs(t, n_out, n_tok, n_in, seed=5 * n_out + n_tok + n_in)
    y = qr.qr_matmul_q8k(t, "q8_k64", torch.from_numpy(w).cuda(), torch.from_numpy(xa).cuda(), n_in)
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    yo, S = oracle.matmul_q8k128(t, w, xa, n_out, n_tok, n_in, with_magnitude=True, act="q8_k64")
    bound = (n_in / (512 if t == "q6_k" else 1024) + 9) * 2.0 ** -24 * S
    tight = 2.0 ** -24 * np.abs(yo) + 8 * 2.0 ** -24 * S + (2 * n_in + 64) * 2.0 ** -52 * S
    assert np.all(np.abs(y - yo) <= bound)
    assert np.all(np.abs(y - yo) <= tight)


@pytest.mark.parametrize("act", ["q8_k64", "q8_k16"])
def test_many_tokens_other_activation_blocks(qr, act):
    # Q8_K16 keeps the lane-parallel kernel at any token count (a group
    # spans two of its blocks); Q8_K64 takes the matrix cores
    say(f"many tokens {act}")
    x, q = synth.q4_0_matrix(48, 1024, seed=96)
    w = oracle.quantize_rows("q4_k", x, q)
    a = synth.calib_activations(40, 1024, seed=196, bf16=False)
    xa = oracle.quantize_q8k(act, a)
    y = qr.qr_matmul_q8k("q4_k", act, torch.from_numpy(w).cuda(), torch.from_numpy(xa).cuda(), 1024)
    torch.cuda.synchronize()
    yo, S = oracle.matmul_q8k128("q4_k", w, xa, 48, 40, 1024, with_magnitude=True, act=act)
    bound = (1024 / 512 + 9) * 2.0 ** -24 * S
    assert np.all(np.abs(y.cpu().numpy().astype(np.float64) - yo) <= bound)


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


def test_full_size_512_tokens_sampled(qr):
    # the 11008x4096 Q4_K matrix with 512 tokens, quantized on the GPU in the
    # launch configuration the benchmark times; 96 rows x all tokens checked
    # against the oracle's product of the same packed bytes
    say("full size mmq_q4_k_11008x4096_t512 (sampled rows)")
    t, x, q, a = synth.matmul_sources("mmq_q4_k_11008x4096_t512")
    xd, qd, ad = (torch.from_numpy(v).cuda() for v in (x, q, a))
    w = qr.qr_quantize_rows(t, xd, qd)
    xa = qr.qr_quantize_activations_q8k("q8_k128", ad)
    y = qr.qr_matmul_q8k128(t, w, xa, x.shape[1]).cpu().numpy().astype(np.float64)
    rows = np.sort(np.random.default_rng(1014).choice(x.shape[0], 96, replace=False))
    rows[-1] = x.shape[0] - 1
    ws = w.cpu().numpy()[rows]
    yo, S = oracle.matmul_q8k128(t, ws, xa.cpu().numpy(), len(rows), a.shape[0], x.shape[1],
                                 with_magnitude=True)
    bound = (x.shape[1] / 1024 + 9) * 2.0 ** -24 * S
    assert np.all(np.abs(y[:, rows] - yo) <= bound)
