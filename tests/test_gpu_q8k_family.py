"""GPU parity of the Q8_K64 and Q8_K16 activation blocks against the CPU
oracle, through the C-ABI: the quantizer and the decoder byte- and
bit-identical, the error statistics to the statistics bar, and the product
with every weight type within its derived bound.

Product bound: as for Q8_K_128 activations (the integer parts exact, at
most three fp32 roundings per term, a fixed order of additions), with the
number of sequential fp32 additions per lane doubled for 16-value blocks
(two terms per 32-weight group): (n_in/1024 + 9) * 2^-24 * S for Q8_K64 and
(n_in/512 + 9) * 2^-24 * S for Q8_K16 or Q6_K weights (whose two 16-weight
halves carry their own scales), S the oracle's magnitude sum.
"""
import numpy as np
import pytest

import oracle
from post_weight_quantization_row_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

F32 = np.float32
ACTS = ["q8_k64", "q8_k16"]
WEIGHT_TYPES = ["q4_0", "q4_1", "q5_0", "q5_1", "q4_k", "q6_0", "q6_k", "q5_k"]


@pytest.fixture(scope="module")
def qr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from post_weight_quantization_row_amd import qrow
    qrow.load_library()
    return qrow


def say(*a):
    print(*a, flush=True)


def to_dev(x, bf16):
    if bf16:
        return torch.from_numpy(synth.f32_to_bf16_bits(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, F32)).cuda()


def host_values(x, bf16):
    return synth.round_to_bf16(x) if bf16 else np.ascontiguousarray(x, F32)


# shapes with ragged iteration tails (32 blocks per wave iteration for
# Q8_K64, 128 for Q8_K16) and odd block counts (a partial 16-byte vector)
SHAPES = {"q8_k64": [(1, 64), (3, 192), (37, 1024), (5, 7168), (129, 320)],
          "q8_k16": [(1, 16), (3, 48), (7, 1040), (33, 4096), (2, 7168)]}


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("outliers", [False, True])
def test_quantizer_bytes(qr, act, bf16, outliers):
    for i, (n_rows, n) in enumerate(SHAPES[act]):
        say(f"{act} bf16={bf16} outliers={outliers} ({n_rows},{n})")
        if outliers:
            x = synth.q8_k128_activations(n_rows, n, seed=600 + i)[0]
        else:
            x = synth.calib_activations(n_rows, n, seed=610 + i, bf16=False)
        got = qr.qr_quantize_activations_q8k(act, to_dev(x, bf16)).cpu().numpy()
        ref = oracle.quantize_q8k(act, host_values(x, bf16))
        assert np.array_equal(got, ref), f"{act} ({n_rows},{n}) differs"


@pytest.mark.parametrize("act", ACTS)
def test_zero_and_tiny_blocks(qr, act):
    B = 64 if act == "q8_k64" else 16
    x = np.zeros((3, 8 * B), F32)
    x[0, B:2 * B] = F32(1e-45)          # 127/amax not finite: stored as zeros
    x[1, 3 * B:4 * B] = np.linspace(-2, 3, B, dtype=F32)
    x[2, :] = F32(-0.0)
    got = qr.qr_quantize_activations_q8k(act, to_dev(x, False)).cpu().numpy()
    assert np.array_equal(got, oracle.quantize_q8k(act, x))


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("n_rows,n", [(3, 48), (5, 1024), (17, 4096)])
def test_decoder_bits(qr, act, n_rows, n):
    if act == "q8_k64" and n % 64:
        n = 64 * (n // 64 + 1)
    x = synth.q8_k128_activations(n_rows, n, seed=620)[0]
    packed = oracle.quantize_q8k(act, x)
    y = qr.qr_dequantize_rows(act, torch.from_numpy(packed).cuda(), n_rows, n).cpu().numpy()
    assert np.array_equal(y.view(np.uint32), oracle.dequantize_rows(act, packed, n_rows, n).view(np.uint32))


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("bf16", [False, True])
def test_stats(qr, act, bf16):
    x = host_values(synth.q8_k128_activations(24, 2048, seed=630)[0], bf16)
    packed = oracle.quantize_q8k(act, x)
    ws = torch.empty(qr.qr_stats_workspace_bytes(24, 2048), dtype=torch.uint8, device="cuda")
    g = qr.qr_quantize_stats(act, to_dev(x, bf16), torch.from_numpy(packed).cuda(), None, workspace=ws)
    o = oracle.quantize_stats(act, x, packed, None)
    assert g["n"] == o["n"]
    assert F32(g["max_abs_err"]) == o["max_abs_err"] and F32(g["p95_abs_err"]) == o["p95_abs_err"]
    tol = 2.0 * o["n"] * 2.0 ** -53
    for k in ("sum_err2", "sum_x2", "sum_werr2", "sum_wx2"):
        assert abs(g[k] - o[k]) <= tol * o[k], k


def product_check(qr, t, act, w, xa, n_in):
    n_out, n_tok = w.shape[0], xa.shape[0]
    y = qr.qr_matmul_q8k(t, act, torch.from_numpy(w).cuda(), torch.from_numpy(xa).cuda(), n_in)
    yg = y.cpu().numpy().astype(np.float64)
    yo, S = oracle.matmul_q8k128(t, w, xa, n_out, n_tok, n_in, with_magnitude=True, act=act)
    per_lane = n_in / (512 if act == "q8_k16" or t == "q6_k" else 1024)
    bound = (per_lane + 9) * 2.0 ** -24 * S
    err = np.abs(yg - yo)
    assert np.all(np.isfinite(yg))
    assert np.all(err <= bound), f"{np.sum(err > bound)} outside; worst {np.max(err / np.maximum(bound, 1e-300)):.3f}x"
    return y


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("t", WEIGHT_TYPES)
@pytest.mark.parametrize("n_out,n_tok,n_in", [(37, 1, 256), (16, 3, 768), (100, 8, 1024), (33, 13, 2048),
                                              (5, 2, 8192), (9, 5, 1280)])
def test_product(qr, t, act, n_out, n_tok, n_in):
    if t in ("q4_k", "q5_k", "q6_k") and n_in % 256:
        n_in = 256 * (n_in // 256 + 1)
    say(f"product {t} x {act} ({n_out},{n_tok},{n_in})")
    x, q = synth.q4_0_matrix(n_out, n_in, seed=n_out + n_in)
    w = oracle.quantize_rows(t, x, q)
    a = synth.q8_k128_activations(n_tok, n_in, seed=n_tok + n_in)[0]
    product_check(qr, t, act, w, oracle.quantize_q8k(act, a), n_in)


def test_product_q8_k64_unaligned_staging(qr):
    # 192 values: three 64-blocks per row, 216 bytes, so the tile is staged
    # one word at a time
    x, q = synth.q4_0_matrix(40, 192, seed=640)
    w = oracle.quantize_rows("q5_1", x, q)
    a = synth.calib_activations(8, 192, seed=641, bf16=False)
    product_check(qr, "q5_1", "q8_k64", w, oracle.quantize_q8k("q8_k64", a), 192)


def test_q8k128_through_the_generic_entry_point_is_identical(qr):
    x, q = synth.q4_0_matrix(64, 2048, seed=650)
    w = torch.from_numpy(oracle.quantize_rows("q4_k", x, q)).cuda()
    a = synth.calib_activations(6, 2048, seed=651, bf16=False)
    xa = torch.from_numpy(oracle.quantize_q8k128(a)).cuda()
    y1 = qr.qr_matmul_q8k128("q4_k", w, xa, 2048)
    y2 = qr.qr_matmul_q8k("q4_k", "q8_k128", w, xa, 2048)
    assert torch.equal(y1, y2)
    ad = to_dev(a, False)
    assert torch.equal(qr.qr_quantize_activations_q8k128(ad), qr.qr_quantize_activations_q8k("q8_k128", ad))


def test_product_reproducible(qr):
    x, q = synth.q4_0_matrix(128, 4096, seed=660)
    w = torch.from_numpy(oracle.quantize_rows("q4_0", x, q)).cuda()
    a = to_dev(synth.calib_activations(8, 4096, seed=661, bf16=False), False)
    xa = qr.qr_quantize_activations_q8k("q8_k16", a)
    assert torch.equal(qr.qr_matmul_q8k("q4_0", "q8_k16", w, xa, 4096),
                       qr.qr_matmul_q8k("q4_0", "q8_k16", w, xa, 4096))


@pytest.mark.parametrize("act", ACTS)
def test_full_size_activations(qr, act):
    # the 8192 x 7168 activation matrix with outlier channels
    x, _ = synth.q8_k128_activations()
    say(f"full size {act}")
    got = qr.qr_quantize_activations_q8k(act, to_dev(x, False)).cpu().numpy()
    assert np.array_equal(got, oracle.quantize_q8k(act, x, threads=16))


def test_full_size_product_q8_k16(qr):
    # first attention projection of the 7B-shaped stack (4096 x 4096, Q4_0)
    # with a tile of 8 tokens in Q8_K16
    _, x, q = synth.stack_matrix(0, 0)
    w = oracle.quantize_rows("q4_0", x, q, threads=16)
    a = synth.calib_activations(8, 4096, seed=670, bf16=False)
    say("full size product q4_0 x q8_k16")
    product_check(qr, "q4_0", "q8_k16", w, oracle.quantize_q8k("q8_k16", a), 4096)
