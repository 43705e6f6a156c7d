"""GPU parity of the row quantizers under every element-importance
weighting ("ik_llama.cpp 量化权重之谜 …", sections 一 and 二), against the CPU
oracle, through the C-ABI.

Bar: as for the default weighting, byte-identical packed rows; the one
tolerated difference is a row whose double sum of x^2 lies at a float
rounding midpoint, which must then equal the oracle run with the
neighbouring sigma2 under the same weighting.
"""
import zlib

import numpy as np
import pytest

import oracle
from post_weight_quantization_row_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

F32 = np.float32
TYPES = ["q4_0", "q4_1", "q5_0", "q5_1", "q4_k", "q6_0", "q6_k", "q5_k"]
MODES = list(oracle.WEIGHTINGS)


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


def sigma2_ambiguous(row):
    s64 = oracle.row_sigma2_f64(row)
    s32 = F32(s64)
    for nb in (np.nextafter(s32, F32(np.inf)), np.nextafter(s32, F32(-np.inf))):
        if abs((float(s32) + float(nb)) / 2 - s64) <= 1e-11 * abs(s64):
            return True
    return False


def assert_rows_equal(t, mode, gpu, ref, x, q):
    for r in np.nonzero((gpu != ref).any(axis=1))[0]:
        ok = False
        if sigma2_ambiguous(x[r]):
            s32 = F32(oracle.row_sigma2_f64(x[r]))
            for s in (np.nextafter(s32, F32(np.inf)), np.nextafter(s32, F32(-np.inf))):
                ok |= np.array_equal(gpu[r], oracle.quantize_row_sigma2_mode(t, x[r], q, s, mode))
        assert ok, f"{t}/{mode}: row {r} differs"


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("t", TYPES)
def test_weighting(qr, t, mode):
    rng = np.random.default_rng(zlib.crc32(f"{t}/{mode}".encode()))
    # (2, 7168) bf16 and (5, 1024) fp32 go through the streaming row kernel
    for bf16, (n_rows, n), qkind in [(False, (5, 2304), "lognormal"), (True, (3, 4096), "none"),
                                     (False, (33, 512), "zero-columns"), (True, (2, 7168), "lognormal"),
                                     (False, (5, 1024), "zero-columns")]:
        if t in ("q4_k", "q5_k", "q6_k") and n % 256:
            n = n // 256 * 256
        x = (0.02 * rng.standard_t(5, (n_rows, n))).astype(F32)
        x[:, ::97] *= 30
        if bf16:
            x = synth.round_to_bf16(x)
        q = {"lognormal": np.exp(1.5 * rng.standard_normal(n)).astype(F32), "none": None,
             "zero-columns": np.where(rng.random(n) < 0.2, 0, np.exp(rng.standard_normal(n))).astype(F32)}[qkind]
        if qkind == "zero-columns":
            q[:64] = 0.0
        say(f"case {t} {mode} bf16={bf16} q={qkind} shape=({n_rows},{n})")
        got = qr.qr_quantize_rows_weighted(t, to_dev(x, bf16), None if q is None else torch.from_numpy(q).cuda(),
                                           mode).cpu().numpy()
        ref = oracle.quantize_rows_weighted(t, x, q, mode, threads=8)
        assert_rows_equal(t, mode, got, ref, x, q)


def test_default_weighting_is_the_plain_quantizer(qr):
    x, q = synth.q4_k_matrix(64, 4096)
    xd, qd = torch.from_numpy(x).cuda(), torch.from_numpy(q).cuda()
    for t in TYPES:
        a = qr.qr_quantize_rows(t, xd, qd)
        b = qr.qr_quantize_rows_weighted(t, xd, qd, "sqrt_sigma2_x2")
        assert torch.equal(a, b)


@pytest.mark.parametrize("mode", ["x2", "abs_x"])
def test_underflowing_importances(qr, mode):
    # magnitudes so small that x^2 underflows: every importance is 0 even
    # after the q = 1 fallback, which must give what the oracle gives
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((4, 256)) * 1e-24).astype(F32)
    x[1] *= 1e20                                      # a normal row beside them
    for t in TYPES:
        got = qr.qr_quantize_rows_weighted(t, torch.from_numpy(x).cuda(), None, mode).cpu().numpy()
        ref = oracle.quantize_rows_weighted(t, x, None, mode)
        assert_rows_equal(t, mode, got, ref, x, None)


def test_full_size_q4_k_every_weighting_sampled(qr):
    # the 11008 x 4096 matrix in the benchmark's launch, every 97th row checked
    x, q = synth.q4_k_matrix()
    xd, qd = torch.from_numpy(x).cuda(), torch.from_numpy(q).cuda()
    rows = np.arange(0, x.shape[0], 97)
    for mode in MODES:
        say(f"full size q4_k {mode}")
        got = qr.qr_quantize_rows_weighted("q4_k", xd, qd, mode).cpu().numpy()[rows]
        ref = oracle.quantize_rows_weighted("q4_k", x[rows], q, mode, threads=8)
        assert_rows_equal("q4_k", mode, got, ref, x[rows], q)
