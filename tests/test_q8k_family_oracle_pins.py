"""Pins for the oracle's Q8_K activation family by block size
("ik_llama.cpp 量化精度修复实录：用 Q8_K_128 替代 Q8_1 …": section 修复方案 fixes
the 128-value block -- fp32 scale, int8 codes, an int16 sum per 32 codes
that is not multiplied by the scale; section 技术启示与后续演进 names Q8_K64
and Q8_K16 as later members that keep the same idea).

Readings: a Q8_K64 block is 64 values, fp32 d, 64 codes and two int16 sums;
a Q8_K16 block is 16 values, fp32 d, 16 codes and one int16 sum over its 16
codes, padded with two zero bytes to 24 (the size of that C struct). The
pins build blocks byte by byte, compare the three block sizes with each
other where they must agree, bound the error from the block maxima with
numpy, and check the product against exact integer arithmetic.
"""
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from post_weight_quantization_row_amd import synth

F32 = np.float32
FAMILY = {"q8_k128": 128, "q8_k64": 64, "q8_k16": 16}


def expected_block(d, codes):
    B = len(codes)
    gs = min(32, B)
    sums = [int(np.sum(codes[g * gs:(g + 1) * gs])) for g in range(B // gs)]
    raw = struct.pack("<f", d) + np.asarray(codes, np.int8).tobytes() + struct.pack(f"<{len(sums)}h", *sums)
    return raw + b"\0" * ((-len(raw)) % 4)


@pytest.mark.parametrize("t", list(FAMILY))
def test_block_bytes_by_hand(t):
    B = FAMILY[t]
    rng = np.random.default_rng(501)
    blocks, want = [], b""
    for b in range(3):
        k = rng.integers(-127, 128, B)
        k[rng.integers(0, B)] = 127 * (1 if b % 2 else -1)   # the block maximum
        d = 2.0 ** -(3 + b)
        blocks.append(k * d)                                  # exact in float
        want += expected_block(d, k)
    x = np.concatenate(blocks).astype(F32)[None, :]
    got = oracle.quantize_q8k(t, x)
    assert oracle.row_bytes(t, 3 * B) == len(want)
    assert got.tobytes() == want
    assert np.array_equal(oracle.dequantize_rows(t, got, 1, 3 * B), x)


def test_block_sizes_agree_where_block_maxima_agree():
    # every 16-value block holds the same maximum magnitude, so all three
    # block sizes pick the same scale and the same codes
    rng = np.random.default_rng(502)
    n = 512
    x = rng.standard_normal((4, n)).astype(F32)
    x = np.clip(x, -2.5, 2.5)
    x[:, ::16] = 3.0
    x[:, 8::32] = -3.0
    q = {t: oracle.quantize_q8k(t, x) for t in FAMILY}
    for t, B in FAMILY.items():
        p = q[t].reshape(4, n // B, -1)
        assert np.all(p[:, :, :4].copy().view(F32) == F32(3.0) / F32(127.0))
    codes = {t: q[t].reshape(4, n // B, -1)[:, :, 4:4 + B].reshape(4, n).view(np.int8)
             for t, B in FAMILY.items()}
    assert np.array_equal(codes["q8_k64"], codes["q8_k128"])
    assert np.array_equal(codes["q8_k16"], codes["q8_k128"])
    s128 = q["q8_k128"].reshape(4, n // 128, 140)[:, :, 132:140].copy().view(np.int16).reshape(4, -1)
    s64 = q["q8_k64"].reshape(4, n // 64, 72)[:, :, 68:72].copy().view(np.int16).reshape(4, -1)
    s16 = q["q8_k16"].reshape(4, n // 16, 24)[:, :, 20:22].copy().view(np.int16).reshape(4, -1)
    assert np.array_equal(s64, s128)
    assert np.array_equal(s16[:, 0::2].astype(int) + s16[:, 1::2], s128)
    assert np.all(q["q8_k16"].reshape(4, n // 16, 24)[:, :, 22:24] == 0)


@pytest.mark.parametrize("t", list(FAMILY))
def test_error_within_half_a_step_of_the_block_maximum(t):
    B = FAMILY[t]
    x, _ = synth.q8_k128_activations(16, 1024, seed=503)
    packed = oracle.quantize_q8k(t, x)
    xh = oracle.dequantize_rows(t, packed, 16, 1024)
    amax = np.abs(x).reshape(16, -1, B).max(axis=2)
    d = (amax / F32(127)).astype(F32)                        # IEEE division in numpy
    dd = packed.reshape(16, 1024 // B, -1)[:, :, :4].copy().view(F32)[:, :, 0]
    assert np.array_equal(dd, d)
    step = np.repeat(d, B, axis=1).astype(np.float64)
    err = np.abs(x.astype(np.float64) - xh)
    # half a step, plus the rounding of x*id and of d*q (a few ulps of x)
    assert np.all(err <= 0.5 * step * (1 + 2.0 ** -20) + 4 * 2.0 ** -24 * np.abs(x))


def test_smaller_blocks_never_coarser_and_closer_on_outliers():
    x, _ = synth.q8_k128_activations(32, 2048, seed=504)
    d = {}
    err = {}
    for t, B in FAMILY.items():
        p = oracle.quantize_q8k(t, x)
        d[t] = np.repeat(p.reshape(32, 2048 // B, -1)[:, :, :4].copy().view(F32)[:, :, 0], B, axis=1)
        err[t] = np.sum((x.astype(np.float64) - oracle.dequantize_rows(t, p, 32, 2048)) ** 2)
    assert np.all(d["q8_k16"] <= d["q8_k64"]) and np.all(d["q8_k64"] <= d["q8_k128"])
    assert err["q8_k16"] < err["q8_k64"] < err["q8_k128"]


def test_zero_and_tiny_blocks_store_zeros():
    x = np.zeros((1, 64), F32)
    x[0, 16:32] = np.float32(1e-45)                  # 127/amax overflows: stored as zeros
    x[0, 32:48] = np.linspace(-1, 1, 16, dtype=F32)
    p = oracle.quantize_q8k("q8_k16", x)
    blocks = p.reshape(4, 24)
    assert not blocks[0].any() and not blocks[1].any() and not blocks[3].any()
    assert blocks[2].any()
    assert not oracle.quantize_q8k("q8_k64", np.zeros((2, 128), F32)).any()


def test_invalid_sizes_are_rejected():
    with pytest.raises(ValueError):
        oracle.quantize_q8k("q8_k64", np.zeros((1, 96), F32))
    with pytest.raises(ValueError):
        oracle.quantize_q8k("q8_k16", np.zeros((1, 40), F32))
    with pytest.raises(ValueError):
        oracle.quantize_q8k("q4_0", np.zeros((1, 64), F32))
    assert oracle.row_bytes("q8_k16", 48) == 72 and oracle.row_bytes("q8_k64", 192) == 216


@pytest.mark.parametrize("act", ["q8_k64", "q8_k16"])
@pytest.mark.parametrize("t", ["q4_0", "q4_1", "q5_1", "q4_k", "q6_0"])
def test_family_product_equals_library_matmul(t, act):
    n = 1024 if t == "q4_k" else 768
    x, q = synth.q4_0_matrix(24, n, seed=505)
    w = oracle.quantize_rows(t, x, q)
    a = synth.q8_k128_activations(5, n, seed=506)[0]
    xa = oracle.quantize_q8k(act, a)
    y, S = oracle.matmul_q8k128(t, w, xa, 24, 5, n, with_magnitude=True, act=act)
    W = oracle.dequantize_rows(t, w, 24, n).astype(np.float64)
    A = oracle.dequantize_rows(act, xa, 5, n).astype(np.float64)
    assert np.all(np.abs(y - A @ W.T) <= 2.0 ** -23 * S + 1e-300)


def test_exact_integer_product_with_two_scales_per_weight_group():
    # Q8_K16 puts two activation scales inside one 32-weight group
    rng = np.random.default_rng(507)
    n = 64
    u = rng.integers(0, 16, n)
    m = 2.0 ** -3
    wrow = b""
    for g in range(2):
        wrow += struct.pack("<ff", 2.0 ** -4, m) + bytes(int(u[32 * g + i] | (u[32 * g + i + 16] << 4))
                                                        for i in range(16))
    wv = [2.0 ** -4 * k + m for k in u]
    xrow = b""
    xv = []
    for b in range(4):
        d = 2.0 ** -int(rng.integers(2, 7))
        k = rng.integers(-127, 128, 16)
        xrow += expected_block(d, k)
        xv += [d * c for c in k]
    y = oracle.matmul_q8k128("q4_1", np.frombuffer(wrow, np.uint8), np.frombuffer(xrow, np.uint8),
                             1, 1, n, act="q8_k16")
    assert y[0, 0] == float(sum(Fraction(a) * Fraction(b) for a, b in zip(wv, xv)))


def test_product_rejects_mismatched_blocks():
    w = np.zeros(oracle.row_bytes("q4_0", 48), np.uint8)
    x = np.zeros(oracle.row_bytes("q8_k16", 48), np.uint8)
    with pytest.raises(ValueError):
        oracle.matmul_q8k128("q4_0", w, x, 1, 1, 48, act="q8_k16")   # 48 is not whole weight blocks
    with pytest.raises(ValueError):
        oracle.matmul_q8k128("q4_0", np.zeros(oracle.row_bytes("q4_0", 96), np.uint8),
                             np.zeros(1, np.uint8), 1, 1, 96, act="q8_k64")
