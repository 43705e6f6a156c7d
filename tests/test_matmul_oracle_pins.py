"""Pins for the oracle of the product of quantized weights with Q8_K_128
activations ("ik_llama.cpp 量化精度修复实录：用 Q8_K_128 替代 Q8_1 …", sections
修复前的数值隐患 and 修复方案).

The oracle is checked against a library matrix product of the decoded
values, against products computed by hand in exact integer arithmetic on
blocks built byte by byte, and against the Q8_1 hazard the page describes.
"""
import struct

import numpy as np
import pytest

import oracle
from post_weight_quantization_row_amd import synth

F32 = np.float32
TYPES = ["q4_0", "q4_1", "q5_0", "q5_1", "q4_k", "q6_0"]


def q8_block(d: float, q) -> bytes:
    q = np.asarray(q, np.int64)
    bs = q.reshape(4, 32).sum(1)
    return (struct.pack("<f", d) + q.astype(np.int8).tobytes()
            + bs.astype(np.int16).tobytes())


def q4_0_block(d: float, u) -> bytes:
    u = np.asarray(u, np.int64)
    return struct.pack("<f", d) + bytes(int(u[i] | (u[i + 16] << 4)) for i in range(16))


def bits6(vals) -> bytes:
    v = 0
    for j, x in enumerate(vals):
        v |= int(x) << (6 * j)
    return v.to_bytes(6, "little")


def q4_k_block(d16: float, dmin16: float, sc, mn, u) -> bytes:
    u = np.asarray(u, np.int64).reshape(8, 32)
    head = (np.float16(d16).tobytes() + np.float16(dmin16).tobytes()
            + bits6(sc) + bits6(mn))
    qs = b"".join(bytes(int(u[j, i] | (u[j, i + 16] << 4)) for i in range(16)) for j in range(8))
    return head + qs


@pytest.mark.parametrize("t", TYPES)
def test_product_equals_library_matmul_of_decoded_values(t):
    x, q = synth.q4_0_matrix(48, 768 if t != "q4_k" else 1024, seed=71)
    n = x.shape[1]
    w = oracle.quantize_rows(t, x, q)
    a = synth.q8_k128_activations(5, n, seed=72)[0]
    xa = oracle.quantize_q8k128(a)
    y, S = oracle.matmul_q8k128(t, w, xa, 48, 5, n, with_magnitude=True)
    W = oracle.dequantize_rows(t, w, 48, n).astype(np.float64)
    A = oracle.dequantize_rows("q8_k128", xa, 5, n).astype(np.float64)
    ref = A @ W.T                                   # [tokens, rows]
    # the decoders round each value once to float: 2^-24 of (|scale| +
    # |offset| part) per element, summed
    assert np.all(np.abs(y - ref) <= 2.0 ** -23 * S + 1e-300)
    assert np.all(S >= np.abs(y))


def test_exact_integer_products_q4_0():
    rng = np.random.default_rng(73)
    n, R, T = 256, 3, 2
    W, Wv, X, Xv = [], [], [], []
    for r in range(R):
        row = b""
        vals = []
        for b in range(n // 32):
            d = 2.0 ** -int(rng.integers(2, 6))
            u = rng.integers(0, 16, 32)
            row += q4_0_block(d, u)
            vals += [d * (k - 8) for k in u]
        W.append(row)
        Wv.append(vals)
    for t in range(T):
        row = b""
        vals = []
        for b in range(n // 128):
            d = 2.0 ** -int(rng.integers(3, 8))
            q = rng.integers(-127, 128, 128)
            row += q8_block(d, q)
            vals += [d * k for k in q]
        X.append(row)
        Xv.append(vals)
    w = np.frombuffer(b"".join(W), np.uint8)
    x = np.frombuffer(b"".join(X), np.uint8)
    y = oracle.matmul_q8k128("q4_0", w, x, R, T, n)
    from fractions import Fraction
    for t in range(T):
        for r in range(R):
            exact = sum(Fraction(a) * Fraction(b) for a, b in zip(Wv[r], Xv[t]))
            assert y[t, r] == float(exact)


def test_q4_k_offset_part_uses_the_unscaled_sums():
    # All sub-scales 0: every weight is -dmin*mn_j, so the product is
    # -sum_B d_B * sum_{j in B} dmin*mn_j*bsum_j, from the int16 sums alone.
    rng = np.random.default_rng(74)
    mn = np.arange(1, 9)
    u = rng.integers(0, 16, 256)
    w = np.frombuffer(q4_k_block(1.0, 2.0 ** -4, [0] * 8, mn, u), np.uint8)
    q = rng.integers(-127, 128, 256)
    x = np.frombuffer(q8_block(0.5, q[:128]) + q8_block(0.25, q[128:]), np.uint8)
    y = oracle.matmul_q8k128("q4_k", w, x, 1, 1, 256)
    bs = q.reshape(8, 32).sum(1)
    dB = np.repeat([0.5, 0.25], 4)
    assert y[0, 0] == -np.sum(dB * 2.0 ** -4 * mn * bs)
    # and the scale part alone: dmin = 0, sc_j = j + 1
    sc = np.arange(1, 9)
    w2 = np.frombuffer(q4_k_block(2.0 ** -3, 0.0, sc, [0] * 8, u), np.uint8)
    y2 = oracle.matmul_q8k128("q4_k", w2, x, 1, 1, 256)
    uq = (u * q).reshape(8, 32).sum(1)
    assert y2[0, 0] == np.sum(dB * 2.0 ** -3 * sc * uq)


def test_tokens_and_rows_are_independent():
    x, q = synth.q4_0_matrix(20, 512, seed=75)
    w = oracle.quantize_rows("q4_1", x, q)
    a = synth.q8_k128_activations(6, 512, seed=76)[0]
    xa = oracle.quantize_q8k128(a)
    y = oracle.matmul_q8k128("q4_1", w, xa, 20, 6, 512)
    rb, ab = oracle.row_bytes("q4_1", 512), oracle.row_bytes("q8_k128", 512)
    for t in (0, 5):
        for r in (0, 7, 19):
            one = oracle.matmul_q8k128("q4_1", w[r], xa[t], 1, 1, 512)
            assert one[0, 0] == y[t, r]
    assert rb > 0 and ab > 0


def test_q8_1_sum_term_breaks_the_product_where_q8k128_does_not():
    # Activations with one outlier channel above the fp16 range [Q8 修复前的
    # 数值隐患]: for asymmetric weights the Q8_1 formulation takes the offset
    # part from s = d*sum(q) in fp16, which overflows; Q8_K_128 takes it from
    # the int16 sums and stays finite and close to the exact product.
    n = 1024
    x, q = synth.q4_0_matrix(16, n, seed=77)
    w = oracle.quantize_rows("q4_1", x, q)
    a, ch = synth.q8_k128_activations(8, n, seed=78)
    y1 = oracle.matmul_q8_1("q4_1", w, a, 16)
    xa = oracle.quantize_q8k128(a)
    yk = oracle.matmul_q8k128("q4_1", w, xa, 16, 8, n)
    amax = np.abs(a[:, ch]).max(axis=1)
    broken = amax >= 65520                      # tokens whose s overflows
    assert broken.any() and (~broken).any()
    assert np.all(~np.isfinite(y1[broken]))
    assert np.all(np.isfinite(y1[~broken]))
    assert np.all(np.isfinite(yk))
    # where Q8_1 survives, the two quantized products agree closely with the
    # product of the decoded weights and the raw activations
    ref = a.astype(np.float64) @ oracle.dequantize_rows("q4_1", w, 16, n).astype(np.float64).T
    scale = np.abs(a).astype(np.float64) @ np.abs(oracle.dequantize_rows("q4_1", w, 16, n)).T
    assert np.all(np.abs(yk - ref) <= 0.02 * scale)
    assert np.all(np.abs(y1[~broken] - ref[~broken]) <= 0.02 * scale[~broken])


def test_invalid_shapes_are_rejected():
    w = np.zeros(oracle.row_bytes("q4_k", 256), np.uint8)
    x = np.zeros(oracle.row_bytes("q8_k128", 128), np.uint8)
    with pytest.raises(ValueError):
        oracle.matmul_q8k128("q4_k", w, x, 1, 1, 128)
    with pytest.raises(ValueError):
        oracle.matmul_q8k128("q8_k128", x, x, 1, 1, 128)
