"""The pins bite: plausible mistakes planted in a copy of the oracle (a dropped
term, a wrong sign, index or operand) must each fail at least one pin.

Each mutant is one textual change to one of the oracle's C sources, built
with the oracle's own flags into a temporary library and loaded in place of
the real one; then the pin tests (test_oracle_pins.py and
test_imatrix_oracle_pins.py) run against it. All of this is CPU work.
"""
import importlib.util
import inspect
import os
import subprocess

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))

MUTANTS = [
    # row statistic
    ("sigma2: sum instead of mean", "return acc / (double)n;", "return acc;"),
    ("sigma2: |x| instead of x^2", "acc += (double)x[j] * (double)x[j];", "acc += fabs((double)x[j]);"),
    # importances
    ("weight: sigma2 term dropped", "sqrtf(fmaf(x[j], x[j], sigma2))", "sqrtf(fmaf(x[j], x[j], 0.0f))"),
    ("weight: imatrix only (no magnitude term)", "w[j] = q ? q[j] * s : s;", "w[j] = q ? q[j] : s;"),
    ("weight: imatrix by in-block offset", "w[j] = q ? q[j] * s : s;", "w[j] = q ? q[j % 32] * s : s;"),
    # symmetric solver
    ("sym: largest element to the short end", "float is = -c / xm;", "float is = c / xm;"),
    ("sym: suml2 without the level", "S2 = fmaf(w[i] * l, l, S2);", "S2 = fmaf(w[i], l, S2);"),
    ("sym: first trial always wins", "better = lhs > rhs;", "better = 0;"),
    ("sym: scale not refitted", "*d_out = A / B;", "*d_out = 1.0f / bis;"),
    # flips
    ("flip: direction reversed", "? -1.0f : 1.0f;", "? 1.0f : -1.0f;"),
    ("flip: +1 dropped from suml2 update", "fmaf(2.0f * s, L[j], 1.0f)", "fmaf(2.0f * s, L[j], 0.0f)"),
    ("flip: operands of the test transposed", "int better = (A1 * A1) * B > (A * A) * B1;",
     "int better = (A1 * A1) * B1 > (A * A) * B;"),
    ("flip: every move kept", "if (better && B1 > 0.0f && lp >= lo_level && lp <= hi_level) {",
     "if (B1 > 0.0f && lp >= lo_level && lp <= hi_level) {"),
    # asymmetric solver
    ("asym: offset formula uses Sx twice", "mm = (Sll * Sx - Sl * Slx) * r;", "mm = (Sll * Sx - Sl * Sx) * r;"),
    ("asym: levels from x instead of x - lo", "xs[i] = x[i] - lo;", "xs[i] = x[i];"),
    ("asym: flips start from Slx + m*Sl", "float A = fmaf(-mf, bSl, bSlx), B = bSll;", "float A = fmaf(mf, bSl, bSlx), B = bSll;"),
    ("asym: Q4_K offset may be positive", "if (k4 && mm > 0.0) {", "if (0 && k4 && mm > 0.0) {"),
    ("asym: constant-code guard at D > 0", "if (D > Sw * Sll * 0x1p-16) {", "if (D > 0.0) {"),
    ("asym: constant-code guard at 2^-6", "if (D > Sw * Sll * 0x1p-16) {", "if (D > Sw * Sll * 0x1p-6) {"),
    # Q4_K super-block
    ("q4k: sub-scale multiplied by d16", "rintf(a[j] / dA0)", "rintf(a[j] * dA0)"),
    ("q4k: re-round with +dm sign flipped", "rintf((x[32 * j + i] + dm) * id)", "rintf((x[32 * j + i] - dm) * id)"),
    ("q4k: super-scale over 64", "orc_f32_to_f16(amx / 63.0f)", "orc_f32_to_f16(amx / 64.0f)"),
    ("f16: subnormals flushed", "if (e < -14) e = -14;", "if (e < -14) return sign;"),
    # Q8_K_128
    ("q8: 128 levels", "127.0f / amax", "128.0f / amax"),
    ("q8: sums over the wrong codes", "for (int i = 0; i < gs; ++i) s += q[gs * g + i];",
     "for (int i = 0; i < gs; ++i) s += q[i];"),
    ("q8k16: sums over 32 codes", "const int gs = B < 32 ? B : 32;", "const int gs = 32;"),
    ("q8k: padding not zero", "        o[k] = 0;", "        o[k] = 0x55;"),
    ("q8k: amax over the first 16 values", "for (int i = 0; i < B; ++i) amax = fmaxf(amax, fabsf(xb[i]));",
     "for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(xb[i]));"),
    # packing and decoding
    ("pack: high nibble from element i+8", "((u[i + 16] & 15) << 4)", "((u[i + 8] & 15) << 4)"),
    ("decode: symmetric offset dropped", "o[i] = d * (float)((int)u[i] - nmax);", "o[i] = d * (float)((int)u[i]);"),
    # importance-matrix accumulator
    ("imatrix: |a| instead of a^2", "acc[c] += (double)a[c] * (double)a[c];", "acc[c] += fabs((double)a[c]);"),
    ("imatrix: repeated expert counted twice", "                    continue;                       /* already counted */",
     "                    ;"),
    ("imatrix: slot row ignored", "const int64_t row = t * n_slots + (n_slots == 1 ? 0 : s);",
     "const int64_t row = t * n_slots;"),
    ("imatrix: count per slot", "counts[e] += 1;", "counts[e] += n_route;"),
    ("imatrix: mean over count + 1", "/ (double)counts[e])", "/ (double)(counts[e] + 1))"),
    ("imatrix: merge drops the counts", "counts[e] += src_counts[e];", "(void)src_counts;"),
    ("imatrix: merge overwrites the sums", "sums[e * n_cols + c] += src_sums[e * n_cols + c];",
     "sums[e * n_cols + c] = src_sums[e * n_cols + c];"),
    # product with Q8_K_128 activations (and the Q8_1 comparison)
    ("matmul: Q4_0 offset 7", "bv = sym ? d * (type == ORC_Q6_0 ? 32 : five ? 16 : 8) : -m;",
     "bv = sym ? d * (type == ORC_Q6_0 ? 32 : five ? 16 : 7) : -m;"),
    ("matmul: Q4_K scale from the offset field", "av = rd_f16(p) * field6(p + 4, j) * u;",
     "av = rd_f16(p) * field6(p + 10, j) * u;"),
    ("matmul: Q4_K high nibble", "int u = k < 16 ? (qs[k] & 15) : (qs[k - 16] >> 4);\n                if (type",
     "int u = k < 16 ? (qs[k] & 15) : (qs[k - 16] & 15);\n                if (type"),
    ("matmul: activation block stride", "const uint8_t *p = row + blk * ab;", "const uint8_t *p = row + blk * (ab - 4);"),
    ("matmul: offset sign", "acc += (a[i] - b[i]) * xt[i];", "acc += (a[i] + b[i]) * xt[i];"),
    ("q8_1: s without d", "orc_f32_to_f16(d * (float)sum)", "orc_f32_to_f16((float)sum)"),
    # weightings
    ("weighting: |x| without abs", "case ORC_W_ABS_X:           return fabsf(x);",
     "case ORC_W_ABS_X:           return x;"),
    ("weighting: sigma not rooted", "const float sigma = sqrtf(sigma2);", "const float sigma = sigma2;"),
    ("weighting: fallback ignores the mode",
     "if (all_zero) orc_row_weights_mode(x + unit * g, NULL, unit, sigma2, mode, w + unit * g);",
     "if (all_zero) orc_row_weights_mode(x + unit * g, NULL, unit, sigma2, 0, w + unit * g);"),
    ("q6k: importance fallback per 32 weights", "const int unit = type == ORC_Q6_K ? 16 : 32;",
     "const int unit = 32;"),
    ("weighting: imatrix dropped", "w[j] = q ? q[j] * m : m;", "w[j] = m;"),
    # Q6_0
    ("q6_0: plane bits shifted by one", "v |= (uint64_t)((u[i] >> 4) & 3) << (2 * i);",
     "v |= (uint64_t)((u[i] >> 4) & 3) << (2 * i + 1);"),
    ("q6_0: decode offset 31", "o[i] = d * (float)((int)u[i] - 32);", "o[i] = d * (float)((int)u[i] - 31);"),
    ("matmul: Q6_0 offset 16", "bv = sym ? d * (type == ORC_Q6_0 ? 32 : five ? 16 : 8) : -m;",
     "bv = sym ? d * (type == ORC_Q6_0 ? 16 : five ? 16 : 8) : -m;"),
    # weighted Q4_K sub-scale fit
    ("fit: largest value below the top level", "float is = c / vmax;", "float is = (c - 1.0f) / vmax;"),
    ("fit: trials scored without the weights", "S2 = fma((double)W[i] * l, l, S2);", "S2 = fma(l, l, S2);"),
    ("fit: flips move against the residual", "double s = ((signbit(A) != 0) != (signbit(e) != 0)) ? -1.0 : 1.0;",
     "double s = ((signbit(A) != 0) != (signbit(e) != 0)) ? 1.0 : -1.0;"),
    ("fit: sub-block weights all one", "W[j] = sw;", "W[j] = 1.0f;"),
    ("fit: offsets fitted from the scales", "orc_fit_levels_pos(8, b, W, 63,", "orc_fit_levels_pos(8, a, W, 63,"),
    # Q6_K super-block
    ("q6k: super-scale over 128", "orc_f32_to_f16(amx / 127.0f)", "orc_f32_to_f16(amx / 128.0f)"),
    ("q6k: sub-scale sign dropped", "(int8_t)clampf(rintf(dj[j] / dA), -127.0f, 127.0f)",
     "(int8_t)clampf(rintf(fabsf(dj[j]) / dA), -127.0f, 127.0f)"),
    ("q6k: level -32 clamped away", "clampf(rintf(x[16 * j + i] * id), -32.0f, 31.0f)",
     "clampf(rintf(x[16 * j + i] * id), -31.0f, 31.0f)"),
    ("q6k: decoder takes the group's first sub-scale", "(int8_t)p[4 + 2 * g + i / 16];", "(int8_t)p[4 + 2 * g];"),
    ("matmul: Q6_K offset 31", "bv = ds * 32;", "bv = ds * 31;"),
    # Q5_K super-block
    ("q5k: fifth-bit words in reverse order", "out[16 + 4 * j + k] = (uint8_t)(qh >> (8 * k));",
     "out[16 + 4 * (7 - j) + k] = (uint8_t)(qh >> (8 * k));"),
    ("q5k: decoder reads the first fifth-bit word", "uint32_t qh = get_u32(p + 16 + 4 * j);",
     "uint32_t qh = get_u32(p + 16);"),
    ("q5k: levels clamped to 0..15", "0.0f, (float)nmax);", "0.0f, 15.0f);"),
    ("matmul: Q5_K nibbles at the Q4_K offset", "p + (type == ORC_Q4_K ? 16 : 48) + 16 * j;",
     "p + 16 + 16 * j;"),
    ("matmul: Q5_K fifth bit of the wrong word", "u |= ((p[16 + 4 * j + k / 8] >> (k % 8)) & 1) << 4;",
     "u |= ((p[16 + k / 8] >> (k % 8)) & 1) << 4;"),
    # error statistics
    ("stats: percentile rank rounded down", "const int64_t k = (95 * n + 99) / 100;",
     "const int64_t k = (95 * n) / 100;"),
    ("stats: weighted error without q", "qe2 += qi * (ed * ed);", "qe2 += ed * ed;"),
    ("stats: RMSE over the signal", "sums[4] = sqrt(e2 / (double)n);", "sums[4] = sqrt(e2 / x2);"),
    ("stats: weighted relative RMSE without q", "sums[6] = qx2 > 0.0 ? sqrt(qe2 / qx2) : 0.0;",
     "sums[6] = x2 > 0.0 ? sqrt(e2 / x2) : 0.0;"),
    ("stats: maximum of the signed error", "mx = fmaxf(mx, ae[i]);", "mx = fmaxf(mx, e);"),
    ("stats: imatrix by row", "const double qi = q ? (double)q[i % n_per_row] : 1.0;",
     "const double qi = q ? (double)q[i / n_per_row] : 1.0;"),
]


PIN_FILES = ("test_oracle_pins.py", "test_imatrix_oracle_pins.py", "test_matmul_oracle_pins.py",
             "test_weighting_oracle_pins.py", "test_stats_oracle_pins.py", "test_q8k_family_oracle_pins.py",
             "test_subscale_fit_oracle_pins.py", "test_q6k_oracle_pins.py",
             "test_q5k_oracle_pins.py")


def _pins_modules():
    mods = []
    for i, f in enumerate(PIN_FILES):
        spec = importlib.util.spec_from_file_location(f"pins_for_mutants_{i}", os.path.join(HERE, f))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mods.append(mod)
    return mods


def _sources():
    return {p: open(p).read() for p in oracle.SOURCES}


def _pin_calls(mods):
    """(name, callable) for every pin; parametrized pins get one small case."""
    params = {
        "test_sym_brute_force_tiny_blocks": dict(n=3, nmax=4, unit_w=False),
        "test_asym_brute_force_tiny_blocks": dict(n=3, nmax=3),
        "test_exact_lattice_rows_round_trip": dict(t="q4_0", nmax=8, sym=True),
        "test_power_of_two_constant_imatrix_equals_none": dict(t="q4_k"),
        "test_product_equals_library_matmul_of_decoded_values": dict(t="q4_k"),
        "test_each_mode_passes_its_weights_to_the_solver": dict(mode="x2"),
        "test_zero_importance_groups_fall_back_per_mode": dict(mode="x2"),
        "test_power_of_two_scaling_scales_the_scales": dict(mode="abs_x"),
        "test_against_numpy_on_the_decoded_rows": dict(t="q4_k"),
        "test_nearest_rank": dict(n=64, k=61),
        "test_block_bytes_by_hand": dict(t="q8_k16"),
        "test_error_within_half_a_step_of_the_block_maximum": dict(t="q8_k16"),
        "test_family_product_equals_library_matmul": dict(t="q4_1", act="q8_k16"),
        "test_product_with_q6_k_weights": dict(act="q8_k16"),
    }
    calls = []
    for mod in mods:
        for name, fn in inspect.getmembers(mod, inspect.isfunction):
            if not name.startswith("test_") or fn.__module__ != mod.__name__:
                continue
            kw = params.get(name, {})
            calls.append((name, lambda fn=fn, kw=kw: fn(**kw)))
    mod = mods[0]
    # extra parametrizations that exercise the other formats
    calls.append(("round trip q5_1", lambda: mod.test_exact_lattice_rows_round_trip("q5_1", 31, False)))
    calls.append(("round trip q5_0", lambda: mod.test_exact_lattice_rows_round_trip("q5_0", 16, True)))
    calls.append(("round trip q6_0", lambda: mod.test_exact_lattice_rows_round_trip("q6_0", 32, True)))
    calls.append(("brute force sym 4/8", lambda: mod.test_sym_brute_force_tiny_blocks(4, 8, True)))
    wm = mods[3]
    for mode in ("abs_x", "sigma_plus_abs_x"):
        calls.append((f"fallback {mode}", lambda mode=mode: wm.test_zero_importance_groups_fall_back_per_mode(mode)))
    mm = mods[2]
    for t in ("q4_0", "q5_1", "q6_0"):
        calls.append((f"matmul {t}", lambda t=t: mm.test_product_equals_library_matmul_of_decoded_values(t)))
    qm = mods[5]
    for t in ("q8_k64", "q8_k128"):
        calls.append((f"q8k bytes {t}", lambda t=t: qm.test_block_bytes_by_hand(t)))
    calls.append(("q8k64 product", lambda: qm.test_family_product_equals_library_matmul("q4_0", "q8_k64")))
    return calls


def test_every_pin_call_passes_on_the_oracle():
    # a pin that fails (or cannot be called) without a mutant would count
    # as catching every mutant
    for name, call in _pin_calls(_pins_modules()):
        call()


def test_every_mutant_is_distinct_and_applies():
    srcs = _sources()
    for name, old, new in MUTANTS:
        assert sum(t.count(old) for t in srcs.values()) == 1, f"{name}: pattern not found exactly once"
        assert old != new


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    paths = []
    for p, text in _sources().items():
        path = tmp_path / os.path.basename(p)
        path.write_text(text.replace(old, new, 1))
        paths.append(str(path))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", *oracle.CFLAGS, "-I", oracle.HERE, "-o", str(so), *paths, "-lm"],
                   check=True, capture_output=True)
    mods = _pins_modules()
    caught = []
    with oracle.using_library(str(so)):
        for pin, call in _pin_calls(mods):
            try:
                call()
            except Exception as e:          # an assertion or a rejected result
                caught.append((pin, type(e).__name__))
                break
    assert caught, f"no pin caught the mutant: {name}"
