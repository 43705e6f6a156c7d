"""CPU oracle for importance-matrix-weighted row quantization.

TEST INFRASTRUCTURE ONLY. This package loads ``liborc_qrow.so`` (a plain C
implementation compiled with gcc, see ``qrow_oracle.c``) through ctypes and
exposes it on numpy arrays. Only the test-suite, the package smoke check and
the benchmark's CPU-baseline leg may import it; the GPU library never does.

Every function here only marshals arguments: all arithmetic of the method is
in the C file.
"""
from __future__ import annotations

import contextlib
import ctypes as C
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qrow_oracle.c")
SOURCES = [SRC, os.path.join(HERE, "imatrix_oracle.c"),
           os.path.join(HERE, "matmul_oracle.c"),
           os.path.join(HERE, "stats_oracle.c")]
LIB = os.path.join(HERE, "liborc_qrow.so")

Q4_0, Q4_1, Q5_0, Q5_1, Q4_K, Q8_K128, Q6_0, Q8_K64, Q8_K16, Q6_K, Q5_K = range(11)
WEIGHTINGS = {"sqrt_sigma2_x2": 0, "x2": 1, "abs_x": 2, "sigma2_plus_x2": 3,
              "sigma_plus_abs_x": 4, "imatrix_only": 5}
TYPE_NAMES = {"q4_0": Q4_0, "q4_1": Q4_1, "q5_0": Q5_0, "q5_1": Q5_1,
              "q4_k": Q4_K, "q8_k128": Q8_K128, "q6_0": Q6_0,
              "q8_k64": Q8_K64, "q8_k16": Q8_K16, "q6_k": Q6_K, "q5_k": Q5_K}
ACT_TYPES = ("q8_k128", "q8_k64", "q8_k16")
FITS = {"max": 0, "weighted": 1}   # Q4_K sub-scale choice

_lib = None
_lock = threading.Lock()

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile liborc_qrow.so with gcc (float contraction off)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, *SOURCES, "-lm"],
                       check=True, cwd=HERE)
        os.replace(tmp, LIB)
    return LIB


_override = None


@contextlib.contextmanager
def using_library(path: str):
    """Temporarily routes every call to another build of the oracle (the
    mutation tests load deliberately broken copies this way)."""
    global _override
    prev = _override
    _override = _load(path)
    try:
        yield
    finally:
        _override = prev


def lib():
    global _lib
    if _override is not None:
        return _override
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB):
                build(force=True)
            _lib = _load(LIB)
    return _lib


def _load(path):
    L = C.CDLL(path)
    f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
    u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
    i8p = np.ctypeslib.ndpointer(np.int8, flags="C_CONTIGUOUS")
    i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
    vp = C.c_void_p
    i64 = C.c_int64
    L.orc_solver_constants.argtypes = [i32p]
    L.orc_block_bytes.argtypes = [C.c_int]
    L.orc_block_bytes.restype = C.c_size_t
    L.orc_block_elems.argtypes = [C.c_int]
    L.orc_row_bytes.argtypes = [C.c_int, i64]
    L.orc_row_bytes.restype = C.c_size_t
    L.orc_row_sigma2.argtypes = [f32p, i64]
    L.orc_row_sigma2.restype = C.c_float
    L.orc_row_sigma2_f64.argtypes = [f32p, i64]
    L.orc_row_sigma2_f64.restype = C.c_double
    L.orc_row_weights.argtypes = [f32p, vp, i64, C.c_float, f32p]
    L.orc_solve_sym.argtypes = [C.c_int, f32p, f32p, C.c_int, C.c_int,
                                C.c_int, i8p, f32p, i32p]
    L.orc_solve_asym.argtypes = [C.c_int, f32p, f32p, C.c_int, C.c_int,
                                 C.c_int, C.c_int, u8p, f32p, f32p,
                                 i32p]
    L.orc_quantize_rows.argtypes = [C.c_int, vp, vp, i64, i64, vp]
    L.orc_quantize_rows_grouped.argtypes = [C.c_int, vp, vp, i64, i64,
                                            i64, vp]
    L.orc_quantize_row_sigma2.argtypes = [C.c_int, f32p, vp, i64,
                                          C.c_float, u8p]
    L.orc_quantize_q8k128.argtypes = [vp, i64, i64, vp]
    L.orc_quantize_q8k.argtypes = [C.c_int, vp, i64, i64, vp]
    L.orc_fit_levels_pos.argtypes = [C.c_int, f32p, f32p, C.c_int, C.c_int, C.c_int, u8p, f32p, i32p]
    L.orc_quantize_rows_ex.argtypes = [C.c_int, vp, vp, i64, i64, i64, C.c_int, C.c_int, vp]
    L.orc_quantize_row_sigma2_ex.argtypes = [C.c_int, f32p, vp, i64, C.c_float, C.c_int, C.c_int, u8p]
    L.orc_row_weights_mode.argtypes = [f32p, vp, i64, C.c_float, C.c_int, f32p]
    L.orc_quantize_rows_weighted.argtypes = [C.c_int, vp, vp, i64, i64, C.c_int, vp]
    L.orc_quantize_row_sigma2_mode.argtypes = [C.c_int, f32p, vp, i64, C.c_float,
                                               C.c_int, u8p]
    L.orc_dequantize_rows.argtypes = [C.c_int, vp, i64, i64, vp]
    f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
    i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
    L.orc_imatrix_accumulate.argtypes = [f32p, i64, i64, i64, vp, i64, i64,
                                         f64p, i64p]
    L.orc_imatrix_merge.argtypes = [f64p, i64p, f64p, i64p, i64, i64]
    L.orc_imatrix_finalize.argtypes = [f64p, i64p, i64, i64, f32p]
    f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
    L.orc_matmul_q8k128.argtypes = [C.c_int, u8p, u8p, i64, i64, i64, f64p, vp]
    L.orc_matmul_q8k.argtypes = [C.c_int, C.c_int, u8p, u8p, i64, i64, i64, f64p, vp]
    L.orc_matmul_q8_1.argtypes = [C.c_int, u8p, f32p, i64, i64, i64, f32p]
    L.orc_quantize_stats.argtypes = [C.c_int, f32p, u8p, vp, i64, i64, f64p, f32p, f32p]
    L.orc_f32_to_f16.argtypes = [C.c_float]
    L.orc_f32_to_f16.restype = C.c_uint16
    L.orc_f16_to_f32.argtypes = [C.c_uint16]
    L.orc_f16_to_f32.restype = C.c_float
    return L


def _tid(t) -> int:
    return TYPE_NAMES[t] if isinstance(t, str) else int(t)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def solver_constants() -> dict:
    c = np.zeros(6, np.int32)
    lib().orc_solver_constants(c)
    return {"cand_step_x4": int(c[0]), "sym_cand": int(c[1]),
            "sym_flip_passes": int(c[2]), "asym_cand": int(c[3]),
            "asym_flip_passes": int(c[4]), "max_block": int(c[5])}


def block_elems(t) -> int:
    return lib().orc_block_elems(_tid(t))


def block_bytes(t) -> int:
    return lib().orc_block_bytes(_tid(t))


def row_bytes(t, n_per_row: int) -> int:
    return lib().orc_row_bytes(_tid(t), n_per_row)


def row_sigma2(x) -> np.float32:
    x = _f32(x)
    return np.float32(lib().orc_row_sigma2(x, x.size))


def row_sigma2_f64(x) -> float:
    x = _f32(x)
    return float(lib().orc_row_sigma2_f64(x, x.size))


def row_weights(x, q, sigma2) -> np.ndarray:
    x = _f32(x)
    qq = None if q is None else _f32(q)
    w = np.empty_like(x)
    lib().orc_row_weights(x, _ptr(qq), x.size, np.float32(sigma2), w)
    return w


def solve_sym(x, w, nmax, K=None, F=None):
    """Returns (levels int8 in [-nmax, nmax-1], d, info)."""
    c = solver_constants()
    K = c["sym_cand"] if K is None else K
    F = c["sym_flip_passes"] if F is None else F
    x, w = _f32(x), _f32(w)
    l = np.zeros(x.size, np.int8)
    d = np.zeros(1, np.float32)
    info = np.zeros(4, np.int32)
    rc = lib().orc_solve_sym(x.size, x, w, nmax, K, F, l, d, info)
    if rc != 0:
        raise ValueError("orc_solve_sym: invalid arguments")
    return l, d[0], info


def fit_levels_pos(v, W, nmax=63, K=None, F=None):
    """Weighted fit of non-negative values v ~ d*l, l in 0..nmax (the Q4_K
    sub-scale fit); returns (levels uint8, d, info)."""
    c = solver_constants()
    K = c["sym_cand"] if K is None else K
    F = c["sym_flip_passes"] if F is None else F
    v, W = _f32(v), _f32(W)
    l = np.zeros(v.size, np.uint8)
    d = np.zeros(1, np.float32)
    info = np.zeros(4, np.int32)
    rc = lib().orc_fit_levels_pos(v.size, v, W, nmax, K, F, l, d, info)
    if rc != 0:
        raise ValueError("orc_fit_levels_pos: invalid arguments")
    return l, d[0], info


def solve_asym(x, w, nmax, K=None, F=None, k4=False):
    """Returns (levels uint8 in [0, nmax], d, m, info)."""
    c = solver_constants()
    K = c["asym_cand"] if K is None else K
    F = c["asym_flip_passes"] if F is None else F
    x, w = _f32(x), _f32(w)
    l = np.zeros(x.size, np.uint8)
    d = np.zeros(1, np.float32)
    m = np.zeros(1, np.float32)
    info = np.zeros(4, np.int32)
    rc = lib().orc_solve_asym(x.size, x, w, nmax, K, F, int(k4), l, d, m, info)
    if rc != 0:
        raise ValueError("orc_solve_asym: invalid arguments")
    return l, d[0], m[0], info


def _wid(mode) -> int:
    return WEIGHTINGS[mode] if isinstance(mode, str) else int(mode)


def row_weights_mode(x, q, sigma2, mode) -> np.ndarray:
    x = _f32(x)
    qq = None if q is None else _f32(q)
    w = np.empty_like(x)
    lib().orc_row_weights_mode(x, _ptr(qq), x.size, np.float32(sigma2), _wid(mode), w)
    return w


def quantize_rows_weighted(t, x, imatrix, mode, threads: int = 1) -> np.ndarray:
    """quantize_rows with a weighting (name or number, see WEIGHTINGS)."""
    t = _tid(t)
    x = _f32(x)
    n_rows, n = x.shape
    rb = row_bytes(t, n)
    q = None if imatrix is None else _f32(imatrix)
    out = np.zeros((n_rows, rb), np.uint8)
    m = _wid(mode)

    def run(r0, r1):
        if r1 > r0:
            rc = lib().orc_quantize_rows_weighted(t, _ptr(x[r0:r1]), _ptr(q), r1 - r0,
                                                  n, m, _ptr(out[r0:r1]))
            if rc != 0:
                raise ValueError("orc_quantize_rows_weighted failed")

    _rows_parallel(n_rows, run, threads)
    return out


def quantize_rows_ex(t, x, imatrix=None, mode=0, fit="max", threads: int = 1) -> np.ndarray:
    """Rows x [n_rows, n] with a weighting and a Q4_K sub-scale fit ("max"
    or "weighted"). imatrix is None, [n], or [n_groups, n] for n_groups
    equal runs of rows (row r uses group r // (n_rows / n_groups))."""
    t = _tid(t)
    x = _f32(x)
    n_rows, n = x.shape
    rb = row_bytes(t, n)
    q = None if imatrix is None else _f32(imatrix).reshape(-1, n)
    G = 1 if q is None else q.shape[0]
    if n_rows % G:
        raise ValueError("imatrix groups do not divide the rows")
    rpg = n_rows // G
    out = np.zeros((n_rows, rb), np.uint8)
    m = _wid(mode)
    f = FITS[fit] if isinstance(fit, str) else int(fit)
    for g in range(G):
        qg = None if q is None else q[g]

        def run(r0, r1, g=g, qg=qg):
            if r1 > r0:
                a, b = g * rpg + r0, g * rpg + r1
                rc = lib().orc_quantize_rows_ex(t, _ptr(x[a:b]), _ptr(qg), 1, b - a, n, m, f,
                                                _ptr(out[a:b]))
                if rc != 0:
                    raise ValueError("orc_quantize_rows_ex failed")

        _rows_parallel(rpg, run, threads)
    return out


def quantize_row_sigma2_ex(t, x, q, sigma2, mode=0, fit="max") -> np.ndarray:
    t = _tid(t)
    x = _f32(x).ravel()
    qq = None if q is None else _f32(q)
    out = np.zeros(row_bytes(t, x.size), np.uint8)
    f = FITS[fit] if isinstance(fit, str) else int(fit)
    rc = lib().orc_quantize_row_sigma2_ex(t, x, _ptr(qq), x.size, np.float32(sigma2), _wid(mode), f, out)
    if rc != 0:
        raise ValueError("orc_quantize_row_sigma2_ex failed")
    return out


def quantize_row_sigma2_mode(t, x, q, sigma2, mode) -> np.ndarray:
    t = _tid(t)
    x = _f32(x).ravel()
    qq = None if q is None else _f32(q)
    out = np.zeros(row_bytes(t, x.size), np.uint8)
    rc = lib().orc_quantize_row_sigma2_mode(t, x, _ptr(qq), x.size,
                                            np.float32(sigma2), _wid(mode), out)
    if rc != 0:
        raise ValueError("orc_quantize_row_sigma2_mode failed")
    return out


def _rows_parallel(n_rows, fn, threads):
    """Runs fn(r0, r1) over contiguous row ranges on `threads` threads
    (ctypes releases the GIL during each foreign call)."""
    threads = max(1, min(threads, n_rows)) if n_rows else 1
    bounds = np.linspace(0, n_rows, threads + 1).astype(np.int64)
    if threads == 1:
        fn(0, n_rows)
        return
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda i: fn(int(bounds[i]), int(bounds[i + 1])),
                    range(threads)))


def quantize_rows(t, x, imatrix=None, threads: int = 1) -> np.ndarray:
    """x: [n_rows, n_per_row] float32. Returns uint8 [n_rows, row_bytes]."""
    t = _tid(t)
    x = _f32(x)
    n_rows, n = x.shape
    rb = row_bytes(t, n)
    if rb == 0:
        raise ValueError("n_per_row is not a multiple of the block length")
    q = None if imatrix is None else _f32(imatrix)
    out = np.zeros((n_rows, rb), np.uint8)

    def run(r0, r1):
        if r1 > r0:
            rc = lib().orc_quantize_rows(t, _ptr(x[r0:r1]), _ptr(q), r1 - r0,
                                         n, _ptr(out[r0:r1]))
            if rc != 0:
                raise ValueError("orc_quantize_rows failed")

    _rows_parallel(n_rows, run, threads)
    return out


def quantize_rows_grouped(t, x, imatrix, rows_per_group: int,
                          threads: int = 1) -> np.ndarray:
    """x: [n_groups*rows_per_group, n] float32; imatrix: [n_groups, n]."""
    t = _tid(t)
    x = _f32(x)
    q = _f32(imatrix)
    n_rows, n = x.shape
    rb = row_bytes(t, n)
    out = np.zeros((n_rows, rb), np.uint8)

    def run(r0, r1):
        # rows [r0, r1) split at group boundaries
        r = r0
        while r < r1:
            g = r // rows_per_group
            e = min(r1, (g + 1) * rows_per_group)
            rc = lib().orc_quantize_rows(t, _ptr(x[r:e]), _ptr(q[g]), e - r, n,
                                         _ptr(out[r:e]))
            if rc != 0:
                raise ValueError("orc_quantize_rows failed")
            r = e

    _rows_parallel(n_rows, run, threads)
    return out


def quantize_row_sigma2(t, x, q, sigma2) -> np.ndarray:
    t = _tid(t)
    x = _f32(x).ravel()
    qq = None if q is None else _f32(q)
    out = np.zeros(row_bytes(t, x.size), np.uint8)
    rc = lib().orc_quantize_row_sigma2(t, x, _ptr(qq), x.size,
                                       np.float32(sigma2), out)
    if rc != 0:
        raise ValueError("orc_quantize_row_sigma2 failed")
    return out


def quantize_q8k(t, x, threads: int = 1) -> np.ndarray:
    """Activation rows x [n_rows, n] to the Q8_K format t (q8_k128, q8_k64
    or q8_k16)."""
    t = _tid(t)
    x = _f32(x)
    n_rows, n = x.shape
    rb = row_bytes(t, n)
    if rb == 0 or t not in (Q8_K128, Q8_K64, Q8_K16):
        raise ValueError("not a Q8_K type, or n_per_row is not a multiple of its block")
    out = np.zeros((n_rows, rb), np.uint8)

    def run(r0, r1):
        if r1 > r0:
            lib().orc_quantize_q8k(t, _ptr(x[r0:r1]), r1 - r0, n, _ptr(out[r0:r1]))

    _rows_parallel(n_rows, run, threads)
    return out


def quantize_q8k128(x, threads: int = 1) -> np.ndarray:
    x = _f32(x)
    n_rows, n = x.shape
    rb = row_bytes(Q8_K128, n)
    if rb == 0:
        raise ValueError("n_per_row is not a multiple of 128")
    out = np.zeros((n_rows, rb), np.uint8)

    def run(r0, r1):
        if r1 > r0:
            lib().orc_quantize_q8k128(_ptr(x[r0:r1]), r1 - r0, n,
                                      _ptr(out[r0:r1]))

    _rows_parallel(n_rows, run, threads)
    return out


def dequantize_rows(t, packed, n_rows: int, n_per_row: int) -> np.ndarray:
    t = _tid(t)
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    if p.size != n_rows * row_bytes(t, n_per_row):
        raise ValueError("packed buffer has the wrong size")
    out = np.zeros((n_rows, n_per_row), np.float32)
    rc = lib().orc_dequantize_rows(t, _ptr(p), n_rows, n_per_row, _ptr(out))
    if rc != 0:
        raise ValueError("orc_dequantize_rows failed")
    return out


def imatrix_new(n_experts: int, n_cols: int):
    """A fresh accumulator state: (sums float64 [E, C], counts int64 [E])."""
    return np.zeros((n_experts, n_cols), np.float64), np.zeros(n_experts, np.int64)


def imatrix_accumulate(state, act, ids=None):
    """Adds one batch to state in place. act: [T, C] (one row per token) or
    [T, S, C] with S == top_k (one row per routed slot); ids: [T, top_k]
    int32 expert ids, or None for a dense tensor."""
    sums, counts = state
    a = _f32(act)
    if a.ndim == 2:
        a = a[:, None, :]
    T, S, Cc = a.shape
    E = sums.shape[0]
    if sums.shape != (E, Cc) or counts.shape != (E,):
        raise ValueError("state does not match the activations")
    if ids is None:
        k = 0
        pid = None
    else:
        idv = np.ascontiguousarray(ids, dtype=np.int32)
        if idv.ndim != 2 or idv.shape[0] != T:
            raise ValueError("ids must be [n_tokens, top_k]")
        k = idv.shape[1]
        pid = idv.ctypes.data_as(C.c_void_p)
    rc = lib().orc_imatrix_accumulate(a, T, S, Cc, pid, k, E, sums, counts)
    if rc != 0:
        raise ValueError("orc_imatrix_accumulate: invalid arguments")
    return state


def imatrix_merge(state, other):
    """Adds other's sums and counts into state (in place)."""
    sums, counts = state
    s2 = np.ascontiguousarray(other[0], np.float64)
    c2 = np.ascontiguousarray(other[1], np.int64)
    if s2.shape != sums.shape or c2.shape != counts.shape:
        raise ValueError("states differ in shape")
    lib().orc_imatrix_merge(sums, counts, s2, c2, sums.shape[0], sums.shape[1])
    return state


def imatrix_finalize(state) -> np.ndarray:
    """Importances q [E, C] float32 (0 for experts with no tokens)."""
    sums, counts = state
    q = np.zeros(sums.shape, np.float32)
    lib().orc_imatrix_finalize(sums, counts, sums.shape[0], sums.shape[1], q)
    return q


def matmul_q8k128(t, w_packed, x_packed, n_out: int, n_tok: int, n_in: int,
                  with_magnitude: bool = False, act="q8_k128"):
    """y [n_tok, n_out] float64 = dequant(w) @ dequant(x).T over the exact
    decoded values; with_magnitude also returns the bound magnitude S. act
    names the activations' Q8_K block size (q8_k128, q8_k64, q8_k16)."""
    t = _tid(t)
    a = _tid(act)
    w = np.ascontiguousarray(w_packed, dtype=np.uint8).reshape(-1)
    x = np.ascontiguousarray(x_packed, dtype=np.uint8).reshape(-1)
    if w.size != n_out * row_bytes(t, n_in) or x.size != n_tok * row_bytes(a, n_in):
        raise ValueError("packed buffers have the wrong size")
    y = np.zeros((n_tok, n_out), np.float64)
    s = np.zeros((n_tok, n_out), np.float64) if with_magnitude else None
    rc = lib().orc_matmul_q8k(t, a, w, x, n_out, n_tok, n_in, y, _ptr(s))
    if rc != 0:
        raise ValueError("orc_matmul_q8k: invalid arguments")
    return (y, s) if with_magnitude else y


def matmul_q8_1(t, w_packed, x, n_out: int):
    """The Q8_1 formulation (fp16 d, fp16 s) for Q4_1/Q5_1 weights and fp32
    activations x [n_tok, n_in]: y [n_tok, n_out] float32."""
    t = _tid(t)
    xv = _f32(x)
    n_tok, n_in = xv.shape
    w = np.ascontiguousarray(w_packed, dtype=np.uint8).reshape(-1)
    y = np.zeros((n_tok, n_out), np.float32)
    rc = lib().orc_matmul_q8_1(t, w, xv, n_out, n_tok, n_in, y)
    if rc != 0:
        raise ValueError("orc_matmul_q8_1: invalid arguments")
    return y


def quantize_stats(t, x, packed, imatrix=None) -> dict:
    """Error statistics of packed rows against x (float32 [n_rows, n]):
    sums of e^2, x^2, q e^2, q x^2 (double), max |e| and the nearest-rank
    95th percentile of |e|, e = x - decoded in float, and the RMSE, relative
    RMSE and importance-weighted relative RMSE."""
    t = _tid(t)
    xv = _f32(x)
    n_rows, n = xv.shape
    p = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1)
    if p.size != n_rows * row_bytes(t, n):
        raise ValueError("packed buffer has the wrong size")
    q = None if imatrix is None else _f32(imatrix)
    sums = np.zeros(7, np.float64)
    mx = np.zeros(1, np.float32)
    p95 = np.zeros(1, np.float32)
    rc = lib().orc_quantize_stats(t, xv, p, _ptr(q), n_rows, n, sums, mx, p95)
    if rc != 0:
        raise ValueError("orc_quantize_stats: invalid arguments")
    return {"sum_err2": sums[0], "sum_x2": sums[1], "sum_werr2": sums[2],
            "sum_wx2": sums[3], "max_abs_err": mx[0], "p95_abs_err": p95[0],
            "n": n_rows * n, "rmse": sums[4], "rel_rmse": sums[5],
            "weighted_rel_rmse": sums[6]}


def f32_to_f16_bits(v: float) -> int:
    return int(lib().orc_f32_to_f16(np.float32(v)))


def f16_bits_to_f32(h: int) -> float:
    return float(lib().orc_f16_to_f32(int(h)))
