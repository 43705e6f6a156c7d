"""Python binding of libqrow.so (argument marshalling only).

Every function has the name of the C entry point it calls (see
include/qrow.h, include/qrow_imatrix.h, include/qrow_matmul.h and
include/qrow_stats.h) and takes torch tensors that live on the GPU; all arithmetic
runs in the library's HIP kernels. torch provides device memory and the
stream. There is no CPU fallback: without the built library or a GPU the
calls raise.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# QROW_LIBRARY may name another build of the same library (A/B timing).
LIB_PATH = os.environ.get("QROW_LIBRARY") or os.path.join(HERE, "libqrow.so")

QR_Q4_0, QR_Q4_1, QR_Q5_0, QR_Q5_1, QR_Q4_K, QR_Q8_K128, QR_Q6_0, QR_Q8_K64, QR_Q8_K16, QR_Q6_K, QR_Q5_K = range(11)
QR_F32, QR_BF16 = 0, 1
# element-importance weightings (qr_weighting)
WEIGHTINGS = {"sqrt_sigma2_x2": 0, "x2": 1, "abs_x": 2, "sigma2_plus_x2": 3,
              "sigma_plus_abs_x": 4, "imatrix_only": 5}
TYPES = {"q4_0": QR_Q4_0, "q4_1": QR_Q4_1, "q5_0": QR_Q5_0, "q5_1": QR_Q5_1,
         "q4_k": QR_Q4_K, "q8_k128": QR_Q8_K128, "q6_0": QR_Q6_0,
         "q8_k64": QR_Q8_K64, "q8_k16": QR_Q8_K16, "q6_k": QR_Q6_K, "q5_k": QR_Q5_K}
ACT_TYPES = ("q8_k128", "q8_k64", "q8_k16")
FITS = {"max": 0, "weighted": 1}   # qr_subscale_fit
ERRORS = {-1: "QR_EINVAL_TYPE", -2: "QR_EINVAL_SHAPE", -3: "QR_EINVAL_PTR",
          -4: "QR_EOVERFLOW", -5: "QR_EDEVICE"}

# Every symbol the headers under include/ declare.
EXPORTS = ("qr_quantize_rows", "qr_quantize_rows_grouped",
           "qr_quantize_activations_q8k128", "qr_dequantize_rows",
           "qr_row_bytes", "qr_block_elems", "qr_solver_constants",
           "qr_last_error", "qr_imatrix_workspace_bytes",
           "qr_imatrix_accumulate", "qr_imatrix_merge",
           "qr_imatrix_finalize", "qr_matmul_q8k128",
           "qr_quantize_rows_weighted", "qr_stats_workspace_bytes",
           "qr_quantize_stats", "qr_quantize_activations_q8k", "qr_matmul_q8k",
           "qr_quantize_rows_ex", "qr_quantize_stats_noalloc")
IMX_MAX_EXPERTS, IMX_MAX_TOP_K = 1024, 64


class QrowError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERRORS.get(code, code)}: {message}")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH):
    """Loads libqrow.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -c 'import "
                "__graft_entry__ as g; g.build()'` (hipcc, gfx950)")
        L = C.CDLL(path)
        vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int
        L.qr_quantize_rows.argtypes = [i32, i32, vp, vp, i64, i64, vp, vp]
        L.qr_quantize_rows_grouped.argtypes = [i32, i32, vp, vp, i64, i64, i64,
                                               vp, vp]
        L.qr_quantize_activations_q8k128.argtypes = [i32, vp, i64, i64, vp, vp]
        L.qr_dequantize_rows.argtypes = [i32, vp, i64, i64, vp, vp]
        L.qr_row_bytes.argtypes = [i32, i64]
        L.qr_row_bytes.restype = C.c_size_t
        L.qr_block_elems.argtypes = [i32]
        L.qr_solver_constants.argtypes = [C.POINTER(C.c_int32)]
        L.qr_last_error.restype = C.c_char_p
        L.qr_imatrix_workspace_bytes.argtypes = [i64, i64, i64, i64]
        L.qr_imatrix_workspace_bytes.restype = C.c_size_t
        L.qr_imatrix_accumulate.argtypes = [i32, vp, i64, i64, i64, vp, i64,
                                            i64, vp, vp, vp, C.c_size_t, vp]
        L.qr_imatrix_merge.argtypes = [vp, vp, vp, vp, i64, i64, vp]
        L.qr_imatrix_finalize.argtypes = [vp, vp, i64, i64, vp, vp]
        L.qr_matmul_q8k128.argtypes = [i32, vp, vp, i64, i64, i64, vp, vp]
        L.qr_matmul_q8k.argtypes = [i32, i32, vp, vp, i64, i64, i64, vp, vp]
        L.qr_quantize_activations_q8k.argtypes = [i32, i32, vp, i64, i64, vp, vp]
        L.qr_quantize_rows_weighted.argtypes = [i32, i32, vp, vp, i64, i64, i32, vp, vp]
        L.qr_quantize_rows_ex.argtypes = [i32, i32, vp, vp, i64, i64, i64, i32, i32, vp, vp]
        L.qr_stats_workspace_bytes.argtypes = [i64, i64]
        L.qr_stats_workspace_bytes.restype = C.c_size_t
        L.qr_quantize_stats.argtypes = [i32, i32, vp, vp, vp, i64, i64, vp, vp, C.c_size_t, vp]
        L.qr_quantize_stats_noalloc.argtypes = [i32, i32, vp, vp, vp, i64, i64, vp, vp]
        for name in (n for n in EXPORTS if n not in
                     ("qr_row_bytes", "qr_block_elems", "qr_last_error",
                      "qr_solver_constants", "qr_imatrix_workspace_bytes",
                      "qr_stats_workspace_bytes")):
            getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def _tid(t) -> int:
    return TYPES[t.lower()] if isinstance(t, str) else int(t)


def _check(rc: int):
    if rc != 0:
        raise QrowError(rc, qr_last_error())


def _stream(x: torch.Tensor, stream):
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    return C.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream")
                      else int(stream))


def _src_dtype(x: torch.Tensor) -> int:
    if x.dtype == torch.float32:
        return QR_F32
    if x.dtype == torch.bfloat16:
        return QR_BF16
    raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")


def _dev2d(x: torch.Tensor, name: str):
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 2-D tensor")


def _cuda_device(t, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    return t.device


def _on(t, name: str, device):
    """Refuses anything but a tensor in the memory of `device`: the kernels
    take raw device addresses, and a host address would reach a kernel as
    one."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.device != torch.device(device):
        raise TypeError(f"{name} is on {t.device}, not on {device}")
    return t


def _imatrix(imatrix, n: int, device):
    """A per-column imatrix of n values (or None) on `device`, contiguous."""
    if imatrix is None:
        return None
    _on(imatrix, "imatrix", device)
    if imatrix.dtype != torch.float32 or imatrix.numel() != n:
        raise ValueError("imatrix must be a CUDA float32 tensor of n_per_row values")
    return imatrix.contiguous()


def qr_last_error() -> str:
    return load_library().qr_last_error().decode()


def qr_row_bytes(t, n_per_row: int) -> int:
    return int(load_library().qr_row_bytes(_tid(t), n_per_row))


def qr_block_elems(t) -> int:
    return int(load_library().qr_block_elems(_tid(t)))


def qr_solver_constants() -> dict:
    c = (C.c_int32 * 6)()
    load_library().qr_solver_constants(c)
    return {"cand_step_x4": c[0], "sym_cand": c[1], "sym_flip_passes": c[2],
            "asym_cand": c[3], "asym_flip_passes": c[4], "group": c[5]}


def _out(out, shape, dtype, device):
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _on(out, "out", device)
    if out.shape != torch.Size(shape) or out.dtype != dtype or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous {dtype} tensor of shape {shape}")
    return out


def qr_quantize_rows(t, x: torch.Tensor, imatrix=None, out=None, stream=None):
    """Quantizes the rows of x ([n_rows, n_per_row], fp32/bf16, on the GPU)
    with importances imatrix ([n_per_row] fp32 or None). Returns uint8
    [n_rows, qr_row_bytes(t, n_per_row)]."""
    _dev2d(x, "x")
    tid = _tid(t)
    n_rows, n = x.shape
    rb = qr_row_bytes(tid, n)
    out = _out(out, (n_rows, rb), torch.uint8, x.device)
    q = _imatrix(imatrix, n, x.device)
    _check(load_library().qr_quantize_rows(
        tid, _src_dtype(x), C.c_void_p(x.data_ptr()),
        None if q is None else C.c_void_p(q.data_ptr()), n_rows, n,
        C.c_void_p(out.data_ptr()), _stream(x, stream)))
    return out


def qr_quantize_rows_weighted(t, x: torch.Tensor, imatrix, weighting, out=None, stream=None):
    """qr_quantize_rows with another element importance: weighting is a
    name of WEIGHTINGS or its number."""
    _dev2d(x, "x")
    tid = _tid(t)
    wid = WEIGHTINGS[weighting] if isinstance(weighting, str) else int(weighting)
    n_rows, n = x.shape
    out = _out(out, (n_rows, qr_row_bytes(tid, n)), torch.uint8, x.device)
    q = _imatrix(imatrix, n, x.device)
    _check(load_library().qr_quantize_rows_weighted(
        tid, _src_dtype(x), C.c_void_p(x.data_ptr()),
        None if q is None else C.c_void_p(q.data_ptr()), n_rows, n, wid,
        C.c_void_p(out.data_ptr()), _stream(x, stream)))
    return out


def qr_quantize_rows_grouped(t, x: torch.Tensor, imatrix, rows_per_group: int,
                             out=None, stream=None):
    """x: [n_groups*rows_per_group, n]; imatrix: [n_groups, n] fp32 or None."""
    _dev2d(x, "x")
    tid = _tid(t)
    n_rows, n = x.shape
    if rows_per_group <= 0 or n_rows % rows_per_group:
        raise ValueError("n_rows must be a multiple of rows_per_group")
    n_groups = n_rows // rows_per_group
    q = None
    if imatrix is not None:
        _on(imatrix, "imatrix", x.device)
        if imatrix.dtype != torch.float32 or tuple(imatrix.shape) != (n_groups, n):
            raise ValueError("imatrix must be float32 [n_groups, n_per_row]")
        q = imatrix.contiguous()
    out = _out(out, (n_rows, qr_row_bytes(tid, n)), torch.uint8, x.device)
    _check(load_library().qr_quantize_rows_grouped(
        tid, _src_dtype(x), C.c_void_p(x.data_ptr()),
        None if q is None else C.c_void_p(q.data_ptr()), n_groups,
        rows_per_group, n, C.c_void_p(out.data_ptr()), _stream(x, stream)))
    return out


def qr_quantize_rows_ex(t, x: torch.Tensor, imatrix=None, rows_per_group=None, weighting=0,
                        subscale_fit="max", out=None, stream=None):
    """Every option of the row quantizer: imatrix is None, [n] or
    [n_groups, n] (rows_per_group = n_rows / n_groups when not given);
    weighting a name of WEIGHTINGS or its number; subscale_fit "max" or
    "weighted" (the Q4_K and Q5_K sub-scales)."""
    _dev2d(x, "x")
    tid = _tid(t)
    n_rows, n = x.shape
    wid = WEIGHTINGS[weighting] if isinstance(weighting, str) else int(weighting)
    fid = FITS[subscale_fit] if isinstance(subscale_fit, str) else int(subscale_fit)
    q = None
    n_groups = 1
    if imatrix is not None:
        _on(imatrix, "imatrix", x.device)
        if imatrix.dtype != torch.float32 or imatrix.numel() % n:
            raise ValueError("imatrix must be a CUDA float32 tensor of whole rows of n_per_row")
        q = imatrix.contiguous()
        n_groups = q.numel() // n
    if rows_per_group is None:
        if n_rows % n_groups:
            raise ValueError("the imatrix groups do not divide the rows")
        rows_per_group = n_rows // n_groups
    if n_groups * rows_per_group != n_rows:
        raise ValueError("n_groups * rows_per_group must equal n_rows")
    out = _out(out, (n_rows, qr_row_bytes(tid, n)), torch.uint8, x.device)
    _check(load_library().qr_quantize_rows_ex(
        tid, _src_dtype(x), C.c_void_p(x.data_ptr()),
        None if q is None else C.c_void_p(q.data_ptr()), n_groups, rows_per_group, n, wid, fid,
        C.c_void_p(out.data_ptr()), _stream(x, stream)))
    return out


def qr_quantize_activations_q8k128(x: torch.Tensor, out=None, stream=None):
    """x: [n_rows, n_per_row] fp32/bf16, n_per_row % 128 == 0."""
    _dev2d(x, "x")
    n_rows, n = x.shape
    out = _out(out, (n_rows, qr_row_bytes(QR_Q8_K128, n)), torch.uint8, x.device)
    _check(load_library().qr_quantize_activations_q8k128(
        _src_dtype(x), C.c_void_p(x.data_ptr()), n_rows, n,
        C.c_void_p(out.data_ptr()), _stream(x, stream)))
    return out


def qr_quantize_activations_q8k(t, x: torch.Tensor, out=None, stream=None):
    """x: [n_rows, n_per_row] fp32/bf16 to the Q8_K format t (q8_k128,
    q8_k64 or q8_k16); n_per_row a multiple of its block length."""
    _dev2d(x, "x")
    tid = _tid(t)
    n_rows, n = x.shape
    out = _out(out, (n_rows, qr_row_bytes(tid, n)), torch.uint8, x.device)
    _check(load_library().qr_quantize_activations_q8k(
        tid, _src_dtype(x), C.c_void_p(x.data_ptr()), n_rows, n,
        C.c_void_p(out.data_ptr()), _stream(x, stream)))
    return out


def qr_dequantize_rows(t, packed: torch.Tensor, n_rows: int, n_per_row: int,
                       out=None, stream=None):
    """packed: uint8 [n_rows, qr_row_bytes]; returns fp32 [n_rows, n_per_row]."""
    tid = _tid(t)
    _on(packed, "packed", _cuda_device(packed, "packed"))
    if packed.dtype != torch.uint8 or not packed.is_contiguous():
        raise ValueError("packed must be a contiguous CUDA uint8 tensor")
    if packed.numel() != n_rows * qr_row_bytes(tid, n_per_row):
        raise ValueError("packed has the wrong size")
    out = _out(out, (n_rows, n_per_row), torch.float32, packed.device)
    _check(load_library().qr_dequantize_rows(
        tid, C.c_void_p(packed.data_ptr()), n_rows, n_per_row,
        C.c_void_p(out.data_ptr()), _stream(packed, stream)))
    return out


# --------------------------------------------------------------------------
# importance-matrix accumulator (include/qrow_imatrix.h)

def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def qr_imatrix_workspace_bytes(n_tokens: int, top_k: int, n_experts: int,
                               n_cols: int) -> int:
    return int(load_library().qr_imatrix_workspace_bytes(n_tokens, top_k,
                                                         n_experts, n_cols))


def imatrix_state(n_experts: int, n_cols: int, device):
    """A fresh accumulator: (sums float64 [E, C], counts int64 [E]), zeros."""
    return (torch.zeros((n_experts, n_cols), dtype=torch.float64, device=device),
            torch.zeros(n_experts, dtype=torch.int64, device=device))


def _check_state(sums, counts, n_experts=None, n_cols=None, device=None):
    _on(sums, "sums", device if device is not None else _cuda_device(sums, "sums"))
    _on(counts, "counts", sums.device)
    if (not isinstance(sums, torch.Tensor) or not sums.is_cuda or sums.dtype != torch.float64
            or sums.dim() != 2 or not sums.is_contiguous()):
        raise ValueError("sums must be a contiguous CUDA float64 [n_experts, n_cols] tensor")
    if (not isinstance(counts, torch.Tensor) or not counts.is_cuda or counts.dtype != torch.int64
            or tuple(counts.shape) != (sums.shape[0],) or not counts.is_contiguous()):
        raise ValueError("counts must be a contiguous CUDA int64 [n_experts] tensor")
    if n_experts is not None and sums.shape[0] != n_experts:
        raise ValueError("sums has the wrong number of experts")
    if n_cols is not None and sums.shape[1] != n_cols:
        raise ValueError("sums has the wrong number of columns")


def qr_imatrix_accumulate(act: torch.Tensor, sums: torch.Tensor, counts: torch.Tensor,
                          ids=None, workspace=None, stream=None):
    """Adds act to the state (sums, counts) in place.

    act: [n_tokens, n_cols] (one row per token) or [n_tokens, top_k, n_cols]
    (one row per routed slot), fp32 or bf16, on the GPU. ids: int32
    [n_tokens, top_k] expert ids on the GPU, or None for a dense tensor.
    workspace: a CUDA uint8 tensor of at least qr_imatrix_workspace_bytes
    bytes, or None to have one allocated here."""
    if not isinstance(act, torch.Tensor) or not act.is_cuda or not act.is_contiguous():
        raise TypeError("act must be a contiguous CUDA tensor")
    if act.dim() == 2:
        n_tokens, n_cols = act.shape
        n_slots = 1
    elif act.dim() == 3:
        n_tokens, n_slots, n_cols = act.shape
    else:
        raise ValueError("act must be [n_tokens, n_cols] or [n_tokens, n_slots, n_cols]")
    _check_state(sums, counts, n_cols=n_cols, device=act.device)
    n_experts = sums.shape[0]
    top_k = 0
    if ids is not None:
        _on(ids, "ids", act.device)
        if (ids.dtype != torch.int32 or ids.dim() != 2
                or ids.shape[0] != n_tokens or not ids.is_contiguous()):
            raise ValueError("ids must be a contiguous CUDA int32 [n_tokens, top_k] tensor")
        top_k = ids.shape[1]
    need = qr_imatrix_workspace_bytes(n_tokens, top_k, n_experts, n_cols)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=act.device)
    if workspace is not None:
        _on(workspace, "workspace", act.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().qr_imatrix_accumulate(
        _src_dtype(act), _ptr(act), n_tokens, n_slots, n_cols, _ptr(ids), top_k,
        n_experts, _ptr(sums), _ptr(counts), _ptr(workspace), ws_bytes,
        _stream(act, stream)))
    return sums, counts


def qr_imatrix_merge(sums, counts, src_sums, src_counts, stream=None):
    """(sums, counts) += (src_sums, src_counts), in place."""
    _check_state(sums, counts)
    _check_state(src_sums, src_counts, sums.shape[0], sums.shape[1], device=sums.device)
    _check(load_library().qr_imatrix_merge(
        _ptr(sums), _ptr(counts), _ptr(src_sums), _ptr(src_counts),
        sums.shape[0], sums.shape[1], _stream(sums, stream)))
    return sums, counts


def qr_imatrix_finalize(sums, counts, out=None, stream=None):
    """Importances q = sums / counts as fp32 [n_experts, n_cols] (0 where a
    count is 0)."""
    _check_state(sums, counts)
    out = _out(out, tuple(sums.shape), torch.float32, sums.device)
    _check(load_library().qr_imatrix_finalize(
        _ptr(sums), _ptr(counts), sums.shape[0], sums.shape[1], _ptr(out),
        _stream(sums, stream)))
    return out


# --------------------------------------------------------------------------
# product with Q8_K_128 activations (include/qrow_matmul.h)

def qr_matmul_q8k(t, act, w: torch.Tensor, x: torch.Tensor, n_in: int, out=None, stream=None):
    """y [n_tok, n_out] fp32 = W @ A.T for packed weight rows w (uint8
    [n_out, qr_row_bytes(t, n_in)]) and packed activation rows x of the
    Q8_K format act (uint8 [n_tok, qr_row_bytes(act, n_in)]), both on the GPU."""
    tid, aid = _tid(t), _tid(act)
    for name, a in (("w", w), ("x", x)):
        _on(a, name, _cuda_device(w, "w"))
        if a.dtype != torch.uint8 or a.dim() != 2 or not a.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 2-D CUDA uint8 tensor")
    if w.shape[1] != qr_row_bytes(tid, n_in) or x.shape[1] != qr_row_bytes(aid, n_in):
        raise ValueError("packed row lengths do not match n_in")
    n_out, n_tok = w.shape[0], x.shape[0]
    out = _out(out, (n_tok, n_out), torch.float32, w.device)
    _check(load_library().qr_matmul_q8k(
        tid, aid, _ptr(w), _ptr(x), n_out, n_tok, n_in, _ptr(out), _stream(w, stream)))
    return out


def qr_matmul_q8k128(t, w: torch.Tensor, x: torch.Tensor, n_in: int, out=None, stream=None):
    """y [n_tok, n_out] fp32 = W @ A.T for packed weight rows w (uint8
    [n_out, qr_row_bytes(t, n_in)]) and packed Q8_K_128 activation rows x
    (uint8 [n_tok, qr_row_bytes("q8_k128", n_in)]), both on the GPU."""
    tid = _tid(t)
    for name, a in (("w", w), ("x", x)):
        _on(a, name, _cuda_device(w, "w"))
        if a.dtype != torch.uint8 or a.dim() != 2 or not a.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 2-D CUDA uint8 tensor")
    if w.shape[1] != qr_row_bytes(tid, n_in) or x.shape[1] != qr_row_bytes(QR_Q8_K128, n_in):
        raise ValueError("packed row lengths do not match n_in")
    n_out, n_tok = w.shape[0], x.shape[0]
    out = _out(out, (n_tok, n_out), torch.float32, w.device)
    _check(load_library().qr_matmul_q8k128(
        tid, _ptr(w), _ptr(x), n_out, n_tok, n_in, _ptr(out), _stream(w, stream)))
    return out


# --------------------------------------------------------------------------
# error statistics (include/qrow_stats.h)

QR_STATS_BYTES = 72   # sizeof(qr_stats)


def qr_stats_workspace_bytes(n_rows: int, n_per_row: int) -> int:
    return int(load_library().qr_stats_workspace_bytes(n_rows, n_per_row))


def qr_quantize_stats(t, x: torch.Tensor, packed: torch.Tensor, imatrix=None, workspace=None,
                      stream=None) -> dict:
    """Error statistics of packed rows against x (see qr_stats); returns the
    struct's fields as a dict (this copies the 72-byte result to the host,
    which waits for the stream)."""
    _dev2d(x, "x")
    tid = _tid(t)
    n_rows, n = x.shape
    _on(packed, "packed", x.device)
    if (packed.dtype != torch.uint8 or not packed.is_contiguous()
            or packed.numel() != n_rows * qr_row_bytes(tid, n)):
        raise ValueError("packed must be a contiguous CUDA uint8 tensor of the rows' packed bytes")
    q = _imatrix(imatrix, n, x.device)
    if workspace is None:
        workspace = torch.empty(qr_stats_workspace_bytes(n_rows, n), dtype=torch.uint8, device=x.device)
    _on(workspace, "workspace", x.device)
    out = torch.zeros(QR_STATS_BYTES, dtype=torch.uint8, device=x.device)
    _check(load_library().qr_quantize_stats(
        tid, _src_dtype(x), _ptr(x), _ptr(packed), _ptr(q), n_rows, n, _ptr(out),
        _ptr(workspace), workspace.numel(), _stream(x, stream)))
    return stats_dict(out)


def stats_dict(out: torch.Tensor) -> dict:
    """The fields of a qr_stats struct held in a 72-byte device buffer (this
    copies it to the host, which waits for its stream)."""
    import numpy as np
    raw = out.cpu().numpy()
    sums = raw[:32].view(np.float64)
    mx, p95 = raw[32:40].view(np.float32)
    ratios = raw[48:72].view(np.float64)
    return {"sum_err2": float(sums[0]), "sum_x2": float(sums[1]), "sum_werr2": float(sums[2]),
            "sum_wx2": float(sums[3]), "max_abs_err": float(mx), "p95_abs_err": float(p95),
            "n": int(raw[40:48].view(np.int64)[0]), "rmse": float(ratios[0]),
            "rel_rmse": float(ratios[1]), "weighted_rel_rmse": float(ratios[2])}


def qr_quantize_stats_noalloc(t, x: torch.Tensor, packed: torch.Tensor, out: torch.Tensor, imatrix=None,
                              stream=None) -> torch.Tensor:
    """qr_quantize_stats without a workspace and without allocating: the
    caller passes `out`, a 72-byte uint8 CUDA buffer that receives the
    qr_stats struct (read it with stats_dict). Returns out."""
    _dev2d(x, "x")
    tid = _tid(t)
    n_rows, n = x.shape
    _on(packed, "packed", x.device)
    if (packed.dtype != torch.uint8 or not packed.is_contiguous()
            or packed.numel() != n_rows * qr_row_bytes(tid, n)):
        raise ValueError("packed must be a contiguous CUDA uint8 tensor of the rows' packed bytes")
    if imatrix is not None and not imatrix.is_contiguous():
        raise ValueError("imatrix must be contiguous (no copy is made here)")
    q = _imatrix(imatrix, n, x.device)
    _on(out, "out", x.device)
    if out.dtype != torch.uint8 or out.numel() != QR_STATS_BYTES or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous uint8 tensor of {QR_STATS_BYTES} bytes")
    _check(load_library().qr_quantize_stats_noalloc(
        tid, _src_dtype(x), _ptr(x), _ptr(packed), _ptr(q), n_rows, n, _ptr(out), _stream(x, stream)))
    return out
