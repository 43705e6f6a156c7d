"""The allocation-free statistics entry point (qr_quantize_stats_noalloc),
called through the C-ABI, against the entry point that takes a caller's
workspace (qr_quantize_stats): the 72-byte qr_stats results must be
identical bit for bit (both run the same kernels over the same grid, and the
sums are combined in a fixed order). Two calls in a row share the static
workspace; the second, smaller one must not see the first one's contents.
Both are also checked against the CPU oracle to the statistics' own bar
(maximum and 95th percentile bit for bit, sums within their rounding bound).
"""
import ctypes as C

import numpy as np
import pytest

import oracle
from post_weight_quantization_row_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from post_weight_quantization_row_amd import qrow
    qrow.load_library()
    return qrow


def say(*a):
    print(*a, flush=True)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _both(qr, t, x, packed, q, stream):
    """(bytes from the workspace entry point, bytes from the static one),
    each written into a buffer poisoned beforehand, both on `stream`."""
    lib = qr.load_library()
    n_rows, n = x.shape
    tid = qr.TYPES[t]
    ws = torch.empty(lib.qr_stats_workspace_bytes(n_rows, n), dtype=torch.uint8, device="cuda")
    a = torch.full((qr.QR_STATS_BYTES,), 0xAB, dtype=torch.uint8, device="cuda")
    b = torch.full((qr.QR_STATS_BYTES,), 0xCD, dtype=torch.uint8, device="cuda")
    h = C.c_void_p(stream.cuda_stream)
    torch.cuda.synchronize()
    rc = lib.qr_quantize_stats(tid, qr.QR_F32, _ptr(x), _ptr(packed), _ptr(q), n_rows, n, _ptr(a),
                               _ptr(ws), ws.numel(), h)
    assert rc == 0, qr.qr_last_error()
    rc = lib.qr_quantize_stats_noalloc(tid, qr.QR_F32, _ptr(x), _ptr(packed), _ptr(q), n_rows, n, _ptr(b), h)
    assert rc == 0, qr.qr_last_error()
    stream.synchronize()
    return a, b


def _against_oracle(qr, t, xh, packed_h, qh, res):
    o = oracle.quantize_stats(t, xh, packed_h, qh)
    g = qr.stats_dict(res)
    assert g["n"] == o["n"]
    assert np.float32(g["max_abs_err"]) == o["max_abs_err"]
    assert np.float32(g["p95_abs_err"]) == o["p95_abs_err"]
    tol = 2.0 * o["n"] * 2.0 ** -53
    for key in ("sum_err2", "sum_x2", "sum_werr2", "sum_wx2"):
        assert abs(g[key] - o[key]) <= tol * o[key], key


def test_static_workspace_matches_the_callers_workspace_on_two_calls(qr):
    stream = torch.cuda.Stream()
    # first call: 2048 x 4096 Q4_K with importances (the largest grid)
    x1, q1 = synth.q4_k_matrix(2048, 4096, seed=2024)
    p1 = oracle.quantize_rows("q4_k", x1, q1)
    xd1, qd1, pd1 = (torch.from_numpy(v).cuda() for v in (x1, q1, p1))
    say("no-alloc stats: call 1, q4_k 2048x4096")
    a1, b1 = _both(qr, "q4_k", xd1, pd1, qd1, stream)
    assert torch.equal(a1, b1)
    _against_oracle(qr, "q4_k", x1, p1, q1, b1)
    # second call, smaller: 33 x 1024 Q4_0 without importances
    x2, _ = synth.q4_0_matrix(33, 1024, seed=2025)
    p2 = oracle.quantize_rows("q4_0", x2, None)
    xd2, pd2 = (torch.from_numpy(v).cuda() for v in (x2, p2))
    say("no-alloc stats: call 2, q4_0 33x1024")
    a2, b2 = _both(qr, "q4_0", xd2, pd2, None, stream)
    assert torch.equal(a2, b2)
    _against_oracle(qr, "q4_0", x2, p2, None, b2)
    assert not torch.equal(b1, b2)


def test_binding_and_default_stream(qr):
    # the Python binding of the same entry point, on torch's current stream
    x, q = synth.q4_k_matrix(64, 2048, seed=2026)
    p = oracle.quantize_rows("q5_k", x, q)
    xd, qd, pd = (torch.from_numpy(v).cuda() for v in (x, q, p))
    out = torch.empty(qr.QR_STATS_BYTES, dtype=torch.uint8, device="cuda")
    say("no-alloc stats: binding, q5_k 64x2048")
    qr.qr_quantize_stats_noalloc("q5_k", xd, pd, out, qd)
    ref = qr.qr_quantize_stats("q5_k", xd, pd, qd)
    assert qr.stats_dict(out) == ref
