"""GPU parity of the importance-matrix accumulator against the CPU oracle,
through the C-ABI.

Bar (derived from the arithmetic): a^2 of an fp32 or bf16 value is exact in
double, so the GPU and the oracle add the same exact terms, in different
orders. Any order of n non-negative double additions is within
(n - 1) * 2^-53 of the exact sum, relative; two orders therefore differ by
at most 2 (n + 1) * 2^-53 of the sum (n = tokens routed to the expert, plus
one for a prior state). Counts are integers: bit-exact. On data whose every
partial sum is exact in double (dyadic values) the sums must be bit-exact.
The finalize and merge kernels are single correctly rounded operations:
bit-exact on identical inputs, and q differs from the oracle's by at most one
float ulp when the sums differ within the bound above.
"""
import numpy as np
import pytest

import oracle
from post_weight_quantization_row_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

F32 = np.float32


@pytest.fixture(scope="module")
def qr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from post_weight_quantization_row_amd import qrow
    qrow.load_library()
    return qrow


def say(*a):
    print(*a, flush=True)


def to_dev(a: np.ndarray, bf16: bool):
    if bf16:
        bits = synth.f32_to_bf16_bits(a)
        return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, F32)).cuda()


def gpu_accumulate(qr, a, ids, n_experts, bf16, state=None, batches=None):
    C = a.shape[-1]
    if state is None:
        state = qr.imatrix_state(n_experts, C, "cuda")
    sums, counts = state
    spans = batches or [(0, a.shape[0])]
    for lo, hi in spans:
        d_ids = None if ids is None else torch.from_numpy(np.ascontiguousarray(ids[lo:hi])).cuda()
        qr.qr_imatrix_accumulate(to_dev(np.ascontiguousarray(a[lo:hi]), bf16), sums, counts, d_ids)
    torch.cuda.synchronize()
    return sums, counts


def oracle_accumulate(a, ids, n_experts, bf16):
    x = synth.round_to_bf16(a) if bf16 else np.ascontiguousarray(a, F32)
    st = oracle.imatrix_new(n_experts, a.shape[-1])
    oracle.imatrix_accumulate(st, x, ids)
    return st


def assert_state_matches(gs, gc, st, exact=False, extra_terms=1):
    sums = gs.cpu().numpy()
    counts = gc.cpu().numpy()
    assert np.array_equal(counts, st[1]), "counts differ"
    if exact:
        assert np.array_equal(sums, st[0]), "sums differ on exact data"
        return
    n = st[1].astype(np.float64)[:, None] + extra_terms
    tol = 2.0 * (n + 1.0) * 2.0 ** -53 * np.abs(st[0])
    bad = np.abs(sums - st[0]) > tol
    assert not bad.any(), f"{bad.sum()} sums outside the rounding bound"


def assert_q_matches(qr, gs, gc, st):
    q = qr.qr_imatrix_finalize(gs, gc).cpu().numpy()
    # the finalize kernel is one double division and one rounding
    sums, counts = gs.cpu().numpy(), gc.cpu().numpy()
    with np.errstate(divide="ignore", invalid="ignore"):
        want = np.where(counts[:, None] > 0, sums / counts[:, None], 0.0).astype(F32)
    assert np.array_equal(q, want)
    qo = oracle.imatrix_finalize(st)
    d = np.abs(q.view(np.int32).astype(np.int64) - qo.view(np.int32).astype(np.int64))
    assert d.max() <= 1


def dyadic(rng, shape, bits=6):
    k = rng.integers(-(2 ** bits) + 1, 2 ** bits, size=shape)
    return (k * 2.0 ** -4).astype(F32)


# --------------------------------------------------------------------------

@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("T,C", [(50, 64), (777, 1000), (5000, 520), (4096, 4096)])
def test_dense(qr, bf16, T, C):
    say(f"dense T={T} C={C} bf16={bf16}")
    a = synth.calib_activations(T, C, seed=T + C, bf16=bf16)
    gs, gc = gpu_accumulate(qr, a, None, 1, bf16)
    st = oracle_accumulate(a, None, 1, bf16)
    assert_state_matches(gs, gc, st)
    assert_q_matches(qr, gs, gc, st)


@pytest.mark.parametrize("T,C,E,K,S", [
    (1000, 1000, 16, 4, 1),      # partial slabs + reduce
    (1000, 1000, 16, 4, 4),      # one row per routed slot
    (300, 136, 8, 2, 1),         # ragged chunk, few tokens
    (10000, 4096, 128, 2, 1),    # one slab of three 4096-token windows
    (2048, 512, 1024, 8, 1),     # the largest expert count (64 KB routing LDS)
    (9000, 64, 4, 2, 2),         # many slabs, per-slot rows
    (600, 256, 128, 64, 1),      # the largest top_k (64 experts per token)
])
def test_routed(qr, T, C, E, K, S):
    say(f"routed T={T} C={C} E={E} K={K} S={S}")
    a = synth.calib_activations(T, C, seed=T + 3 * C + E, n_slots=S, bf16=True)
    ids = synth.routing_ids(T, E, K, seed=T + E, n_dead=min(2, E - K))
    gs, gc = gpu_accumulate(qr, a, ids, E, True)
    st = oracle_accumulate(a, ids, E, True)
    assert_state_matches(gs, gc, st)
    assert_q_matches(qr, gs, gc, st)


@pytest.mark.parametrize("S", [1, 3])
def test_unused_slots_and_repeated_experts(qr, S):
    rng = np.random.default_rng(40 + S)
    T, C, E, K = 700, 96, 9, 3
    ids = rng.integers(-2, E + 2, size=(T, K)).astype(np.int32)
    ids[::7, 1] = ids[::7, 0]            # repeats within a token
    a = dyadic(rng, (T, S, C) if S > 1 else (T, C))
    say(f"unused/repeated S={S}")
    gs, gc = gpu_accumulate(qr, a, ids, E, False)
    st = oracle_accumulate(a, ids, E, False)
    assert_state_matches(gs, gc, st, exact=True)
    assert_q_matches(qr, gs, gc, st)


@pytest.mark.parametrize("routed", [False, True])
def test_exact_data_is_bit_exact_and_batching_free(qr, routed):
    rng = np.random.default_rng(50 + routed)
    T, C = 3000, 1032
    E, K = (32, 4) if routed else (1, 0)
    a = dyadic(rng, (T, C))
    ids = synth.routing_ids(T, E, K, seed=51) if routed else None
    say(f"exact routed={routed}")
    st = oracle_accumulate(a, ids, E, False)
    gs, gc = gpu_accumulate(qr, a, ids, E, False)
    assert_state_matches(gs, gc, st, exact=True)
    gs2, gc2 = gpu_accumulate(qr, a, ids, E, False,
                              batches=[(0, 1), (1, 33), (33, 2000), (2000, 3000)])
    assert_state_matches(gs2, gc2, st, exact=True)


def test_results_are_reproducible(qr):
    a = synth.calib_activations(4096, 2048, seed=60, bf16=True)
    ids = synth.routing_ids(4096, 16, 2, seed=60)
    say("reproducible")
    r1 = gpu_accumulate(qr, a, ids, 16, True)
    r2 = gpu_accumulate(qr, a, ids, 16, True)
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])
    d1 = gpu_accumulate(qr, a, None, 1, True)
    d2 = gpu_accumulate(qr, a, None, 1, True)
    assert torch.equal(d1[0], d2[0]) and torch.equal(d1[1], d2[1])


def test_state_carries_over_calls(qr):
    a = synth.calib_activations(1500, 512, seed=61, bf16=False)
    ids = synth.routing_ids(1500, 12, 3, seed=61, n_dead=1)
    say("carry")
    gs, gc = gpu_accumulate(qr, a, ids, 12, False, batches=[(0, 700), (700, 1500)])
    st = oracle_accumulate(a, ids, 12, False)
    assert_state_matches(gs, gc, st, extra_terms=2)


def test_merge_and_finalize_are_exact(qr):
    rng = np.random.default_rng(62)
    E, C = 37, 328
    s1 = rng.random((E, C)) * 1e3
    s2 = rng.random((E, C)) * 1e-3
    c1 = rng.integers(0, 5000, E).astype(np.int64)
    c2 = rng.integers(0, 5000, E).astype(np.int64)
    c1[:3] = 0
    c2[:2] = 0
    say("merge/finalize")
    gs, gc = torch.from_numpy(s1.copy()).cuda(), torch.from_numpy(c1.copy()).cuda()
    qr.qr_imatrix_merge(gs, gc, torch.from_numpy(s2).cuda(), torch.from_numpy(c2).cuda())
    st = (s1.copy(), c1.copy())
    oracle.imatrix_merge(st, (s2, c2))
    assert np.array_equal(gs.cpu().numpy(), st[0]) and np.array_equal(gc.cpu().numpy(), st[1])
    q = qr.qr_imatrix_finalize(gs, gc).cpu().numpy()
    assert np.array_equal(q, oracle.imatrix_finalize(st))
    assert not q[0].any()


def test_no_tokens_is_a_no_op(qr):
    sums, counts = qr.imatrix_state(4, 64, "cuda")
    sums += 1.5
    qr.qr_imatrix_accumulate(torch.zeros((0, 64), device="cuda"), sums, counts,
                             torch.zeros((0, 2), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert bool((sums == 1.5).all()) and not counts.any()


@pytest.mark.parametrize("name", ["imatrix_moe_256x8_4096x7168", "imatrix_moe_slots_256x8_4096x2048",
                                  "imatrix_dense_4096x4096"])
def test_full_size_workloads(qr, name):
    a, ids, E = synth.imatrix_inputs(name)
    say(f"full size {name}")
    gs, gc = gpu_accumulate(qr, a, ids, E, True)
    st = oracle_accumulate(a, ids, E, True)
    assert_state_matches(gs, gc, st)
    assert_q_matches(qr, gs, gc, st)
    if ids is not None:
        # the never-routed experts of the recipe have no data
        assert (st[1] == 0).sum() == synth.WORKLOADS[name]["n_dead"]
