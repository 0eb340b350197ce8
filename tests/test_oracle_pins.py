"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each pin is a function of an FFN (or reorder) implementation so that the same
check can be run on the oracle (must pass) and on small numpy mutants with a
planted mistake (must fail): that shows every pin has teeth.

What fixes the expected values:
  * reorder: numpy's stable argsort of the "inactive" key is exactly a stable
    partition (library routine), a Python brute-force loop, a hand-derived
    fixture, and the partition invariants;
  * FFN: the all-ones mask is the dense SwiGLU FFN (numpy float64 matmuls), the
    all-zero mask is exactly zero, a token-uniform mask is static width
    pruning (dense FFN on sliced weights), Y is additive over groups, tokens
    are independent (row permutation equivariance, bitwise), and tiny cases
    agree with a 50-digit mpmath evaluation.
"""
import json
import os

import mpmath
import numpy as np
import pytest
import torch

import oracle
from group_sparse_ffn_amd import datagen as dg

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- helpers

def rand_problem(seed, T, d, d_ff, G, density=0.5):
    p = dg.random_small(seed, T, d, d_ff, G, "f32", density)
    return {k: v.numpy() for k, v in p.items()}


def silu64(a):
    return a / (1.0 + np.exp(-a))


def dense_ffn64(X, Wg, Wu, Wd):
    """Unpruned SwiGLU FFN with numpy float64 matmuls (library routine)."""
    X = X.astype(np.float64)
    a = X @ Wg.astype(np.float64).T
    b = X @ Wu.astype(np.float64).T
    return (silu64(a) * b) @ Wd.astype(np.float64).T


def rel(a, b):
    den = max(np.max(np.abs(b)), 1e-300)
    return np.max(np.abs(a - b)) / den


def oracle_ffn_fn(X, Wg, Wu, Wd, mask, G):
    return oracle.ffn(X, Wg, Wu, Wd, mask, G)


# ----------------------------------------------------------------------------- FFN pins
# Each returns True when the implementation passes.

def pin_dense_limit(ffn):
    p = rand_problem(11, T=6, d=24, d_ff=40, G=8)
    ones = np.ones_like(p["mask"])
    _, Y = ffn(p["X"], p["Wg"], p["Wu"], p["Wd"], ones, 8)
    return rel(Y, dense_ffn64(p["X"], p["Wg"], p["Wu"], p["Wd"])) <= 1e-12


def pin_zero_limit(ffn):
    p = rand_problem(12, T=5, d=16, d_ff=32, G=4)
    zeros = np.zeros_like(p["mask"])
    H, Y = ffn(p["X"], p["Wg"], p["Wu"], p["Wd"], zeros, 4)
    return bool(np.all(H == 0.0) and np.all(Y == 0.0))


def pin_token_uniform(ffn):
    """Same active set S for every token == dense FFN on weights sliced to S."""
    G, d_ff, d, T = 4, 36, 20, 5
    ng = d_ff // G
    p = rand_problem(13, T=T, d=d, d_ff=d_ff, G=G)
    S = np.array([1, 2, 5, 8])
    mask = np.zeros((T, ng), dtype=np.uint8)
    mask[:, S] = 1
    ch = np.concatenate([np.arange(g * G, (g + 1) * G) for g in S])
    ref = dense_ffn64(p["X"], p["Wg"][ch], p["Wu"][ch], p["Wd"][:, ch])
    _, Y = ffn(p["X"], p["Wg"], p["Wu"], p["Wd"], mask, G)
    return rel(Y, ref) <= 1e-12


def pin_group_additivity(ffn):
    G, d_ff, d, T = 4, 24, 12, 7
    ng = d_ff // G
    p = rand_problem(14, T=T, d=d, d_ff=d_ff, G=G)
    _, Y = ffn(p["X"], p["Wg"], p["Wu"], p["Wd"], p["mask"], G)
    acc = np.zeros_like(Y)
    for g in range(ng):
        m = np.zeros_like(p["mask"])
        m[:, g] = p["mask"][:, g]
        acc += ffn(p["X"], p["Wg"], p["Wu"], p["Wd"], m, G)[1]
    return rel(Y, acc) <= 1e-12


def pin_token_equivariance(ffn):
    G, d_ff, d, T = 8, 32, 16, 9
    p = rand_problem(15, T=T, d=d, d_ff=d_ff, G=G)
    _, Y = ffn(p["X"], p["Wg"], p["Wu"], p["Wd"], p["mask"], G)
    pi = np.random.default_rng(3).permutation(T)
    _, Yp = ffn(p["X"][pi], p["Wg"], p["Wu"], p["Wd"], p["mask"][pi], G)
    return bool(np.array_equal(Yp, Y[pi]))


def mp_ffn(X, Wg, Wu, Wd, mask, G):
    """50-digit scalar-loop evaluation of the masked SwiGLU FFN."""
    mpmath.mp.dps = 50
    T, d = X.shape
    d_ff = Wg.shape[0]
    Y = np.zeros((T, d), dtype=object)
    for t in range(T):
        h = []
        for c in range(d_ff):
            if mask[t, c // G]:
                a = mpmath.fsum(mpmath.mpf(float(X[t, k])) * mpmath.mpf(float(Wg[c, k])) for k in range(d))
                b = mpmath.fsum(mpmath.mpf(float(X[t, k])) * mpmath.mpf(float(Wu[c, k])) for k in range(d))
                h.append(a / (1 + mpmath.exp(-a)) * b)
            else:
                h.append(mpmath.mpf(0))
        for n in range(d):
            Y[t, n] = mpmath.fsum(mpmath.mpf(float(Wd[n, c])) * h[c] for c in range(d_ff))
    return Y


def pin_mpmath_bruteforce(ffn):
    worst = 0.0
    for seed, (T, d, d_ff, G) in enumerate([(3, 8, 32, 8), (2, 5, 12, 4), (3, 7, 16, 2), (1, 8, 8, 1)]):
        p = rand_problem(100 + seed, T=T, d=d, d_ff=d_ff, G=G, density=0.6)
        p["X"] *= 3.0  # reach the curved part of silu
        ref = mp_ffn(p["X"], p["Wg"] * 10, p["Wu"], p["Wd"], p["mask"], G)
        _, Y = ffn(p["X"], p["Wg"] * 10, p["Wu"], p["Wd"], p["mask"], G)
        scale = max(float(abs(v)) for v in ref.flat) or 1.0
        for y, r in zip(Y.flat, ref.flat):
            worst = max(worst, float(abs(mpmath.mpf(float(y)) - r)) / scale)
    return worst <= 1e-14


FFN_PINS = [pin_dense_limit, pin_zero_limit, pin_token_uniform, pin_group_additivity,
            pin_token_equivariance, pin_mpmath_bruteforce]


@pytest.mark.parametrize("pin", FFN_PINS, ids=lambda f: f.__name__)
def test_oracle_ffn_pins(pin):
    assert pin(oracle_ffn_fn)


def test_oracle_rows_subset_matches_full():
    p = rand_problem(21, T=10, d=16, d_ff=32, G=8)
    H, Y = oracle.ffn(p["X"], p["Wg"], p["Wu"], p["Wd"], p["mask"], 8)
    rows = np.array([9, 0, 4, 4])
    Hs, Ys = oracle.ffn(p["X"], p["Wg"], p["Wu"], p["Wd"], p["mask"], 8, rows=rows)
    assert np.array_equal(Ys, Y[rows]) and np.array_equal(Hs, H[rows])


def test_oracle_masked_channels_are_exact_zero_even_for_huge_inputs():
    # Select, not multiply: a masked group stays +0.0 whatever its inputs.
    p = rand_problem(22, T=4, d=8, d_ff=16, G=4)
    p["Wg"][:4] = np.float32(3e38)
    p["Wu"][:4] = np.float32(-3e38)
    m = p["mask"].copy()
    m[:, 0] = 0
    H, _ = oracle.ffn(p["X"], p["Wg"], p["Wu"], p["Wd"], m, 4)
    assert np.all(H[:, :4] == 0.0) and not np.any(np.signbit(H[:, :4]))


# ----------------------------------------------------------------------------- mutants
# Small numpy variants of the FFN, each with one planted mistake. Every one
# must fail at least one pin; the correct numpy variant must pass them all.

def _np_ffn(X, Wg, Wu, Wd, mask, G, bug=None):
    X = X.astype(np.float64)
    Wg, Wu, Wd = Wg.astype(np.float64), Wu.astype(np.float64), Wd.astype(np.float64)
    T = X.shape[0]
    d_ff = Wg.shape[0]
    ng = d_ff // G
    a = X @ Wg.T
    b = X @ Wu.T
    if bug == "sign":
        h = a / (1 + np.exp(a)) * b
    elif bug == "no_up":
        h = a / (1 + np.exp(-a))
    elif bug == "relu":
        h = np.maximum(a, 0) * b
    else:
        h = a / (1 + np.exp(-a)) * b
    if bug == "interleaved_groups":
        gidx = np.arange(d_ff) % ng
    else:
        gidx = np.arange(d_ff) // G
    if bug == "mask_transposed":
        m = mask.reshape(-1)[(np.arange(ng)[None, :] * T + np.arange(T)[:, None]) % mask.size].reshape(T, ng)
    else:
        m = mask
    keep = m[:, gidx] != 0
    if bug == "mask_ignored":
        keep = np.ones_like(keep)
    H = np.where(keep, h, 0.0)
    if bug == "wd_transposed":
        # Wd read as [d_ff, d] (only type-checks when square, so emulate with a reshape)
        Y = H @ Wd.reshape(d_ff, -1)
    else:
        Y = H @ Wd.T
    if bug == "token_mixing":
        Y = Y + 1e-9 * np.roll(Y, 1, axis=0)
    return H, Y


MUTANTS = ["sign", "no_up", "relu", "interleaved_groups", "mask_transposed", "mask_ignored",
           "wd_transposed", "token_mixing"]


def test_pins_pass_on_correct_numpy_variant():
    fn = lambda *a: _np_ffn(*a)  # noqa: E731
    assert all(pin(fn) for pin in FFN_PINS if pin is not pin_token_equivariance)


@pytest.mark.parametrize("bug", MUTANTS)
def test_pins_catch_planted_mistake(bug):
    fn = lambda *a: _np_ffn(*a, bug=bug)  # noqa: E731
    results = {pin.__name__: pin(fn) for pin in FFN_PINS if pin is not pin_mpmath_bruteforce}
    assert not all(results.values()), f"no pin caught the '{bug}' mutant: {results}"


# ----------------------------------------------------------------------------- reorder pins

def brute_reorder(mask, tile):
    T, ng = mask.shape
    perm = []
    counts = []
    padded = []
    for g in range(ng):
        act = [t for t in range(T) if mask[t, g]]
        ina = [t for t in range(T) if not mask[t, g]]
        perm.append(act + ina)
        counts.append(len(act))
        padded.append(-(-len(act) // tile) * tile)
    return np.array(perm, dtype=np.int32).reshape(ng, T), np.array(counts), np.array(padded)


def check_reorder_invariants(mask, tile, perm, counts, padded):
    T, ng = mask.shape
    for g in range(ng):
        p = perm[g]
        assert np.array_equal(np.sort(p), np.arange(T))
        c = counts[g]
        assert c == int(np.count_nonzero(mask[:, g]))
        assert np.all(mask[p[:c], g] != 0) and np.all(mask[p[c:], g] == 0)
        assert np.all(np.diff(p[:c]) > 0) and np.all(np.diff(p[c:]) > 0)
        assert padded[g] == -(-c // tile) * tile
        assert padded[g] % tile == 0 and padded[g] - tile < c <= padded[g] or c == padded[g] == 0


@pytest.mark.parametrize("T,ng,tile,density", [(1, 1, 1, 0.5), (7, 3, 4, 0.5), (130, 9, 64, 0.3),
                                                (257, 16, 256, 0.5), (1000, 5, 128, 0.9), (64, 40, 3, 0.1)])
def test_oracle_reorder_matches_library_and_bruteforce(T, ng, tile, density):
    mask = dg.mask_bernoulli(T, ng, density, seed=T * 31 + ng)
    perm, counts, padded = oracle.reorder(mask, tile)
    for g in range(ng):
        assert np.array_equal(perm[g], np.argsort(mask[:, g] == 0, kind="stable"))
    bp, bc, bpad = brute_reorder(mask, tile)
    assert np.array_equal(perm, bp) and np.array_equal(counts, bc) and np.array_equal(padded, bpad)
    check_reorder_invariants(mask, tile, perm, counts, padded)


def test_oracle_reorder_special_cases():
    T, ng = 300, 4
    for m, cnt in ((np.ones((T, ng), np.uint8), T), (np.zeros((T, ng), np.uint8), 0)):
        perm, counts, padded = oracle.reorder(m, 128)
        assert np.all(perm == np.arange(T)[None, :]) and np.all(counts == cnt)
        assert np.all(padded == (-(-cnt // 128) * 128))
    m = np.zeros((T, ng), np.uint8)
    m[177, 2] = 5  # any nonzero byte means active
    perm, counts, padded = oracle.reorder(m, 64)
    assert counts[2] == 1 and perm[2, 0] == 177 and padded[2] == 64
    assert np.array_equal(perm[2, 1:], np.delete(np.arange(T), 177))


def test_oracle_reorder_hand_fixture():
    with open(os.path.join(GOLDEN, "reorder_hand.json")) as f:
        fx = json.load(f)
    mask = np.array(fx["mask"], dtype=np.uint8)
    perm, counts, padded = oracle.reorder(mask, fx["tile"])
    assert perm.tolist() == fx["perm"]
    assert counts.tolist() == fx["counts"] and padded.tolist() == fx["padded"]


def test_oracle_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.reorder(np.ones((4, 2), np.uint8), 0)
    p = rand_problem(5, T=2, d=4, d_ff=8, G=4)
    with pytest.raises(ValueError):
        oracle.ffn(p["X"], p["Wg"], p["Wu"], p["Wd"], p["mask"], 4, rows=[0, 2])


# ----------------------------------------------------------------------------- masked GEMM pins
# The N-axis and K-axis group-masked GEMMs (the GEMM-MN and GEMM-K families):
# C[m,n] = mask[m, n/G] ? A[m].B[n] : 0  and  C[m,n] = sum_k mask[m, k/G] A[m,k] B[n,k].

def gemm_problem(seed, M, N, K, G, axis, density=0.5):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = rng.standard_normal((N, K)).astype(np.float32)
    ng = (N if axis == "n" else K) // G
    mask = (rng.random((M, ng)) < density).astype(np.uint8)
    return A, B, mask


def gemm_fn(axis):
    return oracle.gemm_mn if axis == "n" else oracle.gemm_k


def dense64(A, B):
    return A.astype(np.float64) @ B.astype(np.float64).T


def gpin_dense_limit(fn, axis):
    A, B, m = gemm_problem(31, 7, 24, 20, 4, axis)
    return rel(fn(A, B, np.ones_like(m), 4), dense64(A, B)) <= 1e-12


def gpin_zero_limit(fn, axis):
    A, B, m = gemm_problem(32, 5, 16, 12, 4, axis)
    return bool(np.all(fn(A, B, np.zeros_like(m), 4) == 0.0))


def gpin_uniform_mask(fn, axis):
    """A mask shared by every row equals a dense GEMM on the kept columns (N) or K slices."""
    G, M, N, K = 4, 6, 20, 24
    A, B, m = gemm_problem(33, M, N, K, G, axis)
    S = np.array([0, 2, 3])
    m = np.zeros_like(m)
    m[:, S] = 1
    idx = np.concatenate([np.arange(g * G, (g + 1) * G) for g in S])
    C = fn(A, B, m, G)
    if axis == "n":
        ref = np.zeros((M, N))
        ref[:, idx] = dense64(A, B[idx])
    else:
        ref = dense64(A[:, idx], B[:, idx])
    return rel(C, ref) <= 1e-12


def gpin_additivity(fn, axis):
    """K axis: the result is the sum of single-group results; N axis: the groups are disjoint."""
    G, M, N, K = 4, 5, 16, 24
    A, B, m = gemm_problem(34, M, N, K, G, axis)
    C = fn(A, B, m, G)
    acc = np.zeros_like(C)
    for g in range(m.shape[1]):
        mg = np.zeros_like(m)
        mg[:, g] = m[:, g]
        acc += fn(A, B, mg, G)
    return rel(C, acc) <= 1e-12


def gpin_row_equivariance(fn, axis):
    A, B, m = gemm_problem(35, 9, 16, 16, 8, axis)
    C = fn(A, B, m, 8)
    pi = np.random.default_rng(5).permutation(9)
    return bool(np.array_equal(fn(A[pi], B, m[pi], 8), C[pi]))


def gpin_mpmath(fn, axis):
    mpmath.mp.dps = 50
    worst = 0.0
    for seed, (M, N, K, G) in enumerate([(3, 8, 6, 2), (2, 4, 8, 4), (4, 6, 6, 1)]):
        A, B, m = gemm_problem(200 + seed, M, N, K, G, axis, density=0.6)
        C = fn(A, B, m, G)
        ref = np.zeros((M, N), dtype=object)
        for i in range(M):
            for n in range(N):
                if axis == "n":
                    keep = m[i, n // G] != 0
                    ref[i, n] = mpmath.fsum(mpmath.mpf(float(A[i, k])) * mpmath.mpf(float(B[n, k]))
                                            for k in range(K)) if keep else mpmath.mpf(0)
                else:
                    ref[i, n] = mpmath.fsum(mpmath.mpf(float(A[i, k])) * mpmath.mpf(float(B[n, k]))
                                            for k in range(K) if m[i, k // G])
        scale = max(float(abs(v)) for v in ref.flat) or 1.0
        for c, r in zip(C.flat, ref.flat):
            worst = max(worst, float(abs(mpmath.mpf(float(c)) - r)) / scale)
    return worst <= 1e-14


GEMM_PINS = [gpin_dense_limit, gpin_zero_limit, gpin_uniform_mask, gpin_additivity,
             gpin_row_equivariance, gpin_mpmath]


@pytest.mark.parametrize("axis", ["n", "k"])
@pytest.mark.parametrize("pin", GEMM_PINS, ids=lambda f: f.__name__)
def test_oracle_gemm_pins(pin, axis):
    assert pin(gemm_fn(axis), axis)


def test_oracle_gemm_single_group_is_row_skipping():
    """M-axis (dynamic depth) is the N-axis case with one group: rows are dense or zero."""
    A, B, _ = gemm_problem(36, 6, 12, 10, 12, "n")
    m = np.array([[1], [0], [1], [1], [0], [0]], dtype=np.uint8)
    C = oracle.gemm_mn(A, B, m, 12)
    D = dense64(A, B)
    assert np.array_equal(C[m[:, 0] == 0], np.zeros((3, 12)))
    assert rel(C[m[:, 0] != 0], D[m[:, 0] != 0]) <= 1e-12


def test_oracle_ffn_is_the_composition_of_the_masked_gemms():
    """The FFN oracle equals GEMM-K(silu(GEMM-MN(X, Wg)) * GEMM-MN(X, Wu), Wd) with one mask."""
    G = 4
    p = rand_problem(41, T=6, d=12, d_ff=16, G=G)
    a = oracle.gemm_mn(p["X"], p["Wg"], p["mask"], G)
    b = oracle.gemm_mn(p["X"], p["Wu"], p["mask"], G)
    H = silu64(a) * b  # zero wherever the group is masked
    Hf = H.astype(np.float32)  # the GEMM oracle takes float32 operands
    Y = oracle.gemm_k(Hf, p["Wd"], p["mask"], G)
    Href, Yref = oracle.ffn(p["X"], p["Wg"], p["Wu"], p["Wd"], p["mask"], G)
    assert rel(H, Href) <= 1e-12
    assert rel(Y, Yref) <= 1e-6  # float32 rounding of H


def _np_gemm(A, B, mask, G, axis, bug=None):
    A, B = A.astype(np.float64), B.astype(np.float64)
    M, K = A.shape
    N = B.shape[0]
    L = N if axis == "n" else K
    gidx = (np.arange(L) % (L // G)) if bug == "interleaved_groups" else (np.arange(L) // G)
    m = mask
    if bug == "mask_ignored":
        m = np.ones_like(mask)
    if bug == "row_shift":
        m = np.roll(mask, 1, axis=0)
    keep = m[:, gidx] != 0
    if axis == "n":
        C = np.where(keep, A @ B.T, 0.0)
        if bug == "mask_on_k":
            C = A @ B.T
    else:
        C = np.where(keep, A, 0.0) @ B.T
        if bug == "mask_on_n":
            C = np.where(keep[:, :N] if keep.shape[1] >= N else 1.0, A @ B.T, 0.0)
    if bug == "transposed_b":
        C = C.T[:M, :N] if C.shape[0] >= N else C[:, ::-1]
    return C


GEMM_MUTANTS = [(axis, bug) for axis in ("n", "k")
                for bug in ("interleaved_groups", "mask_ignored", "row_shift", "transposed_b")]
GEMM_MUTANTS += [("n", "mask_on_k"), ("k", "mask_on_n")]


@pytest.mark.parametrize("axis", ["n", "k"])
def test_gemm_pins_pass_on_correct_numpy_variant(axis):
    fn = lambda A, B, m, G: _np_gemm(A, B, m, G, axis)  # noqa: E731
    assert all(pin(fn, axis) for pin in GEMM_PINS if pin is not gpin_mpmath)


@pytest.mark.parametrize("axis,bug", GEMM_MUTANTS)
def test_gemm_pins_catch_planted_mistake(axis, bug):
    fn = lambda A, B, m, G: _np_gemm(A, B, m, G, axis, bug=bug)  # noqa: E731
    results = {}
    for pin in GEMM_PINS:
        if pin is gpin_mpmath:
            continue
        try:
            results[pin.__name__] = pin(fn, axis)
        except (ValueError, IndexError):
            results[pin.__name__] = False
    assert not all(results.values()), f"no pin caught '{bug}' on axis {axis}: {results}"


# ----------------------------------------------------------------------------- router
# The bottleneck router (ai.info summary, "How decisions are made"). Pins: a
# hand-derived fixture, closed forms of the two nonlinearities, the argmax's
# invariance to a positive scale of W2 and its flip when each group's two
# class rows are swapped, token independence, and 50-digit brute force.

def router_problem(seed, T, D, r, ng, scale=1.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    X = rng.standard_normal((T, D)).astype(np.float32)
    W1 = (rng.standard_normal((r, D)) / np.sqrt(D)).astype(np.float32)
    W2 = (scale * rng.standard_normal((2 * ng, r)) / np.sqrt(r)).astype(np.float32)
    return X, W1, W2


def oracle_router_fn(X, W1, W2, act):
    return oracle.router(X, W1, W2, act)


def rpin_hand_fixture(fn):
    f = json.load(open(os.path.join(GOLDEN, "router_hand.json")))
    X, W1, W2 = (np.array(f[k], np.float32) for k in ("X", "W1", "W2"))
    logits, mask = fn(X, W1, W2, f["act"])
    return (np.array_equal(mask, np.array(f["mask"], np.uint8))
            and np.allclose(logits, np.array(f["logits"]), rtol=0, atol=1e-12))


def rpin_activation_closed_forms(fn):
    # z = act(a) with a = x0, and one group whose class-0 logit is z, class-1 logit 0
    X = np.array([[1.0, 0.0], [-2.0, 0.0], [0.5, 0.0]], np.float32)
    W1 = np.array([[1.0, 0.0]], np.float32)
    W2 = np.array([[1.0], [0.0]], np.float32)
    ok = True
    expect = {"identity": [1.0, -2.0, 0.5], "relu": [1.0, 0.0, 0.5],
              "silu": [1 / (1 + np.exp(-1.0)), -2.0 / (1 + np.exp(2.0)), 0.5 / (1 + np.exp(-0.5))]}
    for act, want in expect.items():
        logits, mask = fn(X, W1, W2, act)
        ok &= np.allclose(logits[:, 0, 0], want, rtol=0, atol=1e-14)
        ok &= np.array_equal(mask[:, 0], (np.array(want) >= 0).astype(np.uint8))
    return ok


def rpin_scale_and_swap(fn):
    X, W1, W2 = router_problem(11, 64, 48, 16, 12)
    l0, m0 = fn(X, W1, W2, "silu")
    _, m1 = fn(X, W1, (W2 * np.float32(4.0)).astype(np.float32), "silu")
    swapped = W2.reshape(12, 2, 16)[:, ::-1, :].reshape(24, 16).copy()
    _, m2 = fn(X, W1, swapped, "silu")
    ties = l0[:, :, 0] == l0[:, :, 1]
    return np.array_equal(m0, m1) and np.array_equal(m2[~ties], 1 - m0[~ties])


def rpin_token_independence(fn):
    X, W1, W2 = router_problem(12, 40, 32, 8, 6)
    perm = np.random.Generator(np.random.PCG64(3)).permutation(40)
    l, m = fn(X, W1, W2, "relu")
    lp, mp_ = fn(X[perm], W1, W2, "relu")
    return np.array_equal(lp, l[perm]) and np.array_equal(mp_, m[perm])


def rpin_mpmath(fn):
    mpmath.mp.dps = 50
    X, W1, W2 = router_problem(13, 3, 8, 4, 3)
    ok = True
    for act in ("identity", "relu", "silu"):
        logits, mask = fn(X, W1, W2, act)
        for t in range(3):
            z = []
            for j in range(4):
                a = mpmath.fsum(mpmath.mpf(float(X[t, k])) * mpmath.mpf(float(W1[j, k])) for k in range(8))
                z.append(a if act == "identity" else (max(a, 0) if act == "relu" else a / (1 + mpmath.exp(-a))))
            for g in range(3):
                ref = [mpmath.fsum(mpmath.mpf(float(W2[2 * g + c, j])) * z[j] for j in range(4)) for c in (0, 1)]
                ok &= abs(float(ref[0]) - logits[t, g, 0]) <= 1e-14 and abs(float(ref[1]) - logits[t, g, 1]) <= 1e-14
                ok &= int(mask[t, g]) == int(ref[0] >= ref[1])
    return ok


ROUTER_PINS = [rpin_hand_fixture, rpin_activation_closed_forms, rpin_scale_and_swap,
               rpin_token_independence, rpin_mpmath]


@pytest.mark.parametrize("pin", ROUTER_PINS, ids=lambda p: p.__name__)
def test_oracle_router_pins(pin):
    assert pin(oracle_router_fn)


def test_oracle_router_rows_subset_and_rejects_bad_arguments():
    X, W1, W2 = router_problem(14, 30, 16, 8, 5)
    l, m = oracle.router(X, W1, W2, "silu")
    rows = [29, 0, 7]
    lr, mr = oracle.router(X, W1, W2, "silu", rows=rows)
    assert np.array_equal(lr, l[rows]) and np.array_equal(mr, m[rows])
    with pytest.raises(ValueError):
        oracle.router(X, W1, W2, "silu", rows=[30])
    with pytest.raises(ValueError):
        oracle.router(X, W1[:, :8], W2, "silu")


def _np_router(X, W1, W2, act, bug=None):
    x, w1, w2 = (np.asarray(a, np.float64) for a in (X, W1, W2))
    if bug == "w1_transposed":
        w1 = w1.T.reshape(w1.shape) if w1.shape[0] != w1.shape[1] else w1.T
    a = x @ w1.T
    if bug == "act_after_w2":
        z = a
    elif act == "relu":
        z = np.maximum(a, 0)
    elif act == "silu":
        z = a / (1 + np.exp(-a))
    else:
        z = a
    lg = z @ w2.T
    if bug == "act_after_w2" and act != "identity":
        lg = np.maximum(lg, 0) if act == "relu" else lg / (1 + np.exp(-lg))
    ng = w2.shape[0] // 2
    if bug == "class_major_layout":
        logits = lg.reshape(-1, 2, ng).transpose(0, 2, 1)
    else:
        logits = lg.reshape(-1, ng, 2)
    if bug == "polarity":
        mask = (logits[:, :, 1] >= logits[:, :, 0]).astype(np.uint8)
    elif bug == "tie_skips":
        mask = (logits[:, :, 0] > logits[:, :, 1]).astype(np.uint8)
    else:
        mask = (logits[:, :, 0] >= logits[:, :, 1]).astype(np.uint8)
    return logits, mask


ROUTER_MUTANTS = ["polarity", "tie_skips", "class_major_layout", "act_after_w2", "w1_transposed"]


def test_router_pins_pass_on_correct_numpy_variant():
    assert all(pin(_np_router) for pin in ROUTER_PINS if pin is not rpin_mpmath)


@pytest.mark.parametrize("bug", ROUTER_MUTANTS)
def test_router_pins_catch_planted_mistake(bug):
    fn = lambda X, W1, W2, act: _np_router(X, W1, W2, act, bug=bug)  # noqa: E731
    results = {}
    for pin in ROUTER_PINS:
        if pin is rpin_mpmath:
            continue
        try:
            results[pin.__name__] = bool(pin(fn))
        except (ValueError, IndexError):
            results[pin.__name__] = False
    assert not all(results.values()), f"no pin caught '{bug}': {results}"


# ----------------------------------------------------------------------------- attention
# Head-group-pruned causal attention (ai.info summary, "What gets pruned";
# WIDE paper App. B, "Implementation of Attention"). Pins: a hand-derived
# fixture, torch's causal scaled-dot-product attention when every pair is
# active, the closed forms of a zero query (prefix mean of V) and of the first
# token (v0), skipped pairs giving exact zeros while every other pair is
# unchanged, and 50-digit brute force.

def attention_problem(seed, T, Hq, Hk, dh):
    rng = np.random.Generator(np.random.PCG64(seed))
    Q = rng.standard_normal((T, Hq * dh)).astype(np.float32)
    K = rng.standard_normal((T, Hk * dh)).astype(np.float32)
    V = rng.standard_normal((T, Hk * dh)).astype(np.float32)
    return Q, K, V


def oracle_attention_fn(Q, K, V, mask, Hq, Hk):
    return oracle.attention(Q, K, V, mask, Hq, Hk)


def apin_hand_fixture(fn):
    f = json.load(open(os.path.join(GOLDEN, "attention_hand.json")))
    Q, K, V = (np.array(f[k], np.float32) for k in ("Q", "K", "V"))
    ok = True
    for case in f["cases"]:
        O = fn(Q, K, V, np.array(case["mask"], np.uint8), f["Hq"], f["Hk"])
        ok &= np.allclose(O, np.array(case["O"]), rtol=0, atol=1e-12)
    return bool(ok)


def apin_sdpa(fn):
    T, Hq, Hk, dh = 37, 4, 2, 16
    Q, K, V = attention_problem(21, T, Hq, Hk, dh)
    O = fn(Q, K, V, np.ones((T, Hk), np.uint8), Hq, Hk)
    q = torch.from_numpy(Q.astype(np.float64)).view(T, Hq, dh).transpose(0, 1)
    k = torch.from_numpy(K.astype(np.float64)).view(T, Hk, dh).transpose(0, 1)
    v = torch.from_numpy(V.astype(np.float64)).view(T, Hk, dh).transpose(0, 1)
    k = k.repeat_interleave(Hq // Hk, dim=0).contiguous()
    v = v.repeat_interleave(Hq // Hk, dim=0).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None], is_causal=True)
    ref = ref[0].transpose(0, 1).reshape(T, Hq * dh).numpy()
    return bool(np.allclose(O, ref, rtol=0, atol=1e-10))


def apin_zero_query_prefix_mean(fn):
    T, Hq, Hk, dh = 20, 2, 2, 8
    _, K, V = attention_problem(22, T, Hq, Hk, dh)
    O = fn(np.zeros((T, Hq * dh), np.float32), K, V, np.ones((T, Hk), np.uint8), Hq, Hk)
    v = V.astype(np.float64).reshape(T, Hk, dh)
    mean = np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None, None]
    return bool(np.allclose(O.reshape(T, Hq, dh), mean, rtol=0, atol=1e-12)
                and np.array_equal(O.reshape(T, Hq, dh)[0], v[0]))


def apin_skip_is_zero_and_local(fn):
    T, Hq, Hk, dh = 30, 6, 3, 8
    Q, K, V = attention_problem(23, T, Hq, Hk, dh)
    full = fn(Q, K, V, np.ones((T, Hk), np.uint8), Hq, Hk).reshape(T, Hq, dh)
    mask = (np.random.Generator(np.random.PCG64(5)).random((T, Hk)) < 0.5).astype(np.uint8)
    O = fn(Q, K, V, mask, Hq, Hk).reshape(T, Hq, dh)
    on = np.repeat(mask.astype(bool), Hq // Hk, axis=1)  # [T, Hq]
    return bool(np.all(O[~on] == 0.0) and np.array_equal(O[on], full[on]))


def apin_mpmath(fn):
    mpmath.mp.dps = 50
    T, Hq, Hk, dh = 3, 2, 1, 3
    Q, K, V = attention_problem(24, T, Hq, Hk, dh)
    O = fn(Q, K, V, np.ones((T, Hk), np.uint8), Hq, Hk).reshape(T, Hq, dh)
    ok = True
    sc = 1 / mpmath.sqrt(dh)
    for t in range(T):
        for h in range(Hq):
            s = [mpmath.fsum(mpmath.mpf(float(Q[t, h * dh + e])) * mpmath.mpf(float(K[j, e]))
                             for e in range(dh)) * sc for j in range(t + 1)]
            w = [mpmath.exp(x) for x in s]
            z = mpmath.fsum(w)
            for e in range(dh):
                ref = mpmath.fsum(w[j] * mpmath.mpf(float(V[j, e])) for j in range(t + 1)) / z
                ok &= abs(float(ref) - O[t, h, e]) <= 1e-14
    return bool(ok)


ATTENTION_PINS = [apin_hand_fixture, apin_sdpa, apin_zero_query_prefix_mean,
                  apin_skip_is_zero_and_local, apin_mpmath]


@pytest.mark.parametrize("pin", ATTENTION_PINS, ids=lambda p: p.__name__)
def test_oracle_attention_pins(pin):
    assert pin(oracle_attention_fn)


def test_oracle_attention_rows_subset_and_rejects_bad_arguments():
    Q, K, V = attention_problem(25, 12, 4, 2, 8)
    mask = np.ones((12, 2), np.uint8)
    O = oracle.attention(Q, K, V, mask, 4, 2)
    rows = [11, 0, 5]
    assert np.array_equal(oracle.attention(Q, K, V, mask, 4, 2, rows=rows), O[rows])
    with pytest.raises(ValueError):
        oracle.attention(Q, K, V, mask, 4, 2, rows=[12])
    with pytest.raises(ValueError):
        oracle.attention(Q, K, V, mask, 4, 3)
    with pytest.raises(ValueError):
        oracle.attention(Q, K[:, :8], V, mask, 4, 2)


def _np_attention(Q, K, V, mask, Hq, Hk, bug=None):
    T = Q.shape[0]
    dh = Q.shape[1] // Hq
    q = Q.astype(np.float64).reshape(T, Hq, dh)
    k = K.astype(np.float64).reshape(T, Hk, dh)
    v = V.astype(np.float64).reshape(T, Hk, dh)
    O = np.zeros((T, Hq, dh))
    scale = 1.0 if bug == "no_scale" else 1.0 / np.sqrt(dh)
    for t in range(T):
        for h in range(Hq):
            g = h % Hk if bug == "gqa_modulo" else h // (Hq // Hk)
            if not mask[t, g] and bug != "mask_ignored":
                continue
            hi = T if bug == "not_causal" else (t if bug == "causal_off_by_one" else t + 1)
            keys = [j for j in range(hi) if bug != "mask_on_keys" or mask[j, g]]
            if not keys:
                continue
            s = np.array([q[t, h] @ k[j, g] for j in keys]) * scale
            w = np.exp(s - s.max())
            O[t, h] = (w[:, None] * v[keys, g]).sum(0) / w.sum()
    return O.reshape(T, Hq * dh)


ATTENTION_MUTANTS = ["not_causal", "causal_off_by_one", "no_scale", "gqa_modulo", "mask_ignored",
                     "mask_on_keys"]


def test_attention_pins_pass_on_correct_numpy_variant():
    assert all(pin(_np_attention) for pin in ATTENTION_PINS if pin is not apin_mpmath)


@pytest.mark.parametrize("bug", ATTENTION_MUTANTS)
def test_attention_pins_catch_planted_mistake(bug):
    fn = lambda *a: _np_attention(*a, bug=bug)  # noqa: E731
    results = {}
    for pin in ATTENTION_PINS:
        if pin is apin_mpmath:
            continue
        try:
            results[pin.__name__] = bool(pin(fn))
        except (ValueError, IndexError):
            results[pin.__name__] = False
    assert not all(results.values()), f"no pin caught '{bug}': {results}"


def test_native_build_is_bit_identical(tmp_path):
    """The CPU baseline times a gcc -O3 -march=native build of the oracle; it
    must compute the same doubles as the -O2 build the tests use."""
    import ctypes
    path = oracle.build_native(str(tmp_path))
    native = ctypes.CDLL(path)
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    native.oracle_ffn.argtypes = [p, p, p, p, p, i64, i64, i64, i64, p, i64, p, p]
    native.oracle_ffn.restype = ctypes.c_int
    inp = dg.random_small(4242, 9, 64, 256, 32, "bf16", 0.5, wscale=0.05)
    X, Wg, Wu, Wd = (np.ascontiguousarray(inp[k].float().numpy()) for k in ("X", "Wg", "Wu", "Wd"))
    m = np.ascontiguousarray(inp["mask"].numpy())

    H, Y = np.empty((9, 256)), np.empty((9, 64))
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    assert native.oracle_ffn(ptr(X), ptr(Wg), ptr(Wu), ptr(Wd), ptr(m), 9, 64, 256, 32, None, 9,
                             ptr(H), ptr(Y)) == 0
    H0, Y0 = oracle.ffn(X, Wg, Wu, Wd, m, 32)
    assert np.array_equal(H.view(np.int64), H0.view(np.int64))
    assert np.array_equal(Y.view(np.int64), Y0.view(np.int64))
