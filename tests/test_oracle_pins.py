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
