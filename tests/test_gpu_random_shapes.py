"""Seeded random shapes, HIP path vs the fp64 oracle (run with -m gpu).

The fixed cases elsewhere pin the measured workloads and the edges each kernel
was written around; these draw sizes from the whole supported range (one fixed
seed, so every run checks the same cases, each named in its test id): odd
token counts on both sides of the decode limit, group widths that are and are
not multiples of 32 and 64, one to many groups, random mask densities. Every
output element is compared, with the bars of the other parity tests:
  * FFN, bf16: max|Y - ref| / max|ref| <= 2e-2, H exactly 0 at masked
    channels, Y exactly +0.0 for tokens with no active group;
  * masked GEMMs: the same 2e-2 bar; skipped (row, group) outputs of the N
    axis exactly +0.0;
  * router: logits within 1e-3 of the largest oracle logit, the mask equal to
    the kernel's own fp32 argmax, and to the oracle's wherever its two logits
    differ by more than twice that tolerance.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import group_sparse_ffn_amd as wide
from group_sparse_ffn_amd import datagen as dg

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SEED = 20261203


@pytest.fixture(autouse=True)
def announce(request):
    sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


def rel_err(y, ref):
    y = y.detach().float().cpu().numpy().astype(np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(y - ref)) / (den if den > 0 else 1.0))


def _ffn_cases(n=16):
    rng = np.random.Generator(np.random.PCG64(SEED))
    cases = []
    for i in range(n):
        T = int(rng.choice([1, 2, 3, 5, 9, 16])) if i % 3 == 0 else int(rng.integers(17, 1100))
        d = 64 * int(rng.integers(1, 13))
        G = int(rng.choice([16, 32, 48, 64, 80, 96, 128, 192, 256]))
        step = 64 // int(np.gcd(G, 64))  # groups per 64 channels: d_ff % 64 == 0
        ng = step * int(rng.integers(1, max(2, 2048 // (G * step)) + 1))
        density = float(rng.uniform(0.1, 0.9))
        cases.append((i, T, d, int(G * ng), G, round(density, 3)))
    return cases


@pytest.mark.parametrize("i,T,d,d_ff,G,density", _ffn_cases())
def test_ffn_random_shape(i, T, d, d_ff, G, density):
    inp = dg.random_small(SEED + 10 * i, T, d, d_ff, G, "bf16", density)
    Href, Yref = oracle.ffn(inp["X"], inp["Wg"], inp["Wu"], inp["Wd"], inp["mask"], G)
    dv = {k: v.to(DEV) for k, v in inp.items()}
    Y, H = wide.ffn_forward(dv["X"], dv["Wg"], dv["Wu"], dv["Wd"], dv["mask"], G, return_h=True)
    torch.cuda.synchronize()
    assert rel_err(Y, Yref) <= 2e-2
    m = dv["mask"].bool().repeat_interleave(G, dim=1)
    assert bool((H[~m] == 0).all())
    idle = ~dv["mask"].bool().any(dim=1)
    if bool(idle.any()):
        yi = Y[idle]
        assert bool((yi == 0).all()) and not bool(torch.signbit(yi.float()).any())


def _gemm_cases(n=10):
    rng = np.random.Generator(np.random.PCG64(SEED + 1))
    cases = []
    for i in range(n):
        axis = "mn" if i % 2 == 0 else "k"
        M = int(rng.integers(1, 1500))
        G = int(rng.choice([16, 32, 64, 128, 256]))
        if axis == "mn":
            K = 64 * int(rng.integers(1, 17))
            N = G * int(rng.integers(1, max(2, 2048 // G) + 1))
        else:
            step = 64 // int(np.gcd(G, 64))
            K = int(G * step * int(rng.integers(1, max(2, 2048 // (G * step)) + 1)))
            N = 8 * int(rng.integers(1, 160))
        density = round(float(rng.uniform(0.1, 0.9)), 3)
        cases.append((i, axis, M, N, K, G, density))
    return cases


@pytest.mark.parametrize("i,axis,M,N,K,G,density", _gemm_cases())
def test_masked_gemm_random_shape(i, axis, M, N, K, G, density):
    ng = (N if axis == "mn" else K) // G
    A = dg.to_dtype(dg.normal_f32(SEED + 100 + i, (M, K)), "bf16")
    B = dg.to_dtype(dg.normal_f32(SEED + 200 + i, (N, K), 0.05), "bf16")
    mask = torch.from_numpy(dg.mask_bernoulli(M, ng, density, SEED + 300 + i))
    fn, ref_fn = (wide.gemm_mn, oracle.gemm_mn) if axis == "mn" else (wide.gemm_k, oracle.gemm_k)
    C = fn(A.to(DEV), B.to(DEV), mask.to(DEV), G)
    torch.cuda.synchronize()
    ref = ref_fn(A, B, mask, G)
    assert rel_err(C, ref) <= 2e-2
    if axis == "mn":
        m = mask.to(DEV).bool().repeat_interleave(G, dim=1)
        off = C[~m]
        assert bool((off == 0).all()) and not bool(torch.signbit(off.float()).any())


def _router_cases(n=8):
    rng = np.random.Generator(np.random.PCG64(SEED + 2))
    cases = []
    for i in range(n):
        T = int(rng.integers(1, 17)) if i % 2 == 0 else int(rng.integers(17, 3000))
        D = 32 * int(rng.integers(1, 97))
        r = int(rng.choice([16, 32, 64]))
        ng = int(rng.integers(1, 200))
        act = str(rng.choice(["identity", "relu", "silu"]))
        cases.append((i, T, D, r, ng, act))
    return cases


@pytest.mark.parametrize("i,T,D,r,ng,act", _router_cases())
def test_router_random_shape(i, T, D, r, ng, act):
    X = dg.to_dtype(dg.normal_f32(SEED + 400 + i, (T, D)), "bf16")
    w = dg.make_router_weights(SEED + 500 + i, D, r, ng)
    mask, logits = wide.router_forward(X.to(DEV), w["W1"].to(DEV), w["W2"].to(DEV), act,
                                       return_logits=True)
    torch.cuda.synchronize()
    lref, mref = oracle.router(X, w["W1"], w["W2"], act)
    lg = logits.double().cpu().numpy()
    mk = mask.cpu().numpy()
    tol = 1e-3 * max(np.abs(lref).max(), 1e-30)
    assert np.abs(lg - lref).max() <= tol
    assert np.array_equal(mk, (lg[..., 0] >= lg[..., 1]).astype(np.uint8))
    clear = np.abs(lref[..., 0] - lref[..., 1]) > 2 * tol
    assert np.array_equal(mk[clear], mref[clear])
