"""The comparison pipelines (naive gather-scatter and grouped GEMM on
reordered masks, built from framework ops) against the fp64 oracle, on the
CPU. Bars as for the fused kernels: max|err| / max|ref| <= 2e-2 (bf16
operands and result), +0.0 at skipped N-axis pairs, and A's values at skipped
K-axis pairs never matter."""
import numpy as np
import pytest
import torch

import oracle
from group_sparse_ffn_amd import baselines as bl
from group_sparse_ffn_amd import datagen as dg

TOL = 2e-2


def rel_err(c, ref):
    c = c.float().numpy().astype(np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(c - ref)) / (den if den > 0 else 1.0))


def inputs(M, N, K, G, axis, kind, density, seed=40):
    w = dg.GemmWorkload(f"bl-{axis}", seed, M=M, N=N, K=K, G=G, axis=axis, mask_kind=kind,
                        density=density)
    return dg.make_gemm_inputs(w)


CASES = [
    (70, 64, 96, 16, "bernoulli", 0.5),   # ragged counts: padded per-token slots
    (50, 128, 64, 32, "topk", 0.5),       # equal counts: Table 4's exact layout
    (33, 96, 128, 32, "beta", 0.3),
    (20, 64, 64, 16, "ones", 1.0),
]


@pytest.mark.parametrize("M,N,K,G,kind,density", CASES)
def test_naive_and_grouped_mn(M, N, K, G, kind, density):
    inp = inputs(M, N, K, G, "mn", kind, density)
    ref = oracle.gemm_mn(inp["A"], inp["B"], inp["mask"], G)
    off = ~inp["mask"].bool().repeat_interleave(G, dim=1)
    for fn in (bl.naive_gemm_mn, lambda *a: bl.grouped_gemm_mn(*a, use_grouped_mm=False)):
        C = fn(inp["A"], inp["B"], inp["mask"], G)
        assert rel_err(C, ref) <= TOL
        assert bool((C[off] == 0).all()) and not bool(torch.signbit(C[off].float()).any())


@pytest.mark.parametrize("M,N,K,G,kind,density", CASES)
def test_naive_and_grouped_k(M, N, K, G, kind, density):
    inp = inputs(M, N, K, G, "k", kind, density)
    ref = oracle.gemm_k(inp["A"], inp["B"], inp["mask"], G)
    m = inp["mask"].bool().repeat_interleave(G, dim=1)
    A_nan = inp["A"].clone()
    A_nan[~m] = float("nan")
    for fn in (bl.naive_gemm_k, lambda *a: bl.grouped_gemm_k(*a, use_grouped_mm=False)):
        C = fn(A_nan, inp["B"], inp["mask"], G)
        assert bool(torch.isfinite(C.float()).all())
        assert rel_err(C, ref) <= TOL


def test_naive_m_axis_is_the_one_group_case():
    inp = inputs(90, 64, 96, 64, "mn", "bernoulli", 0.5)
    ref = oracle.gemm_mn(inp["A"], inp["B"], inp["mask"], 64)
    C = bl.naive_gemm_m(inp["A"], inp["B"], inp["mask"])
    assert rel_err(C, ref) <= TOL
    assert bool((C[~inp["mask"][:, 0].bool()] == 0).all())


@pytest.mark.parametrize("axis", ["mn", "k"])
def test_all_zero_mask_and_m0(axis):
    inp = inputs(30, 64, 64, 32, axis, "zeros", 0.0)
    naive = bl.naive_gemm_mn if axis == "mn" else bl.naive_gemm_k
    grouped = bl.grouped_gemm_mn if axis == "mn" else bl.grouped_gemm_k
    for fn in (naive, lambda *a: grouped(*a, use_grouped_mm=False)):
        C = fn(inp["A"], inp["B"], inp["mask"], 32)
        assert C.shape == (30, 64) and bool((C == 0).all())
        ng = inp["mask"].shape[1]
        C0 = fn(inp["A"][:0], inp["B"], inp["mask"][:0].reshape(0, ng), 32)
        assert C0.shape == (0, 64)


def test_table4_closed_forms():
    """The closed forms reduce to the dense terms at p = 0 and count the
    token-specific weight subsets (p M N K) three times at p > 0."""
    M, N, K = 256, 512, 128
    assert bl.traffic_elements("n", M, N, K, 0.0) == M * K + M * N
    assert bl.traffic_elements("k", M, N, K, 0.0) == M * N
    assert bl.traffic_elements("m", M, N, K, 0.0) == N * K + M * N
    for axis in "nk":
        d = bl.traffic_elements(axis, M, N, K, 0.5) - bl.traffic_elements(axis, M, N, K, 0.25)
        lin = 0.25 * 3 * (M * N if axis == "n" else M * K)
        assert d == pytest.approx(0.25 * 3 * M * N * K + lin)
    assert bl.materialized_elements("n", M, N, K, 0.5) > 0.5 * M * N * K
