"""The comparison pipelines (naive gather-scatter; grouped GEMM on reordered
masks, with the library's grouped GEMM where this torch build has one for
the device) on the GPU against the fp64 oracle, bars as for the fused
kernels (max|err| / max|ref| <= 2e-2)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from group_sparse_ffn_amd import baselines as bl
from group_sparse_ffn_amd import datagen as dg

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-2


@pytest.fixture(autouse=True)
def announce(request):
    sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


def rel_err(c, ref):
    c = c.float().cpu().numpy().astype(np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(c - ref)) / (den if den > 0 else 1.0))


def grouped_mm_available():
    try:
        a = torch.ones((4, 16), dtype=torch.bfloat16, device=DEV)
        b = torch.ones((2, 16, 16), dtype=torch.bfloat16, device=DEV)
        torch._grouped_mm(a, b, offs=torch.tensor([2, 4], dtype=torch.int32, device=DEV))
        torch.cuda.synchronize()
        return True
    except Exception:
        return False


@pytest.mark.parametrize("axis", ["mn", "k"])
@pytest.mark.parametrize("kind", ["bernoulli", "topk"])
def test_baselines_match_oracle(axis, kind):
    w = dg.GemmWorkload(f"bl-gpu-{axis}", 41, M=300, N=256, K=384, G=64, axis=axis,
                        mask_kind=kind, density=0.5)
    inp = dg.make_gemm_inputs(w)
    ref = (oracle.gemm_mn if axis == "mn" else oracle.gemm_k)(inp["A"], inp["B"], inp["mask"], 64)
    A, B, mask = (inp[k].to(DEV) for k in ("A", "B", "mask"))
    naive = bl.naive_gemm_mn if axis == "mn" else bl.naive_gemm_k
    grouped = bl.grouped_gemm_mn if axis == "mn" else bl.grouped_gemm_k
    outs = {"naive": naive(A, B, mask, 64), "grouped_loop": grouped(A, B, mask, 64, False)}
    if grouped_mm_available():
        outs["grouped_mm"] = grouped(A, B, mask, 64, True)
    torch.cuda.synchronize()
    for name, C in outs.items():
        assert rel_err(C, ref) <= TOL, name


def test_naive_m_axis_gpu():
    w = dg.GemmWorkload("bl-gpu-m", 42, M=500, N=256, K=256, G=256, axis="mn",
                        mask_kind="bernoulli", density=0.5)
    inp = dg.make_gemm_inputs(w)
    ref = oracle.gemm_mn(inp["A"], inp["B"], inp["mask"], 256)
    C = bl.naive_gemm_m(inp["A"].to(DEV), inp["B"].to(DEV), inp["mask"].to(DEV))
    torch.cuda.synchronize()
    assert rel_err(C, ref) <= TOL
