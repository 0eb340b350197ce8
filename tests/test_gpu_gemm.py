"""Group-masked GEMMs (N axis and K axis) on the GPU vs the fp64 oracle.

Bars (applied element by element):
  * C: max|err| / max|ref| <= 2e-2 (bf16 operands, fp32 accumulation, one
    rounding of C);
  * N axis: C exactly +0.0 at every (row, group) the mask skips;
  * K axis: A's values at skipped (row, group) pairs never matter (NaN there
    gives the same bits as zeros there);
  * all-zero masks give C == +0.0 everywhere; M == 0 is a no-op.
Small cases compare every output; the attention-shaped full-size cases
compare a seeded sample of rows and check the exact properties on all rows.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import group_sparse_ffn_amd as wide
from group_sparse_ffn_amd import datagen as dg

pytestmark = pytest.mark.gpu

TOL = 2e-2
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def announce(request):
    sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


def rel_err(c, ref):
    c = c.detach().float().cpu().numpy().astype(np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(c - ref)) / (den if den > 0 else 1.0))


def run(axis, inp, G):
    fn = wide.gemm_mn if axis == "mn" else wide.gemm_k
    C = fn(inp["A"].to(DEV), inp["B"].to(DEV), inp["mask"].to(DEV), G)
    torch.cuda.synchronize()
    return C


def ref(axis, inp, G, rows=None):
    fn = oracle.gemm_mn if axis == "mn" else oracle.gemm_k
    return fn(inp["A"], inp["B"], inp["mask"], G, rows=rows)


def check_mn_zeros(C, mask, G):
    m = mask.to(DEV).bool().repeat_interleave(G, dim=1)
    off = C[~m]
    assert off.numel() == 0 or bool((off == 0).all()), "nonzero C at a skipped (row, group)"
    # +0.0, not -0.0
    assert off.numel() == 0 or not bool(torch.signbit(off.float()).any())


# (M, N, K, G, mask kind, density): ragged M tails, every channel-block width
# (16 .. 256), several N tiles, one group (M axis), and > 768 K-groups (the
# down kernel's global mask-word path).
MN_CASES = [
    (300, 256, 128, 16, "bernoulli", 0.5),
    (40, 48, 64, 16, "bernoulli", 0.5),
    (1000, 512, 256, 32, "beta", 0.4),
    (513, 768, 64, 64, "bernoulli", 0.3),
    (257, 1024, 192, 128, "topk", 0.5),
    (700, 1024, 128, 256, "bernoulli", 0.6),
    (600, 1024, 128, 512, "topk", 0.5),
    (777, 256, 128, 256, "bernoulli", 0.5),   # one group: dynamic depth
    (300, 384, 64, 384, "bernoulli", 0.5),    # one group, G = 384 (128-wide blocks)
]
K_CASES = [
    (300, 256, 128, 16, "bernoulli", 0.5),
    (40, 48, 64, 16, "bernoulli", 0.5),
    (1000, 200, 256, 32, "beta", 0.4),        # N = 200: ragged output tile
    (513, 520, 512, 64, "bernoulli", 0.3),
    (257, 512, 1024, 128, "topk", 0.5),
    (700, 256, 1024, 512, "topk", 0.5),
    (300, 64, 12544, 16, "bernoulli", 0.5),   # 784 groups: mask words from global memory
    (777, 256, 256, 256, "bernoulli", 0.5),   # one group
]


def _w(M, N, K, G, axis, kind, density, wid=20):
    return dg.GemmWorkload(f"gemm-{axis}-{M}x{N}x{K}-G{G}", wid, M=M, N=N, K=K, G=G, axis=axis,
                           mask_kind=kind, density=density)


@pytest.mark.parametrize("M,N,K,G,kind,density", MN_CASES)
def test_gemm_mn_small_all_outputs(M, N, K, G, kind, density):
    w = _w(M, N, K, G, "mn", kind, density)
    inp = dg.make_gemm_inputs(w)
    C = run("mn", inp, G)
    assert rel_err(C, ref("mn", inp, G)) <= TOL
    check_mn_zeros(C, inp["mask"], G)


@pytest.mark.parametrize("M,N,K,G,kind,density", K_CASES)
def test_gemm_k_small_all_outputs(M, N, K, G, kind, density):
    w = _w(M, N, K, G, "k", kind, density, wid=21)
    inp = dg.make_gemm_inputs(w)
    C = run("k", inp, G)
    r = ref("k", inp, G)
    assert rel_err(C, r) <= TOL
    # rows with no active group are exactly +0.0
    dead = ~inp["mask"].bool().any(dim=1)
    if bool(dead.any()):
        assert bool((C[dead.to(DEV)] == 0).all())


@pytest.mark.parametrize("G,K", [(64, 512), (16, 12544)])
def test_gemm_k_ignores_skipped_a_values(G, K):
    w = _w(300, 256, K, G, "k", "bernoulli", 0.5, wid=22)
    inp = dg.make_gemm_inputs(w)
    m = inp["mask"].bool().repeat_interleave(G, dim=1)
    A_nan = inp["A"].clone()
    A_nan[~m] = float("nan")
    A_zero = inp["A"].clone()
    A_zero[~m] = 0
    B, mask = inp["B"].to(DEV), inp["mask"].to(DEV)
    C_nan = wide.gemm_k(A_nan.to(DEV), B, mask, G)
    C_zero = wide.gemm_k(A_zero.to(DEV), B, mask, G)
    torch.cuda.synchronize()
    assert torch.equal(C_nan.view(torch.int16), C_zero.view(torch.int16))
    assert rel_err(C_nan, ref("k", inp, G)) <= TOL


@pytest.mark.parametrize("axis", ["mn", "k"])
def test_gemm_all_zero_mask_and_m0(axis):
    w = _w(500, 512, 256, 128, axis, "zeros", 0.0, wid=23)
    inp = dg.make_gemm_inputs(w)
    C = run(axis, inp, 128)
    assert bool((C == 0).all()) and not bool(torch.signbit(C.float()).any())
    fn = wide.gemm_mn if axis == "mn" else wide.gemm_k
    e = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    ng = 512 // 128 if axis == "mn" else 256 // 128
    C0 = fn(e, inp["B"].to(DEV), torch.empty((0, ng), dtype=torch.uint8, device=DEV), 128)
    torch.cuda.synchronize()
    assert C0.shape == (0, 512)


@pytest.mark.parametrize("axis", ["mn", "k"])
def test_gemm_all_ones_mask_is_dense(axis):
    w = _w(600, 512, 384, 128, axis, "ones", 1.0, wid=24)
    inp = dg.make_gemm_inputs(w)
    C = run(axis, inp, 128)
    dense = inp["A"].double().numpy() @ inp["B"].double().numpy().T
    assert rel_err(C, dense) <= TOL


def test_gemm_k_equals_ffn_down_bitwise():
    """The FFN's down projection is the K-axis GEMM on (H, Wdown, mask)."""
    w = dg.Workload("ffn-vs-gemm-k", 25, T=700, d=256, d_ff=1024, G=64, dtype="bf16",
                    mask_kind="bernoulli")
    inp = {k: v.to(DEV) for k, v in dg.make_inputs(w).items()}
    Y, H = wide.ffn_forward(inp["X"], inp["Wg"], inp["Wu"], inp["Wd"], inp["mask"], 64,
                            return_h=True)
    C = wide.gemm_k(H, inp["Wd"], inp["mask"], 64)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), C.view(torch.int16))


@pytest.mark.parametrize("axis", ["mn", "k"])
def test_gemm_deterministic(axis):
    w = _w(1000, 512, 512, 64, axis, "bernoulli", 0.5, wid=26)
    inp = dg.make_gemm_inputs(w)
    C1 = run(axis, inp, 64)
    C2 = run(axis, inp, 64)
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))


def sampled_rows(M, n_random, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    fixed = [0, 1, 255, 256, M // 2, M - 257, M - 256, M - 1]
    return np.unique(np.concatenate([fixed, rng.integers(0, M, n_random)])).astype(np.int64)


@pytest.mark.parametrize("w", [dg.LLAMA8B_ATTN_Q, dg.LLAMA8B_ATTN_O, dg.LLAMA8B_DEPTH],
                         ids=lambda w: w.name)
def test_attention_shapes_full_size_sampled(w):
    inp = dg.make_gemm_inputs(w)
    C = run(w.axis, inp, w.G)
    rows = sampled_rows(w.M, 48, w.seed)
    r = ref(w.axis, inp, w.G, rows=rows)
    assert rel_err(C[torch.from_numpy(rows).to(DEV)], r) <= TOL
    if w.axis == "mn":
        check_mn_zeros(C, inp["mask"], w.G)
    assert bool(torch.isfinite(C.float()).all())


def test_ffn_many_groups_never_reads_skipped_h():
    """784 groups (past the down kernel's LDS mask table): the H workspace is
    filled with NaN bits before the call and no NaN may reach Y."""
    w = dg.Workload("ffn-784-groups", 27, T=300, d=64, d_ff=12544, G=16, dtype="bf16",
                    mask_kind="bernoulli")
    inp = dg.make_inputs(w)
    d = {k: v.to(DEV) for k, v in inp.items()}
    nbytes = wide.workspace_size(w.T, w.d, w.d_ff, w.G, torch.bfloat16)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=DEV)
    call = wide.FfnCall(d["X"], d["Wg"], d["Wu"], d["Wd"], d["mask"], w.G, workspace=ws,
                        flags=wide.WIDE_FLAG_FORCE_PREFILL)
    Y = call.run()
    torch.cuda.synchronize()
    _, Yref = oracle.ffn(inp["X"], inp["Wg"], inp["Wu"], inp["Wd"], inp["mask"], w.G)
    assert bool(torch.isfinite(Y.float()).all())
    assert rel_err(Y, Yref) <= TOL


def _graph_replays_match(run_fn, out, eager, n=4):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run_fn()
    torch.cuda.current_stream().wait_stream(s)
    for i in range(n):
        out.fill_(3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from eager"
    return g


@pytest.mark.parametrize("axis", ["mn", "k"])
def test_gemm_graph_replay_matches_eager(axis):
    w = _w(700, 512, 512, 128, axis, "bernoulli", 0.5, wid=28)
    inp = {k: v.to(DEV) for k, v in dg.make_gemm_inputs(w).items()}
    fn = wide.gemm_mn if axis == "mn" else wide.gemm_k
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(wide.gemm_workspace_size(w.M, w.ngroups), dtype=torch.uint8, device=DEV)
    fn(inp["A"], inp["B"], inp["mask"], w.G, C=C, workspace=ws)
    torch.cuda.synchronize()
    eager = C.clone()
    g = _graph_replays_match(lambda: fn(inp["A"], inp["B"], inp["mask"], w.G, C=C, workspace=ws),
                             C, eager)
    # the mask is read on the device at replay time
    inp["mask"].zero_()
    g.replay()
    torch.cuda.synchronize()
    assert bool((C == 0).all())
