"""Bottleneck router on the GPU vs the fp64 oracle.

Bars:
  * logits: |gpu - oracle| <= 1e-3 * max|oracle logit| of the case (bf16
    operands, fp32 products and sums over D terms, then over r terms);
  * the GPU mask is its own fp32 argmax, bit for bit: mask == (l0 >= l1) on
    the returned logits (the decision is taken in the kernel's precision);
  * the GPU mask equals the oracle's wherever the oracle's two logits differ
    by more than twice the logit tolerance (elsewhere either answer is right);
  * identical class rows (an exact tie) execute; T == 0 is a no-op.
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
LOGIT_TOL = 1e-3


@pytest.fixture(autouse=True)
def announce(request):
    sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


def inputs(seed, T, D, r, ng):
    X = dg.to_dtype(dg.normal_f32(seed, (T, D)), "bf16")
    w = dg.make_router_weights(seed + 10, D, r, ng)
    return X, w["W1"], w["W2"]


def check(X, W1, W2, act, rows=None):
    mask, logits = wide.router_forward(X.to(DEV), W1.to(DEV), W2.to(DEV), act, return_logits=True)
    torch.cuda.synchronize()
    lref, mref = oracle.router(X, W1, W2, act, rows=rows)
    if rows is not None:
        idx = torch.from_numpy(np.asarray(rows)).to(DEV)
        mask, logits = mask[idx], logits[idx]
    lg = logits.double().cpu().numpy()
    mk = mask.cpu().numpy()
    tol = LOGIT_TOL * max(np.abs(lref).max(), 1e-30)
    assert np.abs(lg - lref).max() <= tol
    assert np.array_equal(mk, (lg[..., 0] >= lg[..., 1]).astype(np.uint8))
    clear = np.abs(lref[..., 0] - lref[..., 1]) > 2 * tol
    assert np.array_equal(mk[clear], mref[clear])
    return mk


@pytest.mark.parametrize("T,D,r,ng,act", [
    (1, 64, 16, 1, "identity"), (15, 256, 32, 3, "relu"), (16, 512, 64, 112, "silu"),
    (17, 4096, 32, 112, "silu"), (300, 1024, 16, 37, "relu"), (1000, 96, 32, 5, "silu"),
    (257, 4096, 64, 8, "identity"), (40, 5120, 32, 136, "silu"),
    (300, 3072, 32, 24, "silu"), (100, 2048, 32, 16, "relu"),
])
def test_router_small_all_outputs(T, D, r, ng, act):
    X, W1, W2 = inputs(T + D + r, T, D, r, ng)
    mk = check(X, W1, W2, act)
    # the synthetic router executes about half of the groups
    if T * ng >= 1000:
        assert 0.3 < mk.mean() < 0.7


def test_router_llama8b_prefill_shape_sampled():
    T, D, r, ng = 16384, 4096, 32, 112
    X, W1, W2 = inputs(9, T, D, r, ng)
    rng = np.random.Generator(np.random.PCG64(9))
    rows = np.unique(np.concatenate([[0, 15, 16, T - 1], rng.integers(0, T, 60)]))
    check(X, W1, W2, "silu", rows=rows)


def test_router_exact_tie_executes():
    T, D, r, ng = 50, 256, 16, 6
    X, W1, W2 = inputs(5, T, D, r, ng)
    W2 = W2.clone()
    W2[1::2] = W2[0::2]  # class 1 row == class 0 row in every group
    mask = wide.router_forward(X.to(DEV), W1.to(DEV), W2.to(DEV), "silu")
    torch.cuda.synchronize()
    assert bool((mask == 1).all())


def test_router_t0_and_feeds_the_ffn():
    w = dg.Workload("router-ffn", 31, T=300, d=512, d_ff=2048, G=128, dtype="bf16",
                    mask_kind="bernoulli")
    inp = dg.make_inputs(w)
    rw = dg.make_router_weights(99, w.d, 32, w.ngroups)
    d = {k: v.to(DEV) for k, v in inp.items()}
    mask = wide.router_forward(d["X"], rw["W1"].to(DEV), rw["W2"].to(DEV), "silu")
    Y = wide.ffn_forward(d["X"], d["Wg"], d["Wu"], d["Wd"], mask, w.G)
    torch.cuda.synchronize()
    _, Yref = oracle.ffn(inp["X"], inp["Wg"], inp["Wu"], inp["Wd"], mask.cpu(), w.G)
    y = Y.float().cpu().numpy().astype(np.float64)
    assert np.abs(y - Yref).max() / np.abs(Yref).max() <= 2e-2
    e = torch.empty((0, w.d), dtype=torch.bfloat16, device=DEV)
    m0 = wide.router_forward(e, rw["W1"].to(DEV), rw["W2"].to(DEV), "silu")
    torch.cuda.synchronize()
    assert m0.shape == (0, w.ngroups)


def test_router_graph_replay_matches_eager():
    T, D, r, ng = 300, 1024, 32, 37
    X, W1, W2 = (t.to(DEV) for t in inputs(21, T, D, r, ng))
    mask = torch.empty((T, ng), dtype=torch.uint8, device=DEV)
    logits = torch.empty((T, ng, 2), dtype=torch.float32, device=DEV)
    wide.router_forward(X, W1, W2, "silu", mask=mask, logits=logits, return_logits=True)
    torch.cuda.synchronize()
    eager = mask.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            wide.router_forward(X, W1, W2, "silu", mask=mask, logits=logits, return_logits=True)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(4):
        mask.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(mask, eager), f"replay {i} differs from eager"


# ----------------------------------------------------------------------------- router fused with the reorder

# wide_router_reorder: the row lists equal the oracle's stable partition of the
# router's own mask, bit for bit (the decision is the kernel's, so the
# reference partition is taken of the GPU mask that the same call returns,
# and that mask is also checked against wide_router_forward's, bit for bit);
# T from 1 to the Llama prefill length, words split over 64-token blocks
# (odd word counts included), tiles of 1, 7 and 256.
@pytest.mark.parametrize("T,D,r,ng,tile", [
    (1, 256, 16, 5, 256), (16, 512, 32, 112, 256), (17, 256, 64, 3, 7), (100, 1024, 32, 37, 1),
    (1000, 4096, 32, 112, 256), (16384, 4096, 32, 112, 256), (4096, 5120, 32, 136, 256),
    (33, 96, 16, 1, 256), (2049, 3072, 16, 512, 128),
])
def test_router_reorder_equals_reorder_of_router_mask(T, D, r, ng, tile):
    X, W1, W2 = inputs(7 * T + ng, T, D, r, ng)
    Xd, W1d, W2d = X.to(DEV), W1.to(DEV), W2.to(DEV)
    call = wide.RouterReorderCall(Xd, W1d, W2d, "silu", tile, return_mask=True)
    call.workspace.fill_(0xA5)
    call.perm.fill_(-7)
    perm, counts, padded = call.run()
    mask_ref = wide.router_forward(Xd, W1d, W2d, "silu")
    torch.cuda.synchronize()
    m = call.mask.cpu().numpy()
    assert np.array_equal(m, mask_ref.cpu().numpy())
    rp, rc, rpad = oracle.reorder(m, tile)
    assert np.array_equal(perm.cpu().numpy(), rp)
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(padded.cpu().numpy(), rpad)
    # and the decisions are the router's (checked against the oracle's logits)
    if T <= 1000:
        check(X, W1, W2, "silu")


def test_router_reorder_without_mask_output_and_t0():
    T, D, r, ng = 300, 512, 32, 24
    X, W1, W2 = inputs(99, T, D, r, ng)
    Xd, W1d, W2d = X.to(DEV), W1.to(DEV), W2.to(DEV)
    perm, counts, padded = wide.router_reorder(Xd, W1d, W2d, "relu", 64)
    mask = wide.router_forward(Xd, W1d, W2d, "relu")
    p2, c2, pad2 = wide.reorder_masks(mask, 64)
    torch.cuda.synchronize()
    assert torch.equal(perm, p2) and torch.equal(counts, c2) and torch.equal(padded, pad2)
    # T == 0: counts and padded are zero
    X0 = torch.empty((0, D), dtype=torch.bfloat16, device=DEV)
    p0, c0, pad0 = wide.router_reorder(X0, W1d, W2d, "relu", 64)
    torch.cuda.synchronize()
    assert p0.numel() == 0 and bool((c0 == 0).all()) and bool((pad0 == 0).all())


def test_router_reorder_graph_replay_matches_eager():
    T, D, r, ng = 1000, 1024, 32, 56
    X, W1, W2 = inputs(5, T, D, r, ng)
    Xd, W1d, W2d = X.to(DEV), W1.to(DEV), W2.to(DEV)
    call = wide.RouterReorderCall(Xd, W1d, W2d, "silu", 256)
    eager = [t.clone() for t in call.run()]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call.run()
    torch.cuda.current_stream().wait_stream(s)
    for i in range(4):
        call.perm.fill_(-1)
        call.counts.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip((call.perm, call.counts, call.padded), eager)), i
