"""HIP path vs the fp64 oracle on the GPU (run with -m gpu on an MI355X).

Bars (written here, applied element by element):
  * mask reorder: permutations, counts and padded counts bit-exact;
  * H: exact zeros at every masked channel;
  * Y: max|err| / max|ref| <= 2e-2 for bf16 inputs (fp32 accumulation),
       <= 1e-5 for fp32 inputs;
  * tokens with no active group, and the all-zero mask: Y exactly +0.0.
Small cases compare every output; the full-size workloads compare a seeded
sample of tokens (first, last, boundary-tile tokens and random ones) and check
the exact-zero and determinism properties on every output.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import group_sparse_ffn_amd as wide
from group_sparse_ffn_amd import datagen as dg

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-5}
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def announce(request):
    # Name the case on the real stderr before any GPU work, so a run that dies
    # still says which case it was in.
    sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


def to_dev(inp):
    return {k: v.to(DEV) for k, v in inp.items()}


def rel_err(y, ref):
    y = y.detach().float().cpu().numpy().astype(np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(y - ref)) / (den if den > 0 else 1.0))


def run_ffn(inp, G, **kw):
    d = to_dev(inp)
    Y, H = wide.ffn_forward(d["X"], d["Wg"], d["Wu"], d["Wd"], d["mask"], G, return_h=True, **kw)
    torch.cuda.synchronize()
    return Y, H


def check_h_zeros(H, mask, G):
    m = mask.to(DEV).bool().repeat_interleave(G, dim=1)
    masked = H[~m]
    assert masked.numel() == 0 or bool((masked == 0).all()), "nonzero H at a masked channel"


# ----------------------------------------------------------------------------- reorder

@pytest.mark.parametrize("T,ng,tile,kind", [
    (64, 16, 256, "bernoulli"), (1, 3, 256, "bernoulli"), (1000, 37, 256, "bernoulli"),
    (1025, 5, 7, "bernoulli"), (4096, 136, 256, "zipf"), (16384, 112, 256, "topk"),
    (300, 8, 1, "ones"), (300, 8, 64, "zeros"), (0, 4, 256, "zeros"),
])
def test_reorder_bit_exact(T, ng, tile, kind):
    if kind == "bernoulli":
        m = dg.mask_bernoulli(T, ng, 0.4, seed=T + ng)
    elif kind == "topk":
        m = dg.mask_topk(T, ng, ng // 2, seed=2004)
    elif kind == "zipf":
        m = dg.mask_zipf(T, ng, 0.5, seed=5004)
    elif kind == "ones":
        m = np.ones((T, ng), np.uint8)
    else:
        m = np.zeros((T, ng), np.uint8)
    perm, counts, padded = wide.reorder_masks(torch.from_numpy(m).to(DEV), tile)
    rp, rc, rpad = oracle.reorder(m, tile)
    assert np.array_equal(perm.cpu().numpy(), rp)
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(padded.cpu().numpy(), rpad)


def _round_up(x, a):
    return (x + a - 1) // a * a


# The FFN's own reorder stage (packed bits, then a per-group partition of each
# bit row) leaves perm / counts / padded at the front of the workspace:
# perm int32 [ng, T], then counts [ng] and padded [ng], each 256-byte aligned.
@pytest.mark.parametrize("T,ng,kind", [
    (64, 16, "bernoulli"), (1, 3, "bernoulli"), (1000, 37, "bernoulli"), (1025, 5, "bernoulli"),
    (16384, 112, "topk"), (300, 8, "ones"), (300, 8, "zeros"), (16385, 7, "zipf"),
    (65, 1, "bernoulli"), (40000, 2, "bernoulli"),
])
def test_ffn_reorder_stage_bit_exact(T, ng, kind):
    G, d = 64, 64
    d_ff = ng * G
    if kind == "bernoulli":
        m = dg.mask_bernoulli(T, ng, 0.4, seed=T + 7 * ng)
    elif kind == "topk":
        m = dg.mask_topk(T, ng, ng // 2, seed=2005)
    elif kind == "zipf":
        m = dg.mask_zipf(T, ng, 0.5, seed=5005)
    elif kind == "ones":
        m = np.ones((T, ng), np.uint8)
    else:
        m = np.zeros((T, ng), np.uint8)
    X = torch.zeros((T, d), dtype=torch.bfloat16, device=DEV)
    W = torch.zeros((d_ff, d), dtype=torch.bfloat16, device=DEV)
    Wd = torch.zeros((d, d_ff), dtype=torch.bfloat16, device=DEV)
    call = wide.FfnCall(X, W, W, Wd, torch.from_numpy(m).to(DEV), G,
                        flags=wide.WIDE_FLAG_FORCE_PREFILL)
    call.workspace.fill_(0xCD)
    wide.ffn_stage(wide.WIDE_STAGE_REORDER, call)
    torch.cuda.synchronize()
    ws = call.workspace
    o_counts = _round_up(ng * T * 4, 256)
    o_padded = o_counts + _round_up(ng * 4, 256)
    perm = ws[: ng * T * 4].view(torch.int32).reshape(ng, T).cpu().numpy()
    counts = ws[o_counts: o_counts + ng * 4].view(torch.int32).cpu().numpy()
    padded = ws[o_padded: o_padded + ng * 4].view(torch.int32).cpu().numpy()
    rp, rc, rpad = oracle.reorder(m, wide.WIDE_TOKEN_TILE)
    assert np.array_equal(perm, rp)
    assert np.array_equal(counts, rc) and np.array_equal(padded, rpad)


def test_reorder_nonzero_bytes_count_as_active():
    m = dg.mask_bernoulli(500, 6, 0.5, seed=1) * np.uint8(200)
    perm, counts, _ = wide.reorder_masks(torch.from_numpy(m).to(DEV), 256)
    rp, rc, _ = oracle.reorder(m, 256)
    assert np.array_equal(perm.cpu().numpy(), rp) and np.array_equal(counts.cpu().numpy(), rc)


# ----------------------------------------------------------------------------- small FFN, every output

SMALL = [
    # (T, d, d_ff, G, dtype, density, flags)
    (64, 256, 1024, 64, "f32", 0.5, 0),      # the tiny SwiGLU workload's shape
    (700, 512, 2048, 128, "bf16", 0.5, 0),    # 3 token tiles (ragged), 2 output tiles
    (700, 320, 1024, 64, "bf16", 0.3, 0),     # partial output tile (d % 256 != 0)
    (513, 256, 1024, 32, "bf16", 0.7, 0),
    (300, 192, 512, 16, "bf16", 0.5, 0),      # G = 16: several groups per K-block
    (257, 128, 512, 256, "bf16", 0.5, 0),     # G = 256: two channel tiles per group
    (40, 64, 128, 64, "bf16", 0.5, 0),        # minimal d
    (1, 256, 1024, 128, "bf16", 0.5, wide.WIDE_FLAG_FORCE_PREFILL),
    (16, 512, 1024, 128, "bf16", 0.5, wide.WIDE_FLAG_FORCE_PREFILL),
    (200, 256, 512, 64, "f32", 0.6, 0),
    (5, 128, 256, 16, "f32", 0.5, 0),
    (300, 256, 1536, 48, "bf16", 0.5, 0),     # G = 48: groups straddle the 64-channel K-blocks
    (40, 128, 960, 80, "f32", 0.5, 0),
]


@pytest.mark.parametrize("T,d,d_ff,G,dtype,density,flags", SMALL)
def test_ffn_small_all_outputs(T, d, d_ff, G, dtype, density, flags):
    inp = dg.random_small(7 * T + G, T, d, d_ff, G, dtype, density, wscale=0.05)
    Y, H = run_ffn(inp, G, flags=flags)
    Href, Yref = oracle.ffn(inp["X"], inp["Wg"], inp["Wu"], inp["Wd"], inp["mask"], G)
    assert rel_err(Y, Yref) <= TOL[dtype]
    check_h_zeros(H, inp["mask"], G)
    # H itself is also within the tolerance of the oracle's H
    assert rel_err(H, Href) <= TOL[dtype]


# T <= 4 runs 8-channel gate/up units, T > 4 16-channel units; G = 16 and 32 put
# several units in one group.
@pytest.mark.parametrize("T,G", [(1, 128), (3, 128), (16, 128), (5, 16), (16, 32), (2, 16),
                                 (4, 32), (1, 64), (8, 256)])
def test_decode_path_vs_oracle(T, G):
    d, d_ff = 512, 2048
    assert T <= wide.decode_max_t() or T <= wide.WIDE_DECODE_T_LIMIT
    inp = dg.random_small(100 + T, T, d, d_ff, G, "bf16", 0.5, wscale=0.05)
    Y, H = run_ffn(inp, G, flags=wide.WIDE_FLAG_FORCE_DECODE)
    _, Yref = oracle.ffn(inp["X"], inp["Wg"], inp["Wu"], inp["Wd"], inp["mask"], G)
    assert rel_err(Y, Yref) <= TOL["bf16"]
    check_h_zeros(H, inp["mask"], G)


# No H_out: the workspace (H included) starts as NaN bits. Groups no token
# executes are never written, and with G = 16 they share 32-channel chunks with
# executed groups, so Y is finite and right only if the down GEMV never reads
# them. T <= 2 with d % 512 == 0 takes the whole-row VALU kernels (also at the
# edges of their LDS capacity: d_ff 18432 at T = 1, 14336 at T = 2, and just
# past it), the rest the MFMA GEMVs.
@pytest.mark.parametrize("T,d,d_ff,G", [
    (1, 1024, 2048, 16), (2, 1024, 2048, 16), (1, 512, 2048, 32), (2, 2048, 2048, 512),
    (3, 1024, 2048, 16), (5, 1024, 2048, 16), (16, 512, 2048, 16), (1, 256, 2048, 16),
    (2, 8192, 1024, 64), (1, 512, 18432, 128), (2, 512, 14336, 128), (1, 512, 18496, 64),
    (2, 512, 14400, 64),
    # G = 48: a 32-channel chunk can hold an executed and a skipped group at any
    # offset, not only at its halves (matrix-core GEMVs at both T)
    (5, 512, 1536, 48), (1, 576, 1536, 48), (16, 512, 1536, 48), (3, 256, 960, 80),
    # past the reach of the gate/up with the activations in LDS, the
    # global-fragment kernel: T * d above the LDS capacity, d not a multiple of 128
    (16, 4224, 1024, 64), (8, 576, 1024, 64),
])
def test_decode_never_reads_unwritten_h(T, d, d_ff, G):
    inp = dg.random_small(500 + T + G, T, d, d_ff, G, "bf16", 0.3, wscale=0.05)
    dv = to_dev(inp)
    call = wide.FfnCall(dv["X"], dv["Wg"], dv["Wu"], dv["Wd"], dv["mask"], G,
                        flags=wide.WIDE_FLAG_FORCE_DECODE)
    call.workspace.fill_(0xFF)
    Y = call.run()
    torch.cuda.synchronize()
    _, Yref = oracle.ffn(inp["X"], inp["Wg"], inp["Wu"], inp["Wd"], inp["mask"], G)
    assert bool(torch.isfinite(Y.float()).all())
    assert rel_err(Y, Yref) <= TOL["bf16"]
    # and with H returned, H holds exact zeros at every masked channel
    Y2, H2 = run_ffn(inp, G, flags=wide.WIDE_FLAG_FORCE_DECODE)
    check_h_zeros(H2, inp["mask"], G)
    assert torch.equal(Y2.view(torch.int16), Y.view(torch.int16))


@pytest.mark.parametrize("T", [1, 4, 9])
def test_decode_edge_masks(T):
    """Decode path: empty groups, tokens with no group, one active group, all-zero mask."""
    d, d_ff, G = 256, 1024, 32
    ng = d_ff // G
    inp = dg.random_small(300 + T, T, d, d_ff, G, "bf16", 0.4, wscale=0.05)
    masks = []
    m = inp["mask"].clone()
    m[:, 2] = 0
    m[0, :] = 0          # token 0 executes nothing
    masks.append(m)
    one = torch.zeros((T, ng), dtype=torch.uint8)
    one[T - 1, ng - 1] = 1   # a single (token, group) pair in the last group
    masks.append(one)
    masks.append(torch.zeros((T, ng), dtype=torch.uint8))
    for m in masks:
        inp["mask"] = m
        Y, H = run_ffn(inp, G, flags=wide.WIDE_FLAG_FORCE_DECODE)
        _, Yref = oracle.ffn(inp["X"], inp["Wg"], inp["Wu"], inp["Wd"], m, G)
        check_h_zeros(H, m, G)
        idle = (m.sum(dim=1) == 0).nonzero().flatten().tolist()
        for t in idle:
            assert bool((Y[t] == 0).all()) and not bool(torch.signbit(Y[t].float()).any())
        if m.any():
            assert rel_err(Y, Yref) <= TOL["bf16"]
        else:
            assert bool((Y == 0).all())


@pytest.mark.parametrize("T,G,d_ff,flags", [
    (700, 128, 1024, 0), (300, 16, 1024, 0), (3, 128, 1024, 0), (12, 64, 1024, 0),
    (12, 64, 1024, wide.WIDE_FLAG_FORCE_PREFILL), (300, 48, 1536, 0), (7, 48, 1536, 0),
    (7, 48, 1536, wide.WIDE_FLAG_FORCE_PREFILL),
])
def test_result_does_not_depend_on_h_out(T, G, d_ff, flags):
    """Y with H kept in the workspace equals Y with H returned, bit for bit."""
    d = 256
    inp = to_dev(dg.random_small(400 + T, T, d, d_ff, G, "bf16", 0.5, wscale=0.05))
    a = wide.FfnCall(inp["X"], inp["Wg"], inp["Wu"], inp["Wd"], inp["mask"], G, flags=flags)
    b = wide.FfnCall(inp["X"], inp["Wg"], inp["Wu"], inp["Wd"], inp["mask"], G, return_h=True,
                     flags=flags)
    # workspace (H included) holds NaN bits and the outputs start as garbage
    a.workspace.fill_(0xFF)
    a.Y.fill_(3.0)
    b.H.fill_(-5.0)
    Ya = a.run().clone()
    Yb = b.run().clone()
    torch.cuda.synchronize()
    assert torch.equal(Ya, Yb)
    check_h_zeros(b.H, inp["mask"], G)


def test_decode_equals_prefill_within_tolerance_t16():
    T, d, d_ff, G = 16, 1024, 2048, 128
    inp = dg.random_small(77, T, d, d_ff, G, "bf16", 0.5, wscale=0.05)
    Yd, _ = run_ffn(inp, G, flags=wide.WIDE_FLAG_FORCE_DECODE)
    Yp, _ = run_ffn(inp, G, flags=wide.WIDE_FLAG_FORCE_PREFILL)
    ref = Yp.float().cpu().numpy().astype(np.float64)
    assert rel_err(Yd, ref) <= TOL["bf16"]


def test_edge_masks_small():
    T, d, d_ff, G = 300, 256, 1024, 64
    inp = dg.random_small(5, T, d, d_ff, G, "bf16", 0.5, wscale=0.05)
    ng = d_ff // G
    m = inp["mask"].clone()
    m[7, :] = 0                    # a token with no active group
    m[:, 3] = 0                    # a group no token executes
    m[:, 5] = 0
    m[123, 5] = 1                  # a group exactly one token executes
    inp["mask"] = m
    for flags in (0, wide.WIDE_FLAG_FORCE_PREFILL):
        Y, H = run_ffn(inp, G, flags=flags)
        _, Yref = oracle.ffn(inp["X"], inp["Wg"], inp["Wu"], inp["Wd"], m, G)
        assert rel_err(Y, Yref) <= TOL["bf16"]
        assert bool((Y[7] == 0).all()) and not bool(torch.signbit(Y[7].float()).any())
        check_h_zeros(H, m, G)
    # all-zero mask: Y and H exactly zero; all-ones: dense
    inp["mask"] = torch.zeros((T, ng), dtype=torch.uint8)
    Y, H = run_ffn(inp, G)
    assert bool((Y == 0).all()) and bool((H == 0).all())
    inp["mask"] = torch.ones((T, ng), dtype=torch.uint8)
    Y, _ = run_ffn(inp, G)
    _, Yref = oracle.ffn(inp["X"], inp["Wg"], inp["Wu"], inp["Wd"], inp["mask"], G)
    assert rel_err(Y, Yref) <= TOL["bf16"]


def test_t0_is_a_no_op():
    inp = dg.random_small(3, 0, 256, 512, 64, "bf16", 0.5)
    d = to_dev(inp)
    Y = wide.ffn_forward(d["X"], d["Wg"], d["Wu"], d["Wd"], d["mask"], 64)
    assert Y.shape == (0, 256)


def test_stages_equal_forward_and_are_deterministic():
    T, d, d_ff, G = 600, 512, 1024, 128
    inp = to_dev(dg.random_small(9, T, d, d_ff, G, "bf16", 0.5, wscale=0.05))
    call = wide.FfnCall(inp["X"], inp["Wg"], inp["Wu"], inp["Wd"], inp["mask"], G)
    Y1 = call.run().clone()
    Y2 = call.run().clone()
    call.Y.zero_()
    for s in (wide.WIDE_STAGE_REORDER, wide.WIDE_STAGE_GATE_UP, wide.WIDE_STAGE_DOWN):
        call.stage(s)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2), "two identical calls differ"
    assert torch.equal(Y1, call.Y), "stages differ from forward"


def test_hip_graph_replay_matches_eager():
    T, d, d_ff, G = 512, 512, 1024, 64
    inp = to_dev(dg.random_small(13, T, d, d_ff, G, "bf16", 0.5, wscale=0.05))
    call = wide.FfnCall(inp["X"], inp["Wg"], inp["Wu"], inp["Wd"], inp["mask"], G)
    eager = call.run().clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call.run()
    torch.cuda.current_stream().wait_stream(s)
    for i in range(4):
        call.Y.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(call.Y, eager), f"replay {i} differs from eager"
    # the mask is read on the device at replay time: a new mask changes the result
    inp["mask"].copy_(torch.zeros_like(inp["mask"]))
    g.replay()
    torch.cuda.synchronize()
    assert bool((call.Y == 0).all())


# ----------------------------------------------------------------------------- full-size workloads

def sample_rows(T, must, n_random, seed, min_rows=0):
    """Token rows to compare: 0, T/2, T-1, the `must` rows, and random ones
    (at least n_random, and enough for min_rows rows in all)."""
    rng = np.random.default_rng(seed)
    rows = {0, T - 1, T // 2}
    rows.update(int(r) for r in must)
    rows = {r for r in rows if 0 <= r < T}
    rest = np.setdiff1d(np.arange(T), np.fromiter(rows, dtype=np.int64, count=len(rows)))
    n = min(len(rest), max(n_random, min_rows - len(rows)))
    rows.update(int(r) for r in rng.choice(rest, size=n, replace=False))
    return np.array(sorted(rows), dtype=np.int64)


def full_size_check(w, n_random, mask_kind=None, min_rows=0):
    """One workload at its full size, in the launch configuration the bench times.

    * Y at a seeded sample of tokens against the oracle (one token from the
      boundary tile of EVERY group, i.e. its last active token, plus the first,
      middle and last tokens and random ones);
    * H exactly zero at every masked channel (whole H);
    * the call without H_out, with the workspace (where H then lives) holding
      NaN bits, gives the same Y bit for bit (whole Y): the bench times that
      call, in which skipped (token, group) pairs of H are never written;
    * a second identical call gives the same Y bit for bit.
    """
    inp = dg.make_inputs(w, mask_kind=mask_kind)
    m = inp["mask"].numpy()
    d = to_dev(inp)
    call = wide.FfnCall(d["X"], d["Wg"], d["Wu"], d["Wd"], d["mask"], w.G, return_h=True)
    Y = call.run()
    bare = wide.FfnCall(d["X"], d["Wg"], d["Wu"], d["Wd"], d["mask"], w.G)
    bare.workspace.fill_(0xFF)
    Yb = bare.run()
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Yb.view(torch.int16)), \
        f"{w.name}: Y without H_out differs from Y with H_out"
    del bare
    perm, counts, _ = oracle.reorder(m, wide.WIDE_TOKEN_TILE)
    bnd = [perm[g, c - 1] for g, c in enumerate(counts) if c > 0]
    rows = sample_rows(w.T, bnd, n_random, seed=w.seed, min_rows=min_rows)
    assert set(bnd) <= set(rows.tolist())
    Hs, Ys = oracle.ffn(inp["X"], inp["Wg"], inp["Wu"], inp["Wd"], m, w.G, rows=rows)
    err = rel_err(Y[torch.from_numpy(rows).to(DEV)], Ys)
    sys.__stderr__.write(f"[gpu-case] {w.name}: {len(rows)} rows, rel err {err:.3e}\n")
    assert err <= TOL[w.dtype], f"{w.name}: rel err {err}"
    check_h_zeros(call.H, inp["mask"], w.G)
    Y2 = call.run().clone()
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2), "not deterministic at full size"
    return Y


def test_llama8b_prefill_full_size_sampled():
    full_size_check(dg.LLAMA8B_PREFILL, n_random=48, min_rows=256)


@pytest.mark.parametrize("w", [dg.LLAMA8B_DECODE_T1, dg.LLAMA8B_DECODE_T16], ids=lambda w: w.name)
def test_llama8b_decode_full_size(w):
    full_size_check(w, n_random=16)


def test_qwen14b_skewed_full_size_sampled():
    full_size_check(dg.QWEN14B_SKEW, n_random=24, min_rows=256)


def test_qwen14b_all_zero_and_all_ones():
    w = dg.QWEN14B_SKEW
    Y = full_size_check(w, n_random=4, mask_kind="ones")
    # all-ones equals the dense FFN: also compare with torch's dense GEMMs (fp32 on the GPU)
    inp = dg.make_inputs(w, mask_kind="ones")
    X = inp["X"].to(DEV).float()
    rows = torch.arange(0, w.T, 97, device=DEV)
    a = X[rows] @ inp["Wg"].to(DEV).float().t()
    b = X[rows] @ inp["Wu"].to(DEV).float().t()
    ref = ((a * torch.sigmoid(a)) * b) @ inp["Wd"].to(DEV).float().t()
    err = (Y[rows].float() - ref).abs().max() / ref.abs().max()
    assert float(err) <= TOL["bf16"]
    inp = dg.make_inputs(w, mask_kind="zeros")
    d = to_dev(inp)
    Yz, Hz = wide.ffn_forward(d["X"], d["Wg"], d["Wu"], d["Wd"], d["mask"], w.G, return_h=True)
    torch.cuda.synchronize()
    assert bool((Yz == 0).all()) and bool((Hz == 0).all())


# Llama3.2-3B-shaped sweep cells: every G of the sweep and every sparsity level
# at a prefill length (T = 2048 or 8192), and T = 1 at three G.
SWEEP_CELLS = [
    (16, 10, 2048), (32, 25, 8192), (64, 50, 2048), (128, 70, 8192), (256, 10, 8192),
    (512, 70, 2048), (128, 50, 8192), (16, 70, 8192), (512, 25, 8192), (256, 50, 2048),
    (64, 50, 1), (256, 25, 1), (16, 10, 1),
]


def _sweep_cell(G, s, T):
    for c in dg.llama3b_sweep_cells():
        if c.G == G and round((1 - c.density) * 100) == s and c.T == T:
            return c
    raise KeyError((G, s, T))


@pytest.mark.parametrize("G,s,T", SWEEP_CELLS, ids=lambda v: str(v))
def test_llama3b_sweep_cell_sampled(G, s, T):
    full_size_check(_sweep_cell(G, s, T), n_random=16)


def test_sweep_cells_cover_every_g_and_sparsity():
    pre = [(G, s) for G, s, T in SWEEP_CELLS if T > 1]
    assert {G for G, _ in pre} == {16, 32, 64, 128, 256, 512}
    assert {s for _, s in pre} == {10, 25, 50, 70}
    assert len({G for G, _, T in SWEEP_CELLS if T == 1}) >= 2


# ----------------------------------------------------------------------------- down projection

# The gate/up with 128-channel blocks and 256-position tiles over 1024-1280
# tiles (four to five rounds of the chip, so every XCD's share holds full,
# boundary and past-count tiles): ragged T, K of one to four 64-wide stages, a
# group no token executes and one every token executes; Y and H against the
# oracle, with and without H returned (past-count tiles are cleared only when
# it is), and two calls bit-identical.
@pytest.mark.parametrize("T,d,d_ff,G,density", [
    (2048, 256, 16384, 128, 0.5), (2000, 192, 16384, 128, 0.5), (1100, 64, 32768, 256, 0.6),
    (2500, 128, 16384, 128, 0.2),
])
def test_gate_up_many_tiles(T, d, d_ff, G, density):
    inp = dg.random_small(53 * T + G, T, d, d_ff, G, "bf16", density, wscale=0.05)
    m = inp["mask"].clone()
    m[:, 3] = 0
    m[:, 5] = 1
    inp["mask"] = m
    Y, H = run_ffn(inp, G)
    Href, Yref = oracle.ffn(inp["X"], inp["Wg"], inp["Wu"], inp["Wd"], m, G)
    assert rel_err(Y, Yref) <= TOL["bf16"]
    assert rel_err(H, Href) <= TOL["bf16"]
    check_h_zeros(H, m, G)
    x = to_dev(inp)
    a = wide.FfnCall(x["X"], x["Wg"], x["Wu"], x["Wd"], x["mask"], G)
    a.workspace.fill_(0xFF)
    Ya = a.run().clone()
    Ya2 = a.run().clone()
    torch.cuda.synchronize()
    assert torch.equal(Ya.view(torch.int16), Ya2.view(torch.int16)), "not deterministic"
    assert torch.equal(Ya.view(torch.int16), Y.view(torch.int16)), "H returned or not differ"


# The down kernel on ragged shapes: T not a multiple of the 256-token tile, d
# not a multiple of the 256-column tile, G from 64 to 512 (one to eight
# 64-channel K-blocks per group), densities from nearly empty to full, a
# 128-token run that executes no group and a token that executes every group;
# workspace (where H lives) filled with NaN bits, two calls bit-identical.
@pytest.mark.parametrize("T,d,d_ff,G,density", [
    (700, 512, 2048, 128, 0.5), (1000, 320, 1536, 64, 0.3), (129, 256, 1024, 256, 0.7),
    (300, 576, 3072, 192, 0.5), (257, 256, 4096, 512, 0.5), (128, 256, 1024, 64, 1.0),
    (333, 256, 1024, 64, 0.05), (4096, 512, 2048, 128, 0.5), (300, 256, 257 * 64, 64, 0.5),
    # partial 256 x 256 tiles in both dimensions
    (2000, 4032, 1024, 128, 0.5),
])
def test_down_ragged_tiles_and_idle_runs(T, d, d_ff, G, density):
    inp = dg.random_small(31 * T + G, T, d, d_ff, G, "bf16", density, wscale=0.05)
    m = inp["mask"].clone()
    if T >= 400:
        m[128:256, :] = 0   # a run of 128 tokens with no live group
        m[300, :] = 1       # a token executing every group
    inp["mask"] = m
    x = to_dev(inp)
    a = wide.FfnCall(x["X"], x["Wg"], x["Wu"], x["Wd"], x["mask"], G)
    a.workspace.fill_(0xFF)
    Ya = a.run().clone()
    Ya2 = a.run().clone()
    torch.cuda.synchronize()
    assert torch.equal(Ya.view(torch.int16), Ya2.view(torch.int16)), "not deterministic"
    _, Yref = oracle.ffn(inp["X"], inp["Wg"], inp["Wu"], inp["Wd"], m, G)
    assert rel_err(Ya, Yref) <= TOL["bf16"]
    idle = (m.sum(dim=1) == 0).nonzero().flatten().tolist()
    for t in idle[:64]:
        assert bool((Ya[t] == 0).all()) and not bool(torch.signbit(Ya[t].float()).any())
