"""Decode with operand-order weights (wide_decode_prepare_weights and
wide_ffn_decode_prepared) on the GPU.

Bars:
  * the prepared copy is a pure permutation of the nn.Linear weights: every
    byte equals the one the documented block order names (bit-exact);
  * the prepared decode equals wide_ffn_forward's decode path bit for bit
    (Y and H): the kernels run the same MFMAs in the same order, only the
    weight addresses differ; and both meet the oracle's bf16 bar.
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


@pytest.fixture(autouse=True)
def announce(request):
    sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


def operand_order(W: torch.Tensor) -> torch.Tensor:
    """[R, C] -> blocks (R/16, C/32); lane 16 q + r of a block holds row 16 rb + r,
    columns 32 kc + 8 q .. + 7 (written out with views, independently of the kernel)."""
    R, C = W.shape
    return W.view(R // 16, 16, C // 32, 4, 8).permute(0, 2, 3, 1, 4).reshape(-1)


def test_prepared_layout_bit_exact():
    d, d_ff = 192, 320
    inp = dg.random_small(41, 1, d, d_ff, 64, "bf16")
    Wg, Wu, Wd = (inp[k].to(DEV) for k in ("Wg", "Wu", "Wd"))
    prep = wide.decode_prepare_weights(Wg, Wu, Wd)
    torch.cuda.synchronize()
    region = (d * d_ff * 2 + 255) // 256 * 256
    assert prep.numel() == wide.decode_weights_size(d, d_ff) == 3 * region
    p16 = prep.cpu()
    for r, W in enumerate((inp["Wg"], inp["Wu"], inp["Wd"])):
        got = p16[r * region: r * region + d * d_ff * 2].view(torch.bfloat16)
        want = operand_order(W)
        assert torch.equal(got.view(torch.int16), want.contiguous().view(torch.int16))


CASES = [
    # (T, d, d_ff, G, density): G = 128 / 32 / 16 units, T across the 8-channel,
    # 32-channel and whole-row thresholds, a d that the whole-row kernels do
    # not take (576: T = 1 and 2 run on the matrix cores too)
    (16, 512, 1024, 128, 0.5), (5, 512, 1024, 128, 0.5), (3, 512, 1024, 128, 0.5),
    (16, 512, 1024, 16, 0.5), (9, 512, 1024, 32, 0.4), (1, 576, 1024, 128, 0.5),
    (2, 576, 512, 16, 0.6), (1, 512, 1024, 128, 0.5), (16, 512, 1024, 128, 0.0),
    (16, 512, 1024, 128, 1.0), (5, 512, 1536, 48, 0.3), (1, 576, 1536, 48, 0.3),
]


@pytest.mark.parametrize("T,d,d_ff,G,density", CASES)
def test_prepared_decode_equals_forward(T, d, d_ff, G, density):
    inp = dg.random_small(500 + T + G, T, d, d_ff, G, "bf16", density, wscale=0.05)
    x = {k: v.to(DEV) for k, v in inp.items()}
    prep = wide.decode_prepare_weights(x["Wg"], x["Wu"], x["Wd"])
    Y0, H0 = wide.ffn_forward(x["X"], x["Wg"], x["Wu"], x["Wd"], x["mask"], G, return_h=True,
                              flags=wide.WIDE_FLAG_FORCE_DECODE)
    Y1, H1 = wide.ffn_decode_prepared(x["X"], x["Wg"], x["Wu"], x["Wd"], prep, x["mask"], G,
                                      return_h=True)
    torch.cuda.synchronize()
    assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))
    assert torch.equal(H0.view(torch.int16), H1.view(torch.int16))
    _, Yref = oracle.ffn(inp["X"], inp["Wg"], inp["Wu"], inp["Wd"], inp["mask"], G)
    den = np.max(np.abs(Yref))
    if den == 0:
        assert bool((Y1 == 0).all())
    else:
        err = np.max(np.abs(Y1.float().cpu().numpy() - Yref)) / den
        assert err <= 2e-2, err


def test_prepared_decode_llama8b_t16_equals_forward():
    w = dg.LLAMA8B_DECODE_T16
    inp = dg.make_inputs(w)
    x = {k: v.to(DEV) for k, v in inp.items()}
    prep = wide.decode_prepare_weights(x["Wg"], x["Wu"], x["Wd"])
    Y0 = wide.ffn_forward(x["X"], x["Wg"], x["Wu"], x["Wd"], x["mask"], w.G)
    Y1 = wide.ffn_decode_prepared(x["X"], x["Wg"], x["Wu"], x["Wd"], prep, x["mask"], w.G)
    torch.cuda.synchronize()
    assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))


def test_prepared_copy_follows_weight_changes():
    # the copy is a snapshot: preparing again after the weights change gives
    # the new results, and a stale copy gives the old ones
    T, d, d_ff, G = 8, 512, 512, 64
    inp = dg.random_small(77, T, d, d_ff, G, "bf16", 0.5, wscale=0.05)
    x = {k: v.to(DEV) for k, v in inp.items()}
    prep = wide.decode_prepare_weights(x["Wg"], x["Wu"], x["Wd"])
    Ya = wide.ffn_decode_prepared(x["X"], x["Wg"], x["Wu"], x["Wd"], prep, x["mask"], G).clone()
    x["Wd"].mul_(2)
    Ystale = wide.ffn_decode_prepared(x["X"], x["Wg"], x["Wu"], x["Wd"], prep, x["mask"], G).clone()
    wide.decode_prepare_weights(x["Wg"], x["Wu"], x["Wd"], out=prep)
    Yb = wide.ffn_decode_prepared(x["X"], x["Wg"], x["Wu"], x["Wd"], prep, x["mask"], G)
    torch.cuda.synchronize()
    assert torch.equal(Ya, Ystale)
    assert torch.allclose(Yb.float(), 2 * Ya.float(), rtol=1e-2, atol=1e-3)


def test_prepared_decode_graph_replay_matches_eager():
    # the prepared call allocates nothing and never synchronises, so it can be
    # captured; every replay (with eager work in between) equals the eager call
    T, d, d_ff, G = 12, 512, 1024, 128
    inp = dg.random_small(91, T, d, d_ff, G, "bf16", 0.5, wscale=0.05)
    x = {k: v.to(DEV) for k, v in inp.items()}
    prep = wide.decode_prepare_weights(x["Wg"], x["Wu"], x["Wd"])
    call = wide.FfnCall(x["X"], x["Wg"], x["Wu"], x["Wd"], x["mask"], G, prepared=prep)
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
    # the mask is read at replay time
    x["mask"].zero_()
    g.replay()
    torch.cuda.synchronize()
    assert bool((call.Y == 0).all())


# No H_out: the workspace (H included) holds NaN bits. With G = 16 or 48 a
# 32-channel chunk of the down GEMV can hold a group no token executes, whose
# H is never written; Y must equal the unprepared decode bit for bit and be
# finite.
@pytest.mark.parametrize("T,d,d_ff,G", [(5, 512, 1536, 48), (1, 576, 1536, 48), (16, 512, 1024, 16),
                                        (3, 512, 960, 80)])
def test_prepared_never_reads_unwritten_h(T, d, d_ff, G):
    inp = dg.random_small(900 + T + G, T, d, d_ff, G, "bf16", 0.3, wscale=0.05)
    x = {k: v.to(DEV) for k, v in inp.items()}
    prep = wide.decode_prepare_weights(x["Wg"], x["Wu"], x["Wd"])
    a = wide.FfnCall(x["X"], x["Wg"], x["Wu"], x["Wd"], x["mask"], G,
                     flags=wide.WIDE_FLAG_FORCE_DECODE)
    b = wide.FfnCall(x["X"], x["Wg"], x["Wu"], x["Wd"], x["mask"], G, prepared=prep)
    a.workspace.fill_(0xFF)
    b.workspace.fill_(0xFF)
    Ya = a.run().clone()
    Yb = b.run().clone()
    torch.cuda.synchronize()
    assert bool(torch.isfinite(Yb.float()).all())
    assert torch.equal(Ya.view(torch.int16), Yb.view(torch.int16))
    _, Yref = oracle.ffn(inp["X"], inp["Wg"], inp["Wu"], inp["Wd"], inp["mask"], G)
    err = np.max(np.abs(Yb.float().cpu().numpy() - Yref)) / max(np.max(np.abs(Yref)), 1e-30)
    assert err <= 2e-2
