"""wide_ffn_forward_noalloc on the GPU, called through the raw C ABI (ctypes).

Bar: Y and H bit-identical to wide_ffn_forward with a caller workspace (the
same kernels run on the same data; only the workspace address differs), on
two calls in a row whose second is smaller than the first, for the prefill
and the decode path; and the results meet the oracle's bf16 bar. The
scratch array keeps the first call's contents when the second runs, so the
second call also shows that nothing in it needs to start cleared.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import group_sparse_ffn_amd as wide
from group_sparse_ffn_amd import _lib
from group_sparse_ffn_amd import datagen as dg

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def announce(request):
    sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


def noalloc_raw(x, G, flags=0):
    """The C entry point with torch-allocated outputs; returns (status, Y, H)."""
    T, d = x["X"].shape
    d_ff = x["Wg"].shape[0]
    Y = torch.full((T, d), 7.0, dtype=x["X"].dtype, device=DEV)
    H = torch.full((T, d_ff), -3.0, dtype=x["X"].dtype, device=DEV)
    lib = _lib.load()
    st = lib.wide_ffn_forward_noalloc(
        x["X"].data_ptr(), x["Wg"].data_ptr(), x["Wu"].data_ptr(), x["Wd"].data_ptr(),
        x["mask"].data_ptr(), T, d, d_ff, G, _lib.WIDE_BF16 if x["X"].dtype == torch.bfloat16
        else _lib.WIDE_F32, Y.data_ptr(), H.data_ptr(), flags,
        torch.cuda.current_stream().cuda_stream)
    return st, Y, H


def with_workspace(x, G, flags=0):
    call = wide.FfnCall(x["X"], x["Wg"], x["Wu"], x["Wd"], x["mask"], G, return_h=True,
                        flags=flags)
    call.workspace.fill_(0xFF)
    Y = call.run()
    return Y, call.H


def same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.mark.parametrize("sizes,G,dtype", [
    # prefill, then a smaller prefill
    ([(700, 512, 2048), (300, 512, 2048)], 128, "bf16"),
    ([(513, 256, 1536), (65, 256, 1536)], 48, "bf16"),
    # decode T = 16, then T = 3 (matrix-core GEMVs), then T = 1 (whole-row kernels)
    ([(16, 512, 1024), (3, 512, 1024), (1, 512, 1024)], 64, "bf16"),
    # fp32 prefill, then a smaller one
    ([(64, 256, 1024), (20, 256, 1024)], 64, "f32"),
])
def test_noalloc_equals_forward_two_calls(sizes, G, dtype):
    for i, (T, d, d_ff) in enumerate(sizes):
        inp = dg.random_small(800 + 17 * i + T, T, d, d_ff, G, dtype, 0.5, wscale=0.05)
        x = {k: v.to(DEV) for k, v in inp.items()}
        st, Y, H = noalloc_raw(x, G)
        Yw, Hw = with_workspace(x, G)
        torch.cuda.synchronize()
        assert st == _lib.WIDE_OK, _lib.load().wide_last_error().decode()
        assert same_bits(Y, Yw), f"call {i}: Y differs from wide_ffn_forward"
        assert same_bits(H, Hw), f"call {i}: H differs from wide_ffn_forward"
        _, Yref = oracle.ffn(inp["X"], inp["Wg"], inp["Wu"], inp["Wd"], inp["mask"], G)
        err = np.max(np.abs(Y.float().cpu().numpy() - Yref)) / max(np.max(np.abs(Yref)), 1e-30)
        assert err <= (2e-2 if dtype == "bf16" else 1e-5), f"call {i}: rel err {err}"


def test_noalloc_llama8b_prefill_then_decode():
    # the largest workload of the bench fits the array: T = 16384, 112 groups
    w = dg.LLAMA8B_PREFILL
    need = _lib.load().wide_ffn_workspace_size_for(w.T, w.d, w.d_ff, w.G, _lib.WIDE_BF16, 1)
    assert need <= _lib.WIDE_NOALLOC_SCRATCH_BYTES
    for T in (w.T, 16):
        inp = dg.make_inputs(w, T=T)
        x = {k: v.to(DEV) for k, v in inp.items()}
        st, Y, H = noalloc_raw(x, w.G)
        Yw, Hw = with_workspace(x, w.G)
        torch.cuda.synchronize()
        assert st == _lib.WIDE_OK, _lib.load().wide_last_error().decode()
        assert same_bits(Y, Yw) and same_bits(H, Hw)
        del x, Y, H, Yw, Hw
    torch.cuda.empty_cache()


def test_noalloc_rejects_without_enqueueing():
    lib = _lib.load()
    x = {k: v.to(DEV) for k, v in dg.random_small(5, 64, 256, 1024, 64, "bf16").items()}
    Y = torch.zeros((64, 256), dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    # H_out missing
    st = lib.wide_ffn_forward_noalloc(x["X"].data_ptr(), x["Wg"].data_ptr(), x["Wu"].data_ptr(),
                                      x["Wd"].data_ptr(), x["mask"].data_ptr(), 64, 256, 1024, 64,
                                      _lib.WIDE_BF16, Y.data_ptr(), None, 0, s)
    assert st == _lib.WIDE_ERR_NULL
    torch.cuda.synchronize()
    assert bool((Y == 0).all())


def test_noalloc_qwen14b_split_down():
    # the down projection's last round is split (320 tiles: 64 remainder tiles
    # x 4 parts), so its partial sums live in the static array too
    w = dg.QWEN14B_SKEW
    need = _lib.load().wide_ffn_workspace_size_for(w.T, w.d, w.d_ff, w.G, _lib.WIDE_BF16, 1)
    assert need <= _lib.WIDE_NOALLOC_SCRATCH_BYTES
    inp = dg.make_inputs(w)
    x = {k: v.to(DEV) for k, v in inp.items()}
    st, Y, H = noalloc_raw(x, w.G)
    Yw, Hw = with_workspace(x, w.G)
    torch.cuda.synchronize()
    assert st == _lib.WIDE_OK, _lib.load().wide_last_error().decode()
    assert same_bits(Y, Yw), "Y differs from wide_ffn_forward"
    assert same_bits(H, Hw), "H differs from wide_ffn_forward"
