"""C-ABI checks that need no GPU: the library loads, exports exactly what
include/wide.h declares, and rejects bad arguments on the host before any
HIP call (so these calls are safe without a device)."""
import ctypes
import os
import re
import subprocess

import pytest

from group_sparse_ffn_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wide.h")
FAKE = 1 << 20  # a 256-byte aligned non-NULL address that is never dereferenced


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return set(re.findall(r"\b(wide_[a-z_]+)\s*\(", src))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from group_sparse_ffn_amd import build
        build.build()
    return _lib.load()


def test_exports_match_header(lib):
    declared = declared_functions()
    assert declared == set(_lib.SIGNATURES), "binding and header disagree"
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert declared <= exported
    assert {s for s in exported if s.startswith("wide_")} == declared
    for name in declared:
        assert getattr(lib, name) is not None


def ffn_call(lib, **kw):
    a = dict(X=FAKE, Wg=FAKE, Wu=FAKE, Wd=FAKE, mask=FAKE, T=64, d=256, d_ff=1024, G=64,
             dtype=_lib.WIDE_BF16, Y=FAKE, H=None, ws=FAKE, ws_bytes=1 << 40, flags=0, stream=None)
    a.update(kw)
    return lib.wide_ffn_forward(a["X"], a["Wg"], a["Wu"], a["Wd"], a["mask"], a["T"], a["d"],
                                a["d_ff"], a["G"], a["dtype"], a["Y"], a["H"], a["ws"],
                                a["ws_bytes"], a["flags"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), _lib.WIDE_ERR_NULL),
    (dict(Wd=None, T=0), _lib.WIDE_ERR_NULL),
    (dict(mask=None), _lib.WIDE_ERR_NULL),
    (dict(Y=None), _lib.WIDE_ERR_NULL),
    (dict(dtype=7), _lib.WIDE_ERR_DTYPE),
    (dict(T=-1), _lib.WIDE_ERR_SHAPE),
    (dict(d=0), _lib.WIDE_ERR_SHAPE),
    (dict(G=0), _lib.WIDE_ERR_SHAPE),
    (dict(d_ff=1000, G=64), _lib.WIDE_ERR_SHAPE),
    (dict(d=96), _lib.WIDE_ERR_UNSUPPORTED),
    (dict(d_ff=1040, G=40), _lib.WIDE_ERR_UNSUPPORTED),
    (dict(d_ff=1024, G=8), _lib.WIDE_ERR_UNSUPPORTED),
    (dict(d_ff=131072, G=128), _lib.WIDE_ERR_UNSUPPORTED),
    (dict(T=1 << 20, d_ff=4096, G=128), _lib.WIDE_ERR_UNSUPPORTED),
    (dict(X=FAKE + 8), _lib.WIDE_ERR_ALIGN),
    (dict(H=FAKE + 4), _lib.WIDE_ERR_ALIGN),
    (dict(ws=FAKE + 16), _lib.WIDE_ERR_ALIGN),
    (dict(ws=None), _lib.WIDE_ERR_WORKSPACE),
    (dict(ws_bytes=1024), _lib.WIDE_ERR_WORKSPACE),
    (dict(flags=3), _lib.WIDE_ERR_SHAPE),
    (dict(flags=8), _lib.WIDE_ERR_SHAPE),
    (dict(flags=_lib.WIDE_FLAG_FORCE_DECODE, T=17), _lib.WIDE_ERR_UNSUPPORTED),
    (dict(flags=_lib.WIDE_FLAG_FORCE_DECODE, dtype=_lib.WIDE_F32, T=4), _lib.WIDE_ERR_UNSUPPORTED),
])
def test_forward_validation(lib, kw, status):
    assert ffn_call(lib, **kw) == status
    assert lib.wide_last_error().decode() != ""
    assert lib.wide_status_string(status).decode() not in ("", "unknown status")


def test_forward_t0_is_a_no_op(lib):
    # valid arguments with T == 0 enqueue nothing and succeed
    assert ffn_call(lib, T=0) == _lib.WIDE_OK
    assert ffn_call(lib, T=0, X=None, mask=None, Y=None) == _lib.WIDE_OK
    assert lib.wide_last_error().decode() == ""


def test_stage_rejects_the_other_path(lib):
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 64, 256, 1024, 64, _lib.WIDE_BF16, FAKE, None, FAKE,
            1 << 40, 0, None]
    # T = 64 > decode limit -> prefill; a decode stage must be refused
    assert lib.wide_ffn_stage(_lib.WIDE_STAGE_DECODE_DOWN, *args) == _lib.WIDE_ERR_UNSUPPORTED
    args[5] = 4  # T = 4 -> decode; a prefill stage must be refused
    assert lib.wide_ffn_stage(_lib.WIDE_STAGE_GATE_UP, *args) == _lib.WIDE_ERR_UNSUPPORTED
    assert lib.wide_ffn_stage(9, *args) == _lib.WIDE_ERR_SHAPE


@pytest.mark.parametrize("args,status", [
    ((None, 8, 2, 4, FAKE, FAKE, FAKE, None), _lib.WIDE_ERR_NULL),
    ((FAKE, 0, 2, 4, FAKE, None, FAKE, None), _lib.WIDE_ERR_NULL),
    ((FAKE, 8, 2, 4, None, FAKE, FAKE, None), _lib.WIDE_ERR_NULL),
    ((FAKE, -1, 2, 4, FAKE, FAKE, FAKE, None), _lib.WIDE_ERR_SHAPE),
    ((FAKE, 8, 0, 4, FAKE, FAKE, FAKE, None), _lib.WIDE_ERR_SHAPE),
    ((FAKE, 8, 2, 0, FAKE, FAKE, FAKE, None), _lib.WIDE_ERR_SHAPE),
    ((FAKE, 1 << 30, 8, 4, FAKE, FAKE, FAKE, None), _lib.WIDE_ERR_SHAPE),
])
def test_reorder_validation(lib, args, status):
    assert lib.wide_reorder_masks(*args) == status


def test_workspace_size(lib):
    ws = lib.wide_ffn_workspace_size(16384, 4096, 14336, 128, _lib.WIDE_BF16)
    ng, T = 112, 16384
    need = ng * T * 4 + 2 * ng * 4 + ng * (T // 32) * 4 + T * 14336 * 2
    assert need <= ws <= need + 5 * 256
    assert lib.wide_ffn_workspace_size(16, 4096, 14336, 100, _lib.WIDE_BF16) == 0
    assert lib.wide_ffn_workspace_size(16, 4096, 14336, 128, 5) == 0
    # with H_out given the workspace holds no H
    assert lib.wide_ffn_workspace_size_for(16384, 4096, 14336, 128, _lib.WIDE_BF16, 0) == ws
    small = lib.wide_ffn_workspace_size_for(16384, 4096, 14336, 128, _lib.WIDE_BF16, 1)
    assert need - T * 14336 * 2 <= small <= need - T * 14336 * 2 + 5 * 256
    # decode sizes hold the split partial sums either way
    dec = lib.wide_ffn_workspace_size_for(16, 4096, 14336, 128, _lib.WIDE_BF16, 1)
    assert dec >= 4 * 16 * 4096 * 4
    assert lib.wide_ffn_workspace_size_for(16, 4096, 14336, 128, _lib.WIDE_BF16, 0) >= \
        dec + 16 * 14336 * 2


def test_workspace_check_follows_h_out(lib):
    # a workspace sized for a call with H_out is accepted with H_out and
    # refused without it (T = 0 would skip the check, so T stays positive;
    # the check runs before anything is enqueued)
    small = lib.wide_ffn_workspace_size_for(64, 256, 1024, 64, _lib.WIDE_BF16, 1)
    full = lib.wide_ffn_workspace_size_for(64, 256, 1024, 64, _lib.WIDE_BF16, 0)
    assert full == small + 64 * 1024 * 2
    assert ffn_call(lib, ws_bytes=small, d=96) == _lib.WIDE_ERR_UNSUPPORTED  # checks run in order
    assert ffn_call(lib, ws_bytes=small) == _lib.WIDE_ERR_WORKSPACE
    assert "needs %d" % full in lib.wide_last_error().decode()
    assert ffn_call(lib, ws_bytes=small - 1, H=FAKE) == _lib.WIDE_ERR_WORKSPACE
    assert "needs %d" % small in lib.wide_last_error().decode()


def test_decode_threshold_default(lib):
    assert 0 <= lib.wide_decode_max_t() <= _lib.WIDE_DECODE_T_LIMIT


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        _lib.load()


def gemm_call(lib, fn, **kw):
    a = dict(A=FAKE, B=FAKE, mask=FAKE, M=300, N=512, K=256, G=64, dtype=_lib.WIDE_BF16, C=FAKE,
             ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return getattr(lib, fn)(a["A"], a["B"], a["mask"], a["M"], a["N"], a["K"], a["G"], a["dtype"],
                            a["C"], a["ws"], a["ws_bytes"], a["stream"])


GEMM_BAD = [
    (dict(A=None), _lib.WIDE_ERR_NULL),
    (dict(B=None, M=0), _lib.WIDE_ERR_NULL),
    (dict(mask=None), _lib.WIDE_ERR_NULL),
    (dict(C=None), _lib.WIDE_ERR_NULL),
    (dict(dtype=9), _lib.WIDE_ERR_DTYPE),
    (dict(dtype=_lib.WIDE_F32), _lib.WIDE_ERR_UNSUPPORTED),
    (dict(M=-1), _lib.WIDE_ERR_SHAPE),
    (dict(N=0), _lib.WIDE_ERR_SHAPE),
    (dict(K=0), _lib.WIDE_ERR_SHAPE),
    (dict(G=0), _lib.WIDE_ERR_SHAPE),
    (dict(K=96, N=96, G=32), _lib.WIDE_ERR_UNSUPPORTED),        # K % 64
    (dict(N=520, K=520, G=40), _lib.WIDE_ERR_UNSUPPORTED),      # K % 64 and G % 16
    (dict(N=1 << 17, K=1 << 17, G=1 << 10), _lib.WIDE_ERR_UNSUPPORTED),  # K > 65536
    (dict(M=1 << 20, N=2048, K=2048, G=128), _lib.WIDE_ERR_UNSUPPORTED),  # M*K >= 2^30
    (dict(A=FAKE + 8), _lib.WIDE_ERR_ALIGN),
    (dict(C=FAKE + 2), _lib.WIDE_ERR_ALIGN),
    (dict(ws=FAKE + 64), _lib.WIDE_ERR_ALIGN),
    (dict(ws=None), _lib.WIDE_ERR_WORKSPACE),
    (dict(ws_bytes=256), _lib.WIDE_ERR_WORKSPACE),
]


@pytest.mark.parametrize("kw,status", GEMM_BAD + [(dict(N=500, G=64), _lib.WIDE_ERR_SHAPE)])
def test_gemm_mn_validation(lib, kw, status):
    assert gemm_call(lib, "wide_gemm_mn", **kw) == status
    assert lib.wide_last_error().decode() != ""


@pytest.mark.parametrize("kw,status", GEMM_BAD + [
    (dict(K=320, G=128), _lib.WIDE_ERR_SHAPE),                  # G does not divide K
    (dict(N=500), _lib.WIDE_ERR_UNSUPPORTED),                   # N % 8
])
def test_gemm_k_validation(lib, kw, status):
    assert gemm_call(lib, "wide_gemm_k", **kw) == status
    assert lib.wide_last_error().decode() != ""


def test_gemm_m0_is_a_no_op(lib):
    for fn in ("wide_gemm_mn", "wide_gemm_k"):
        assert gemm_call(lib, fn, M=0, A=None, mask=None, C=None) == _lib.WIDE_OK
        assert lib.wide_last_error().decode() == ""


def test_gemm_workspace_size(lib):
    M, ng = 16384, 8
    ws = lib.wide_gemm_workspace_size(M, ng)
    need = ng * M * 4 + 2 * ng * 4 + ng * (M // 32) * 4
    assert need <= ws <= need + 4 * 256
    assert lib.wide_gemm_workspace_size(-1, 8) == 0
    assert lib.wide_gemm_workspace_size(16, 0) == 0


def router_call(lib, **kw):
    a = dict(X=FAKE, W1=FAKE, W2=FAKE, T=64, D=256, r=32, ng=8, act=_lib.WIDE_ACT_SILU,
             dtype=_lib.WIDE_BF16, mask=FAKE, logits=None, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.wide_router_forward(a["X"], a["W1"], a["W2"], a["T"], a["D"], a["r"], a["ng"],
                                   a["act"], a["dtype"], a["mask"], a["logits"], a["ws"],
                                   a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(W1=None), _lib.WIDE_ERR_NULL),
    (dict(X=None), _lib.WIDE_ERR_NULL),
    (dict(mask=None), _lib.WIDE_ERR_NULL),
    (dict(dtype=4), _lib.WIDE_ERR_DTYPE),
    (dict(dtype=_lib.WIDE_F32), _lib.WIDE_ERR_UNSUPPORTED),
    (dict(T=-1), _lib.WIDE_ERR_SHAPE),
    (dict(D=0), _lib.WIDE_ERR_SHAPE),
    (dict(ng=0), _lib.WIDE_ERR_SHAPE),
    (dict(act=7), _lib.WIDE_ERR_SHAPE),
    (dict(D=48), _lib.WIDE_ERR_UNSUPPORTED),
    (dict(r=24), _lib.WIDE_ERR_UNSUPPORTED),
    (dict(T=1 << 24, D=256), _lib.WIDE_ERR_UNSUPPORTED),
    (dict(X=FAKE + 8), _lib.WIDE_ERR_ALIGN),
    (dict(W2=FAKE + 2), _lib.WIDE_ERR_ALIGN),
    (dict(logits=FAKE + 4), _lib.WIDE_ERR_ALIGN),
])
def test_router_validation(lib, kw, status):
    assert router_call(lib, **kw) == status
    assert lib.wide_last_error().decode() != ""


def test_router_t0_is_a_no_op(lib):
    assert router_call(lib, T=0, X=None, mask=None) == _lib.WIDE_OK


def test_router_workspace(lib):
    # partial sums of the split first map: 8 slices x 16 token rows x r floats, for 1 <= T <= 16
    for r in (16, 32, 64):
        for T in (1, 7, 16):
            assert lib.wide_router_workspace_size(T, r) == 8 * 16 * r * 4
        for T in (0, 17, 16384, -1):
            assert lib.wide_router_workspace_size(T, r) == 0
    assert lib.wide_router_workspace_size(4, 24) == 0
    need = 8 * 16 * 32 * 4
    assert router_call(lib, T=16, ws=None) == _lib.WIDE_ERR_WORKSPACE
    assert router_call(lib, T=1, ws=FAKE, ws_bytes=need - 1) == _lib.WIDE_ERR_WORKSPACE
    assert router_call(lib, T=1, ws=FAKE + 16, ws_bytes=need) == _lib.WIDE_ERR_ALIGN
    # T > 16 needs none (validation of such a call is covered above)
    assert lib.wide_router_workspace_size(17, 32) == 0


def attn_call(lib, fn, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, mask=FAKE, T=300, Hq=32, Hk=8, dh=128, dtype=_lib.WIDE_BF16,
             O=FAKE, flags=0, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return getattr(lib, fn)(a["Q"], a["K"], a["V"], a["mask"], a["T"], a["Hq"], a["Hk"], a["dh"],
                            a["dtype"], a["O"], a["flags"], a["ws"], a["ws_bytes"], a["stream"])


ATTN_BAD = [
    (dict(Q=None), _lib.WIDE_ERR_NULL),
    (dict(mask=None), _lib.WIDE_ERR_NULL),
    (dict(O=None), _lib.WIDE_ERR_NULL),
    (dict(dtype=9), _lib.WIDE_ERR_DTYPE),
    (dict(dtype=_lib.WIDE_F32), _lib.WIDE_ERR_UNSUPPORTED),
    (dict(Hk=0), _lib.WIDE_ERR_SHAPE),
    (dict(Hq=12, Hk=8), _lib.WIDE_ERR_SHAPE),                 # Hk does not divide Hq
    (dict(flags=4), _lib.WIDE_ERR_SHAPE),
    (dict(dh=64), _lib.WIDE_ERR_UNSUPPORTED),
    (dict(Q=FAKE + 8), _lib.WIDE_ERR_ALIGN),
    (dict(O=FAKE + 2), _lib.WIDE_ERR_ALIGN),
    (dict(ws=FAKE + 64), _lib.WIDE_ERR_ALIGN),
    (dict(ws=None), _lib.WIDE_ERR_WORKSPACE),
    (dict(ws_bytes=256), _lib.WIDE_ERR_WORKSPACE),
]


@pytest.mark.parametrize("kw,status", ATTN_BAD + [
    (dict(T=-1), _lib.WIDE_ERR_SHAPE),
    (dict(T=1 << 20), _lib.WIDE_ERR_UNSUPPORTED),             # T*Hq*dh >= 2^31
])
def test_attention_prefill_validation(lib, kw, status):
    assert attn_call(lib, "wide_attention_prefill", **kw) == status
    assert lib.wide_last_error().decode() != ""


@pytest.mark.parametrize("kw,status", ATTN_BAD + [
    (dict(T=0), _lib.WIDE_ERR_SHAPE),                          # a step needs its own key
    (dict(Hq=48, Hk=3), _lib.WIDE_ERR_UNSUPPORTED),            # 16 heads per group
])
def test_attention_decode_validation(lib, kw, status):
    assert attn_call(lib, "wide_attention_decode", **kw) == status
    assert lib.wide_last_error().decode() != ""


def test_attention_prefill_t0_is_a_no_op(lib):
    assert attn_call(lib, "wide_attention_prefill", T=0, Q=None, K=None, V=None, mask=None,
                     O=None) == _lib.WIDE_OK


def test_attention_workspace_sizes(lib):
    T, Hk, Hq, dh = 16384, 8, 32, 128
    ws = lib.wide_attention_workspace_size(T, Hk, dh)
    reorder = Hk * T * 4 + 2 * Hk * 4 + Hk * (T // 32) * 4
    vt = Hk * dh * T * 2  # T is a multiple of the 64-key tile here
    assert reorder + vt <= ws <= reorder + vt + 5 * 256
    assert lib.wide_attention_workspace_size(-1, Hk, dh) == 0
    d = lib.wide_attention_decode_workspace_size(T, Hq, dh)
    assert (T // 128) * Hq * (dh + 2) * 4 <= d <= (T // 128) * Hq * (dh + 2) * 4 + 256
    assert lib.wide_attention_decode_workspace_size(0, Hq, dh) == 0
    assert lib.wide_attention_decode_workspace_size(T, Hq, 64) == 0


# ---------------------------------------------------------------- operand-order decode weights

def test_decode_weights_size(lib):
    d, d_ff = 4096, 14336
    assert lib.wide_decode_weights_size(d, d_ff) == 3 * d * d_ff * 2
    assert lib.wide_decode_weights_size(4096 + 32, d_ff) == 0
    assert lib.wide_decode_weights_size(d, 0) == 0
    assert lib.wide_decode_weights_size(32768, 32768) == 0  # d * d_ff >= 2^30


@pytest.mark.parametrize("kw,status", [
    (dict(Wg=None), _lib.WIDE_ERR_NULL),
    (dict(out=None), _lib.WIDE_ERR_NULL),
    (dict(d=100), _lib.WIDE_ERR_SHAPE),
    (dict(Wu=FAKE + 8), _lib.WIDE_ERR_ALIGN),
    (dict(out=FAKE + 16), _lib.WIDE_ERR_ALIGN),
    (dict(nbytes=1024), _lib.WIDE_ERR_WORKSPACE),
])
def test_decode_prepare_validation(lib, kw, status):
    a = dict(Wg=FAKE, Wu=FAKE, Wd=FAKE, d=256, d_ff=1024, out=FAKE, nbytes=1 << 40)
    a.update(kw)
    assert lib.wide_decode_prepare_weights(a["Wg"], a["Wu"], a["Wd"], a["d"], a["d_ff"], a["out"],
                                           a["nbytes"], None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(prep=None), _lib.WIDE_ERR_NULL),
    (dict(prep=FAKE + 16), _lib.WIDE_ERR_ALIGN),
    (dict(T=17), _lib.WIDE_ERR_UNSUPPORTED),   # decode only: T <= 16
    (dict(X=None), _lib.WIDE_ERR_NULL),
    (dict(G=8), _lib.WIDE_ERR_UNSUPPORTED),
    (dict(ws_bytes=16), _lib.WIDE_ERR_WORKSPACE),
    (dict(prep_bytes=3 * 256 * 1024 * 2 - 1), _lib.WIDE_ERR_WORKSPACE),
])
def test_decode_prepared_validation(lib, kw, status):
    a = dict(X=FAKE, Wg=FAKE, Wu=FAKE, Wd=FAKE, prep=FAKE, prep_bytes=1 << 40, mask=FAKE, T=4,
             d=256, d_ff=1024, G=64, Y=FAKE, H=None, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    assert lib.wide_ffn_decode_prepared(a["X"], a["Wg"], a["Wu"], a["Wd"], a["prep"],
                                        a["prep_bytes"], a["mask"], a["T"], a["d"], a["d_ff"],
                                        a["G"], a["Y"], a["H"], a["ws"], a["ws_bytes"],
                                        None) == status


def test_noalloc_rejects_before_any_hip_call(lib):
    # validation and the size limit come before the scratch lookup, so these
    # return without touching a device
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, 64, 256, 1024, 64, _lib.WIDE_BF16, FAKE, FAKE, 0, None]

    def call(**kw):
        a = list(base)
        for k, v in kw.items():
            a[{"T": 5, "d": 6, "d_ff": 7, "G": 8, "dtype": 9, "Y": 10, "H": 11, "flags": 12}[k]] = v
        return lib.wide_ffn_forward_noalloc(*a)

    assert call(H=None) == _lib.WIDE_ERR_NULL
    assert call(d=96) == _lib.WIDE_ERR_UNSUPPORTED
    assert call(dtype=9) == _lib.WIDE_ERR_DTYPE
    assert call(H=FAKE + 4) == _lib.WIDE_ERR_ALIGN
    # T * ngroups too large for the array: 2^19 tokens x 64 groups needs 128 MiB of row lists
    assert call(T=1 << 19, d_ff=1024, G=16) == _lib.WIDE_ERR_WORKSPACE
    assert "WIDE_NOALLOC_SCRATCH_BYTES" in lib.wide_last_error().decode()
    assert lib.wide_ffn_workspace_size_for(1 << 19, 256, 1024, 16, _lib.WIDE_BF16, 1) > \
        _lib.WIDE_NOALLOC_SCRATCH_BYTES
    # the largest workload of the bench fits, and so does the Qwen3-14B shape,
    # whose down projection splits its last round (64 tiles x 4 parts of
    # fp32 partial sums in the workspace)
    assert lib.wide_ffn_workspace_size_for(16384, 4096, 14336, 128, _lib.WIDE_BF16, 1) <= \
        _lib.WIDE_NOALLOC_SCRATCH_BYTES
    qwen = lib.wide_ffn_workspace_size_for(4096, 5120, 17408, 128, _lib.WIDE_BF16, 1)
    assert 64 * 4 * 256 * 256 * 4 < qwen <= _lib.WIDE_NOALLOC_SCRATCH_BYTES
    # T == 0 with H_out NULL is a valid no-op
    assert call(T=0, H=None) == _lib.WIDE_OK


def test_router_reorder_validation(lib):
    ws = lib.wide_router_reorder_workspace_size(1000, 112)
    assert ws == (112 * 32 * 4 + 255) // 256 * 256
    # T <= 16: one bit word per group, then the first map's partial sums (sized for r = 64)
    assert lib.wide_router_reorder_workspace_size(16, 112) == (112 * 4 + 255) // 256 * 256 + 8 * 16 * 64 * 4
    assert lib.wide_router_reorder_workspace_size(-1, 4) == 0
    base = [FAKE, FAKE, FAKE, 64, 256, 32, 8, _lib.WIDE_ACT_SILU, _lib.WIDE_BF16, 256, None, None,
            FAKE, FAKE, FAKE, FAKE, 1 << 30, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return lib.wide_router_reorder(*a)

    assert call(0, None) == _lib.WIDE_ERR_NULL          # X
    assert call(12, None) == _lib.WIDE_ERR_NULL         # perm
    assert call(13, None) == _lib.WIDE_ERR_NULL         # counts
    assert call(9, 0) == _lib.WIDE_ERR_SHAPE            # tile
    assert call(5, 24) == _lib.WIDE_ERR_UNSUPPORTED     # r
    assert call(7, 5) == _lib.WIDE_ERR_SHAPE            # activation
    assert call(8, _lib.WIDE_F32) == _lib.WIDE_ERR_UNSUPPORTED
    assert call(15, None) == _lib.WIDE_ERR_WORKSPACE
    assert call(16, 16) == _lib.WIDE_ERR_WORKSPACE
    assert call(15, FAKE + 16) == _lib.WIDE_ERR_ALIGN
    assert call(11, FAKE + 4) == _lib.WIDE_ERR_ALIGN    # logits
