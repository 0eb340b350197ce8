"""Group-sparse (token-wise dynamic-width) SwiGLU FFN for MI355X.

Thin Python binding over libwide.so: it checks devices, dtypes and shapes,
allocates outputs and workspace with torch, and passes raw device pointers
and torch's current HIP stream to the C ABI. Every step of the computation
runs in the library's HIP kernels.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib
from ._lib import (WIDE_BF16, WIDE_DECODE_T_LIMIT, WIDE_F32, WIDE_FLAG_FORCE_DECODE,
                   WIDE_FLAG_FORCE_PREFILL, WIDE_STAGE_DECODE_DOWN, WIDE_STAGE_DECODE_GATE_UP,
                   WIDE_STAGE_DOWN, WIDE_STAGE_GATE_UP, WIDE_STAGE_REORDER, WIDE_TOKEN_TILE,
                   WideError)

__all__ = ["reorder_masks", "ffn_forward", "ffn_stage", "workspace_size", "decode_max_t",
           "gemm_mn", "gemm_k", "gemm_workspace_size", "router_forward", "router_reorder",
           "RouterReorderCall", "router_reorder_workspace_size", "router_workspace_size",
           "FfnCall", "WideError", "WIDE_TOKEN_TILE", "WIDE_DECODE_T_LIMIT",
           "WIDE_FLAG_FORCE_PREFILL", "WIDE_FLAG_FORCE_DECODE", "WIDE_STAGE_REORDER",
           "WIDE_STAGE_GATE_UP", "WIDE_STAGE_DOWN", "WIDE_STAGE_DECODE_GATE_UP",
           "WIDE_STAGE_DECODE_DOWN", "decode_weights_size", "decode_prepare_weights",
           "ffn_decode_prepared", "ffn_forward_noalloc"]

_DTYPES = {torch.bfloat16: WIDE_BF16, torch.float32: WIDE_F32}


def _stream_ptr(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need_cuda(name: str, t: torch.Tensor) -> None:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def decode_max_t() -> int:
    return int(_lib.load().wide_decode_max_t())


def workspace_size(T: int, d: int, d_ff: int, G: int, dtype: torch.dtype,
                   h_out_given: bool = False) -> int:
    return int(_lib.load().wide_ffn_workspace_size_for(T, d, d_ff, G, _DTYPES[dtype],
                                                       1 if h_out_given else 0))


def reorder_masks(mask: torch.Tensor, tile: int = WIDE_TOKEN_TILE):
    """Per-group stable active-first partition -> (perm [ng, T], counts [ng], padded [ng]) int32."""
    _need_cuda("mask", mask)
    if mask.dtype != torch.uint8 or mask.dim() != 2:
        raise ValueError("mask must be a 2-D uint8 tensor [T, ngroups]")
    T, ng = mask.shape
    perm = torch.empty((ng, T), dtype=torch.int32, device=mask.device)
    counts = torch.empty(ng, dtype=torch.int32, device=mask.device)
    padded = torch.empty(ng, dtype=torch.int32, device=mask.device)
    _lib.check(_lib.load().wide_reorder_masks(mask.data_ptr(), T, ng, tile, perm.data_ptr(),
                                              counts.data_ptr(), padded.data_ptr(),
                                              _stream_ptr(mask.device)))
    return perm, counts, padded


class FfnCall:
    """Validated arguments of one FFN call, with outputs and workspace allocated once.

    `run()` enqueues wide_ffn_forward; `stage(s)` enqueues one stage of it
    with the same arguments (used to time the kernels separately).
    """

    def __init__(self, X, Wg, Wu, Wd, mask, G: int, return_h: bool = False, flags: int = 0,
                 Y: Optional[torch.Tensor] = None, H: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None,
                 prepared: Optional[torch.Tensor] = None):
        for name, t in (("X", X), ("Wgate", Wg), ("Wup", Wu), ("Wdown", Wd), ("mask", mask)):
            _need_cuda(name, t)
        if X.dtype not in _DTYPES or any(w.dtype != X.dtype for w in (Wg, Wu, Wd)):
            raise ValueError("X and the weights must share one dtype, bfloat16 or float32")
        if mask.dtype != torch.uint8:
            raise ValueError("mask must be uint8")
        T, d = X.shape
        d_ff = Wg.shape[0]
        if Wg.shape != (d_ff, d) or Wu.shape != (d_ff, d) or Wd.shape != (d, d_ff):
            raise ValueError("expected Wgate, Wup [d_ff, d] and Wdown [d, d_ff]")
        if d_ff % G != 0 or mask.shape != (T, d_ff // G):
            raise ValueError("mask must be [T, d_ff // G] with G dividing d_ff")
        dev = X.device
        self.args = (X, Wg, Wu, Wd, mask)
        self.T, self.d, self.d_ff, self.G = T, d, d_ff, G
        self.dtype = _DTYPES[X.dtype]
        self.flags = flags
        self.Y = Y if Y is not None else torch.empty((T, d), dtype=X.dtype, device=dev)
        self.H = H if H is not None else (torch.empty((T, d_ff), dtype=X.dtype, device=dev)
                                          if return_h else None)
        if self.H is not None:
            _need_cuda("H", self.H)
        nbytes = workspace_size(T, d, d_ff, G, X.dtype, h_out_given=self.H is not None)
        if workspace is None:
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        self.workspace = workspace
        self.ws_bytes = workspace.numel() * workspace.element_size()
        # operand-order weights (decode_prepare_weights): run() then takes the
        # decode path through wide_ffn_decode_prepared
        self.prepared = prepared
        if prepared is not None:
            _need_cuda("prepared", prepared)
            if flags != 0:
                raise ValueError("a call with prepared weights takes no flags (it is decode only)")

    def _ffn_args(self):
        X, Wg, Wu, Wd, mask = self.args
        return (X.data_ptr(), Wg.data_ptr(), Wu.data_ptr(), Wd.data_ptr(), mask.data_ptr(), self.T,
                self.d, self.d_ff, self.G, self.dtype, self.Y.data_ptr(),
                None if self.H is None else self.H.data_ptr(), self.workspace.data_ptr(),
                self.ws_bytes, self.flags, _stream_ptr(X.device))

    def run(self):
        if self.prepared is not None:
            X, Wg, Wu, Wd, mask = self.args
            _lib.check(_lib.load().wide_ffn_decode_prepared(
                X.data_ptr(), Wg.data_ptr(), Wu.data_ptr(), Wd.data_ptr(), self.prepared.data_ptr(),
                self.prepared.numel() * self.prepared.element_size(), mask.data_ptr(), self.T,
                self.d, self.d_ff, self.G, self.Y.data_ptr(),
                None if self.H is None else self.H.data_ptr(), self.workspace.data_ptr(),
                self.ws_bytes, _stream_ptr(X.device)))
        else:
            _lib.check(_lib.load().wide_ffn_forward(*self._ffn_args()))
        return self.Y

    def stage(self, stage: int):
        if self.prepared is not None:
            raise ValueError("stages run the nn.Linear weights; time a prepared call with run()")
        _lib.check(_lib.load().wide_ffn_stage(stage, *self._ffn_args()))


def ffn_forward(X, Wg, Wu, Wd, mask, G: int, return_h: bool = False, flags: int = 0):
    """Masked SwiGLU FFN -> Y (and H with exact zeros at masked channels if return_h)."""
    call = FfnCall(X, Wg, Wu, Wd, mask, G, return_h=return_h, flags=flags)
    Y = call.run()
    return (Y, call.H) if return_h else Y


def ffn_forward_noalloc(X, Wg, Wu, Wd, mask, G: int, flags: int = 0,
                        Y: Optional[torch.Tensor] = None, H: Optional[torch.Tensor] = None):
    """ffn_forward through wide_ffn_forward_noalloc (the library's own scratch
    array instead of a workspace) -> (Y, H). Y and H are allocated here unless
    given; the library call itself allocates nothing."""
    for name, t in (("X", X), ("Wgate", Wg), ("Wup", Wu), ("Wdown", Wd), ("mask", mask)):
        _need_cuda(name, t)
    if X.dtype not in _DTYPES or any(w.dtype != X.dtype for w in (Wg, Wu, Wd)):
        raise ValueError("X and the weights must share one dtype, bfloat16 or float32")
    T, d = X.shape
    d_ff = Wg.shape[0]
    if Wg.shape != (d_ff, d) or Wu.shape != (d_ff, d) or Wd.shape != (d, d_ff):
        raise ValueError("expected Wgate, Wup [d_ff, d] and Wdown [d, d_ff]")
    if mask.dtype != torch.uint8 or d_ff % G != 0 or mask.shape != (T, d_ff // G):
        raise ValueError("mask must be uint8 [T, d_ff // G] with G dividing d_ff")
    Y = Y if Y is not None else torch.empty((T, d), dtype=X.dtype, device=X.device)
    H = H if H is not None else torch.empty((T, d_ff), dtype=X.dtype, device=X.device)
    _need_cuda("Y", Y)
    _need_cuda("H", H)
    _lib.check(_lib.load().wide_ffn_forward_noalloc(
        X.data_ptr(), Wg.data_ptr(), Wu.data_ptr(), Wd.data_ptr(), mask.data_ptr(), T, d, d_ff, G,
        _DTYPES[X.dtype], Y.data_ptr(), H.data_ptr(), flags, _stream_ptr(X.device)))
    return Y, H


def ffn_stage(stage: int, call: FfnCall) -> None:
    call.stage(stage)


def decode_weights_size(d: int, d_ff: int) -> int:
    return int(_lib.load().wide_decode_weights_size(d, d_ff))


def decode_prepare_weights(Wg, Wu, Wd, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Operand-order copy of the bf16 weights for the decode kernels (uint8 bytes)."""
    for name, t in (("Wgate", Wg), ("Wup", Wu), ("Wdown", Wd)):
        _need_cuda(name, t)
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16")
    d_ff, d = Wg.shape
    if Wu.shape != (d_ff, d) or Wd.shape != (d, d_ff):
        raise ValueError("expected Wgate, Wup [d_ff, d] and Wdown [d, d_ff]")
    nbytes = decode_weights_size(d, d_ff)
    if out is None:
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=Wg.device)
    _need_cuda("out", out)
    _lib.check(_lib.load().wide_decode_prepare_weights(
        Wg.data_ptr(), Wu.data_ptr(), Wd.data_ptr(), d, d_ff, out.data_ptr(),
        out.numel() * out.element_size(), _stream_ptr(Wg.device)))
    return out


def ffn_decode_prepared(X, Wg, Wu, Wd, prepared, mask, G: int, return_h: bool = False):
    """The decode path of ffn_forward with the matrix-core kernels reading `prepared`."""
    call = FfnCall(X, Wg, Wu, Wd, mask, G, return_h=return_h, prepared=prepared)
    Y = call.run()
    return (Y, call.H) if return_h else Y


# ---------------------------------------------------------------- masked GEMMs


def gemm_workspace_size(M: int, ngroups: int) -> int:
    return int(_lib.load().wide_gemm_workspace_size(M, ngroups))


def _gemm(fn_name: str, A, B, mask, G: int, routed_axis: str, C=None, workspace=None):
    for name, t in (("A", A), ("B", B), ("mask", mask)):
        _need_cuda(name, t)
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise ValueError("A and B must be bfloat16")
    if mask.dtype != torch.uint8:
        raise ValueError("mask must be uint8")
    M, K = A.shape
    N = B.shape[0]
    if B.shape != (N, K):
        raise ValueError("expected A [M, K] and B [N, K]")
    routed = N if routed_axis == "n" else K
    if routed % G != 0 or mask.shape != (M, routed // G):
        raise ValueError(f"mask must be [M, {routed_axis.upper()} // G] with G dividing "
                         f"{routed_axis.upper()}")
    dev = A.device
    if C is None:
        C = torch.empty((M, N), dtype=A.dtype, device=dev)
    _need_cuda("C", C)
    nbytes = gemm_workspace_size(M, routed // G)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    fn = getattr(_lib.load(), fn_name)
    _lib.check(fn(A.data_ptr(), B.data_ptr(), mask.data_ptr(), M, N, K, G, WIDE_BF16, C.data_ptr(),
                  workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                  _stream_ptr(dev)))
    return C


def gemm_mn(A, B, mask, G: int, C=None, workspace=None):
    """N-axis masked GEMM: C[m, n] = A[m] . B[n] if mask[m, n // G] else 0 (bf16)."""
    return _gemm("wide_gemm_mn", A, B, mask, G, "n", C, workspace)


def gemm_k(A, B, mask, G: int, C=None, workspace=None):
    """K-axis masked GEMM: C[m, n] = sum over active groups g of A[m, g] . B[n, g] (bf16)."""
    return _gemm("wide_gemm_k", A, B, mask, G, "k", C, workspace)


# ---------------------------------------------------------------- router

_ACTS = {"identity": _lib.WIDE_ACT_IDENTITY, "relu": _lib.WIDE_ACT_RELU, "silu": _lib.WIDE_ACT_SILU}


def router_workspace_size(T: int, r: int) -> int:
    return int(_lib.load().wide_router_workspace_size(T, r))


def router_forward(X, W1, W2, act: str = "silu", return_logits: bool = False, mask=None,
                   logits=None, workspace=None):
    """Bottleneck router -> mask [T, N_G] uint8 (1 = execute), and logits [T, N_G, 2] fp32.
    `workspace` (uint8 device tensor of router_workspace_size(T, r) bytes) is allocated when
    not given and needed (1 <= T <= 16)."""
    for name, t in (("X", X), ("W1", W1), ("W2", W2)):
        _need_cuda(name, t)
    if any(t.dtype != torch.bfloat16 for t in (X, W1, W2)):
        raise ValueError("X, W1 and W2 must be bfloat16")
    T, D = X.shape
    r = W1.shape[0]
    if W1.shape != (r, D) or W2.dim() != 2 or W2.shape[1] != r or W2.shape[0] % 2:
        raise ValueError("expected W1 [r, D] and W2 [2 * ngroups, r]")
    ng = W2.shape[0] // 2
    dev = X.device
    if mask is None:
        mask = torch.empty((T, ng), dtype=torch.uint8, device=dev)
    if return_logits and logits is None:
        logits = torch.empty((T, ng, 2), dtype=torch.float32, device=dev)
    need = router_workspace_size(T, r)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _lib.check(_lib.load().wide_router_forward(
        X.data_ptr(), W1.data_ptr(), W2.data_ptr(), T, D, r, ng, _ACTS[act], WIDE_BF16,
        mask.data_ptr(), None if logits is None else logits.data_ptr(),
        None if workspace is None else workspace.data_ptr(),
        0 if workspace is None else workspace.numel(), _stream_ptr(dev)))
    return (mask, logits) if return_logits else mask


def router_reorder_workspace_size(T: int, ngroups: int) -> int:
    return int(_lib.load().wide_router_reorder_workspace_size(T, ngroups))


class RouterReorderCall:
    """Arguments of wide_router_reorder with outputs and workspace allocated once:
    run() enqueues router -> packed bits -> per-group partition."""

    def __init__(self, X, W1, W2, act: str = "silu", tile: int = WIDE_TOKEN_TILE,
                 return_mask: bool = False, return_logits: bool = False):
        for name, t in (("X", X), ("W1", W1), ("W2", W2)):
            _need_cuda(name, t)
        if any(t.dtype != torch.bfloat16 for t in (X, W1, W2)):
            raise ValueError("X, W1 and W2 must be bfloat16")
        T, D = X.shape
        r = W1.shape[0]
        if W1.shape != (r, D) or W2.dim() != 2 or W2.shape[1] != r or W2.shape[0] % 2:
            raise ValueError("expected W1 [r, D] and W2 [2 * ngroups, r]")
        ng = W2.shape[0] // 2
        dev = X.device
        self.args = (X, W1, W2)
        self.T, self.D, self.r, self.ng, self.act, self.tile = T, D, r, ng, _ACTS[act], tile
        self.mask = torch.empty((T, ng), dtype=torch.uint8, device=dev) if return_mask else None
        self.logits = (torch.empty((T, ng, 2), dtype=torch.float32, device=dev)
                       if return_logits else None)
        self.perm = torch.empty((ng, T), dtype=torch.int32, device=dev)
        self.counts = torch.empty(ng, dtype=torch.int32, device=dev)
        self.padded = torch.empty(ng, dtype=torch.int32, device=dev)
        n = router_reorder_workspace_size(T, ng)
        self.workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)

    def run(self):
        X, W1, W2 = self.args
        _lib.check(_lib.load().wide_router_reorder(
            X.data_ptr(), W1.data_ptr(), W2.data_ptr(), self.T, self.D, self.r, self.ng, self.act,
            WIDE_BF16, self.tile, None if self.mask is None else self.mask.data_ptr(),
            None if self.logits is None else self.logits.data_ptr(), self.perm.data_ptr(),
            self.counts.data_ptr(), self.padded.data_ptr(), self.workspace.data_ptr(),
            self.workspace.numel(), _stream_ptr(X.device)))
        return self.perm, self.counts, self.padded


def router_reorder(X, W1, W2, act: str = "silu", tile: int = WIDE_TOKEN_TILE,
                   return_mask: bool = False):
    """Router fused with the mask reorder -> (perm [ng, T], counts [ng], padded [ng]) int32,
    plus the mask [T, ng] uint8 if return_mask."""
    call = RouterReorderCall(X, W1, W2, act, tile, return_mask=return_mask)
    out = call.run()
    return (*out, call.mask) if return_mask else out


# ---------------------------------------------------------------- attention


def attention_workspace_size(T: int, Hk: int, dh: int) -> int:
    return int(_lib.load().wide_attention_workspace_size(T, Hk, dh))


def attention_prefill(Q, K, V, mask, Hq: int, Hk: int, O=None, workspace=None,
                      zero_inactive: bool = False):
    """Head-group-pruned causal attention -> O [T, Hq*dh] bf16.

    Q [T, Hq*dh], K and V [T, Hk*dh] bf16; mask [T, Hk] uint8 (group g = KV
    head g and its Hq/Hk query heads). O is written where the token keeps the
    group (and +0.0 elsewhere with zero_inactive; else left as it was).
    """
    for name, t in (("Q", Q), ("K", K), ("V", V), ("mask", mask)):
        _need_cuda(name, t)
    if any(t.dtype != torch.bfloat16 for t in (Q, K, V)):
        raise ValueError("Q, K and V must be bfloat16")
    if mask.dtype != torch.uint8:
        raise ValueError("mask must be uint8")
    if Q.dim() != 2 or Hq <= 0 or Hk <= 0 or Hq % Hk or Q.shape[1] % Hq:
        raise ValueError("expected Q [T, Hq*dh] with Hk dividing Hq")
    T = Q.shape[0]
    dh = Q.shape[1] // Hq
    if K.shape != (T, Hk * dh) or V.shape != (T, Hk * dh) or mask.shape != (T, Hk):
        raise ValueError("expected K and V [T, Hk*dh] and mask [T, Hk]")
    dev = Q.device
    if O is None:
        # a fresh output holds +0.0 at skipped pairs either way
        alloc = torch.empty if zero_inactive else torch.zeros
        O = alloc((T, Hq * dh), dtype=Q.dtype, device=dev)
    _need_cuda("O", O)
    nbytes = attention_workspace_size(T, Hk, dh)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    flags = _lib.WIDE_ATTN_ZERO_INACTIVE if zero_inactive else 0
    _lib.check(_lib.load().wide_attention_prefill(
        Q.data_ptr(), K.data_ptr(), V.data_ptr(), mask.data_ptr(), T, Hq, Hk, dh, WIDE_BF16,
        O.data_ptr(), flags, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream_ptr(dev)))
    return O


def attention_decode_workspace_size(T: int, Hq: int, dh: int) -> int:
    return int(_lib.load().wide_attention_decode_workspace_size(T, Hq, dh))


def attention_decode(q, K, V, mask, Hq: int, Hk: int, O=None, workspace=None,
                     zero_inactive: bool = False):
    """One decoding step: q [Hq*dh] (position T - 1) over the cache K, V
    [T, Hk*dh]; mask [Hk] uint8. Returns O [Hq*dh] bf16 (kept heads written;
    +0.0 elsewhere with zero_inactive or on a fresh output)."""
    for name, t in (("q", q), ("K", K), ("V", V), ("mask", mask)):
        _need_cuda(name, t)
    if any(t.dtype != torch.bfloat16 for t in (q, K, V)):
        raise ValueError("q, K and V must be bfloat16")
    if mask.dtype != torch.uint8:
        raise ValueError("mask must be uint8")
    if q.dim() != 1 or Hq <= 0 or Hk <= 0 or Hq % Hk or q.shape[0] % Hq:
        raise ValueError("expected q [Hq*dh] with Hk dividing Hq")
    dh = q.shape[0] // Hq
    T = K.shape[0]
    if K.shape != (T, Hk * dh) or V.shape != (T, Hk * dh) or mask.shape != (Hk,):
        raise ValueError("expected K and V [T, Hk*dh] and mask [Hk]")
    dev = q.device
    if O is None:
        alloc = torch.empty if zero_inactive else torch.zeros
        O = alloc((Hq * dh,), dtype=q.dtype, device=dev)
    _need_cuda("O", O)
    nbytes = attention_decode_workspace_size(T, Hq, dh)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    flags = _lib.WIDE_ATTN_ZERO_INACTIVE if zero_inactive else 0
    _lib.check(_lib.load().wide_attention_decode(
        q.data_ptr(), K.data_ptr(), V.data_ptr(), mask.data_ptr(), T, Hq, Hk, dh, WIDE_BF16,
        O.data_ptr(), flags, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream_ptr(dev)))
    return O
