"""fp64 CPU oracle for the group-sparse FFN (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. It loads `liboracle.so`, built from `wide_oracle.c` by
`build_oracle()` with plain gcc (no HIP), and exposes numpy-level wrappers.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wide_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build_oracle(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math so no reassociation)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_native(out_dir: str) -> str:
    """A copy of the oracle for timing on the host that runs it: gcc -O3
    -march=native -fopenmp, built there (the build container's CPU may differ).

    The arithmetic is unchanged: ISO C mode (-std=c11) keeps floating-point
    contraction off and there is no fast-math, so every product and sum is
    the same double operation in the same order as in the -O2 build (the
    pins compare the two bit for bit)."""
    os.makedirs(out_dir, exist_ok=True)
    path = os.path.join(out_dir, "liboracle_native.so")
    tmp = path + ".tmp"
    subprocess.check_call(["gcc", "-O3", "-march=native", "-std=c11", "-fopenmp", "-fPIC",
                           "-shared", _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, path)
    return path


def use_library(path: str) -> None:
    """Load the oracle from `path` (a build of wide_oracle.c) from now on."""
    global _LIB_PATH, _lib
    _LIB_PATH = path
    _lib = None
    _load()


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_oracle(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_reorder.argtypes = [p, i64, i64, i64, p, p, p]
        lib.oracle_reorder.restype = ctypes.c_int
        lib.oracle_ffn.argtypes = [p, p, p, p, p, i64, i64, i64, i64, p, i64, p, p]
        lib.oracle_ffn.restype = ctypes.c_int
        lib.oracle_gemm_mn.argtypes = [p, p, p, i64, i64, i64, i64, p, i64, p]
        lib.oracle_gemm_mn.restype = ctypes.c_int
        lib.oracle_gemm_k.argtypes = [p, p, p, i64, i64, i64, i64, p, i64, p]
        lib.oracle_gemm_k.restype = ctypes.c_int
        lib.oracle_router.argtypes = [p, p, p, i64, i64, i64, i64, ctypes.c_int, p, i64, p, p]
        lib.oracle_router.restype = ctypes.c_int
        lib.oracle_attention.argtypes = [p, p, p, p, i64, i64, i64, i64, p, i64, p]
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _as_f32(x) -> np.ndarray:
    """Exact float32 copy of a float tensor/array (bf16 widens exactly)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu").float().numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _as_u8(m) -> np.ndarray:
    try:
        import torch
        if isinstance(m, torch.Tensor):
            m = m.detach().to("cpu").numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(m, dtype=np.uint8))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def reorder(mask, tile: int):
    """Per-group stable partition -> (perm [ng, T] int32, counts [ng], padded [ng])."""
    m = _as_u8(mask)
    T, ng = m.shape
    perm = np.empty((ng, T), dtype=np.int32)
    counts = np.empty(ng, dtype=np.int32)
    padded = np.empty(ng, dtype=np.int32)
    rc = _load().oracle_reorder(_ptr(m), T, ng, tile, _ptr(perm), _ptr(counts), _ptr(padded))
    if rc != 0:
        raise ValueError(f"oracle_reorder rejected its arguments (rc={rc})")
    return perm, counts, padded


def ffn(X, Wg, Wu, Wd, mask, G: int, rows=None):
    """Masked SwiGLU FFN in fp64 -> (H [n, d_ff], Y [n, d]) for all tokens or `rows`."""
    x, wg, wu, wd = _as_f32(X), _as_f32(Wg), _as_f32(Wu), _as_f32(Wd)
    m = _as_u8(mask)
    T, d = x.shape
    d_ff = wg.shape[0]
    if wg.shape != (d_ff, d) or wu.shape != (d_ff, d) or wd.shape != (d, d_ff):
        raise ValueError("weight shapes must be Wg,Wu [d_ff,d] and Wd [d,d_ff]")
    if m.shape != (T, d_ff // G):
        raise ValueError("mask must be [T, d_ff/G]")
    if rows is None:
        r = None
        n = T
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = r.shape[0]
    H = np.empty((n, d_ff), dtype=np.float64)
    Y = np.empty((n, d), dtype=np.float64)
    rc = _load().oracle_ffn(_ptr(x), _ptr(wg), _ptr(wu), _ptr(wd), _ptr(m), T, d, d_ff, G,
                            None if r is None else _ptr(r), n, _ptr(H), _ptr(Y))
    if rc != 0:
        raise ValueError(f"oracle_ffn rejected its arguments (rc={rc})")
    return H, Y


def _gemm(fn_name, A, B, mask, G, rows, axis_len):
    a, b = _as_f32(A), _as_f32(B)
    m = _as_u8(mask)
    M, K = a.shape
    N = b.shape[0]
    if b.shape != (N, K):
        raise ValueError("A must be [M, K] and B [N, K]")
    if m.shape != (M, axis_len // G):
        raise ValueError("mask has the wrong shape")
    if rows is None:
        r, n = None, M
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = r.shape[0]
    C = np.empty((n, N), dtype=np.float64)
    rc = getattr(_load(), fn_name)(_ptr(a), _ptr(b), _ptr(m), M, N, K, G,
                                   None if r is None else _ptr(r), n, _ptr(C))
    if rc != 0:
        raise ValueError(f"{fn_name} rejected its arguments (rc={rc})")
    return C


def gemm_mn(A, B, mask, G: int, rows=None):
    """N-axis group-masked C = A B^T in fp64: C[m,n] = mask[m, n/G] ? A[m].B[n] : 0."""
    return _gemm("oracle_gemm_mn", A, B, mask, G, rows, _as_f32(B).shape[0])


def gemm_k(A, B, mask, G: int, rows=None):
    """K-axis group-masked C in fp64: C[m,n] = sum_k mask[m, k/G] A[m,k] B[n,k]."""
    return _gemm("oracle_gemm_k", A, B, mask, G, rows, _as_f32(A).shape[1])


ROUTER_ACTS = {"identity": 0, "relu": 1, "silu": 2}


def router(X, W1, W2, act: str = "silu", rows=None):
    """Bottleneck router in fp64 -> (logits [n, N_G, 2] float64, mask [n, N_G] uint8).

    z = act(X W1^T), logits = z W2^T viewed as [N_G, 2]; a group executes
    (mask 1) when its class-0 logit is >= its class-1 logit.
    """
    x, w1, w2 = _as_f32(X), _as_f32(W1), _as_f32(W2)
    T, D = x.shape
    r = w1.shape[0]
    if w1.shape != (r, D) or w2.ndim != 2 or w2.shape[1] != r or w2.shape[0] % 2:
        raise ValueError("W1 must be [r, D] and W2 [2*N_G, r]")
    ng = w2.shape[0] // 2
    if rows is None:
        rr, n = None, T
    else:
        rr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = rr.shape[0]
    logits = np.empty((n, ng, 2), dtype=np.float64)
    mask = np.empty((n, ng), dtype=np.uint8)
    rc = _load().oracle_router(_ptr(x), _ptr(w1), _ptr(w2), T, D, r, ng, ROUTER_ACTS[act],
                               None if rr is None else _ptr(rr), n, _ptr(logits), _ptr(mask))
    if rc != 0:
        raise ValueError(f"oracle_router rejected its arguments (rc={rc})")
    return logits, mask


def attention(Q, K, V, mask, Hq: int, Hk: int, rows=None):
    """Head-group-pruned causal attention in fp64 -> O [n, Hq*dh] float64.

    Q [T, Hq*dh], K and V [T, Hk*dh], mask [T, Hk] (group g = KV head g =
    query heads g*Hq/Hk .. (g+1)*Hq/Hk - 1). For an active (t, g) and each of
    its query heads h: O[t,h] = softmax_j<=t(Q[t,h].K[j,g] / sqrt(dh)) V[:,g];
    a skipped pair gives +0.0.
    """
    q, k, v = _as_f32(Q), _as_f32(K), _as_f32(V)
    m = _as_u8(mask)
    T = q.shape[0]
    if Hq <= 0 or Hk <= 0 or Hq % Hk or q.ndim != 2 or q.shape[1] % Hq:
        raise ValueError("Q must be [T, Hq*dh] with Hk dividing Hq")
    dh = q.shape[1] // Hq
    if k.shape != (T, Hk * dh) or v.shape != (T, Hk * dh) or m.shape != (T, Hk):
        raise ValueError("K and V must be [T, Hk*dh] and mask [T, Hk]")
    if rows is None:
        r, n = None, T
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = r.shape[0]
    O = np.empty((n, Hq * dh), dtype=np.float64)
    rc = _load().oracle_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(m), T, Hq, Hk, dh,
                                  None if r is None else _ptr(r), n, _ptr(O))
    if rc != 0:
        raise ValueError(f"oracle_attention rejected its arguments (rc={rc})")
    return O
