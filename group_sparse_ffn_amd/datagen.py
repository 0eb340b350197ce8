"""Seeded synthetic inputs for the group-sparse FFN: activations, weights and masks.

This module only draws random numbers and shapes them; it holds none of the
FFN's arithmetic. Both the fp64 oracle and the HIP path consume exactly the
arrays produced here, so the two sides see identical bits.

Recipe (per workload, base seed s = 1000 * workload id):
  X      ~ N(0, 1)        drawn with seed s
  Wgate  ~ 0.02 * N(0, 1) seed s + 1   ([d_ff, d], nn.Linear layout)
  Wup    ~ 0.02 * N(0, 1) seed s + 2   ([d_ff, d])
  Wdown  ~ 0.02 * N(0, 1) seed s + 3   ([d, d_ff])
  mask                    seed s + 4 (+ cell index for sweep cells)
All values are drawn in float32 with numpy's PCG64 and, for bf16 workloads,
rounded once to bfloat16 (round-to-nearest-even) on the host.

Masks are uint8 [T, ngroups], row-major, nonzero = the token executes the
group (WIDE paper, Sec. 3.1 "Preliminaries": one mask matrix per FFN layer,
contiguous channel groups of size G).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """One FFN problem: sizes, dtype and the mask recipe."""
    name: str
    wid: int                 # workload id (seed base = 1000 * wid)
    T: int
    d: int
    d_ff: int
    G: int
    dtype: str               # "bf16" or "f32"
    mask_kind: str           # "bernoulli", "topk", "beta", "zipf", "ones", "zeros"
    density: float = 0.5     # target fraction of active (token, group) pairs
    cell: int = 0            # sweep-cell index (offsets the mask seed)

    @property
    def ngroups(self) -> int:
        return self.d_ff // self.G

    @property
    def seed(self) -> int:
        return 1000 * self.wid


# The workloads the library is measured and checked on.
TINY = Workload("tiny-swiglu", 1, T=64, d=256, d_ff=1024, G=64, dtype="f32", mask_kind="bernoulli")
LLAMA8B_PREFILL = Workload("llama3.1-8b-ffn-prefill", 2, T=16384, d=4096, d_ff=14336, G=128,
                           dtype="bf16", mask_kind="topk")
LLAMA8B_DECODE_T1 = Workload("llama3.1-8b-ffn-decode-t1", 3, T=1, d=4096, d_ff=14336, G=128,
                             dtype="bf16", mask_kind="topk")
LLAMA8B_DECODE_T16 = Workload("llama3.1-8b-ffn-decode-t16", 3, T=16, d=4096, d_ff=14336, G=128,
                              dtype="bf16", mask_kind="topk")
QWEN14B_SKEW = Workload("qwen3-14b-ffn-skew", 5, T=4096, d=5120, d_ff=17408, G=128,
                        dtype="bf16", mask_kind="zipf")


def llama3b_sweep_cells():
    """Llama3.2-3B-shaped sweep: G x sparsity x T, Beta(2,2) per-group rates."""
    cells = []
    idx = 0
    for G in (16, 32, 64, 128, 256, 512):
        for s in (0.10, 0.25, 0.50, 0.70):
            for T in (1, 2048, 8192):
                cells.append(Workload(f"llama3.2-3b-sweep-G{G}-s{int(s * 100)}-T{T}", 4, T=T, d=3072,
                                      d_ff=8192, G=G, dtype="bf16", mask_kind="beta",
                                      density=1.0 - s, cell=idx))
                idx += 1
    return cells


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal_f32(seed: int, shape, scale: float = 1.0) -> np.ndarray:
    x = _rng(seed).standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def to_dtype(x: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 numpy -> torch CPU tensor of the workload dtype (bf16 rounds once, RNE)."""
    t = torch.from_numpy(x)
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t.clone()
    raise ValueError(dtype)


def waterfill(w: np.ndarray, m: float, iters: int = 200) -> np.ndarray:
    """Scale nonnegative weights w so that mean(min(1, c*w)) == m.

    Plain clipping after a single rescale misses the target whenever some
    entries saturate, so the scale is found by bisection on c.
    """
    w = np.asarray(w, dtype=np.float64)
    if m <= 0.0:
        return np.zeros_like(w)
    if m >= 1.0:
        return np.ones_like(w)
    lo, hi = 0.0, 1.0
    while np.mean(np.minimum(1.0, hi * w)) < m:
        hi *= 2.0
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if np.mean(np.minimum(1.0, mid * w)) < m:
            lo = mid
        else:
            hi = mid
    return np.minimum(1.0, hi * w)


def mask_bernoulli(T: int, ng: int, p, seed: int) -> np.ndarray:
    """M[t, g] = (u < p_g), u ~ U[0,1); p is a scalar or a per-group vector."""
    u = _rng(seed).random(size=(T, ng))
    return (u < np.asarray(p)[None, ...] if np.ndim(p) else u < p).astype(np.uint8)


def mask_topk(T: int, ng: int, k: int, seed: int) -> np.ndarray:
    """Per token, the k groups with the largest Gaussian router score.

    Ties (measure zero for continuous scores) go to the lower group index.
    """
    scores = _rng(seed).standard_normal(size=(T, ng))
    order = np.argsort(-scores, axis=1, kind="stable")
    m = np.zeros((T, ng), dtype=np.uint8)
    np.put_along_axis(m, order[:, :k], 1, axis=1)
    return m


def mask_beta(T: int, ng: int, density: float, seed: int) -> np.ndarray:
    """Bernoulli mask with per-group rates b_g ~ Beta(2,2) water-filled to `density`."""
    rng = _rng(seed)
    b = rng.beta(2.0, 2.0, size=ng)
    p = waterfill(b, density)
    u = rng.random(size=(T, ng))
    return (u < p[None, :]).astype(np.uint8)


def zipf_profile(ng: int, density: float, seed: int, s: float = 1.2) -> np.ndarray:
    """Per-group activation probabilities from a Zipf(s)-ranked profile averaging `density`.

    Rank r (1-based) has weight r^-s; ranks are assigned to groups by a seeded permutation.
    """
    rng = _rng(seed)
    w = np.arange(1, ng + 1, dtype=np.float64) ** (-s)
    p_rank = waterfill(w, density)
    perm = rng.permutation(ng)
    p = np.empty(ng)
    p[perm] = p_rank
    return p


def mask_zipf(T: int, ng: int, density: float, seed: int) -> np.ndarray:
    p = zipf_profile(ng, density, seed)
    u = _rng(seed + 7919).random(size=(T, ng))
    return (u < p[None, :]).astype(np.uint8)


def make_mask(w: Workload, kind: Optional[str] = None, T: Optional[int] = None) -> np.ndarray:
    kind = kind or w.mask_kind
    T = w.T if T is None else T
    ng = w.ngroups
    seed = w.seed + 4 + w.cell
    if kind == "bernoulli":
        return mask_bernoulli(T, ng, w.density, seed)
    if kind == "topk":
        return mask_topk(T, ng, int(round(ng * w.density)), seed)
    if kind == "beta":
        return mask_beta(T, ng, w.density, seed)
    if kind == "zipf":
        return mask_zipf(T, ng, w.density, seed)
    if kind == "ones":
        return np.ones((T, ng), dtype=np.uint8)
    if kind == "zeros":
        return np.zeros((T, ng), dtype=np.uint8)
    raise ValueError(kind)


def make_inputs(w: Workload, T: Optional[int] = None, mask_kind: Optional[str] = None,
                weights: bool = True) -> dict:
    """All inputs of one workload as CPU tensors (X, Wg, Wu, Wd in the workload dtype, mask uint8)."""
    T = w.T if T is None else T
    s = w.seed
    out = {"X": to_dtype(normal_f32(s, (T, w.d)), w.dtype)}
    if weights:
        out["Wg"] = to_dtype(normal_f32(s + 1, (w.d_ff, w.d), 0.02), w.dtype)
        out["Wu"] = to_dtype(normal_f32(s + 2, (w.d_ff, w.d), 0.02), w.dtype)
        out["Wd"] = to_dtype(normal_f32(s + 3, (w.d, w.d_ff), 0.02), w.dtype)
    out["mask"] = torch.from_numpy(make_mask(w, mask_kind, T))
    return out


def random_small(seed: int, T: int, d: int, d_ff: int, G: int, dtype: str = "f32",
                 density: float = 0.5, wscale: float = 0.1) -> dict:
    """Small random problem for property tests (Bernoulli mask)."""
    ng = d_ff // G
    return {
        "X": to_dtype(normal_f32(seed, (T, d)), dtype),
        "Wg": to_dtype(normal_f32(seed + 1, (d_ff, d), wscale), dtype),
        "Wu": to_dtype(normal_f32(seed + 2, (d_ff, d), wscale), dtype),
        "Wd": to_dtype(normal_f32(seed + 3, (d, d_ff), wscale), dtype),
        "mask": torch.from_numpy(mask_bernoulli(T, ng, density, seed + 4)),
    }


# ---------------------------------------------------------------- masked GEMMs

@dataclasses.dataclass(frozen=True)
class GemmWorkload:
    """One group-masked GEMM C = A B^T (A [M, K], B [N, K]) routed on `axis`.

    axis "mn": the mask [M, N/G] routes output columns (an attention W_q
    projection; with G = N, one group, the M-axis / dynamic-depth case);
    axis "k": the mask [M, K/G] routes the reduction (an attention W_o
    projection). Recipe: A ~ N(0,1) with seed s, B ~ 0.02 N(0,1) with seed
    s + 1, mask with seed s + 4, s = 1000 * wid; bf16 rounded once.
    """
    name: str
    wid: int
    M: int
    N: int
    K: int
    G: int
    axis: str                # "mn" or "k"
    mask_kind: str           # as for Workload
    density: float = 0.5

    @property
    def ngroups(self) -> int:
        return (self.N if self.axis == "mn" else self.K) // self.G

    @property
    def seed(self) -> int:
        return 1000 * self.wid


# Llama3.1-8B attention projections at the prefill length: 32 query heads of
# 128 channels in 8 GQA groups, so one routed group = 4 heads = 512 channels.
LLAMA8B_ATTN_Q = GemmWorkload("llama3.1-8b-attn-wq-prefill", 6, M=16384, N=4096, K=4096, G=512,
                              axis="mn", mask_kind="topk")
LLAMA8B_ATTN_O = GemmWorkload("llama3.1-8b-attn-wo-prefill", 7, M=16384, N=4096, K=4096, G=512,
                              axis="k", mask_kind="topk")
# Dynamic depth: one group spanning all N outputs, a token keeps or skips the layer.
LLAMA8B_DEPTH = GemmWorkload("llama3.1-8b-depth-wq-prefill", 8, M=16384, N=4096, K=4096, G=4096,
                             axis="mn", mask_kind="bernoulli")


def make_gemm_mask(w: GemmWorkload, kind: Optional[str] = None, M: Optional[int] = None):
    kind = kind or w.mask_kind
    M = w.M if M is None else M
    ng = w.ngroups
    seed = w.seed + 4
    if kind == "bernoulli":
        return mask_bernoulli(M, ng, w.density, seed)
    if kind == "topk":
        return mask_topk(M, ng, int(round(ng * w.density)), seed)
    if kind == "beta":
        return mask_beta(M, ng, w.density, seed)
    if kind == "ones":
        return np.ones((M, ng), dtype=np.uint8)
    if kind == "zeros":
        return np.zeros((M, ng), dtype=np.uint8)
    raise ValueError(kind)


def make_gemm_inputs(w: GemmWorkload, M: Optional[int] = None,
                     mask_kind: Optional[str] = None) -> dict:
    """A [M, K], B [N, K] bf16 and mask uint8 as CPU tensors."""
    M = w.M if M is None else M
    s = w.seed
    return {"A": to_dtype(normal_f32(s, (M, w.K)), "bf16"),
            "B": to_dtype(normal_f32(s + 1, (w.N, w.K), 0.02), "bf16"),
            "mask": torch.from_numpy(make_gemm_mask(w, mask_kind, M))}


# ---------------------------------------------------------------- router

def make_router_weights(seed: int, D: int, r: int, ngroups: int) -> dict:
    """Synthetic bottleneck-router weights (no trained ones exist here):
    W1 [r, D] ~ N(0, 1/D) with seed `seed`, W2 [2*ngroups, r] ~ N(0, 1/r) with
    seed `seed + 1`, both rounded once to bf16. With these scales the two
    logits of a group are exchangeable, so about half the groups execute."""
    return {"W1": to_dtype(normal_f32(seed, (r, D), 1.0 / np.sqrt(D)), "bf16"),
            "W2": to_dtype(normal_f32(seed + 1, (2 * ngroups, r), 1.0 / np.sqrt(r)), "bf16")}


# ---------------------------------------------------------------- attention

@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    """Head-group-pruned causal attention over one sequence: Q [T, Hq*dh],
    K and V [T, Hk*dh], mask [T, Hk] (one routing group per KV head)."""
    name: str
    seed: int
    T: int
    Hq: int
    Hk: int
    dh: int = 128
    mask_kind: str = "bernoulli"
    density: float = 0.5


# Llama3.1-8B attention at the prefill length: 32 query heads, 8 KV heads,
# head dim 128 (G_attn = 4 * 128 = 512 channels of W_q per group).
LLAMA8B_ATTN_PREFILL = AttnWorkload("llama3.1-8b-attention-prefill", 9, T=16384, Hq=32, Hk=8)


def make_attention_inputs(w: AttnWorkload, T: Optional[int] = None,
                          mask_kind: Optional[str] = None) -> dict:
    """Q, K, V ~ N(0, 1) rounded to bf16 (scores q.k / sqrt(dh) ~ N(0, 1)) and
    the [T, Hk] mask, as CPU tensors."""
    T = w.T if T is None else T
    kind = mask_kind or w.mask_kind
    s = w.seed
    out = {"Q": to_dtype(normal_f32(s, (T, w.Hq * w.dh)), "bf16"),
           "K": to_dtype(normal_f32(s + 1, (T, w.Hk * w.dh)), "bf16"),
           "V": to_dtype(normal_f32(s + 2, (T, w.Hk * w.dh)), "bf16")}
    ms = s + 3
    if kind == "bernoulli":
        m = mask_bernoulli(T, w.Hk, w.density, ms)
    elif kind == "topk":
        m = mask_topk(T, w.Hk, int(round(w.Hk * w.density)), ms)
    elif kind == "beta":
        m = mask_beta(T, w.Hk, w.density, ms)
    elif kind == "ones":
        m = np.ones((T, w.Hk), dtype=np.uint8)
    elif kind == "zeros":
        m = np.zeros((T, w.Hk), dtype=np.uint8)
    else:
        raise ValueError(kind)
    out["mask"] = torch.from_numpy(m)
    return out
