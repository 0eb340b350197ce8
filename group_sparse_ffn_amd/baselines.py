"""Comparison pipelines for group-masked GEMMs, written the way a framework user
would write them: plain PyTorch ops, no custom kernels. They are measured next
to the fused kernels of this package and are never part of its compute path.

WIDE paper, Sec. 3.2 "Inference-time Group Skipping with Unified Mask
Reordering" and App. A ("Naive M/N/K-axis pruning", Table 4, Fig. 8):
  * naive gather-scatter: the mask is turned into exact active indices (a
    device-to-host read of their number, so the pipeline cannot be captured in
    a graph), the token-specific subsets of the operands are materialized, a
    batched product runs on them and the results are scattered into C;
  * grouped GEMM on reordered masks: every group's active tokens are brought
    to a prefix (a stable per-group partition), gathered, multiplied by the
    group's weight slice in one GEMM per group, and scattered back.

C = A B^T with A [M, K], B [N, K] (weights stored [out, in]); mask [M, N_G]
uint8, nonzero = active; N-axis groups are G consecutive columns of C (rows of
B), K-axis groups are G consecutive channels of K. The M axis is the N_G = 1
case (one decision per token and row).

Table 4's traffic (elements; masks, indices and offsets excluded) for a
density p of active (token, group) pairs:
  M axis: 3pMK + NK + 3pMN + MN       (our reading: gather A rows, dense GEMM
                                       on them, zero C, scatter the rows)
  N axis: MK + 3pMNK + 3pMN + MN
  K axis: 3pMK + 3pMNK + MN
The naive N- and K-axis pipelines below follow those terms exactly when every
token has the same number of active groups (the per-token subsets are padded to
the largest count otherwise). `traffic_elements` gives the closed forms and
`materialized_elements` the token-specific storage.
"""
from __future__ import annotations

import torch

__all__ = [
    "naive_gemm_m",
    "naive_gemm_mn",
    "naive_gemm_k",
    "grouped_gemm_mn",
    "grouped_gemm_k",
    "traffic_elements",
    "materialized_elements",
]


def _check(A, B, mask, G, axis):
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[1]:
        raise ValueError("expected A [M, K] and B [N, K]")
    M, K = A.shape
    N = B.shape[0]
    routed = N if axis == "n" else K
    if G <= 0 or routed % G != 0 or mask.shape != (M, routed // G):
        raise ValueError(f"mask must be [M, {axis.upper()} // G] with G dividing {axis.upper()}")
    return M, N, K, routed // G


def _per_token_slots(maskb):
    """Active groups of every token first (ascending), then its inactive ones;
    returns (slot -> group [M, kmax], slot valid [M, kmax], kmax, uniform).
    Reading kmax back to the host is the pipeline's device-to-host sync."""
    counts = maskb.sum(dim=1)
    kmax, kmin = (int(v) for v in torch.stack([counts.max(), counts.min()]).tolist())
    order = torch.argsort((~maskb).to(torch.int8), dim=1, stable=True)[:, :kmax]
    valid = torch.arange(kmax, device=maskb.device)[None, :] < counts[:, None]
    return order, valid, kmax, kmax == kmin


def naive_gemm_m(A, B, mask):
    """M axis (mask [M, 1]): gather the active rows of A, dense GEMM, scatter."""
    M, N, K, _ = _check(A, B, mask, B.shape[0], "n")
    rows = torch.nonzero(mask[:, 0] != 0).squeeze(1)  # device-to-host sync on its size
    C = torch.zeros((M, N), dtype=A.dtype, device=A.device)
    if rows.numel():
        C[rows] = A[rows] @ B.t()
    return C


def naive_gemm_mn(A, B, mask, G: int):
    """N axis: every token's active rows of B are materialized ([M, k G, K],
    the token-specific weight subsets), one batched GEMV per token, scatter."""
    M, N, K, ng = _check(A, B, mask, G, "n")
    C = torch.zeros((M, N), dtype=A.dtype, device=A.device)
    if M == 0:
        return C
    order, valid, kmax, uniform = _per_token_slots(mask != 0)
    if kmax == 0:
        return C
    Bs = B.view(ng, G, K)[order].view(M, kmax * G, K)  # gather: pMNK read + pMNK written
    out = torch.bmm(Bs, A.unsqueeze(2).contiguous()).view(M, kmax, G)  # pMNK + MK read, pMN written
    if not uniform:  # padded slots hold inactive groups: their C stays +0.0
        out = torch.where(valid[:, :, None], out, torch.zeros((), dtype=out.dtype, device=out.device))
    C.view(M, ng, G).scatter_(1, order[:, :, None].expand(M, kmax, G), out)  # pMN read + written
    return C


def naive_gemm_k(A, B, mask, G: int):
    """K axis: every token's active channels of A ([M, k G]) and the matching
    columns of B ([M, k G, N], the token-specific weight subsets) are
    materialized, one batched GEMV per token gives C directly."""
    M, N, K, ng = _check(A, B, mask, G, "k")
    C = torch.zeros((M, N), dtype=A.dtype, device=A.device)
    if M == 0:
        return C
    order, valid, kmax, _ = _per_token_slots(mask != 0)
    if kmax == 0:
        return C
    As = torch.gather(A.view(M, ng, G), 1, order[:, :, None].expand(M, kmax, G))  # pMK + pMK
    # A's values at skipped pairs never count (also when they are not finite)
    As = torch.where(valid[:, :, None], As, torch.zeros((), dtype=As.dtype, device=As.device))
    Bt = B.t().contiguous().view(ng, G, N)  # weight layout [K, N] (not counted in Table 4)
    Bs = Bt[order].view(M, kmax * G, N)  # gather: pMNK read + pMNK written
    return torch.bmm(As.view(M, 1, kmax * G), Bs).view(M, N)  # pMNK + pMK read, MN written


def _grouped_mm(a_cat, b3, offs):
    return torch._grouped_mm(a_cat, b3, offs=offs)


def _group_prefixes(maskb):
    """Per group, its active tokens in ascending order (a stable partition of
    the column); returns the concatenated token list and per-group counts."""
    M, ng = maskb.shape
    order = torch.argsort((~maskb).to(torch.int8).t(), dim=1, stable=True)  # [ng, M]
    counts = maskb.sum(dim=0)
    counts_h = counts.tolist()  # device-to-host sync: the GEMM sizes
    toks = torch.cat([order[g, :c] for g, c in enumerate(counts_h)]) if M else order.flatten()
    return toks, counts, counts_h


def grouped_gemm_mn(A, B, mask, G: int, use_grouped_mm: bool = True):
    """N axis on reordered masks: for every group, its active tokens' rows of A
    are gathered and multiplied by the group's G rows of B in one GEMM (one
    grouped-GEMM call with per-group offsets where the library has it, else one
    GEMM per group); the results are scattered into C."""
    M, N, K, ng = _check(A, B, mask, G, "n")
    C = torch.zeros((M, N), dtype=A.dtype, device=A.device)
    if M == 0:
        return C
    toks, counts, counts_h = _group_prefixes(mask != 0)
    if toks.numel() == 0:
        return C
    Ag = A[toks]  # [sum of counts, K]
    gid = torch.repeat_interleave(torch.arange(ng, device=A.device), counts)
    if use_grouped_mm:
        offs = torch.cumsum(counts, 0).to(torch.int32)
        out = _grouped_mm(Ag, B.view(ng, G, K).transpose(1, 2), offs)  # [sum, G]
    else:
        parts, s = [], 0
        Bg = B.view(ng, G, K)
        for g, c in enumerate(counts_h):
            parts.append(Ag[s:s + c] @ Bg[g].t())
            s += c
        out = torch.cat(parts)
    C.view(M, ng, G)[toks, gid] = out
    return C


def grouped_gemm_k(A, B, mask, G: int, use_grouped_mm: bool = True):
    """K axis on reordered masks: for every group, its active tokens' G channels
    of A times the group's G columns of B give partial rows of C, summed in
    fp32 into the tokens' rows."""
    M, N, K, ng = _check(A, B, mask, G, "k")
    if M == 0:
        return torch.zeros((M, N), dtype=A.dtype, device=A.device)
    toks, counts, counts_h = _group_prefixes(mask != 0)
    acc = torch.zeros((M, N), dtype=torch.float32, device=A.device)
    if toks.numel() == 0:
        return acc.to(A.dtype)
    gid = torch.repeat_interleave(torch.arange(ng, device=A.device), counts)
    Ag = A.view(M, ng, G)[toks, gid]  # [sum of counts, G]
    if use_grouped_mm:
        offs = torch.cumsum(counts, 0).to(torch.int32)
        Bk = B.view(N, ng, G).permute(1, 2, 0)  # [ng, G, N]
        out = _grouped_mm(Ag, Bk, offs)  # [sum, N]
    else:
        parts, s = [], 0
        Bv = B.view(N, ng, G)
        for g, c in enumerate(counts_h):
            parts.append(Ag[s:s + c] @ Bv[:, g, :].t())
            s += c
        out = torch.cat(parts)
    acc.index_add_(0, toks, out.float())
    return acc.to(A.dtype)


def traffic_elements(axis: str, M: int, N: int, K: int, p: float) -> float:
    """Table 4's data-tensor traffic of the naive pipelines, in elements."""
    if axis == "m":
        return 3 * p * M * K + N * K + 3 * p * M * N + M * N
    if axis == "n":
        return M * K + 3 * p * M * N * K + 3 * p * M * N + M * N
    if axis == "k":
        return 3 * p * M * K + 3 * p * M * N * K + M * N
    raise ValueError(axis)


def materialized_elements(axis: str, M: int, N: int, K: int, p: float) -> float:
    """Intermediate storage the naive pipelines materialize (outputs excluded)."""
    if axis == "m":
        return p * M * K + p * M * N  # gathered rows of A and their products
    if axis == "n":
        return p * M * N * K + p * M * N  # token-specific rows of B, per-token products
    if axis == "k":
        return p * M * K + p * M * N * K  # token-specific channels of A and columns of B
    raise ValueError(axis)
