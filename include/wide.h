/*
 * wide.h - C ABI of libwide.so, a group-sparse (token-wise dynamic-width)
 * SwiGLU FFN for AMD Instinct MI355X (gfx950).
 *
 * The method: WIDE ("Boosting Adaptive LLM Inference via Token-level Dynamic
 * Width Pruning"). The FFN intermediate dimension d_ff is cut into contiguous
 * groups of G channels and every token keeps or skips each group; one mask
 * matrix covers the whole FFN layer (ai.info summary, "Methodology in Plain
 * English"; WIDE paper, Sec. 3.1 "Preliminaries"). Skipped groups are turned
 * into skipped work in the gate/up projection (N axis, App. B
 * "Implementation of GEMM-MN") and in the down projection (K axis, App. B
 * "Implementation of GEMM-K").
 *
 * Computed definition, for token t, channel c in group g = c / G:
 *   H[t,c] = silu(X[t,:] . Wgate[c,:]) * (X[t,:] . Wup[c,:])  if mask[t,g] != 0
 *   H[t,c] = 0                                                otherwise
 *   Y[t,n] = sum_c Wdown[n,c] * H[t,c]            silu(a) = a / (1 + exp(-a))
 *
 * Conventions shared by every entry point:
 *   - All array arguments are DEVICE pointers (hipMalloc'd or equivalent),
 *     row-major and contiguous, 16-byte aligned. The caller owns every
 *     buffer; the library never allocates, frees or synchronises.
 *   - `stream` is a hipStream_t (NULL = the null stream). All work is
 *     enqueued on it and the call returns before the work completes. No
 *     call reads device memory on the host or decides anything from mask
 *     contents on the host, so every call can be captured in a hipGraph.
 *   - Arguments are validated on the host before anything is enqueued. A
 *     failed check returns a status code and enqueues nothing; the message is
 *     kept per host thread and returned by wide_last_error(). A failed launch
 *     returns WIDE_ERR_HIP. No C++ exception crosses the ABI.
 *   - Masks are uint8 [T, ngroups], nonzero = the token executes the group.
 *     (The pages' router emits class 0 = execute; whoever builds the mask
 *     inverts that.)
 */
#ifndef WIDE_H
#define WIDE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WIDE_OK = 0,
  WIDE_ERR_NULL = 1,        /* a required pointer is NULL */
  WIDE_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  WIDE_ERR_DTYPE = 3,       /* unknown dtype */
  WIDE_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  WIDE_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than wide_ffn_workspace_size() */
  WIDE_ERR_UNSUPPORTED = 6, /* valid for the definition but not for these kernels */
  WIDE_ERR_HIP = 7          /* a HIP launch failed (detail in wide_last_error()) */
} wide_status_t;

typedef enum {
  WIDE_F32 = 0,  /* X, W*, H and Y are float32; fp32 arithmetic throughout */
  WIDE_BF16 = 1  /* X, W*, H and Y are bfloat16; fp32 accumulation, H and Y rounded once (RNE) */
} wide_dtype_t;

/* Token tile of the gate/up kernel: the tile that wide_ffn_forward's reorder
 * aligns the per-group counts to. */
#define WIDE_TOKEN_TILE 256

/* Largest token count the bf16 decode kernels take in one pass. */
#define WIDE_DECODE_T_LIMIT 16

/* Flags for wide_ffn_forward / wide_ffn_stage. */
#define WIDE_FLAG_FORCE_PREFILL 0x1u /* never take the decode path */
#define WIDE_FLAG_FORCE_DECODE 0x2u  /* take the decode path (needs bf16 and T <= 16) */

/*
 * wide_reorder_masks - per-group stable partition of the mask columns.
 *
 * For every group g the tokens are reordered so that the active ones form a
 * contiguous prefix (ai.info summary, "How the speedups are obtained": sorting
 * each routing column gives a contiguous active prefix with at most one
 * boundary tile per group; WIDE paper Sec. 1, "tile-aligned prefixes").
 * The order is stable: perm[g, 0:counts[g]] lists the active tokens in
 * ascending order, perm[g, counts[g]:T] the inactive ones in ascending order.
 *
 *   mask    [T, ngroups] uint8, device, read only.
 *   perm    [ngroups, T] int32, device, written (a permutation of 0..T-1 per row).
 *   counts  [ngroups] int32, device, written: active tokens per group.
 *   padded  [ngroups] int32, device, written: ceil(counts[g] / tile) * tile
 *           (0 when counts[g] == 0; may exceed T, so consumers bound rows by counts).
 *   T >= 0, ngroups >= 1, tile >= 1. T == 0 enqueues only the counts/padded
 *   writes, and mask and perm may then be NULL.
 * Errors: WIDE_ERR_NULL, WIDE_ERR_SHAPE, WIDE_ERR_HIP.
 */
wide_status_t wide_reorder_masks(const uint8_t* mask, int32_t T, int32_t ngroups, int32_t tile,
                                 int32_t* perm, int32_t* counts, int32_t* padded, void* stream);

/*
 * wide_ffn_workspace_size - bytes of device workspace wide_ffn_forward needs
 * for a call without H_out: the per-group permutations, counts, packed mask
 * bits, the decode path's partial sums (T <= WIDE_DECODE_T_LIMIT) and the
 * intermediate H [T, d_ff]. Returns 0 for invalid sizes.
 *
 * wide_ffn_workspace_size_for - the same for a call that passes H_out
 * (h_out_given != 0) or not (h_out_given == 0). With H_out the workspace
 * holds no H (at T = 16384, d_ff = 14336 in bf16 that is 470 MB less).
 * wide_ffn_forward, wide_ffn_stage and wide_ffn_decode_prepared check the
 * workspace against the size that matches the H_out they receive.
 */
size_t wide_ffn_workspace_size(int32_t T, int32_t d, int32_t d_ff, int32_t G, wide_dtype_t dtype);
size_t wide_ffn_workspace_size_for(int32_t T, int32_t d, int32_t d_ff, int32_t G,
                                   wide_dtype_t dtype, int32_t h_out_given);

/*
 * wide_ffn_forward - the masked SwiGLU FFN defined at the top of this file.
 *
 *   X      [T, d]      device, dtype, read only.
 *   Wgate  [d_ff, d]   device, dtype, read only ([out, in], as nn.Linear).
 *   Wup    [d_ff, d]   device, dtype, read only.
 *   Wdown  [d, d_ff]   device, dtype, read only.
 *   mask   [T, d_ff/G] device, uint8, read only.
 *   Y      [T, d]      device, dtype, written. Rows of tokens with no active
 *                      group are exactly +0.0.
 *   H_out  [T, d_ff]   device, dtype, optional (NULL = keep H in the workspace).
 *                      When given, it receives H with exact +0.0 at every
 *                      masked channel.
 *   workspace          device, >= wide_ffn_workspace_size_for(..., H_out != NULL)
 *                      bytes, 256-byte aligned; contents on entry are ignored.
 *   flags              WIDE_FLAG_* (0 = choose the path from T).
 *
 * Prefill path (T > wide_decode_max_t(), or WIDE_FLAG_FORCE_PREFILL): mask
 * reorder, then the gate/up kernel over each group's active prefix (tiles past
 * the prefix do no MFMA work, rows past it are not fetched, fragments past it
 * are not multiplied; SiLU(gate)*up fused in the epilogue and scattered to H
 * for the active (token, group) pairs only, plus +0.0 at the others when
 * H_out is given), then the down kernel, which owns each [token tile x output
 * tile] of Y, accumulates over the channels in registers, skips every
 * 64-channel K-block whose groups are inactive for the whole token tile and
 * never reads H at an inactive (token, group) (WIDE paper App. B, GEMM-MN
 * and GEMM-K).
 * Decode path (bf16, T <= wide_decode_max_t()): no reorder (WIDE paper App. B:
 * the T_q = 1 case checks routing directly); a gate/up GEMV and a down GEMV
 * that stream only the weight rows/segments of groups active for some token.
 *
 * Sizes: T >= 0 (T == 0 enqueues nothing; X, mask and Y may then be NULL);
 * d, d_ff, G >= 1 with d_ff % G == 0. The kernels also need d % 64 == 0,
 * d_ff % 64 == 0, G % 16 == 0, d_ff <= 65536 and T*d, T*d_ff, d*d_ff < 2^30
 * (each operand within 2^31 bytes), else WIDE_ERR_UNSUPPORTED.
 * bf16 results differ from exact arithmetic by fp32 accumulation and the two
 * roundings; the reduction order is fixed, so a call is deterministic.
 * Errors: WIDE_ERR_NULL, WIDE_ERR_SHAPE, WIDE_ERR_DTYPE, WIDE_ERR_ALIGN,
 * WIDE_ERR_WORKSPACE, WIDE_ERR_UNSUPPORTED, WIDE_ERR_HIP.
 */
wide_status_t wide_ffn_forward(const void* X, const void* Wgate, const void* Wup, const void* Wdown,
                               const uint8_t* mask, int32_t T, int32_t d, int32_t d_ff, int32_t G,
                               wide_dtype_t dtype, void* Y, void* H_out, void* workspace,
                               size_t workspace_bytes, uint32_t flags, void* stream);

/*
 * wide_ffn_forward_noalloc - wide_ffn_forward for callers that cannot
 * allocate device memory: code under hipGraph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments, kernels and results (bit
 * for bit) as wide_ffn_forward, without the workspace: the library keeps its
 * workspace in a static device array of WIDE_NOALLOC_SCRATCH_BYTES on each GPU
 * (placed when the library is loaded on that GPU, held until the process
 * ends). The call allocates and frees nothing.
 *   H_out  required (non-NULL when T > 0): the array does not hold H.
 *   Limit: wide_ffn_workspace_size_for(T, d, d_ff, G, dtype, 1) must not
 *          exceed WIDE_NOALLOC_SCRATCH_BYTES, else WIDE_ERR_WORKSPACE and
 *          nothing is enqueued. 64 MiB of the array cover the largest
 *          partial sums of the prefill down projection's split last round;
 *          the rest holds T * ngroups up to about 7.9 million at d <= 16384.
 *   The array is shared by every call on one GPU and keeps the last call's
 *   contents (nothing in it needs to start at zero: every call writes what it
 *   reads). Calls that overlap on one GPU (different streams, or host
 *   threads racing) race on it: serialise them.
 * The first call on a GPU looks up the array's device address
 * (hipGetSymbolAddress) and keeps it. Errors: as wide_ffn_forward, plus
 * WIDE_ERR_HIP when the device or the address cannot be obtained.
 */
#define WIDE_NOALLOC_SCRATCH_BYTES (96u << 20)
wide_status_t wide_ffn_forward_noalloc(const void* X, const void* Wgate, const void* Wup,
                                       const void* Wdown, const uint8_t* mask, int32_t T,
                                       int32_t d, int32_t d_ff, int32_t G, wide_dtype_t dtype,
                                       void* Y, void* H_out, uint32_t flags, void* stream);

/* Stages of wide_ffn_forward, for callers that time or interleave them. */
typedef enum {
  WIDE_STAGE_REORDER = 0,   /* prefill: mask reorder into the workspace */
  WIDE_STAGE_GATE_UP = 1,   /* prefill: gate/up kernel -> H */
  WIDE_STAGE_DOWN = 2,      /* prefill: down kernel -> Y */
  WIDE_STAGE_DECODE_GATE_UP = 3, /* decode: gate/up GEMV -> H */
  WIDE_STAGE_DECODE_DOWN = 4     /* decode: down GEMV -> Y */
} wide_stage_t;

/*
 * wide_ffn_stage - enqueue one stage of wide_ffn_forward with the same
 * arguments. Running the prefill stages 0,1,2 (or the decode stages 3,4) in
 * order on one stream with one workspace is exactly wide_ffn_forward on that
 * path; the path must be the one wide_ffn_forward would take for these
 * arguments and flags (else WIDE_ERR_UNSUPPORTED). A stage reads what the
 * previous stages left in the workspace (and in H_out when given).
 */
wide_status_t wide_ffn_stage(wide_stage_t stage, const void* X, const void* Wgate, const void* Wup,
                             const void* Wdown, const uint8_t* mask, int32_t T, int32_t d,
                             int32_t d_ff, int32_t G, wide_dtype_t dtype, void* Y, void* H_out,
                             void* workspace, size_t workspace_bytes, uint32_t flags, void* stream);

/*
 * Decode with operand-order weights (bf16). The decode GEMV kernels that run
 * on the matrix cores (T > 2, or shapes the whole-row kernels do not take)
 * load their weight operands as 16 rows x 32 columns; in the nn.Linear
 * layout that is 16 separate 64-byte pieces per load. A copy of the weights
 * in operand order makes each such load one contiguous 1 KB block. (The
 * pages give decoding its own fast path and GEMV variants for small M: WIDE
 * paper Sec. 1 and App. B, GEMM-MN / GEMM-K; the layout is chosen here for
 * the gfx950 MFMA operand shape.)
 *
 * wide_decode_weights_size - bytes of the copy for [d_ff, d] Wgate and Wup and
 *   [d, d_ff] Wdown: three regions of d * d_ff bf16, each 256-byte aligned.
 *   Returns 0 unless d and d_ff are multiples of 64 and d * d_ff < 2^30.
 *
 * wide_decode_prepare_weights - writes the copy (device, caller-owned,
 *   256-byte aligned, >= wide_decode_weights_size bytes) from the nn.Linear
 *   weights on `stream`. Region r holds matrix r (Wgate, Wup, Wdown) of R rows
 *   and C columns as 1 KB blocks ordered by 16-row block, then by 32-column
 *   slice; within block (rb, kc) lane l's 16 bytes (at byte 16 l) are row
 *   16 rb + l % 16, columns 32 kc + 8 (l / 16) .. + 7. A pure permutation: no
 *   value changes. Run it again whenever the weights change.
 *
 * wide_ffn_decode_prepared - wide_ffn_forward forced onto the decode path
 *   (bf16, 0 <= T <= 16; same arguments, workspace and results, bit for bit),
 *   with the matrix-core kernels reading `prepared` instead of Wgate, Wup and
 *   Wdown. The whole-row kernels (T <= 2 at shapes they take) still read the
 *   nn.Linear weights, so both must be passed. `prepared_bytes` is the size
 *   of `prepared`. Errors as wide_ffn_forward, plus WIDE_ERR_NULL /
 *   WIDE_ERR_ALIGN for `prepared` and WIDE_ERR_WORKSPACE when it is smaller
 *   than wide_decode_weights_size(d, d_ff).
 */
size_t wide_decode_weights_size(int32_t d, int32_t d_ff);
wide_status_t wide_decode_prepare_weights(const void* Wgate, const void* Wup, const void* Wdown,
                                          int32_t d, int32_t d_ff, void* prepared,
                                          size_t prepared_bytes, void* stream);
wide_status_t wide_ffn_decode_prepared(const void* X, const void* Wgate, const void* Wup,
                                       const void* Wdown, const void* prepared,
                                       size_t prepared_bytes, const uint8_t* mask, int32_t T,
                                       int32_t d, int32_t d_ff,
                                       int32_t G, void* Y, void* H_out, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * The two group-masked GEMM families the FFN kernels are built from, exposed
 * on their own (WIDE paper App. B, "Implementation of GEMM-MN" and
 * "Implementation of GEMM-K"). C = A B^T with A [M, K] and B [N, K]; a mask
 * uint8 [M, ngroups] (nonzero = active) routes each row of A over groups of G
 * consecutive indices of one axis:
 *
 *   wide_gemm_mn (N axis; ngroups = N / G):
 *     C[m,n] = A[m,:] . B[n,:]   if mask[m, n / G] != 0,   else C[m,n] = +0.0
 *     The N-axis path covers an attention W_q projection (groups of query
 *     heads) and the FFN gate/up; with G = N (ngroups = 1) it is the M-axis
 *     case, dynamic depth: a row with mask 0 gets an all-zero output row.
 *   wide_gemm_k (K axis; ngroups = K / G):
 *     C[m,n] = sum_k [mask[m, k / G] != 0] A[m,k] B[n,k]
 *     The K-axis path covers an attention W_o projection (groups of heads in
 *     its input) and the FFN down projection. A's values at inactive
 *     (row, group) pairs are never read: they may hold anything, NaN included.
 *
 * Both run bf16 operands with fp32 accumulation over the full K range in a
 * fixed order (one writer per output, no atomics) and round C once (RNE).
 * wide_gemm_mn reorders the mask columns on the device (as
 * wide_reorder_masks) and runs one workgroup per (G-aligned channel block,
 * 256-row tile of the group's active prefix); wide_gemm_k packs the mask into
 * bits on the device and runs one workgroup per 256 x 256 output tile,
 * skipping every 64-wide K-block inactive for all its rows.
 *
 *   A        [M, K]  device, bf16, read only.
 *   B        [N, K]  device, bf16, read only ([out, in], as nn.Linear).
 *   mask     [M, ngroups] device, uint8, read only.
 *   C        [M, N]  device, bf16, written in full (every element).
 *   workspace        device, >= wide_gemm_workspace_size(M, ngroups) bytes,
 *                    256-byte aligned; contents on entry are ignored.
 *   dtype            WIDE_BF16 (WIDE_F32 returns WIDE_ERR_UNSUPPORTED).
 * Sizes: M >= 0 (M == 0 enqueues nothing; A, mask and C may then be NULL),
 * N, K, G >= 1, G divides the routed axis (N for wide_gemm_mn, K for
 * wide_gemm_k). The kernels also need K % 64 == 0, G % 16 == 0, N % 8 == 0,
 * K <= 65536 and M*K, N*K, M*N < 2^30, else WIDE_ERR_UNSUPPORTED.
 * Errors: WIDE_ERR_NULL, WIDE_ERR_SHAPE, WIDE_ERR_DTYPE, WIDE_ERR_ALIGN,
 * WIDE_ERR_WORKSPACE, WIDE_ERR_UNSUPPORTED, WIDE_ERR_HIP.
 */
size_t wide_gemm_workspace_size(int32_t M, int32_t ngroups);

wide_status_t wide_gemm_mn(const void* A, const void* B, const uint8_t* mask, int32_t M, int32_t N,
                           int32_t K, int32_t G, wide_dtype_t dtype, void* C, void* workspace,
                           size_t workspace_bytes, void* stream);

wide_status_t wide_gemm_k(const void* A, const void* B, const uint8_t* mask, int32_t M, int32_t N,
                          int32_t K, int32_t G, wide_dtype_t dtype, void* C, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * wide_router_forward - the bottleneck router that produces the group mask
 * (ai.info summary, "How decisions are made": input activations -> N_G
 * two-way decisions per token through an inner dimension r, typically 16 or
 * 32; argmax at inference; class 0 = execute, class 1 = skip). The paper's
 * Sec. 3.1 "Routing Components" prints no formula; the readings taken are no
 * biases, an activation chosen by the caller, logits [T, N_G, 2] with the
 * class fastest, and a tie going to class 0 (the first maximum):
 *   z[t,j]       = act( X[t,:] . W1[j,:] )          j < r
 *   logit[t,g,c] = W2[2g + c, :] . z[t,:]             c in {0, 1}
 *   mask[t,g]    = 1 if logit[t,g,0] >= logit[t,g,1] else 0
 * The mask is exactly what wide_ffn_forward, wide_gemm_mn and wide_gemm_k take.
 *
 *   X       [T, D]          device, bf16, read only (the FFN's input for an FFN router).
 *   W1      [r, D]          device, bf16, read only.
 *   W2      [2*ngroups, r]  device, bf16, read only (row 2g + c: class c of group g).
 *   act     WIDE_ACT_*.
 *   mask    [T, ngroups]    device, uint8, written.
 *   logits  [T, ngroups, 2] device, fp32, written when non-NULL.
 *   workspace  device scratch of wide_router_workspace_size(T, r) bytes,
 *              256-byte aligned, contents on entry ignored, owned by the
 *              caller; may be NULL when that size is 0 (T > 16 or T == 0).
 *              For 1 <= T <= 16 it holds the first map's partial sums: that
 *              map is split over D into 8 workgroups, so that W1 streams
 *              through 8 CUs instead of one.
 * z and the logits are computed in fp32 from bf16 operands (fp32 products and
 * sums, fixed order: the same result every call), and the argmax is taken on
 * those fp32 logits.
 * Sizes: T >= 0 (T == 0 enqueues nothing; X, mask and logits may then be
 * NULL), ngroups >= 1; the kernels need D % 32 == 0, r in {16, 32, 64} and
 * T*D, T*ngroups < 2^31, else WIDE_ERR_UNSUPPORTED. bf16 only.
 * Errors: WIDE_ERR_NULL, WIDE_ERR_SHAPE, WIDE_ERR_DTYPE, WIDE_ERR_ALIGN,
 * WIDE_ERR_WORKSPACE (workspace NULL or smaller than its size while that size
 * is not 0), WIDE_ERR_UNSUPPORTED, WIDE_ERR_HIP.
 */
typedef enum {
  WIDE_ACT_IDENTITY = 0,
  WIDE_ACT_RELU = 1, /* max(a, 0) */
  WIDE_ACT_SILU = 2  /* a / (1 + exp(-a)) */
} wide_act_t;

/* Workspace bytes of wide_router_forward: 8 * 16 * r * 4 for 1 <= T <= 16,
   else 0 (also 0 for T < 0 or r not in {16, 32, 64}). */
size_t wide_router_workspace_size(int32_t T, int32_t r);
wide_status_t wide_router_forward(const void* X, const void* W1, const void* W2, int32_t T,
                                  int32_t D, int32_t r, int32_t ngroups, wide_act_t act,
                                  wide_dtype_t dtype, uint8_t* mask, float* logits,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * wide_router_reorder - the router of wide_router_forward fused with the mask
 * reorder of wide_reorder_masks: from the activations straight to the per-group
 * row lists, with no mask round trip (the pages count router execution and
 * mask reordering in the work that pruning does not accelerate: WIDE paper
 * Sec. 4.2, the layer-time breakdown; ai.info summary, "How decisions are
 * made"). The router kernel packs its decisions into bits [ngroups,
 * ceil(T/32)] in the workspace as it makes them (one ballot per group over
 * each block of 64 tokens), and a partition kernel turns the bits into the
 * stable per-group partition.
 *
 *   X, W1, W2, T, D, r, ngroups, act, dtype: as wide_router_forward.
 *   tile            >= 1: padded[g] = ceil(counts[g] / tile) * tile.
 *   mask            [T, ngroups] uint8, optional (NULL = not written): the
 *                   decisions, as wide_router_forward writes them.
 *   logits          [T, ngroups, 2] fp32, optional, 8-byte aligned.
 *   perm, counts, padded: as wide_reorder_masks (perm may be NULL when T == 0):
 *                   exactly wide_reorder_masks applied to the mask above.
 *   workspace       device, 256-byte aligned, at least
 *                   wide_router_reorder_workspace_size(T, ngroups) bytes
 *                   (the packed bits, and for T <= 16 the first map's
 *                   partial sums as in wide_router_forward).
 * Errors: as wide_router_forward, plus WIDE_ERR_SHAPE (tile < 1),
 * WIDE_ERR_WORKSPACE.
 */
size_t wide_router_reorder_workspace_size(int32_t T, int32_t ngroups);
wide_status_t wide_router_reorder(const void* X, const void* W1, const void* W2, int32_t T,
                                  int32_t D, int32_t r, int32_t ngroups, wide_act_t act,
                                  wide_dtype_t dtype, int32_t tile, uint8_t* mask, float* logits,
                                  int32_t* perm, int32_t* counts, int32_t* padded,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * wide_attention_prefill - head-group-pruned causal attention for one sequence
 * (ai.info summary, "What gets pruned": the attention unit is a GQA-aligned
 * group of H_q/H_k query heads, and each token keeps or skips each group;
 * WIDE paper App. B, "Implementation of Attention": query tiles of one query
 * head are admitted, gathered, run through a dense K/V mainloop with the
 * FlashAttention online softmax, and scattered back). Readings where the text
 * is silent: causal (key j is valid for query t when j <= t), scale
 * 1/sqrt(dh), group g = KV head g = query heads [g*H_q/H_k, (g+1)*H_q/H_k):
 *   for t and query head h with mask[t, g] != 0:
 *     O[t,h,:] = sum_{j<=t} softmax_j(Q[t,h,:].K[j,g,:] / sqrt(dh)) V[j,g,:]
 * The mask is reordered on the device (the per-group stable partition of
 * wide_reorder_masks, tiles of 128 queries); K and V stay dense.
 *
 *   Q     [T, Hq*dh]  device, bf16, read only (the W_q projection's output).
 *   K, V  [T, Hk*dh]  device, bf16, read only.
 *   mask  [T, Hk]     device, uint8, nonzero = the token keeps the head group.
 *   O     [T, Hq*dh]  device, bf16, written at every (t, h) whose group t
 *                     keeps; with WIDE_ATTN_ZERO_INACTIVE also +0.0 at the
 *                     others, else they are left untouched (wide_gemm_k with
 *                     G = (Hq/Hk)*dh never reads them for the W_o projection).
 *   workspace         device, 256-byte aligned, at least
 *                     wide_attention_workspace_size(T, Hk, dh) bytes; holds the
 *                     reorder and a transposed copy of V. Overwritten; the
 *                     caller owns it.
 * P is rounded to bf16 before the P.V product (fp32 accumulation, fp32
 * softmax statistics); O is rounded once to bf16.
 * Sizes: T >= 0 (T == 0 enqueues nothing), Hk >= 1, Hq a multiple of Hk; the
 * kernel needs dh == 128 and T*Hq*dh < 2^31, else WIDE_ERR_UNSUPPORTED. bf16
 * only. Q, K, V and O 16-byte aligned. Asynchronous on `stream`; nothing is
 * allocated and the host never waits, so the call can be captured in a graph.
 * Errors: WIDE_ERR_NULL, WIDE_ERR_SHAPE, WIDE_ERR_DTYPE, WIDE_ERR_ALIGN,
 * WIDE_ERR_WORKSPACE, WIDE_ERR_UNSUPPORTED, WIDE_ERR_HIP.
 */
#define WIDE_ATTN_ZERO_INACTIVE 1u

size_t wide_attention_workspace_size(int32_t T, int32_t Hk, int32_t dh);

wide_status_t wide_attention_prefill(const void* Q, const void* K, const void* V,
                                     const uint8_t* mask, int32_t T, int32_t Hq, int32_t Hk,
                                     int32_t dh, wide_dtype_t dtype, void* O, uint32_t flags,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * wide_attention_decode - one decoding step of the head-group-pruned attention
 * (WIDE paper App. B, "Implementation of Attention": for decoding the routing
 * is checked directly, without mask reordering, and the softmax is split over
 * the keys): the new token's query at position T - 1 attends to the T cached
 * keys 0..T-1 (its own included), the definition of wide_attention_prefill at
 * query row T - 1:
 *   for query head h with mask[g] != 0, g = h / (Hq/Hk):
 *     O[h,:] = sum_{j<T} softmax_j(q[h,:].K[j,g,:] / sqrt(dh)) V[j,g,:]
 * A group the token skips costs nothing: its K/V rows are never read.
 *
 *   q     [Hq*dh]     device, bf16, read only.
 *   K, V  [T, Hk*dh]  device, bf16, read only (the cache, new token included).
 *   mask  [Hk]        device, uint8, nonzero = the token keeps the head group.
 *   O     [Hq*dh]     device, bf16, written at kept heads (and +0.0 at the
 *                     others with WIDE_ATTN_ZERO_INACTIVE, else untouched).
 *   workspace         device, 256-byte aligned, at least
 *                     wide_attention_decode_workspace_size(T, Hq, dh) bytes:
 *                     the fp32 partials of the key splits.
 * fp32 scores, softmax statistics and sums from bf16 operands; O rounded once.
 * Sizes: T >= 1, Hk >= 1, Hq a multiple of Hk; the kernel needs dh == 128 and
 * Hq/Hk in {1, 2, 4, 8}, else WIDE_ERR_UNSUPPORTED. bf16 only; q, K, V, O
 * 16-byte aligned. Asynchronous, allocation-free, capturable in a graph.
 * Errors: as wide_attention_prefill.
 */
size_t wide_attention_decode_workspace_size(int32_t T, int32_t Hq, int32_t dh);

wide_status_t wide_attention_decode(const void* q, const void* K, const void* V,
                                    const uint8_t* mask, int32_t T, int32_t Hq, int32_t Hk,
                                    int32_t dh, wide_dtype_t dtype, void* O, uint32_t flags,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code. */
const char* wide_status_string(wide_status_t status);

/* Detail of the last failure on the calling host thread ("" if none). */
const char* wide_last_error(void);

/* Largest T that takes the decode path (WIDE_DECODE_T_LIMIT unless the
 * environment variable WIDE_DECODE_MAX_T, read once, sets 0..16). */
int32_t wide_decode_max_t(void);

#ifdef __cplusplus
}
#endif

#endif /* WIDE_H */
