// Internal declarations shared by the HIP translation units of libwide.so:
// device helpers (bf16 rounding, silu, MFMA operand types, LDS swizzle) and
// the host-side launchers that wide_api.cpp calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wide {

// ---------------------------------------------------------------- device helpers

// s_waitcnt immediate that waits only for the vector-memory counter to reach n.
#define WIDE_VMCNT(n) ((((n) & 15)) | ((((n) >> 4) & 3) << 14) | (7 << 4) | (15 << 8))

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even float -> bfloat16 bits (quiet NaN kept a NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// silu(a) * b with the hardware exp2 and reciprocal (v_exp_f32, v_rcp_f32).
// For a -> -inf, exp2 overflows to +inf and the reciprocal gives 0, so the
// result is a signed zero, never NaN.
__device__ __forceinline__ float silu_mul(float a, float b) {
  const float e = __builtin_amdgcn_exp2f(-a * 1.4426950408889634f);
  return a * __builtin_amdgcn_rcpf(1.0f + e) * b;
}

// Pack two floats into two bf16 in one 32-bit word (low = first): one
// v_cvt_pk_bf16_f32 (round to nearest even, NaN stays NaN). The bit-level
// f32_to_bf16_bits above compiles to a branch per value on its NaN test.
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_v v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v));
}

// Workgroup barrier for LDS hand-offs only: orders this workgroup's LDS
// accesses across the barrier (fences scoped to LDS) without the release
// fence of __syncthreads, which also waits for every outstanding global
// store to complete.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// LDS tiles hold rows of 64 bf16 (128 bytes = 8 chunks of 16 bytes). Chunk c
// of row r is stored at chunk position c ^ (r & 7): eight consecutive rows
// reading the same logical chunk then hit eight different 16-byte bank groups.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

}  // namespace wide

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; none allocates or synchronises.

namespace wide {

// Mask reorder (+ optional packed mask bits [ngroups, ceil(T/32)] uint32).
hipError_t launch_reorder(const uint8_t* mask, int T, int ng, int tile, int32_t* perm,
                          int32_t* counts, int32_t* padded, uint32_t* maskbits,
                          hipStream_t stream);

// The same reorder from packed mask bits (made by launch_pack_mask_bits or by
// the router kernel).
hipError_t launch_reorder_from_bits(const uint32_t* maskbits, int T, int ng, int tile,
                                    int32_t* perm, int32_t* counts, int32_t* padded,
                                    hipStream_t stream);

// Packed mask bits alone: maskbits[g, w] bit b = mask[32w + b, g] != 0.
hipError_t launch_pack_mask_bits(const uint8_t* mask, int T, int ng, uint32_t* maskbits,
                                 hipStream_t stream);

// Keys of the transposed V copy per KV head (T rounded up to the key tile;
// 64-bit so that a size query with any int32 T cannot overflow).
int64_t attention_tpad(int64_t T);

// Head-group-pruned causal attention, prefill (dh = 128): V is transposed into
// Vt [Hk, dh, attention_tpad(T)], then one workgroup per (query tile of the
// group's reordered tokens, query head). perm/counts: the reorder of the
// [T, Hk] mask with tiles of 128.
hipError_t launch_attention_prefill_bf16(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                                         const int32_t* perm, const int32_t* counts, int T, int Hq,
                                         int Hk, int dh, uint16_t* O, bool zero_inactive,
                                         uint16_t* Vt, hipStream_t stream);

// One decoding step of the head-group-pruned attention (dh = 128, Hq/Hk in
// {1, 2, 4, 8}): per (128-key split, kept KV group) fp32 partials into `part`
// (attention_decode_part_floats(T, Hq) floats), then a per-head merge.
int64_t attention_decode_splits(int64_t T);
size_t attention_decode_part_floats(int64_t T, int64_t Hq);
hipError_t launch_attention_decode_bf16(const uint16_t* q, const uint16_t* K, const uint16_t* V,
                                        const uint8_t* mask, int T, int Hq, int Hk, int dh,
                                        uint16_t* O, bool zero_inactive, float* part,
                                        hipStream_t stream);

// Largest group count for which the bf16 down kernel keeps the token tile's
// mask bits in an LDS table (beyond it, it reads them from global memory).
constexpr int kDownMaxGroups = 768;

// Whether the bf16 prefill gate/up runs dense-masked: groups narrower than
// 64 channels (G % 64 != 0) with d_ff a multiple of 128. Measured at the
// Llama3.2-3B shape, T = 8192, 50% masks: the per-group tiles at G = 16 and
// 32 made the FFN 0.52x and 0.75x as fast as the dense one. The reorder then
// only packs the mask bits (no row lists are read).
inline bool gate_up_dense(int G, int d_ff) { return G % 64 != 0 && d_ff % 128 == 0; }

// bf16 prefill gate/up over the reordered tokens (tile = 256 tokens). Writes
// H[t, c] for every active (token, group); with zero_inactive it also writes
// +0.0 at every (token, channel) whose group the token skips. In the
// dense-masked form (gate_up_dense) it reads maskbits [ngroups, ceil(T/32)]
// instead of the row lists and writes every (token, channel), +0.0 at
// skipped pairs.
hipError_t launch_gate_up_bf16(const uint16_t* X, const uint16_t* Wg, const uint16_t* Wu,
                               const int32_t* perm, const int32_t* counts,
                               const uint32_t* maskbits, int T, int d, int d_ff, int G,
                               uint16_t* H, bool zero_inactive, hipStream_t stream);

// bf16 N-axis masked GEMM over reordered rows: C[m, n] = A[m] . B[n] where
// row m takes group n / G, else +0.0 (every element of C is written).
hipError_t launch_gemm_mn_bf16(const uint16_t* A, const uint16_t* B, const int32_t* perm,
                               const int32_t* counts, int M, int K, int N, int G, uint16_t* C,
                               hipStream_t stream);

// Tile edge of the prefill down projection: 256 x 256 tiles unless fewer
// than 128 of them would leave most of the 256 CUs idle; then 128 x 128
// tiles run four times as many workgroups. Measured at 50% masks: 2048^3
// 60 -> 41 us with 128-tiles (64 large tiles), but 4096^3 127 -> 183 us (256
// large tiles) and 384 / 320 large tiles (Llama3.2-3B T = 8192, Qwen3-14B
// T = 4096) slower by 0.1 ms.
inline int down_tile(int T, int d) {
  const long long t256 = (((long long)T + 255) / 256) * (((long long)d + 255) / 256);
  return t256 < 128 ? 128 : 256;
}

// The last round of 256 x 256 down tiles: with nt tiles on kDownRoundCUs CUs
// the nrem = nt % kDownRoundCUs tiles of the last round are split nsplit
// ways along their live K-blocks (nsplit = 1: no split). A function of the
// shape only (the CU count of MI355X is a constant here), so the workspace
// size and the launch always agree.
constexpr int kDownRoundCUs = 256;
constexpr int kDownMaxSplit = 8;
struct DownSplit {
  int nrem, nsplit;
};
inline DownSplit down_split(int T, int d, int d_ff) {
  DownSplit ds{0, 1};
  if (T <= 0 || down_tile(T, d) != 256) return ds;
  const long long nt = (((long long)T + 255) / 256) * (((long long)d + 255) / 256);
  const int rem = (int)(nt % kDownRoundCUs);
  if (rem == 0) return ds;
  int s = kDownRoundCUs / rem;
  if (s > kDownMaxSplit) s = kDownMaxSplit;
  if (s > (d_ff / 64) / 8) s = (d_ff / 64) / 8;  // at least 8 K-blocks of 64 channels per part
  if (s < 2) return ds;
  ds.nrem = rem;
  ds.nsplit = s;
  return ds;
}
// bytes of the fp32 partial sums of the split tiles (0 without a split)
inline size_t down_split_bytes(int T, int d, int d_ff) {
  const DownSplit ds = down_split(T, d, d_ff);
  return ds.nsplit > 1 ? (size_t)ds.nrem * ds.nsplit * 256 * 256 * 4 : 0;
}

// bf16 prefill down projection, also the K-axis masked GEMM (output-stationary;
// K-blocks inactive for a whole token tile are skipped and the H copies of
// inactive (token, group) pairs read zeros, so H's values there never matter).
// part: down_split_bytes(T, d, d_ff) bytes of workspace for the split
// last-round tiles, or NULL (no split).
hipError_t launch_down_bf16(const uint16_t* H, const uint16_t* Wd, const uint32_t* maskbits, int T,
                            int d, int d_ff, int G, uint16_t* Y, float* part, hipStream_t stream);

// Operand-order copy of a bf16 [rows, cols] matrix (rows % 16 == 0, cols % 32
// == 0): each 16-row x 32-column MFMA operand becomes one contiguous 1 KB
// block (lane l's 16 bytes at byte 16 l: row l % 16, columns 8 (l / 16) ..),
// blocks ordered by 16-row block, then by 32-column slice.
hipError_t launch_decode_pack_bf16(const uint16_t* W, int rows, int cols, uint16_t* out,
                                   hipStream_t stream);

// bf16 decode GEMVs (T <= 16). Wg_op / Wu_op / Wd_op: operand-order copies of
// the weights, or NULL. With them the MFMA kernels (T > 2, or shapes the
// whole-row kernels do not take) read contiguous 1 KB operands; the
// whole-row kernels always read the nn.Linear layout.
hipError_t launch_decode_gate_up_bf16(const uint16_t* X, const uint16_t* Wg, const uint16_t* Wu,
                                      const uint16_t* Wg_op, const uint16_t* Wu_op,
                                      const uint8_t* mask, int T, int d, int d_ff, int G,
                                      uint16_t* H, bool zero_inactive, hipStream_t stream);
// For T > 2 (or shapes the whole-row kernels do not take) the down GEMV is
// split over the live channel chunks: `part` holds kDecodeDownSplit * T * d
// fp32 partial sums (workspace; contents on entry ignored).
constexpr int kDecodeDownSplit = 4;  // measured best of 2, 4, 8 and 16 at the Llama3.1-8B shape, T = 16
hipError_t launch_decode_down_bf16(const uint16_t* H, const uint16_t* Wd, const uint16_t* Wd_op,
                                   const uint8_t* mask, int T, int d, int d_ff, int G, uint16_t* Y,
                                   float* part, hipStream_t stream);

// Bottleneck router: mask[t, g] = argmax over the two logits of group g is
// class 0 (act 0 identity, 1 relu, 2 silu). Each output is optional (NULL =
// not written): mask bytes [T, ng], logits [T, ng, 2], and the decisions packed
// as maskbits [ng, ceil(T/32)] (the layout of launch_pack_mask_bits). For
// 1 <= T <= kRouterSmallT the first map's partial sums go to `zpart`
// (router_zpart_bytes(T, r) bytes of workspace, 16-byte aligned; contents on
// entry ignored); otherwise zpart is not used and may be null.
constexpr int kRouterSmallT = 16;
constexpr int kRouterSlices = 8;  // workgroups (slices of D) of the small-T first map
hipError_t launch_router_bf16(const uint16_t* X, const uint16_t* W1, const uint16_t* W2, int T,
                              int D, int r, int ng, int act, uint8_t* mask, float* logits,
                              uint32_t* maskbits, float* zpart, hipStream_t stream);
inline size_t router_zpart_bytes(int T, int r) {
  return T >= 1 && T <= kRouterSmallT ? (size_t)kRouterSlices * 16 * r * sizeof(float) : 0;
}

// Device address of the no-allocation entry point's scratch array
// (WIDE_NOALLOC_SCRATCH_BYTES, 256-byte aligned) on the device that runs
// `stream` (the current device for the null stream); looked up on the first
// call per device and kept. Allocates nothing.
hipError_t noalloc_scratch(hipStream_t stream, void** out);

// fp32 prefill kernels (VALU, same structure as the bf16 ones).
hipError_t launch_gate_up_f32(const float* X, const float* Wg, const float* Wu,
                              const int32_t* perm, const int32_t* counts, int T, int d, int d_ff,
                              int G, float* H, bool zero_inactive, hipStream_t stream);
hipError_t launch_down_f32(const float* H, const float* Wd, const uint32_t* maskbits, int T, int d,
                           int d_ff, int G, float* Y, hipStream_t stream);

}  // namespace wide
