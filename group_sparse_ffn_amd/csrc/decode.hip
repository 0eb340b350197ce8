// Decode fast path (T <= 16 tokens): no mask reorder; routing is checked
// directly (WIDE paper App. B, "Implementation of Attention": for decoding
// the routing can be checked without reordering; App. B GEMM-MN/GEMM-K:
// GEMV variants for small M; Sec. 1: dedicated fast paths for decoding).
//
// Both kernels are bound by streaming weights from HBM, so they are built for
// balance and memory-level parallelism:
//   * weights are read with 16-byte loads in batches per lane; the next batch
//     is issued before the MFMAs of the current one, so loads stay in flight
//     while the wave computes. The MFMA operand layout reads half of a 128-byte
//     line per load and the other half with the next one, so these loads keep
//     the default cache policy (with the non-temporal hint the second half
//     missed again: the T = 16 gate/up took 63 instead of 58 us); the
//     whole-row kernels below read whole lines and stream them non-temporally;
//   * the tokens sit on the N side of v_mfma_f32_16x16x32_bf16 (tokens past T
//     read as zeros), so the matrix core does the dot products and every
//     weight byte is loaded exactly once per call;
//   * gate/up: the work is cut into units of 8 channels of one group (their
//     8 gate rows and 8 up rows form one 16-row MFMA operand; for T > 4,
//     16 channels with separate gate and up operands that share each
//     activation fragment; where the activations fit in LDS, 32-channel
//     units read them from there, see decode_gate_up_xlds_kernel). Every
//     workgroup lists the groups that some token executes (U) and takes the
//     blockIdx-th unit of U, so the active units are packed onto the first
//     workgroups and spread evenly over the CUs; workgroups past the last
//     unit exit. Four waves split K and meet in LDS.
//     Output: H[t, c] = silu(gate)*up, or +0.0 where token t skips the group.
//   * down: every workgroup lists the 32-channel chunks whose group is in U;
//     a workgroup owns 64 output rows and one of kDecodeDownSplit slices of
//     that list, its four waves take every fourth chunk of the slice, and
//     each H fragment feeds four 16-row blocks of Wdown. Only those segments
//     of each Wdown row are read. The slices' fp32 partial sums are added in
//     a fixed order by a second kernel, which rounds Y once. H is never read
//     at a group no token executes (when G is not a multiple of 32 such a
//     group may share a 32-channel chunk with an executed one): those lanes
//     use zeros.
// For one or two tokens the matrix core gains nothing and its operand layout
// (16 rows x 64 bytes per load) costs HBM efficiency, so a second pair of
// kernels streams whole weight rows with contiguous 1 KB loads and VALU dot
// products (v_dot2_f32_bf16) on a persistent grid (at T = 1 on the
// Llama3.1-8B shape: gate/up 27 -> 21 us, down 17 -> 15 us):
//   * gate/up: every wave takes channels of U in turn and reads its gate and
//     up rows end to end; X sits in LDS;
//   * down: every wave takes output rows in turn; one load covers 16 live
//     32-channel chunks (64 bytes each) of the row; the live part of H is
//     compacted into LDS once per workgroup, with zeros for groups no token
//     executes.
#include "common.h"

namespace wide {

namespace {

constexpr int kUnroll = 8;      // gate/up loads in flight per lane
constexpr int kMaxGroups = 4096;  // d_ff / 16
constexpr int kDecodeSmallT = 4;  // largest T that uses 8-channel gate/up units
constexpr int kValuMaxT = 2;      // largest T of the contiguous VALU kernels
// Channels of compacted H the VALU down kernel holds per token in LDS: one
// token fits four workgroups per CU, two tokens two.
__host__ __device__ constexpr int valu_cap(int nt) { return nt == 1 ? 18432 : 14336; }
constexpr int kValuMaxD = 8192;   // the VALU gate/up holds d / 512 loads per row per lane

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// dot of the eight bf16 held in each of two u32x4, accumulated in fp32 by
// four v_dot2_f32_bf16. (The whole vector is reinterpreted and the pairs are
// built from its elements: a bit cast of one 32-bit element of a u32x4 is
// compiled by this toolchain into a reuse of element 0.)
__device__ __forceinline__ float dot8(const u32x4& a, const u32x4& b, float acc) {
  const bf16x8 av = __builtin_bit_cast(bf16x8, a), bv = __builtin_bit_cast(bf16x8, b);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf16x2 p = {av[2 * e], av[2 * e + 1]}, q = {bv[2 * e], bv[2 * e + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(p, q, acc, false);
  }
  return acc;
}

// Sum over the 64 lanes, left in every lane: four DPP row rotations give
// each 16-lane row its sum, and the four row sums are read lane by lane (no
// LDS-crossbar permutes, which a chain of __shfl_xor compiles to).
__device__ __forceinline__ float wave_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false));
  const int b = __builtin_bit_cast(int, v);
  return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
         (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}

__device__ __forceinline__ u32x4 ld16_nt(const uint16_t* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}
__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *(const u32x4*)p; }

// Lists the items i < nitems with pred(i) into s_list (ascending) and returns
// their number. Every thread of the block must call it.
template <int kThreads, class Pred>
__device__ __forceinline__ int list_where(int nitems, Pred pred, uint16_t* s_list,
                                          int* s_wave_cnt) {
  constexpr int kWaves = kThreads / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int n = 0;
  for (int b0 = 0; b0 < nitems; b0 += kThreads) {
    const int it = b0 + tid;
    const bool any = it < nitems && pred(it);
    const uint64_t bal = __ballot(any);
    if (lane == 0) s_wave_cnt[wave] = __popcll(bal);
    __syncthreads();
    int base = n;
    for (int w = 0; w < wave; ++w) base += s_wave_cnt[w];
    if (any) {
      const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      s_list[base + rank] = (uint16_t)it;
    }
    for (int w = 0; w < kWaves; ++w) n += s_wave_cnt[w];
    __syncthreads();
  }
  return n;
}

// Whether some token executes group g. All mask bytes are requested before
// any is tested: token rows past T - 1 are clamped to T - 1 (T >= 1), which
// leaves the OR unchanged and keeps the loads out of branches.
template <int kMaxT>
__device__ __forceinline__ bool group_live(const uint8_t* __restrict__ mask, int T, int ng, int g) {
  uint32_t m = 0;
#pragma unroll
  for (int t = 0; t < kMaxT; ++t) m |= mask[(size_t)min(t, T - 1) * ng + g];
  return m != 0;
}

// Lists the groups executed by some token (1 <= T <= kMaxT) into s_list.
template <int kThreads, int kMaxT>
__device__ __forceinline__ int list_active(const uint8_t* __restrict__ mask, int T, int ng,
                                           uint16_t* s_list, int* s_wave_cnt) {
  return list_where<kThreads>(
      ng, [&](int g) { return group_live<kMaxT>(mask, T, ng, g); }, s_list, s_wave_cnt);
}

// Flags the groups executed by some token into s_gact[0, ng) and lists the
// 32-channel chunks that hold at least one of them into s_list (one pass
// over the mask; the chunk test reads the flags in LDS).
template <int kThreads, int kMaxT>
__device__ __forceinline__ int list_active_chunks(const uint8_t* __restrict__ mask, int T, int ng,
                                                  int G, int nchunks, uint8_t* s_gact,
                                                  uint16_t* s_list, int* s_wave_cnt) {
  for (int g = threadIdx.x; g < ng; g += kThreads) s_gact[g] = group_live<kMaxT>(mask, T, ng, g);
  __syncthreads();
  return list_where<kThreads>(
      nchunks,
      [&](int c) {
        bool any = false;
        for (int g = (c * 32) / G; g <= (c * 32 + 31) / G; ++g) any |= s_gact[g] != 0;
        return any;
      },
      s_list, s_wave_cnt);
}

constexpr int kGuThreads = 256;
constexpr int kGuWaves = kGuThreads / 64;

// One work unit: UC channels of one group, all T tokens, full K split over
// the four waves. UC = 8: the 8 gate rows and 8 up rows form one 16-row MFMA
// operand (finest balance; for few tokens the activation fragment costs
// almost nothing). UC = 16 / 32: UC/16 gate operands and UC/16 up operands of
// 16 rows share each activation fragment (a half / a quarter of the
// activation traffic per weight byte, for many tokens).
// PACKED (UC >= 16): Wg and Wu are operand-order copies, in which the 16 rows
// x 32 columns of each MFMA operand are one contiguous 1 KB block (lane l's
// 16 bytes at byte 16 l), blocks ordered by 16-row block, then by 32-column
// slice; every weight load then reads 1 KB of contiguous memory.
template <int UC, bool PACKED = false>
__device__ __forceinline__ void gate_up_unit(const uint16_t* __restrict__ X,
                                             const uint16_t* __restrict__ Wg,
                                             const uint16_t* __restrict__ Wu,
                                             const uint8_t* __restrict__ mask, int T, int d,
                                             int d_ff, int G, uint16_t* __restrict__ H,
                                             int zero_inactive, uint16_t* s_groups,
                                             int* s_wave_cnt, float (*s_red)[64][16]) {
  constexpr int NF = UC / 8;  // 16-row A operands per unit
  constexpr int kU = NF >= 4 ? 4 : kUnroll;  // loads per lane per batch and operand
  const int ng = d_ff / G;
  const int upg = G / UC;  // units per group
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  const int nact = list_active<kGuThreads, 16>(mask, T, ng, s_groups, s_wave_cnt);
  const int u = blockIdx.x;
  if (u >= nact * upg) {
    // Past the active units: when H must hold exact zeros, the units of the
    // groups no token executes (in unit order after the active ones) are
    // cleared here.
    if (!zero_inactive) return;
    const int k = u - nact * upg;  // k-th unit of an inactive group
    if (k >= (ng - nact) * upg) return;
    const int want = k / upg;  // the want-th group (ascending) that no token executes
    int g = -1;
    for (int gg = 0, seen = 0, ai = 0; gg < ng; ++gg) {
      if (ai < nact && s_groups[ai] == gg) {
        ++ai;
        continue;
      }
      if (seen++ == want) {
        g = gg;
        break;
      }
    }
    if (g >= 0 && tid < T * NF) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      *(u32x4*)(H + (size_t)(tid / NF) * d_ff + g * G + (k % upg) * UC + (tid % NF) * 8) = z;
    }
    return;
  }
  const int g = s_groups[u / upg];
  const int c0 = g * G + (u % upg) * UC;

  // wave w takes the 32-wide K slices [s_lo, s_hi) of d / 32
  const int nsub_all = d / 32;
  const int s_lo = (wave * nsub_all) / kGuWaves;
  const int s_hi = ((wave + 1) * nsub_all) / kGuWaves;
  const int kbase = s_lo * 32 + 8 * (lane >> 4);
  const int r = lane & 15;
  // operand rows: UC == 8: rows 0..7 gate, 8..15 up of channels c0..c0+7;
  //   else operand f < NF/2: gate rows c0 + 16 f + r, operand f + NF/2: the up
  //   rows of the same channels
  static_assert(!PACKED || NF >= 2, "operand-order weights need 16-row gate and up operands");
  // elements between the operands of consecutive 32-wide K slices
  constexpr int kStep = PACKED ? 512 : 32;
  const uint16_t* pw[NF];
  if (NF == 1) {
    pw[0] = (r < 8 ? Wg : Wu) + (size_t)(c0 + (r & 7)) * d + kbase;
  } else {
#pragma unroll
    for (int f = 0; f < NF / 2; ++f) {
      const size_t off = PACKED ? ((size_t)((c0 + 16 * f) / 16) * (d / 32) + s_lo) * 512 + 8 * lane
                                : (size_t)(c0 + 16 * f + r) * d + kbase;
      pw[f] = Wg + off;
      pw[f + NF / 2] = Wu + off;
    }
  }
  // B operand column = token; columns past T - 1 repeat token T - 1's row
  // (each output column depends on its own B column only, and those columns
  // are never stored), so no load sits in a branch and the wait counts stay
  // exact across the double buffer
  const int tok = lane & 15;
  const uint16_t* px = X + (size_t)min(tok, T - 1) * d + kbase;

  f32x4 acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nsub = s_hi - s_lo;
  // Software pipeline: the loads of batch b+1 are issued before the MFMAs of
  // batch b, so every wave keeps a batch of loads in flight while it computes.
  const int nb = nsub / kU;
  u32x4 aw[2][NF][kU], bx[2][kU];
  // the scheduling barrier keeps a batch's loads together, ahead of the
  // MFMAs that follow (the scheduler would otherwise sink them between those
  // MFMAs, behind waits for the previous batch)
  auto load_batch = [&](int b, int set) {
#pragma unroll
    for (int q = 0; q < kU; ++q) {
#pragma unroll
      for (int f = 0; f < NF; ++f) aw[set][f][q] = ld16(pw[f] + kStep * (b * kU + q));
      bx[set][q] = ld16(px + 32 * (b * kU + q));
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto mma_batch = [&](int set) {
#pragma unroll
    for (int q = 0; q < kU; ++q)
#pragma unroll
      for (int f = 0; f < NF; ++f)
        acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, aw[set][f][q]),
                                                         __builtin_bit_cast(bf16x8, bx[set][q]),
                                                         acc[f], 0, 0, 0);
  };
  // (No load is issued under a condition inside the loop: the wait counts
  // then stay exact, and the MFMAs of one batch wait only for that batch.)
  if (nb > 0) {
    load_batch(0, 0);
    int b = 0;
    for (; b + 2 < nb; b += 2) {
      load_batch(b + 1, 1);
      mma_batch(0);
      load_batch(b + 2, 0);
      mma_batch(1);
    }
    if (b + 1 < nb) {
      load_batch(b + 1, 1);
      mma_batch(0);
      mma_batch(1);
    } else {
      mma_batch(0);
    }
  }
  for (int s = nb * kU; s < nsub; ++s) {
    const bf16x8 bv = __builtin_bit_cast(bf16x8, ld16(px + 32 * s));
#pragma unroll
    for (int f = 0; f < NF; ++f)
      acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ld16(pw[f] + kStep * s)),
                                                       bv, acc[f], 0, 0, 0);
  }

  // lane holds token (lane % 16) and operand rows 4*(lane/16) + e.
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_red[wave][lane][4 * f + e] = acc[f][e];
  __syncthreads();
  if (wave != 0 || tok >= T) return;
  // UC == 8: gate channels 0..7 sit in lanes 0..31, the matching up rows in
  // lanes 32..63; else gate operand f and up operand f + NF/2 share a lane.
  if (NF == 1 && lane >= 32) return;
  // A token that skips this group still gets +0.0 here: the down GEMV reads
  // every channel of a group that some token executes.
  const bool act = mask[(size_t)tok * ng + g] != 0;
  constexpr int NP = NF == 1 ? 1 : NF / 2;  // 16-channel (or 8-channel) blocks
#pragma unroll
  for (int f = 0; f < NP; ++f) {
    float h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float gs = 0.0f, us = 0.0f;
#pragma unroll
      for (int w = 0; w < kGuWaves; ++w) {
        gs += s_red[w][lane][4 * f + e];
        us += (NF == 1) ? s_red[w][lane + 32][e] : s_red[w][lane][4 * (f + NP) + e];
      }
      h[e] = act ? silu_mul(gs, us) : 0.0f;
    }
    const u32x2 v = {pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
    *(u32x2*)(H + (size_t)tok * d_ff + c0 + 16 * f + 4 * (lane >> 4)) = v;
  }
}

#define WIDE_DECODE_GATE_UP_KERNEL(NAME, UC, PACKED)                                            \
  __global__ __launch_bounds__(kGuThreads) void NAME(                                           \
      const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wg,                          \
      const uint16_t* __restrict__ Wu, const uint8_t* __restrict__ mask, int T, int d,          \
      int d_ff, int G, uint16_t* __restrict__ H, int zero_inactive) {                           \
    __shared__ uint16_t s_groups[kMaxGroups];                                                   \
    __shared__ int s_wave_cnt[kGuWaves];                                                        \
    __shared__ float s_red[kGuWaves][64][16];                                                   \
    gate_up_unit<UC, PACKED>(X, Wg, Wu, mask, T, d, d_ff, G, H, zero_inactive, s_groups,        \
                             s_wave_cnt, s_red);                                                \
  }
WIDE_DECODE_GATE_UP_KERNEL(decode_gate_up_kernel_8, 8, false)
WIDE_DECODE_GATE_UP_KERNEL(decode_gate_up_kernel_16, 16, false)
WIDE_DECODE_GATE_UP_KERNEL(decode_gate_up_kernel_32, 32, false)
WIDE_DECODE_GATE_UP_KERNEL(decode_gate_up_packed_kernel_16, 16, true)
WIDE_DECODE_GATE_UP_KERNEL(decode_gate_up_packed_kernel_32, 32, true)
#undef WIDE_DECODE_GATE_UP_KERNEL

// gate/up with the activations in LDS, for nn.Linear weights (3 <= T,
// T * d <= kXldsElems, G % 32 == 0, d % 128 == 0). The activation fragments
// of the kernels above are global loads (L2 hits) that join every batch of
// weight loads in the wave's memory queue; at T = 16 on the Llama3.1-8B shape
// the kernel without them took 45 instead of 51 us. Here a workgroup of
// 8 waves takes two 32-channel units (waves 0-3 and 4-7, each wave one
// quarter of K) and first copies the T activation rows into LDS, where the
// fragment reads cost no memory-queue slots; only weights stream from HBM.
// Row t's 16-byte chunk c sits at chunk c ^ (t % 16) of the row (d % 128 == 0
// keeps that inside the row), so the 16 token lanes of a fragment read hit
// distinct banks. Per unit the arithmetic, the operand order and the sum
// over the four quarters are those of gate_up_unit<32>, so H is the same bit
// for bit. Measured at T = 16 on the Llama3.1-8B shape: 47.4 against 50.8 us.
constexpr int kXThreads = 512;
constexpr int kXWaves = kXThreads / 64;
constexpr int kXldsElems = 65536;  // activation elements held in LDS (128 KB)

__global__ __launch_bounds__(kXThreads) void decode_gate_up_xlds_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wg,
    const uint16_t* __restrict__ Wu, const uint8_t* __restrict__ mask, int T, int d, int d_ff,
    int G, uint16_t* __restrict__ H, int zero_inactive) {
  constexpr int UC = 32, NF = 4, kU = 4;
  __shared__ uint16_t s_groups[kMaxGroups];
  __shared__ int s_wave_cnt[kXWaves];
  // the T activation rows; after the MFMA loop, the partial sums [wave][lane][16]
  __shared__ __attribute__((aligned(16))) uint16_t s_x[kXldsElems];
  const int ng = d_ff / G;
  const int upg = G / UC;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  const int nact = list_active<kXThreads, 16>(mask, T, ng, s_groups, s_wave_cnt);
  const int u = 2 * (int)blockIdx.x + (wave >> 2);  // this wave's unit
  const int quarter = wave & 3;
  const bool active = u < nact * upg;
  const int g = active ? s_groups[u / upg] : 0;
  const int c0 = g * G + (u % upg) * UC;

  const int nsub_all = d / 32;
  const int s_lo = (quarter * nsub_all) / 4;
  const int s_hi = ((quarter + 1) * nsub_all) / 4;
  const int kbase = s_lo * 32 + 8 * (lane >> 4);
  const int r = lane & 15;
  constexpr int kStep = 32;  // elements between the operands of consecutive K slices
  const uint16_t* pw[NF];
#pragma unroll
  for (int f = 0; f < NF / 2; ++f) {
    const size_t off = (size_t)(c0 + 16 * f + r) * d + kbase;
    pw[f] = Wg + off;
    pw[f + NF / 2] = Wu + off;
  }
  const int nsub = active ? s_hi - s_lo : 0;
  const int nb = nsub / kU;
  u32x4 aw[2][NF][kU];
  auto load_batch = [&](int b, int set) {
#pragma unroll
    for (int q = 0; q < kU; ++q)
#pragma unroll
      for (int f = 0; f < NF; ++f) aw[set][f][q] = ld16(pw[f] + kStep * (b * kU + q));
    __builtin_amdgcn_sched_barrier(0);
  };
  // Issue order: the activation loads, then this wave's first weight batch,
  // then the LDS writes of the activations, which wait only for the
  // activation loads, so the first batch's latency overlaps the copy and the
  // barrier (47.9 -> 47.5 us for gate/up at T = 16 on the Llama3.1-8B shape).
  // Issuing the first batch before the activation loads measured 4 us slower.
  const int cpr = d / 8;  // 16-byte chunks per row
  const int nchunk = T * cpr;
  constexpr int kXPer = kXldsElems / 8 / kXThreads;  // chunks per thread at most
  u32x4 xv[kXPer];
#pragma unroll
  for (int i = 0; i < kXPer; ++i) {
    const int e = min(tid + kXThreads * i, nchunk - 1);
    xv[i] = ld16(X + (size_t)8 * e);
  }
  if (nb > 0) load_batch(0, 0);
#pragma unroll
  for (int i = 0; i < kXPer; ++i) {
    const int e = tid + kXThreads * i;
    if (e < nchunk) {
      const int t = e / cpr, c = e % cpr;
      *(u32x4*)(s_x + (size_t)t * d + 8 * (c ^ (t & 15))) = xv[i];
    }
  }
  __syncthreads();

  // B operand column = token; columns past T - 1 read token T - 1's row (each
  // output column depends on its own B column only, and those columns are
  // never stored)
  const int tok = lane & 15;
  const int xrow = min(tok, T - 1);
  const uint16_t* sxr = s_x + (size_t)xrow * d;
  const int xsw = xrow & 15;
  auto xfrag = [&](int s) -> bf16x8 {
    const int c = 4 * s + (lane >> 4);
    return *(const bf16x8*)(sxr + 8 * (c ^ xsw));
  };
  f32x4 acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma_batch = [&](int b, int set) {
    bf16x8 bv[kU];
#pragma unroll
    for (int q = 0; q < kU; ++q) bv[q] = xfrag(s_lo + b * kU + q);
#pragma unroll
    for (int q = 0; q < kU; ++q)
#pragma unroll
      for (int f = 0; f < NF; ++f)
        acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, aw[set][f][q]),
                                                         bv[q], acc[f], 0, 0, 0);
  };
  if (nb > 0) {
    int b = 0;
    for (; b + 2 < nb; b += 2) {
      load_batch(b + 1, 1);
      mma_batch(b, 0);
      load_batch(b + 2, 0);
      mma_batch(b + 1, 1);
    }
    if (b + 1 < nb) {
      load_batch(b + 1, 1);
      mma_batch(b, 0);
      mma_batch(b + 1, 1);
    } else {
      mma_batch(b, 0);
    }
  }
  for (int s = nb * kU; s < nsub; ++s) {
    const bf16x8 bv = xfrag(s_lo + s);
#pragma unroll
    for (int f = 0; f < NF; ++f)
      acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ld16(pw[f] + kStep * s)),
                                                       bv, acc[f], 0, 0, 0);
  }

  __syncthreads();  // every wave is done with the activation rows
  float(*s_red)[64][16] = (float(*)[64][16])s_x;
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_red[wave][lane][4 * f + e] = acc[f][e];
  __syncthreads();
  if (quarter != 0) return;
  if (!active) {
    // a unit of a group no token executes gets +0.0 when H must hold it
    // (units in order after the active ones, as in gate_up_unit)
    if (!zero_inactive) return;
    const int k = u - nact * upg;
    if (k >= (ng - nact) * upg) return;
    const int want = k / upg;
    int gz = -1;
    for (int gg = 0, seen = 0, ai = 0; gg < ng; ++gg) {
      if (ai < nact && s_groups[ai] == gg) {
        ++ai;
        continue;
      }
      if (seen++ == want) {
        gz = gg;
        break;
      }
    }
    if (gz >= 0 && lane < T * NF) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      *(u32x4*)(H + (size_t)(lane / NF) * d_ff + gz * G + (k % upg) * UC + (lane % NF) * 8) = z;
    }
    return;
  }
  if (tok >= T) return;
  const bool act = mask[(size_t)tok * ng + g] != 0;
  const int w0 = wave;  // first of the unit's four waves
#pragma unroll
  for (int f = 0; f < NF / 2; ++f) {
    float h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float gs = 0.0f, us = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        gs += s_red[w0 + w][lane][4 * f + e];
        us += s_red[w0 + w][lane][4 * (f + NF / 2) + e];
      }
      h[e] = act ? silu_mul(gs, us) : 0.0f;
    }
    const u32x2 v = {pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
    *(u32x2*)(H + (size_t)tok * d_ff + c0 + 16 * f + 4 * (lane >> 4)) = v;
  }
}

// Shapes the LDS-activation gate/up takes.
bool xlds_shape(int T, int d, int G) {
  return T > kValuMaxT && T <= 16 && G % 32 == 0 && d % 128 == 0 && (long)T * d <= kXldsElems;
}

// Down GEMV for T > 2: split over the live chunks. A workgroup owns 64
// output rows and one kDecodeDownSplit-th of the live 32-channel chunk list;
// each wave multiplies every H fragment it loads by four 16-row blocks of
// Wdown (a quarter of the H traffic of one block per fragment), and the four
// waves meet in LDS. The fp32 partial sums go to `part` [split, T, d]; a
// second kernel adds the splits in a fixed order and rounds once to bf16.
constexpr int kSkRows = 64;
constexpr int kSkThreads = 256;
constexpr int kSkWaves = kSkThreads / 64;
constexpr int kSkU = 4;  // chunks per batch per wave
constexpr int kMaxChunks = 2048;  // d_ff / 32 limit

// PIECES (G % 32 != 0): a live 32-channel chunk can also hold a group that no
// token executes (its H was never written), so each lane's 8-channel piece is
// tested on its own group and uses zeros there. A piece never straddles two
// groups: G is a multiple of 16 and pieces start at multiples of 8.
// PACKED: Wd is the operand-order copy (see gate_up_unit): the 16 rows x 32
// channels of each operand are one contiguous 1 KB block.
template <bool PIECES, bool PACKED = false>
__global__ __launch_bounds__(kSkThreads) void decode_down_splitk_kernel(
    const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wd,
    const uint8_t* __restrict__ mask, int T, int d, int d_ff, int G, float* __restrict__ part) {
  __shared__ uint16_t s_chunks[kMaxChunks];
  __shared__ int s_wave_cnt[kSkWaves];
  __shared__ float s_red[kSkWaves][64][16];
  __shared__ uint8_t s_gact[kMaxGroups];  // PIECES: group executed by some token
  const int ng = d_ff / G;
  const int n0 = (int)(blockIdx.x / kDecodeDownSplit) * kSkRows;
  const int split = (int)(blockIdx.x % kDecodeDownSplit);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // groups some token executes (s_gact) and the 32-channel chunks that hold one
  const int nch =
      list_active_chunks<kSkThreads, 16>(mask, T, ng, G, d_ff / 32, s_gact, s_chunks, s_wave_cnt);
  const int lo = (split * nch) / kDecodeDownSplit;
  const int hi = ((split + 1) * nch) / kDecodeDownSplit;

  const int koff = 8 * (lane >> 4);
  const int tok = lane & 15;
  // weight operand of chunk k (its first channel) for row block rb: pw[rb] +
  // k, or with the operand-order copy pw[rb] + 16 k (1 KB per 32 channels)
  const uint16_t* pw[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
    pw[rb] = PACKED ? Wd + (size_t)((n0 + 16 * rb) / 16) * (d_ff / 32) * 512 + 8 * lane
                    : Wd + (size_t)(n0 + 16 * rb + (lane & 15)) * d_ff + koff;
  constexpr int kScale = PACKED ? 16 : 1;
  // token columns past T - 1 repeat token T - 1 (never stored, see gate/up)
  const uint16_t* ph = H + (size_t)min(tok, T - 1) * d_ff + koff;
  f32x4 acc[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // this wave takes chunks lo + wave, lo + wave + 4, ...; batches of kSkU
  // chunks, the loads of batch b+1 issued before the MFMAs of batch b
  const int mine = hi - lo > wave ? (hi - lo - wave + kSkWaves - 1) / kSkWaves : 0;
  const int nb = mine / kSkU;
  u32x4 a[2][4][kSkU], bb[2][kSkU];
  auto chunk_k = [&](int i) { return (int)s_chunks[lo + wave + kSkWaves * i] * 32; };
  // H loads are unconditional (inside H's bounds). With PIECES, the lanes of
  // a group no token executes get an all-zero AND mask, applied when the
  // fragment is used, so nothing unwritten reaches the sums and no load or
  // move of a loaded value sits in a branch.
  uint32_t hm[2][kSkU];
  auto h_mask = [&](int k) -> uint32_t {
    return PIECES ? (s_gact[(k + koff) / G] ? 0xFFFFFFFFu : 0u) : 0xFFFFFFFFu;
  };
  auto masked = [](const u32x4& v, uint32_t m) {
    const u32x4 mv = {m, m, m, m};
    return __builtin_bit_cast(bf16x8, v & mv);
  };
  auto load_batch = [&](int b, int set) {
#pragma unroll
    for (int q = 0; q < kSkU; ++q) {
      const int k = chunk_k(b * kSkU + q);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) a[set][rb][q] = ld16(pw[rb] + kScale * k);
      bb[set][q] = ld16(ph + k);
      hm[set][q] = h_mask(k);
    }
    __builtin_amdgcn_sched_barrier(0);  // the batch's loads stay together (see gate/up)
  };
  auto mma_batch = [&](int set) {
#pragma unroll
    for (int q = 0; q < kSkU; ++q) {
      const bf16x8 hv = PIECES ? masked(bb[set][q], hm[set][q]) : __builtin_bit_cast(bf16x8, bb[set][q]);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[set][rb][q]),
                                                          hv, acc[rb], 0, 0, 0);
    }
  };
  // (no load is issued under a condition inside the loop; see gate/up)
  if (nb > 0) {
    load_batch(0, 0);
    int b = 0;
    for (; b + 2 < nb; b += 2) {
      load_batch(b + 1, 1);
      mma_batch(0);
      load_batch(b + 2, 0);
      mma_batch(1);
    }
    if (b + 1 < nb) {
      load_batch(b + 1, 1);
      mma_batch(0);
      mma_batch(1);
    } else {
      mma_batch(0);
    }
  }
  for (int i = nb * kSkU; i < mine; ++i) {
    const int k = chunk_k(i);
    const bf16x8 hv = PIECES ? masked(ld16(ph + k), h_mask(k)) : __builtin_bit_cast(bf16x8, ld16(ph + k));
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
      acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ld16(pw[rb] + kScale * k)),
                                                        hv, acc[rb], 0, 0, 0);
  }
  // lane holds token (lane % 16) and rows 16 rb + 4 (lane / 16) + e
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_red[wave][lane][4 * rb + e] = acc[rb][e];
  __syncthreads();
  if (wave != 0 || tok >= T) return;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kSkWaves; ++w)
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] += s_red[w][lane][4 * rb + e];
    *(f32x4*)(part + ((size_t)split * T + tok) * d + n0 + 16 * rb + 4 * (lane >> 4)) = y;
  }
}

// Y[t, n] = bf16(sum over the splits of part[s, t, n]), splits added in order.
__global__ __launch_bounds__(256) void decode_down_reduce_kernel(const float* __restrict__ part,
                                                                 int T, int d,
                                                                 uint16_t* __restrict__ Y) {
  const int i = (int)blockIdx.x * 256 + (int)threadIdx.x;  // 4 outputs per thread
  if (i >= T * d / 4) return;
  f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sp = 0; sp < kDecodeDownSplit; ++sp) y += *(const f32x4*)(part + (size_t)sp * T * d + 4 * i);
  const u32x2 v = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
  *(u32x2*)(Y + 4 * (size_t)i) = v;
}

// ---------------------------------------------------------------- T <= 2: VALU

constexpr int kValuThreads = 256;
constexpr int kValuWaves = kValuThreads / 64;
// Threads of a VALU down workgroup: one token, 8 waves (two workgroups per
// CU, so at d = 4096 each wave takes exactly one output row, and one chunk
// list per 8 waves; measured 13.2 us against 13.4 for three 4-wave
// workgroups per CU and 13.9 for one of 16 waves); two tokens, 4 waves.
__host__ __device__ constexpr int down_valu_threads(int nt) { return nt == 1 ? 512 : 256; }

// gate/up for T <= NT tokens. Wave items are the channels of the groups some
// token executes; lane l reads 16 bytes at k = 8 l + 512 j of the item's gate
// and up rows (whole 1 KB blocks per load), against X staged in LDS.
template <int NT>
__device__ __forceinline__ void gate_up_valu(const uint16_t* __restrict__ X,
                                             const uint16_t* __restrict__ Wg,
                                             const uint16_t* __restrict__ Wu,
                                             const uint8_t* __restrict__ mask, int T, int d,
                                             int d_ff, int G, uint16_t* __restrict__ H,
                                             int zero_inactive, uint16_t* s_groups,
                                             int* s_wave_cnt, uint16_t* s_x) {
  constexpr int kJ = 8;  // 1 KB loads per row and k-block (4096 channels)
  const int ng = d_ff / G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nact = list_active<kValuThreads, NT>(mask, T, ng, s_groups, s_wave_cnt);
  const int nj = d / 512;
  const int gw = blockIdx.x * kValuWaves + wave, nw = gridDim.x * kValuWaves;
  const int nitems = nact * G;
  // blocks past the row's end re-read its last block (never used), so no
  // load sits in a branch
  u32x4 vg[kJ], vu[kJ];
  auto load_rows = [&](int it, int j0) {
    const int c = (int)s_groups[it / G] * G + it % G;
    const uint16_t* pg = Wg + (size_t)c * d + 8 * lane;
    const uint16_t* pu = Wu + (size_t)c * d + 8 * lane;
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int jj = min(j0 + j, nj - 1);
      vg[j] = ld16_nt(pg + 512 * jj);
      vu[j] = ld16_nt(pu + 512 * jj);
    }
  };
  // the first batch of this wave's first row is requested before X is
  // staged, so the two latencies overlap (a wave without rows re-reads the
  // last row; the values are never used)
  if (nitems > 0) load_rows(min(gw, nitems - 1), 0);
  // X rows of the NT tokens (rows past T are zeros)
  const int cpr = d / 8;
  for (int e = tid; e < NT * cpr; e += kValuThreads) {
    const int t = e / cpr, c = e % cpr;
    const u32x4 z = {0u, 0u, 0u, 0u};
    const u32x4 v = ld16(X + (size_t)min(t, T - 1) * d + 8 * c);
    *(u32x4*)(s_x + t * d + 8 * c) = t < T ? v : z;
  }
  __syncthreads();
  bool loaded = true;
  for (int it = gw; it < nitems; it += nw) {
    const int g = s_groups[it / G];
    const int c = g * G + it % G;
    float sg[NT], su[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) sg[t] = su[t] = 0.0f;
    for (int j0 = 0; j0 < nj; j0 += kJ) {
      if (!loaded) load_rows(it, j0);
      loaded = false;
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        if (j0 + j < nj) {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const u32x4 xv = *(const u32x4*)(s_x + t * d + 512 * (j0 + j) + 8 * lane);
            sg[t] = dot8(vg[j], xv, sg[t]);
            su[t] = dot8(vu[j], xv, su[t]);
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      sg[t] = wave_sum(sg[t]);
      su[t] = wave_sum(su[t]);
    }
    // lane t writes token t; a token that skips the group gets +0.0
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (lane == t && t < T) {
        const bool act = mask[(size_t)t * ng + g] != 0;
        H[(size_t)t * d_ff + c] = f32_to_bf16_bits(act ? silu_mul(sg[t], su[t]) : 0.0f);
      }
    }
  }
  if (!zero_inactive) return;
  // groups no token executes: +0.0 over their channels (workgroup-strided)
  for (int g = blockIdx.x; g < ng; g += gridDim.x) {
    bool any = false;
#pragma unroll
    for (int t = 0; t < NT; ++t) any |= mask[(size_t)min(t, T - 1) * ng + g] != 0;
    if (any) continue;
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int e = tid; e < T * (G / 8); e += kValuThreads) {
      const int t = e / (G / 8), c = e % (G / 8);
      *(u32x4*)(H + (size_t)t * d_ff + g * G + 8 * c) = z;
    }
  }
}

// down for T <= NT tokens. Wave items are output rows; the live 32-channel
// chunks are listed once, and H over them is compacted into LDS (zeros for
// groups no token executes and for tokens past T). Lane l reads 16 bytes of
// chunk 16 i + l / 4, piece l % 4, of the item's row.
template <int NT, int kTh>
__device__ __forceinline__ void down_valu(const uint16_t* __restrict__ H,
                                          const uint16_t* __restrict__ Wd,
                                          const uint8_t* __restrict__ mask, int T, int d, int d_ff,
                                          int G, uint16_t* __restrict__ Y, uint16_t* s_chunks,
                                          uint8_t* s_gact, int* s_wave_cnt, uint16_t* s_h) {
  constexpr int kBatch = 16;  // loads in flight per lane (a whole row of 256 live chunks)
  const int ng = d_ff / G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch =
      list_active_chunks<kTh, NT>(mask, T, ng, G, d_ff / 32, s_gact, s_chunks, s_wave_cnt);
  const int stride = nch * 32;  // compacted channels per token
  const int ninstr = (nch + 15) / 16;
  const int gw = blockIdx.x * (kTh / 64) + wave, nw = gridDim.x * (kTh / 64);
  const int piece = 8 * (lane & 3);
  // chunk slots past the list's end re-read its last chunk (never used), so
  // no load sits in a branch
  u32x4 w[kBatch];
  auto load_row = [&](int n, int i0) {
    const uint16_t* pw = Wd + (size_t)n * d_ff + piece;
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int j = min(16 * (i0 + q) + (lane >> 2), nch - 1);
      w[q] = ld16_nt(pw + (int)s_chunks[j] * 32);
    }
  };
  // the first batch of this wave's first row is requested before H is
  // compacted, so the two latencies overlap (a wave without rows re-reads
  // the last row; the values are never used)
  if (nch > 0) load_row(min(gw, d - 1), 0);
  for (int e = tid; e < NT * nch * 4; e += kTh) {
    const int t = e / (nch * 4), r = e % (nch * 4);
    const int j = r >> 2, q = r & 3;
    const int ch = (int)s_chunks[j] * 32 + 8 * q;
    const bool live = s_gact[ch / G] != 0;
    const u32x4 z = {0u, 0u, 0u, 0u};
    // an H fragment of a group no token executes may be unwritten: it is
    // loaded (in bounds) and replaced by zeros, never summed
    const u32x4 v = ld16(H + (size_t)min(t, T - 1) * d_ff + ch);
    *(u32x4*)(s_h + t * stride + 32 * j + 8 * q) = (t < T && live) ? v : z;
  }
  __syncthreads();
  bool loaded = true;
  for (int n = gw; n < d; n += nw) {
    float y[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) y[t] = 0.0f;
    for (int i0 = 0; i0 < ninstr; i0 += kBatch) {
      if (!loaded) load_row(n, i0);
      loaded = false;
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int j = 16 * (i0 + q) + (lane >> 2);
        if (j < nch) {
#pragma unroll
          for (int t = 0; t < NT; ++t)
            y[t] = dot8(w[q], *(const u32x4*)(s_h + t * stride + 32 * j + piece), y[t]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) y[t] = wave_sum(y[t]);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      if (lane == t && t < T) Y[(size_t)t * d + n] = f32_to_bf16_bits(y[t]);
  }
}

#define WIDE_DECODE_VALU_KERNELS(NT)                                                            \
  __global__ __launch_bounds__(kValuThreads) void decode_gate_up_valu_kernel_##NT(               \
      const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wg,                          \
      const uint16_t* __restrict__ Wu, const uint8_t* __restrict__ mask, int T, int d,          \
      int d_ff, int G, uint16_t* __restrict__ H, int zero_inactive) {                           \
    __shared__ uint16_t s_groups[kMaxGroups];                                                   \
    __shared__ int s_wave_cnt[kValuWaves];                                                      \
    __shared__ __attribute__((aligned(16))) uint16_t s_x[NT * kValuMaxD];                       \
    gate_up_valu<NT>(X, Wg, Wu, mask, T, d, d_ff, G, H, zero_inactive, s_groups, s_wave_cnt,    \
                     s_x);                                                                      \
  }                                                                                             \
  __global__ __launch_bounds__(down_valu_threads(NT)) void decode_down_valu_kernel_##NT(        \
      const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wd,                          \
      const uint8_t* __restrict__ mask, int T, int d, int d_ff, int G,                          \
      uint16_t* __restrict__ Y) {                                                               \
    __shared__ uint16_t s_chunks[valu_cap(NT) / 32];                                            \
    __shared__ uint8_t s_gact[valu_cap(NT) / 16];                                               \
    __shared__ int s_wave_cnt[down_valu_threads(NT) / 64];                                      \
    __shared__ __attribute__((aligned(16))) uint16_t s_h[NT * valu_cap(NT)];                    \
    down_valu<NT, down_valu_threads(NT)>(H, Wd, mask, T, d, d_ff, G, Y, s_chunks, s_gact,       \
                                         s_wave_cnt, s_h);                                      \
  }
WIDE_DECODE_VALU_KERNELS(1)
WIDE_DECODE_VALU_KERNELS(2)
#undef WIDE_DECODE_VALU_KERNELS

// Shapes the VALU kernels take: whole 1 KB blocks per row, X in LDS, H over
// every channel compactable into LDS.
bool valu_shape(int T, int d, int d_ff) {
  return T >= 1 && T <= kValuMaxT && d % 512 == 0 && d <= kValuMaxD && d_ff <= valu_cap(T) &&
         d_ff % 32 == 0;
}

int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace

namespace {

// Operand-order copy of a [rows, cols] bf16 matrix: 16-byte chunk i of the
// output is lane l = i % 64 of block b = i / 64, i.e. row 16 (b / (cols/32)) +
// l % 16, columns 32 (b % (cols/32)) + 8 (l / 16) .. + 7 of the input.
__global__ __launch_bounds__(256) void decode_pack_kernel(const uint16_t* __restrict__ W, int rows,
                                                          int cols, uint16_t* __restrict__ out) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)rows * cols / 8) return;
  const size_t b = i / 64;
  const int l = (int)(i % 64);
  const size_t rb = b / (size_t)(cols / 32);
  const int kc = (int)(b % (size_t)(cols / 32));
  *(u32x4*)(out + 8 * i) = ld16(W + (16 * rb + (size_t)(l & 15)) * cols + 32 * kc + 8 * (l >> 4));
}

}  // namespace

hipError_t launch_decode_pack_bf16(const uint16_t* W, int rows, int cols, uint16_t* out,
                                   hipStream_t stream) {
  if (rows % 16 != 0 || cols % 32 != 0) return hipErrorInvalidValue;
  const size_t chunks = (size_t)rows * cols / 8;
  if (chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_pack_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0,
                     stream, W, rows, cols, out);
  return hipGetLastError();
}

hipError_t launch_decode_gate_up_bf16(const uint16_t* X, const uint16_t* Wg, const uint16_t* Wu,
                                      const uint16_t* Wg_op, const uint16_t* Wu_op,
                                      const uint8_t* mask, int T, int d, int d_ff, int G,
                                      uint16_t* H, bool zero_inactive, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  // one or two tokens: whole-row streaming on a persistent grid of four
  // workgroups per CU for one token (measured best of three, four, five and
  // seven at the Llama3.1-8B shape), three for two tokens
  if (valu_shape(T, d, d_ff)) {
    if (T == 1)
      hipLaunchKernelGGL(decode_gate_up_valu_kernel_1, dim3(4 * num_cus()), dim3(kValuThreads), 0,
                         stream, X, Wg, Wu, mask, T, d, d_ff, G, H, zero_inactive ? 1 : 0);
    else
      hipLaunchKernelGGL(decode_gate_up_valu_kernel_2, dim3(3 * num_cus()), dim3(kValuThreads), 0,
                         stream, X, Wg, Wu, mask, T, d, d_ff, G, H, zero_inactive ? 1 : 0);
    return hipGetLastError();
  }
  // nn.Linear weights: activations in LDS, two 32-channel units per
  // workgroup. (With operand-order weights the kernels below, whose loads
  // read contiguous 1 KB blocks, measured faster: 69.9 against 76.4 us per
  // T = 16 step on the Llama3.1-8B shape.)
  if (Wg_op == nullptr && xlds_shape(T, d, G)) {
    hipLaunchKernelGGL(decode_gate_up_xlds_kernel, dim3((unsigned)((d_ff / 32 + 1) / 2)),
                       dim3(kXThreads), 0, stream, X, Wg, Wu, mask, T, d, d_ff, G, H,
                       zero_inactive ? 1 : 0);
    return hipGetLastError();
  }
  // operand-order weights: 32-channel units (16 when G is not a multiple of
  // 32) for any T
  if (Wg_op != nullptr) {
    if (G % 32 == 0)
      hipLaunchKernelGGL(decode_gate_up_packed_kernel_32, dim3(d_ff / 32), dim3(kGuThreads), 0,
                         stream, X, Wg_op, Wu_op, mask, T, d, d_ff, G, H, zero_inactive ? 1 : 0);
    else
      hipLaunchKernelGGL(decode_gate_up_packed_kernel_16, dim3(d_ff / 16), dim3(kGuThreads), 0,
                         stream, X, Wg_op, Wu_op, mask, T, d, d_ff, G, H, zero_inactive ? 1 : 0);
    return hipGetLastError();
  }
  // few tokens: 8-channel units (finest balance); more tokens: 32-channel
  // units (16 when G is not a multiple of 32) whose gate and up operands
  // share each activation fragment
  if (T <= kDecodeSmallT)
    hipLaunchKernelGGL(decode_gate_up_kernel_8, dim3(d_ff / 8), dim3(kGuThreads), 0, stream, X, Wg,
                       Wu, mask, T, d, d_ff, G, H, zero_inactive ? 1 : 0);
  else if (G % 32 == 0)
    hipLaunchKernelGGL(decode_gate_up_kernel_32, dim3(d_ff / 32), dim3(kGuThreads), 0, stream, X,
                       Wg, Wu, mask, T, d, d_ff, G, H, zero_inactive ? 1 : 0);
  else
    hipLaunchKernelGGL(decode_gate_up_kernel_16, dim3(d_ff / 16), dim3(kGuThreads), 0, stream, X,
                       Wg, Wu, mask, T, d, d_ff, G, H, zero_inactive ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_decode_down_bf16(const uint16_t* H, const uint16_t* Wd, const uint16_t* Wd_op,
                                   const uint8_t* mask, int T, int d, int d_ff, int G, uint16_t* Y,
                                   float* part, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (valu_shape(T, d, d_ff)) {
    // waves strided over the output rows, two workgroups per CU (the LDS
    // copy of H holds two per CU with two tokens)
    if (T == 1)
      hipLaunchKernelGGL(decode_down_valu_kernel_1, dim3(2 * num_cus()), dim3(down_valu_threads(1)),
                         0, stream, H, Wd, mask, T, d, d_ff, G, Y);
    else
      hipLaunchKernelGGL(decode_down_valu_kernel_2, dim3(2 * num_cus()), dim3(down_valu_threads(2)),
                         0, stream, H, Wd, mask, T, d, d_ff, G, Y);
    return hipGetLastError();
  }
  // G is a multiple of 16; unless it is a multiple of 32, a 32-channel chunk
  // can straddle an executed and a skipped group (G = 16, 48, 80, ...)
  if (G % 16 != 0) return hipErrorInvalidValue;
  const bool pieces = G % 32 != 0;
  const dim3 grid((d / kSkRows) * kDecodeDownSplit);
  if (Wd_op != nullptr && pieces)
    hipLaunchKernelGGL((decode_down_splitk_kernel<true, true>), grid, dim3(kSkThreads), 0, stream, H,
                       Wd_op, mask, T, d, d_ff, G, part);
  else if (Wd_op != nullptr)
    hipLaunchKernelGGL((decode_down_splitk_kernel<false, true>), grid, dim3(kSkThreads), 0, stream,
                       H, Wd_op, mask, T, d, d_ff, G, part);
  else if (pieces)
    hipLaunchKernelGGL(decode_down_splitk_kernel<true>, grid, dim3(kSkThreads), 0, stream, H, Wd,
                       mask, T, d, d_ff, G, part);
  else
    hipLaunchKernelGGL(decode_down_splitk_kernel<false>, grid, dim3(kSkThreads), 0, stream, H, Wd,
                       mask, T, d, d_ff, G, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_down_reduce_kernel, dim3((T * d / 4 + 255) / 256), dim3(256), 0, stream,
                     part, T, d, Y);
  return hipGetLastError();
}

}  // namespace wide
