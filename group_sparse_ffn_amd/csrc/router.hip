// Bottleneck router producing the group mask (ai.info summary, "How decisions
// are made": input activations -> N_G two-way decisions per token through an
// inner dimension r; argmax at inference; class 0 = execute, class 1 = skip).
// Readings (the paper's Sec. 3.1 "Routing Components" gives no formula): no
// biases, a caller-chosen activation between the two maps, logits laid out
// [T, N_G, 2] with the class fastest, and a tie taking the first maximum
// (execute):
//   z[t,j]       = act( X[t,:] . W1[j,:] )          j < r
//   logit[t,g,c] = W2[2g + c, :] . z[t,:]
//   mask[t,g]    = logit[t,g,0] >= logit[t,g,1]
//
// The first map reads every activation byte once and is bound by HBM, so the
// many-token kernel is built to stream X: a workgroup owns 64 tokens and its eight waves
// split D; each wave reads 16-byte pieces of X in the layout of a
// v_mfma_f32_16x16x32_bf16 operand (16 tokens x 32 channels per load) against
// the r / 16 matching fragments of W1 (shared by every workgroup, served from
// L2, each fragment used for all four 16-token blocks), with the loads of the next
// batch in flight during the current MFMAs. The partial sums meet in LDS,
// where the activation is applied; the second map (a small fp32 MFMA
// product), the argmax and the mask bytes follow in the same kernel (no
// logits round trip through memory unless the caller asks).
#include "common.h"

namespace wide {

namespace {

// The many-token workgroup: 8 waves over 64 tokens (every W1 fragment serves
// four 16-token blocks; measured against 4 and 16 waves and 16- or 32-token
// workgroups).
constexpr int kRtGC = 64;  // groups whose mask bytes gather in LDS at a time

// X pieces are read in the MFMA operand layout (half of a 128-byte line per
// load, the other half with the next), so they keep the default cache policy.
__device__ __forceinline__ u32x4 rt_ld(const uint16_t* p) { return *(const u32x4*)p; }

__device__ __forceinline__ float router_act(float a, int act) {
  if (act == 1) return a > 0.0f ? a : 0.0f;
  if (act == 2) return a * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a * 1.4426950408889634f));
  return a;
}

// Copies the decisions of tokens t0 .. t0 + ntok - 1 for the groups
// g0 .. g0 + gc - 1 from the LDS tile to their mask rows, VW bytes per lane
// (VW divides ng, gc, g0 and the mask address).
template <int VW>
__device__ __forceinline__ void store_mask_rows(uint8_t* __restrict__ mask,
                                                const uint8_t (*s_mask)[kRtGC], int t0, int ntok,
                                                int ng, int g0, int gc, int tid, int nthreads) {
  typedef uint32_t vec4 __attribute__((ext_vector_type(4)));
  typedef uint32_t vec2 __attribute__((ext_vector_type(2)));
  const int per_row = gc / VW;
  for (int e = tid; e < ntok * per_row; e += nthreads) {
    const int t = e / per_row, c = VW * (e % per_row);
    uint8_t* dst = mask + (size_t)(t0 + t) * ng + g0 + c;
    const uint8_t* src = &s_mask[t][c];
    if constexpr (VW == 16)
      *(vec4*)dst = *(const vec4*)src;
    else if constexpr (VW == 8)
      *(vec2*)dst = *(const vec2*)src;
    else if constexpr (VW == 4)
      *(uint32_t*)dst = *(const uint32_t*)src;
    else
      *dst = *src;
  }
}

template <int R, int kRtRB, int kRtWaves>
__device__ __forceinline__ void router_body(const uint16_t* __restrict__ X,
                                            const uint16_t* __restrict__ W1,
                                            const uint16_t* __restrict__ W2, int T, int D, int ng,
                                            int act, uint8_t* __restrict__ mask,
                                            float* __restrict__ logits,
                                            uint32_t* __restrict__ maskbits, int words,
                                            float (*s_part)[16 * kRtRB][R],
                                            float (*s_z)[R + 1], uint8_t (*s_mask)[kRtGC]) {
  constexpr int kRtTok = 16 * kRtRB;
  constexpr int kRtThreads = 64 * kRtWaves;
  constexpr int NF = R / 16;  // W1 fragments of 16 outputs
  // k-steps per load batch: two batches of kRtRB blocks in flight
  constexpr int kU = R >= 64 ? 1 : 2;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // XCD-aware: workgroup ids go to the 8 XCDs in turn, and XCD x takes the
  // x-th contiguous range of token blocks, so the neighbouring blocks whose
  // 8-byte pieces of a group's packed-bit row share a 128-byte line write it
  // through one L2
  const int nblk = (T + kRtTok - 1) / kRtTok;
  const int per_xcd = (nblk + 7) / 8;
  const int blk = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (blk >= nblk) return;
  const int t0 = blk * kRtTok;

  // ---- z partials: wave w takes the 32-wide K slices [s_lo, s_hi) of D / 32;
  // every W1 fragment it loads serves the workgroup's kRtRB token blocks
  const int nsub_all = D / 32;
  const int s_lo = (wave * nsub_all) / kRtWaves;
  const int s_hi = ((wave + 1) * nsub_all) / kRtWaves;
  const int kbase = s_lo * 32 + 8 * (lane >> 4);
  // A operand row = token; rows past T - 1 repeat token T - 1 (each output
  // row depends on its own A row only, and those rows are never stored), so
  // no load sits in a branch and the wait counts stay exact across the
  // double buffer
  const uint16_t* px[kRtRB];
#pragma unroll
  for (int b = 0; b < kRtRB; ++b) {
    const int tok = min(t0 + 16 * b + (lane & 15), T - 1);
    px[b] = X + (size_t)tok * D + kbase;
  }
  const uint16_t* pw[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) pw[f] = W1 + (size_t)(16 * f + (lane & 15)) * D + kbase;
  f32x4 acc[kRtRB][NF];
#pragma unroll
  for (int b = 0; b < kRtRB; ++b)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[b][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nsub = s_hi - s_lo;
  const int nb = nsub / kU;
  u32x4 ax[2][kRtRB][kU], bw[2][NF][kU];
  auto load_batch = [&](int bt, int set) {
#pragma unroll
    for (int q = 0; q < kU; ++q) {
      const int k = 32 * (bt * kU + q);
#pragma unroll
      for (int b = 0; b < kRtRB; ++b) ax[set][b][q] = rt_ld(px[b] + k);
#pragma unroll
      for (int f = 0; f < NF; ++f) bw[set][f][q] = *(const u32x4*)(pw[f] + k);
    }
    // keeps the batch's loads together, ahead of the MFMAs that follow
    __builtin_amdgcn_sched_barrier(0);
  };
  auto mma_batch = [&](int set) {
#pragma unroll
    for (int q = 0; q < kU; ++q)
#pragma unroll
      for (int b = 0; b < kRtRB; ++b)
#pragma unroll
        for (int f = 0; f < NF; ++f)
          acc[b][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, ax[set][b][q]), __builtin_bit_cast(bf16x8, bw[set][f][q]),
              acc[b][f], 0, 0, 0);
  };
  // no load is issued under a condition inside the loop
  if (nb > 0) {
    load_batch(0, 0);
    int bt = 0;
    for (; bt + 2 < nb; bt += 2) {
      load_batch(bt + 1, 1);
      mma_batch(0);
      load_batch(bt + 2, 0);
      mma_batch(1);
    }
    if (bt + 1 < nb) {
      load_batch(bt + 1, 1);
      mma_batch(0);
      mma_batch(1);
    } else {
      mma_batch(0);
    }
  }
  for (int s = nb * kU; s < nsub; ++s) {
#pragma unroll
    for (int b = 0; b < kRtRB; ++b) {
      const bf16x8 xv = __builtin_bit_cast(bf16x8, rt_ld(px[b] + 32 * s));
#pragma unroll
      for (int f = 0; f < NF; ++f)
        acc[b][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            xv, __builtin_bit_cast(bf16x8, *(const u32x4*)(pw[f] + 32 * s)), acc[b][f], 0, 0, 0);
    }
  }
  // W2 rows of one chunk of kRtGC groups (2 kRtGC rows of R bf16) pass
  // through registers into LDS; each chunk's rows are requested one step
  // ahead (the first chunk's now, while the partial sums meet in LDS), so the
  // products below read W2 from LDS instead of putting an L2 round trip on
  // every wave for each of its items (about 0.8 us of the kernel at the
  // Llama3.1-8B prefill shape).
  constexpr int kW2Vec = 2 * kRtGC * R / 8;  // 16-byte pieces of a full chunk
  constexpr int kW2Per = (kW2Vec + kRtThreads - 1) / kRtThreads;
  u32x4 w2r[kW2Per];
  auto w2_pieces = [&](int g0) { return 2 * min(kRtGC, ng - g0) * R / 8; };
  auto load_w2 = [&](int g0) {
    const int n = w2_pieces(g0);
    const u32x4* src = (const u32x4*)(W2 + (size_t)2 * g0 * R);
#pragma unroll
    for (int i = 0; i < kW2Per; ++i) w2r[i] = src[min(tid + kRtThreads * i, n - 1)];
  };
  // the chunk's rows in LDS, in the partial-sum array (free once z is formed)
  uint16_t* s_w2 = reinterpret_cast<uint16_t*>(&s_part[0][0][0]);
  static_assert(2 * kRtGC * R * 2 <= kRtWaves * kRtTok * R * 4, "a W2 chunk fits the partial sums");
  auto store_w2 = [&](int g0) {
    const int n = w2_pieces(g0);
#pragma unroll
    for (int i = 0; i < kW2Per; ++i) {
      const int e = tid + kRtThreads * i;
      if (e < n) *(u32x4*)(s_w2 + 8 * e) = w2r[i];
    }
  };
  load_w2(0);

  // lane holds z for token 16 b + 4 (lane / 16) + e and output 16 f + lane % 16
#pragma unroll
  for (int b = 0; b < kRtRB; ++b)
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s_part[wave][16 * b + 4 * (lane >> 4) + e][16 * f + (lane & 15)] = acc[b][f][e];
  lds_barrier();
  for (int e = tid; e < kRtTok * R; e += kRtThreads) {
    const int t = e / R, j = e % R;
    float a = 0.0f;
#pragma unroll
    for (int w = 0; w < kRtWaves; ++w) a += s_part[w][t][j];
    s_z[t][j] = router_act(a, act);
  }

  // ---- logits, argmax and mask: [tokens x 2 N_G] = z [tokens x R] . W2^T on
  // v_mfma_f32_16x16x4_f32 (fp32 products and fp32 sums, like a scalar fma
  // chain). Work items are (16-token block, 16-column block = 8 groups x 2
  // classes). The sum over k is order-free, so the MFMA's k slot is permuted:
  // lane group q = lane / 16 takes k = KQ q + kk in step kk, which gives every
  // lane contiguous pieces of z and of a W2 row. Groups go kRtGC at a time;
  // their mask bytes gather in LDS and leave as contiguous row segments.
  constexpr int KQ = R / 4;
  const int ntok = min(kRtTok, T - t0);
  const int q = lane >> 4, c16 = lane & 15;
  lds_barrier();  // s_z complete; the partial sums are no longer read
  for (int g0 = 0; g0 < ng; g0 += kRtGC) {
    const int gc = min(kRtGC, ng - g0);
    store_w2(g0);
    if (g0 + kRtGC < ng) load_w2(g0 + kRtGC);
    lds_barrier();  // the chunk's W2 rows in LDS
    // A wave keeps one 16-token block (its z operands are read from LDS once)
    // and takes every kWpb-th 16-column block of the chunk; the MFMA chains
    // of its blocks run interleaved, one k-step at a time. (One item at a
    // time, with z re-read per item, these products took about 6 us of the
    // kernel's 40 at the Llama3.1-8B prefill shape.) Blocks past the chunk multiply zeros and
    // store nothing.
    static_assert(kRtWaves % kRtRB == 0, "waves per token block");
    constexpr int kWpb = kRtWaves / kRtRB;
    constexpr int kObMax = (2 * kRtGC / 16 + kWpb - 1) / kWpb;
    const int tb = wave % kRtRB, ob0 = wave / kRtRB;
    float zv[KQ];
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) zv[kk] = s_z[16 * tb + c16][KQ * q + kk];
    uint32_t wv[kObMax][KQ / 2];
    f32x4 acc[kObMax];
#pragma unroll
    for (int j = 0; j < kObMax; ++j) {
      const int col = 16 * (ob0 + kWpb * j) + c16;  // chunk-local column: group col / 2, class col % 2
      const bool colok = col < 2 * gc;
      // W2 row of this column from LDS (row 0 stands in past the chunk; zeroed)
      const uint32_t* pw2 = (const uint32_t*)(s_w2 + (colok ? col : 0) * R + KQ * q);
#pragma unroll
      for (int i = 0; i < KQ / 2; ++i) wv[j][i] = colok ? pw2[i] : 0u;
      acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk)
#pragma unroll
      for (int j = 0; j < kObMax; ++j) {
        const uint32_t bits =
            (kk & 1) ? (wv[j][kk >> 1] & 0xFFFF0000u) : (wv[j][kk >> 1] << 16);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(zv[kk], __builtin_bit_cast(float, bits),
                                                      acc[j], 0, 0, 0);
      }
#pragma unroll
    for (int j = 0; j < kObMax; ++j) {
      const int col = 16 * (ob0 + kWpb * j) + c16;
      const bool colok = col < 2 * gc;
      // lane holds tokens 16 tb + 4 q + e of column col; lane ^ 1 holds the
      // other class of the same group and tokens. (A DPP quad permute here,
      // reading the MFMA result a few cycles after the MFMA, gave wrong
      // values with this toolchain; the permute through LDS is correct.)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float other = __shfl_xor(acc[j][e], 1);
        const int t = 16 * tb + 4 * q + e;
        if (colok && (c16 & 1) == 0) s_mask[t][col >> 1] = acc[j][e] >= other ? 1 : 0;
        if (logits && colok && t < ntok) logits[((size_t)(t0 + t) * ng + g0) * 2 + col] = acc[j][e];
      }
    }
    lds_barrier();
    if (mask != nullptr) {
      // row segments of the chunk in pieces of vw bytes: the widest of 16, 8
      // and 4 that divides the row length and the mask address (g0 and a
      // full chunk are multiples of 64), else single bytes. (One byte per
      // lane these stores took about 2.4 us of the kernel at the Llama3.1-8B
      // prefill shape.)
      const uintptr_t am = reinterpret_cast<uintptr_t>(mask) | (uintptr_t)ng;
      if ((am & 15) == 0)
        store_mask_rows<16>(mask, s_mask, t0, ntok, ng, g0, gc, tid, kRtThreads);
      else if ((am & 7) == 0)
        store_mask_rows<8>(mask, s_mask, t0, ntok, ng, g0, gc, tid, kRtThreads);
      else if ((am & 3) == 0)
        store_mask_rows<4>(mask, s_mask, t0, ntok, ng, g0, gc, tid, kRtThreads);
      else
        store_mask_rows<1>(mask, s_mask, t0, ntok, ng, g0, gc, tid, kRtThreads);
    }
    if (maskbits != nullptr) {
      // packed bits straight from the decisions in LDS, one wave ballot per
      // group: lane t holds token t0 + t (a workgroup owns 64 tokens, one
      // per lane), and the 64 decision bits are the group's two words of
      // this workgroup. maskbits[g, w] bit b = decision of token 32 w + b;
      // tokens past T give 0 bits and words past T are not stored.
      // Wave w takes the chunk's groups 8 w .. 8 w + 7: one 8-byte LDS read
      // per token gives its 8 decisions, 8 ballots give the 16 words, and
      // lanes 2 i + h store word h of group 8 w + i in one instruction.
      static_assert(kRtTok == 64 && kRtGC == 8 * kRtWaves, "one token per lane, 8 groups per wave");
      const int gw0 = 8 * wave;
      if (gw0 < gc) {
        const uint64_t row8 = lane < ntok ? *(const uint64_t*)&s_mask[lane][gw0] : 0ull;
        uint32_t word = 0u;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint64_t b = __ballot(((row8 >> (8 * i)) & 0xFFull) != 0ull);
          if (lane == 2 * i) word = (uint32_t)b;
          if (lane == 2 * i + 1) word = (uint32_t)(b >> 32);
        }
        const int gi = lane >> 1, h = lane & 1;
        if (lane < 16 && gw0 + gi < gc && 32 * h < ntok)
          maskbits[(size_t)(g0 + gw0 + gi) * words + (t0 >> 5) + h] = word;
      }
    }
    lds_barrier();  // s_mask and the W2 rows are refilled by the next chunk
  }
}

#define WIDE_ROUTER_KERNEL(NAME, R, RB, NW)                                                    \
  __global__ __launch_bounds__(64 * NW) void NAME(                                             \
      const uint16_t* __restrict__ X, const uint16_t* __restrict__ W1,                         \
      const uint16_t* __restrict__ W2, int T, int D, int ng, int act,                          \
      uint8_t* __restrict__ mask, float* __restrict__ logits, uint32_t* __restrict__ maskbits, \
      int words) {                                                                             \
    __shared__ float s_part[NW][16 * RB][R];                                                   \
    __shared__ float s_z[16 * RB][R + 1];                                                      \
    __shared__ __attribute__((aligned(16))) uint8_t s_mask[16 * RB][kRtGC];                    \
    router_body<R, RB, NW>(X, W1, W2, T, D, ng, act, mask, logits, maskbits, words, s_part,    \
                           s_z, s_mask);                                                       \
  }
WIDE_ROUTER_KERNEL(router_kernel_16, 16, 4, 8)
WIDE_ROUTER_KERNEL(router_kernel_32, 32, 4, 8)
WIDE_ROUTER_KERNEL(router_kernel_64, 64, 4, 8)
#undef WIDE_ROUTER_KERNEL

// ---- At most 16 tokens: two kernels instead of one workgroup.
// One workgroup streaming all of W1 (r * D * 2 bytes, 256 KB at D = 4096,
// r = 32) is bound by the misses a single CU keeps in flight: its last wave
// finished the first map 8 us after the first (timestamps inside the kernel,
// T = 1). So the first map is split over kRtSlices workgroups, each taking a
// slice of D for all tokens and outputs and writing fp32 partial sums
// [kRtSlices][16][r] (D = 4096, r = 32, per call in a graph at T = 1: one
// workgroup 12.9 us; 4, 8, 16 and 32 slices 6.7, 5.8, 6.3 and 6.9 us; 8
// slices of 8 waves 6.6 us); a second kernel with one wave per 16 logit columns
// (8 groups) requests its W2 rows at once, adds the partial sums in slice
// order (fixed order: the same z every call), applies the activation and takes
// the decisions as the many-token kernel does.
constexpr int kRtSlices = kRouterSlices;

template <int R>
__global__ __launch_bounds__(256) void router_zpart_kernel(const uint16_t* __restrict__ X,
                                                           const uint16_t* __restrict__ W1, int T,
                                                           int D, float* __restrict__ zpart) {
  constexpr int NF = R / 16;
  __shared__ float s_part[4][16][R];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nsub = D / 32;  // 32-channel k-steps
  const int sbeg = (int)(((long long)blockIdx.x * nsub) / kRtSlices);
  const int send = (int)(((long long)(blockIdx.x + 1) * nsub) / kRtSlices);
  // A operand row = token (rows past T - 1 repeat token T - 1; never stored),
  // B operand row = output 16 f + lane % 16; lane group lane / 16 holds k 8 (lane / 16) ..
  const int kof = 8 * (lane >> 4);
  const uint16_t* px = X + (size_t)min(lane & 15, T - 1) * D + kof;
  const uint16_t* pw[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) pw[f] = W1 + (size_t)(16 * f + (lane & 15)) * D + kof;
  f32x4 acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
  // wave w takes k-steps sbeg + w, + 4, + 8, ...: four per pass, loads clamped
  // into the slice (so none sits under a condition), MFMAs only for real steps
  for (int s0 = sbeg + wave; s0 < send; s0 += 16) {
    u32x4 xa[4], wb[4][NF];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = 32 * min(s0 + 4 * i, send - 1);
      xa[i] = *(const u32x4*)(px + k);
#pragma unroll
      for (int f = 0; f < NF; ++f) wb[i][f] = *(const u32x4*)(pw[f] + k);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (s0 + 4 * i < send)
#pragma unroll
        for (int f = 0; f < NF; ++f)
          acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[i]),
                                                           __builtin_bit_cast(bf16x8, wb[i][f]),
                                                           acc[f], 0, 0, 0);
  }
  // lane holds the partial z of token 4 (lane / 16) + e, output 16 f + lane % 16
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_part[wave][4 * (lane >> 4) + e][16 * f + (lane & 15)] = acc[f][e];
  __syncthreads();
  float* out = zpart + (size_t)blockIdx.x * 16 * R;
  for (int e = tid; e < 16 * R; e += 256) {
    const int t = e / R, j = e % R;
    out[e] = ((s_part[0][t][j] + s_part[1][t][j]) + s_part[2][t][j]) + s_part[3][t][j];
  }
}

template <int R>
__global__ __launch_bounds__(64) void router_decide_kernel(
    const uint16_t* __restrict__ W2, const float* __restrict__ zpart, int T, int ng, int act,
    uint8_t* __restrict__ mask, float* __restrict__ logits, uint32_t* __restrict__ maskbits,
    int words) {
  constexpr int KQ = R / 4;
  const int lane = threadIdx.x, q = lane >> 4, c16 = lane & 15;
  const int col = 16 * (int)blockIdx.x + c16;  // logit column 2 g + c
  const bool colok = col < 2 * ng;
  // this lane's W2 piece: row col, k = KQ q .. KQ q + KQ (row 0 stands in past the end)
  const uint32_t* pw2 = (const uint32_t*)(W2 + (size_t)(colok ? col : 0) * R + KQ * q);
  uint32_t wv[KQ / 2];
#pragma unroll
  for (int i = 0; i < KQ / 2; ++i) wv[i] = pw2[i];
  // z of token c16 at k = KQ q .. KQ q + KQ: the slices' partial sums (in slice
  // order), CS slices' loads in flight at a time (64 floats per lane)
  constexpr int CS = 64 / KQ < kRtSlices ? 64 / KQ : kRtSlices;
  static_assert(kRtSlices % CS == 0, "slice chunks");
  float z[KQ];
#pragma unroll
  for (int i = 0; i < KQ; ++i) z[i] = 0.0f;
#pragma unroll
  for (int s0 = 0; s0 < kRtSlices; s0 += CS) {
    f32x4 zp[CS][KQ / 4];
#pragma unroll
    for (int s = 0; s < CS; ++s)
#pragma unroll
      for (int i = 0; i < KQ / 4; ++i)
        zp[s][i] = *(const f32x4*)(zpart + ((size_t)(s0 + s) * 16 + c16) * R + KQ * q + 4 * i);
#pragma unroll
    for (int s = 0; s < CS; ++s)
#pragma unroll
      for (int i = 0; i < KQ / 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) z[4 * i + e] += zp[s][i][e];
  }
  // logits of tokens 4 q + e, column c16 (v_mfma_f32_16x16x4_f32 with the k
  // slot permuted as in the many-token kernel)
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < KQ; ++kk) {
    const uint32_t w = colok ? wv[kk >> 1] : 0u;
    const uint32_t bits = (kk & 1) ? (w & 0xFFFF0000u) : (w << 16);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(router_act(z[kk], act),
                                               __builtin_bit_cast(float, bits), acc, 0, 0, 0);
  }
  // lane ^ 1 holds the other class of the same group and tokens
  const int g = col >> 1;
  const bool dec_lane = colok && (c16 & 1) == 0;
  uint64_t bal[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float other = __shfl_xor(acc[e], 1);
    const int t = 4 * q + e;
    const bool exec = acc[e] >= other;
    if (mask && dec_lane && t < T) mask[(size_t)t * ng + g] = exec ? 1 : 0;
    if (logits && colok && t < T) logits[(size_t)t * ng * 2 + col] = acc[e];
    bal[e] = __ballot(dec_lane && t < T && exec);
  }
  // packed decisions: lane gl < 8 builds the word of group 8 blockIdx.x + gl
  // (T <= 16: one word per group, bit t = token t)
  if (maskbits) {
    const int gg = 8 * (int)blockIdx.x + lane;
    if (lane < 8 && gg < ng) {
      uint32_t w = 0u;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
#pragma unroll
        for (int e = 0; e < 4; ++e) w |= (uint32_t)((bal[e] >> (16 * qq + 2 * lane)) & 1u) << (4 * qq + e);
      maskbits[(size_t)gg * words] = w;
    }
  }
}

}  // namespace

hipError_t launch_router_bf16(const uint16_t* X, const uint16_t* W1, const uint16_t* W2, int T,
                              int D, int r, int ng, int act, uint8_t* mask, float* logits,
                              uint32_t* maskbits, float* zpart, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int words = (T + 31) / 32;
  if (T <= kRouterSmallT) {
    typedef void (*KZ)(const uint16_t*, const uint16_t*, int, int, float*);
    typedef void (*KD)(const uint16_t*, const float*, int, int, int, uint8_t*, float*, uint32_t*,
                       int);
    const KZ kz = r == 16 ? router_zpart_kernel<16> : r == 32 ? router_zpart_kernel<32>
                                                              : router_zpart_kernel<64>;
    const KD kd = r == 16 ? router_decide_kernel<16> : r == 32 ? router_decide_kernel<32>
                                                               : router_decide_kernel<64>;
    hipLaunchKernelGGL(kz, dim3(kRtSlices), dim3(256), 0, stream, X, W1, T, D, zpart);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kd, dim3((ng + 7) / 8), dim3(64), 0, stream, W2, zpart, T, ng, act, mask,
                       logits, maskbits, words);
    return hipGetLastError();
  }
  typedef void (*K)(const uint16_t*, const uint16_t*, const uint16_t*, int, int, int, int, uint8_t*,
                    float*, uint32_t*, int);
  const K k = r == 16 ? router_kernel_16 : r == 32 ? router_kernel_32 : router_kernel_64;
  const int nblk = (T + 63) / 64;
  hipLaunchKernelGGL(k, dim3((nblk + 7) / 8 * 8), dim3(512), 0, stream, X, W1, W2, T, D, ng, act,
                     mask, logits, maskbits, words);
  return hipGetLastError();
}


}  // namespace wide
