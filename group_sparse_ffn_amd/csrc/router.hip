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
// kernel is built to stream X: a workgroup owns 64 tokens and its eight waves
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

// Two shapes of workgroup: for many tokens, 8 waves over 64 tokens (every W1
// fragment serves four 16-token blocks; measured against 4 and 16 waves and
// 16- or 32-token workgroups); for at most 16 tokens, 16 waves over one
// block, so that the chain of dependent loads along D is 16 times shorter.
constexpr int kRtGC = 64;  // groups whose mask bytes gather in LDS at a time

// X pieces are read in the MFMA operand layout (half of a 128-byte line per
// load, the other half with the next), so they keep the default cache policy.
__device__ __forceinline__ u32x4 rt_ld(const uint16_t* p) { return *(const u32x4*)p; }

__device__ __forceinline__ float router_act(float a, int act) {
  if (act == 1) return a > 0.0f ? a : 0.0f;
  if (act == 2) return a * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a * 1.4426950408889634f));
  return a;
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
  // k-steps per load batch: the many-token shape keeps two batches of four
  // blocks in flight; the one-block shape loads a quarter of its D slice at once
  constexpr int kU = kRtRB == 1 ? (R >= 64 ? 2 : 4) : (R >= 64 ? 1 : 2);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t0 = (int)blockIdx.x * kRtTok;

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
  lds_barrier();  // s_z complete
  for (int g0 = 0; g0 < ng; g0 += kRtGC) {
    const int gc = min(kRtGC, ng - g0);
    const int nob = (gc + 7) / 8;  // 16-column blocks of the chunk
    for (int it = wave; it < kRtRB * nob; it += kRtWaves) {
      const int tb = it / nob, ob = it % nob;
      const int col = 16 * ob + c16;  // chunk-local column: group col / 2, class col % 2
      const bool colok = col < 2 * gc;
      // W2 row of this column (row 2 g0 stands in past the chunk; zeroed)
      const uint32_t* pw2 =
          (const uint32_t*)(W2 + (size_t)(2 * g0 + (colok ? col : 0)) * R + KQ * q);
      uint32_t wv[KQ / 2];
#pragma unroll
      for (int i = 0; i < KQ / 2; ++i) wv[i] = colok ? pw2[i] : 0u;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KQ; ++kk) {
        const uint32_t bits = (kk & 1) ? (wv[kk >> 1] & 0xFFFF0000u) : (wv[kk >> 1] << 16);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(s_z[16 * tb + c16][KQ * q + kk],
                                                   __builtin_bit_cast(float, bits), acc, 0, 0, 0);
      }
      // lane holds tokens 16 tb + 4 q + e of column col; lane ^ 1 holds the
      // other class of the same group and tokens
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float other = __shfl_xor(acc[e], 1);
        const int t = 16 * tb + 4 * q + e;
        if (colok && (c16 & 1) == 0) s_mask[t][col >> 1] = acc[e] >= other ? 1 : 0;
        if (logits && colok && t < ntok) logits[((size_t)(t0 + t) * ng + g0) * 2 + col] = acc[e];
      }
    }
    lds_barrier();
    if (mask != nullptr) {
      for (int e = tid; e < ntok * gc; e += kRtThreads) {
        const int t = e / gc, gl = e % gc;
        mask[(size_t)(t0 + t) * ng + g0 + gl] = s_mask[t][gl];
      }
    }
    if (maskbits != nullptr) {
      // packed bits straight from the decisions in LDS: thread (j, h) reads
      // the 4-group words of tokens 32 h .. 32 h + 31 (consecutive threads,
      // consecutive words: no bank conflict) and builds the bit words of
      // groups 4 j .. 4 j + 3; tokens past T give 0 bits.
      // maskbits[g, w] bit b = decision of token 32 w + b.
      constexpr int kHalves = (kRtTok + 31) / 32;
      const int nj = (gc + 3) / 4;
      const int j = tid / kHalves, h = tid % kHalves;
      const int nt = min(32, ntok - 32 * h);  // <= 0: the word lies past T (none stored)
      if (tid < nj * kHalves && nt > 0) {
        uint32_t b[4] = {0u, 0u, 0u, 0u};
        for (int t = 0; t < nt; ++t) {
          const uint32_t w = *(const uint32_t*)&s_mask[32 * h + t][4 * j];
#pragma unroll
          for (int q = 0; q < 4; ++q) b[q] |= ((w >> (8 * q)) & 0xFFu) != 0 ? (1u << t) : 0u;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (4 * j + q < gc) maskbits[(size_t)(g0 + 4 * j + q) * words + (t0 >> 5) + h] = b[q];
      }
    }
    lds_barrier();  // s_mask is refilled by the next chunk
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
    __shared__ uint8_t s_mask[16 * RB][kRtGC];                                                 \
    router_body<R, RB, NW>(X, W1, W2, T, D, ng, act, mask, logits, maskbits, words, s_part,    \
                           s_z, s_mask);                                                       \
  }
WIDE_ROUTER_KERNEL(router_kernel_16, 16, 4, 8)
WIDE_ROUTER_KERNEL(router_kernel_32, 32, 4, 8)
WIDE_ROUTER_KERNEL(router_kernel_64, 64, 4, 8)
WIDE_ROUTER_KERNEL(router_small_kernel_16, 16, 1, 16)
WIDE_ROUTER_KERNEL(router_small_kernel_32, 32, 1, 16)
WIDE_ROUTER_KERNEL(router_small_kernel_64, 64, 1, 16)
#undef WIDE_ROUTER_KERNEL

}  // namespace

hipError_t launch_router_bf16(const uint16_t* X, const uint16_t* W1, const uint16_t* W2, int T,
                              int D, int r, int ng, int act, uint8_t* mask, float* logits,
                              uint32_t* maskbits, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int words = (T + 31) / 32;
  typedef void (*K)(const uint16_t*, const uint16_t*, const uint16_t*, int, int, int, int, uint8_t*,
                    float*, uint32_t*, int);
  const bool small = T <= 16;
  const K k = small ? (r == 16 ? router_small_kernel_16 : r == 32 ? router_small_kernel_32
                                                                  : router_small_kernel_64)
                    : (r == 16 ? router_kernel_16 : r == 32 ? router_kernel_32 : router_kernel_64);
  const dim3 grid(small ? 1 : (T + 63) / 64), block(small ? 1024 : 512);
  hipLaunchKernelGGL(k, grid, block, 0, stream, X, W1, W2, T, D, ng, act, mask, logits, maskbits,
                     words);
  return hipGetLastError();
}

}  // namespace wide
