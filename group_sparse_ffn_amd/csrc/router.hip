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
// kernel is built to stream X: a workgroup owns 64 tokens and its four waves
// split D; each wave reads 16-byte pieces of X in the layout of a
// v_mfma_f32_16x16x32_bf16 operand (16 tokens x 32 channels per load) against
// the r / 16 matching fragments of W1 (shared by every workgroup, served from
// L2, each fragment used for all four 16-token blocks), with the loads of the next
// batch in flight during the current MFMAs. The partial sums meet in LDS,
// where the activation is applied; the second map (W2 staged in LDS a chunk
// of groups at a time), the argmax and the mask bytes follow in the same
// kernel (no logits round trip through memory unless the caller asks).
#include "common.h"

namespace wide {

namespace {

// Two shapes of workgroup: for many tokens, 4 waves over 64 tokens (every W1
// fragment serves four 16-token blocks); for at most 16 tokens, 16 waves over
// one block, so that the chain of dependent loads along D is 16 times shorter.
constexpr int kRtGC = 64;  // groups whose W2 rows are staged in LDS at a time

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
                                            float (*s_part)[16 * kRtRB][R],
                                            float (*s_z)[R + 1], float (*s_w2)[2 * kRtGC]) {
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
  const uint16_t* px[kRtRB];
#pragma unroll
  for (int b = 0; b < kRtRB; ++b) {
    const int tok = t0 + 16 * b + (lane & 15);
    px[b] = tok < T ? X + (size_t)tok * D + kbase : nullptr;
  }
  const uint16_t* pw[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) pw[f] = W1 + (size_t)(16 * f + (lane & 15)) * D + kbase;
  const u32x4 zero = {0u, 0u, 0u, 0u};
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
      for (int b = 0; b < kRtRB; ++b) ax[set][b][q] = px[b] ? rt_ld(px[b] + k) : zero;
#pragma unroll
      for (int f = 0; f < NF; ++f) bw[set][f][q] = *(const u32x4*)(pw[f] + k);
    }
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
  if (nb > 0) load_batch(0, 0);
  for (int bt = 0; bt < nb; bt += 2) {
    if (bt + 1 < nb) load_batch(bt + 1, 1);
    mma_batch(0);
    if (bt + 1 >= nb) break;
    if (bt + 2 < nb) load_batch(bt + 2, 0);
    mma_batch(1);
  }
  for (int s = nb * kU; s < nsub; ++s) {
#pragma unroll
    for (int b = 0; b < kRtRB; ++b) {
      const bf16x8 xv = __builtin_bit_cast(bf16x8, px[b] ? rt_ld(px[b] + 32 * s) : zero);
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
  __syncthreads();
  for (int e = tid; e < kRtTok * R; e += kRtThreads) {
    const int t = e / R, j = e % R;
    float a = 0.0f;
#pragma unroll
    for (int w = 0; w < kRtWaves; ++w) a += s_part[w][t][j];
    s_z[t][j] = router_act(a, act);
  }

  // ---- logits, argmax and mask, kRtGC groups at a time with their W2 rows in
  // LDS, transposed to [j][2 g + c] fp32. Thread (token tid % 32, phase
  // tid / 32) holds its token's z in registers and takes every eighth group
  // of the chunk; the 32 lanes of a phase read the same W2 pair (broadcast).
  const int ntok = min(kRtTok, T - t0);
  const int my_t = tid % kRtTok, phase = tid / kRtTok;
  constexpr int kPhases = kRtThreads / kRtTok;
  __syncthreads();  // s_z complete
  float zr[R];
#pragma unroll
  for (int j = 0; j < R; ++j) zr[j] = s_z[my_t][j];
  for (int g0 = 0; g0 < ng; g0 += kRtGC) {
    const int gc = min(kRtGC, ng - g0);
    __syncthreads();  // the previous chunk's rows consumed
    for (int e = tid; e < 2 * gc * (R / 8); e += kRtThreads) {
      const int row = e / (R / 8), c8 = e % (R / 8);
      const bf16x8 v = __builtin_bit_cast(bf16x8, *(const u32x4*)(W2 + (size_t)(2 * g0 + row) * R + 8 * c8));
#pragma unroll
      for (int i = 0; i < 8; ++i) s_w2[8 * c8 + i][row] = (float)v[i];
    }
    __syncthreads();
    if (my_t >= ntok) continue;
    for (int gl = phase; gl < gc; gl += kPhases) {
      float l0 = 0.0f, l1 = 0.0f;
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const float2 w = *(const float2*)&s_w2[j][2 * gl];
        l0 = fmaf(w.x, zr[j], l0);
        l1 = fmaf(w.y, zr[j], l1);
      }
      const size_t o = (size_t)(t0 + my_t) * ng + g0 + gl;
      mask[o] = l0 >= l1 ? 1 : 0;
      if (logits) {
        logits[2 * o] = l0;
        logits[2 * o + 1] = l1;
      }
    }
  }
}

#define WIDE_ROUTER_KERNEL(NAME, R, RB, NW)                                                    \
  __global__ __launch_bounds__(64 * NW) void NAME(                                             \
      const uint16_t* __restrict__ X, const uint16_t* __restrict__ W1,                         \
      const uint16_t* __restrict__ W2, int T, int D, int ng, int act,                          \
      uint8_t* __restrict__ mask, float* __restrict__ logits) {                                \
    __shared__ float s_part[NW][16 * RB][R];                                                   \
    __shared__ float s_z[16 * RB][R + 1];                                                      \
    __shared__ __attribute__((aligned(8))) float s_w2[R][2 * kRtGC];                           \
    router_body<R, RB, NW>(X, W1, W2, T, D, ng, act, mask, logits, s_part, s_z, s_w2);         \
  }
WIDE_ROUTER_KERNEL(router_kernel_16, 16, 4, 4)
WIDE_ROUTER_KERNEL(router_kernel_32, 32, 4, 4)
WIDE_ROUTER_KERNEL(router_kernel_64, 64, 4, 4)
WIDE_ROUTER_KERNEL(router_small_kernel_16, 16, 1, 16)
WIDE_ROUTER_KERNEL(router_small_kernel_32, 32, 1, 16)
WIDE_ROUTER_KERNEL(router_small_kernel_64, 64, 1, 16)
#undef WIDE_ROUTER_KERNEL

}  // namespace

hipError_t launch_router_bf16(const uint16_t* X, const uint16_t* W1, const uint16_t* W2, int T,
                              int D, int r, int ng, int act, uint8_t* mask, float* logits,
                              hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (T <= 16) {
    const dim3 grid(1), block(1024);
    if (r == 16)
      hipLaunchKernelGGL(router_small_kernel_16, grid, block, 0, stream, X, W1, W2, T, D, ng, act,
                         mask, logits);
    else if (r == 32)
      hipLaunchKernelGGL(router_small_kernel_32, grid, block, 0, stream, X, W1, W2, T, D, ng, act,
                         mask, logits);
    else
      hipLaunchKernelGGL(router_small_kernel_64, grid, block, 0, stream, X, W1, W2, T, D, ng, act,
                         mask, logits);
    return hipGetLastError();
  }
  const dim3 grid((T + 63) / 64), block(256);
  if (r == 16)
    hipLaunchKernelGGL(router_kernel_16, grid, block, 0, stream, X, W1, W2, T, D, ng, act, mask,
                       logits);
  else if (r == 32)
    hipLaunchKernelGGL(router_kernel_32, grid, block, 0, stream, X, W1, W2, T, D, ng, act, mask,
                       logits);
  else
    hipLaunchKernelGGL(router_kernel_64, grid, block, 0, stream, X, W1, W2, T, D, ng, act, mask,
                       logits);
  return hipGetLastError();
}

}  // namespace wide
