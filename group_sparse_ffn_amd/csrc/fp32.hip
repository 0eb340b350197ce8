// fp32 instantiation of the prefill path, on the vector ALUs (fp32 FMA, no
// reduced-precision mode). Same structure as the bf16 kernels:
//   gate/up: a workgroup owns 16 channels of one group x 64 positions of the
//            group's reordered token list; tiles past the active count exit,
//            rows past it load zeros; silu(gate)*up is formed in the epilogue
//            and scattered to H[token, channel].
//   down:    a workgroup owns Y[64 tokens, 64 output columns]; 16-channel
//            K-blocks inactive for the whole token tile are skipped and H is
//            loaded only for active (token, group) pairs.
// Used for every T when the dtype is fp32 (there is no fp32 decode kernel).
#include "common.h"

namespace wide {

namespace {

constexpr int kTok = 64;
constexpr int kCh = 16;
constexpr int kK = 32;

__global__ __launch_bounds__(256) void gate_up_f32_kernel(
    const float* __restrict__ X, const float* __restrict__ Wg, const float* __restrict__ Wu,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ counts, int T, int d, int d_ff,
    int G, float* __restrict__ H, int zero_inactive, int ntok_tiles, int nct) {
  __shared__ float sx[kTok][kK + 1];
  __shared__ float sg[kCh][kK + 1];
  __shared__ float su[kCh][kK + 1];
  __shared__ int stok[kTok];
  const int tile = blockIdx.x % ntok_tiles;
  const int blk = blockIdx.x / ntok_tiles;
  const int g = blk / nct;
  const int ch0 = g * G + (blk % nct) * kCh;
  const int tile0 = tile * kTok;
  const int count = counts[g];
  const int tid = threadIdx.x;
  if (tile0 >= T) return;
  if (tile0 >= count && !zero_inactive) return;
  if (tid < kTok) stok[tid] = (tile0 + tid < T) ? perm[(size_t)g * T + tile0 + tid] : -1;
  __syncthreads();
  const int tx = tid & 15;  // channel
  const int ty = tid >> 4;  // rows ty*4 .. ty*4+3
  float ag[4] = {0.f, 0.f, 0.f, 0.f}, au[4] = {0.f, 0.f, 0.f, 0.f};
  if (tile0 < count) {
    for (int k0 = 0; k0 < d; k0 += kK) {
      for (int e = tid; e < kTok * kK; e += 256) {
        const int r = e / kK, k = e % kK;
        sx[r][k] = (tile0 + r < count && k0 + k < d) ? X[(size_t)stok[r] * d + k0 + k] : 0.f;
      }
      for (int e = tid; e < kCh * kK; e += 256) {
        const int r = e / kK, k = e % kK;
        const bool ok = k0 + k < d;
        sg[r][k] = ok ? Wg[(size_t)(ch0 + r) * d + k0 + k] : 0.f;
        su[r][k] = ok ? Wu[(size_t)(ch0 + r) * d + k0 + k] : 0.f;
      }
      __syncthreads();
      for (int k = 0; k < kK; ++k) {
        const float wgk = sg[tx][k], wuk = su[tx][k];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ag[i] = fmaf(sx[ty * 4 + i][k], wgk, ag[i]);
          au[i] = fmaf(sx[ty * 4 + i][k], wuk, au[i]);
        }
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty * 4 + i;
    const int pos = tile0 + r;
    if (pos >= T) continue;
    const bool act = pos < count;
    if (!act && !zero_inactive) continue;
    H[(size_t)stok[r] * d_ff + ch0 + tx] = act ? silu_mul(ag[i], au[i]) : 0.0f;
  }
}

__global__ __launch_bounds__(256) void down_f32_kernel(const float* __restrict__ H,
                                                       const float* __restrict__ Wd,
                                                       const uint32_t* __restrict__ maskbits, int T,
                                                       int d, int d_ff, int G,
                                                       float* __restrict__ Y, int nnt, int words) {
  __shared__ float sh[kTok][kCh + 1];
  __shared__ float sw[kTok][kCh + 1];
  __shared__ int s_any;
  const int t0 = (blockIdx.x / nnt) * kTok;
  const int n0 = (blockIdx.x % nnt) * kTok;
  const int tid = threadIdx.x;
  const int tx = tid & 15;  // output columns tx*4 .. tx*4+3
  const int ty = tid >> 4;  // tokens ty*4 .. ty*4+3
  const int w0 = t0 / 32;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < d_ff; k0 += kCh) {
    const int g = k0 / G;
    const uint32_t* mw = maskbits + (size_t)g * words;
    if (tid == 0) {
      uint32_t a = 0;
      if (w0 < words) a |= mw[w0];
      if (w0 + 1 < words) a |= mw[w0 + 1];
      s_any = a != 0;
    }
    __syncthreads();
    const bool any = s_any != 0;
    if (any) {
      for (int e = tid; e < kTok * kCh; e += 256) {
        const int r = e / kCh, k = e % kCh;
        const int t = t0 + r;
        const bool on = t < T && ((mw[t / 32] >> (t % 32)) & 1u);
        sh[r][k] = on ? H[(size_t)t * d_ff + k0 + k] : 0.f;
        sw[r][k] = (n0 + r < d) ? Wd[(size_t)(n0 + r) * d_ff + k0 + k] : 0.f;
      }
    }
    __syncthreads();
    if (any) {
      for (int k = 0; k < kCh; ++k) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(sh[ty * 4 + i][k], sw[tx * 4 + j][k], acc[i][j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < d) Y[(size_t)t * d + n] = acc[i][j];
    }
  }
}

}  // namespace

hipError_t launch_gate_up_f32(const float* X, const float* Wg, const float* Wu,
                              const int32_t* perm, const int32_t* counts, int T, int d, int d_ff,
                              int G, float* H, bool zero_inactive, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int ng = d_ff / G;
  const int nct = G / kCh;
  const int ntok_tiles = (T + kTok - 1) / kTok;
  hipLaunchKernelGGL(gate_up_f32_kernel, dim3(ntok_tiles * ng * nct), dim3(256), 0, stream, X, Wg,
                     Wu, perm, counts, T, d, d_ff, G, H, zero_inactive ? 1 : 0, ntok_tiles, nct);
  return hipGetLastError();
}

hipError_t launch_down_f32(const float* H, const float* Wd, const uint32_t* maskbits, int T, int d,
                           int d_ff, int G, float* Y, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int ntt = (T + kTok - 1) / kTok;
  const int nnt = (d + kTok - 1) / kTok;
  hipLaunchKernelGGL(down_f32_kernel, dim3(ntt * nnt), dim3(256), 0, stream, H, Wd, maskbits, T, d,
                     d_ff, G, Y, nnt, (T + 31) / 32);
  return hipGetLastError();
}

}  // namespace wide
