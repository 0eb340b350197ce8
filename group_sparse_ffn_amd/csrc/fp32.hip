// fp32 instantiation of the prefill path, on the vector ALUs (fp32 FMA, no
// reduced-precision mode). Same structure as the bf16 kernels:
//   gate/up: a workgroup owns 16 channels of one group x 64 positions of the
//            group's reordered token list; tiles past the active count exit,
//            rows past it load zeros; silu(gate)*up is formed in the epilogue
//            and scattered to H[token, channel].
//   down:    a workgroup owns Y[32 tokens, 64 output columns]; the 16-channel
//            K-blocks inactive for the whole token tile are skipped (listed
//            once) and H counts only at active (token, group) pairs.
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

constexpr int kDnTok = 32;     // tokens per down tile
constexpr int kDnCol = 64;     // output columns per down tile
constexpr int kMaxBlocks = 4096;  // 16-channel K-blocks (d_ff <= 65536)

// Down projection, fp32: a workgroup owns Y[32 tokens, 64 columns]. The
// 16-channel K-blocks with an active token in the tile are listed once; the
// operands of block i + 1 are loaded into registers while block i is
// multiplied from LDS (double-buffered), so the loop waits on one barrier per
// block and its loads overlap the FMAs. H is loaded in bounds and replaced by
// 0 where the (token, group) is inactive, so its value there never matters.
__global__ __launch_bounds__(256) void down_f32_kernel(const float* __restrict__ H,
                                                       const float* __restrict__ Wd,
                                                       const uint32_t* __restrict__ maskbits, int T,
                                                       int d, int d_ff, int G,
                                                       float* __restrict__ Y, int nnt, int words) {
  __shared__ float sh[2][kDnTok][kCh + 1];
  __shared__ float sw[2][kDnCol][kCh + 1];
  __shared__ uint16_t s_blk[kMaxBlocks];
  __shared__ int s_wave_cnt[4];
  const int t0 = (blockIdx.x / nnt) * kDnTok;
  const int n0 = (blockIdx.x % nnt) * kDnCol;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int w0 = t0 / 32;  // one mask word covers the 32-token tile
  const int nblk = d_ff / kCh;
  int nlive = 0;
  for (int b0 = 0; b0 < nblk; b0 += 256) {
    const int b = b0 + tid;
    const bool any = b < nblk && w0 < words && maskbits[(size_t)((b * kCh) / G) * words + w0] != 0;
    const uint64_t bal = __ballot(any);
    if (lane == 0) s_wave_cnt[wave] = __popcll(bal);
    __syncthreads();
    int base = nlive;
    for (int w = 0; w < wave; ++w) base += s_wave_cnt[w];
    if (any) {
      const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      s_blk[base + rank] = (uint16_t)b;
    }
    for (int w = 0; w < 4; ++w) nlive += s_wave_cnt[w];
    __syncthreads();
  }
  // this thread's operand elements per block: H row r = tid / 8, channels
  // 2 (tid % 8) .. +1; Wd rows tid / 8 and 32 + tid / 8, the same channels.
  // Loads run kAhead blocks ahead in a ring of register sets (the loop is
  // unrolled by kAhead so every set index is a constant).
  constexpr int kAhead = 4;
  const int hr = tid >> 3, hk = 2 * (tid & 7);
  const int th = min(t0 + hr, T - 1);
  const int nw0 = min(n0 + hr, d - 1), nw1 = min(n0 + 32 + hr, d - 1);
  float rh[kAhead][2], rw[kAhead][4];
  uint32_t rm[kAhead];
  auto load = [&](int i, float (&h)[2], float (&w)[4], uint32_t& m) {
    const int k0 = (int)s_blk[i] * kCh + hk;
    m = maskbits[(size_t)(k0 / G) * words + w0];
    h[0] = H[(size_t)th * d_ff + k0];
    h[1] = H[(size_t)th * d_ff + k0 + 1];
    w[0] = Wd[(size_t)nw0 * d_ff + k0];
    w[1] = Wd[(size_t)nw0 * d_ff + k0 + 1];
    w[2] = Wd[(size_t)nw1 * d_ff + k0];
    w[3] = Wd[(size_t)nw1 * d_ff + k0 + 1];
  };
  const int tx = tid & 15;  // output columns tx * 4 .. + 3
  const int ty = tid >> 4;  // tokens ty * 2 .. + 1
  float acc[2][4] = {};
#pragma unroll
  for (int q = 0; q < kAhead; ++q)
    if (q < nlive) load(q, rh[q], rw[q], rm[q]);
  auto step = [&](int i, float (&h)[2], float (&w)[4], uint32_t& m) {
    const int buf = i & 1;
    const bool on = t0 + hr < T && ((m >> hr) & 1u);
    sh[buf][hr][hk] = on ? h[0] : 0.f;
    sh[buf][hr][hk + 1] = on ? h[1] : 0.f;
    sw[buf][hr][hk] = w[0];
    sw[buf][hr][hk + 1] = w[1];
    sw[buf][32 + hr][hk] = w[2];
    sw[buf][32 + hr][hk + 1] = w[3];
    __syncthreads();
    if (i + kAhead < nlive) load(i + kAhead, h, w, m);
    for (int k = 0; k < kCh; ++k) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[a][j] = fmaf(sh[buf][ty * 2 + a][k], sw[buf][tx * 4 + j][k], acc[a][j]);
    }
  };
  for (int i = 0; i < nlive; i += kAhead) {
#pragma unroll
    for (int q = 0; q < kAhead; ++q)
      if (i + q < nlive) step(i + q, rh[q], rw[q], rm[q]);
  }
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int t = t0 + ty * 2 + a;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < d) Y[(size_t)t * d + n] = acc[a][j];
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
  const int ntt = (T + kDnTok - 1) / kDnTok;
  const int nnt = (d + kDnCol - 1) / kDnCol;
  hipLaunchKernelGGL(down_f32_kernel, dim3(ntt * nnt), dim3(256), 0, stream, H, Wd, maskbits, T, d,
                     d_ff, G, Y, nnt, (T + 31) / 32);
  return hipGetLastError();
}

}  // namespace wide
