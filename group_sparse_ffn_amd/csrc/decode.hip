// Decode fast path (T <= 16 tokens): no mask reorder; routing is checked
// directly (WIDE paper App. B, "Implementation of Attention": for decoding
// the routing can be checked without reordering; App. B GEMM-MN/GEMM-K:
// GEMV variants for small M; Sec. 1: dedicated fast paths for decoding).
//
// Both kernels are bound by streaming weights from HBM. The 16 tokens sit on
// the N side of v_mfma_f32_16x16x32_bf16 (tokens past T read as zeros), so
// the matrix core does the dot products and every weight byte is loaded once
// per call with 16-byte lane loads (four lanes cover 64 contiguous bytes of a
// row per instruction).
//
// gate/up: a workgroup owns 16 channels of one group; its four waves split
//   K = d and meet in LDS. A group no token executes costs one mask read.
//   Output: H[t, c] = silu(gate)*up, or +0.0 where the token skips the group.
// down:    a workgroup owns 16 output rows; it lists the 32-channel chunks
//   whose group some token executes and its four waves split that list. Only
//   those segments of each Wdown row are read; one writer per output.
#include "common.h"

namespace wide {

namespace {

constexpr int kUnroll = 8;

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *(const u32x4*)p; }

__global__ __launch_bounds__(256) void decode_gate_up_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wg,
    const uint16_t* __restrict__ Wu, const uint8_t* __restrict__ mask, int T, int d, int d_ff,
    int G, uint16_t* __restrict__ H, int zero_inactive) {
  __shared__ float s_red[4][64][8];
  const int ng = d_ff / G;
  const int c0 = blockIdx.x * 16;
  const int g = c0 / G;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  const bool mine = lane < T && mask[(size_t)lane * ng + g] != 0;
  if (__ballot(mine) == 0) {
    // no token executes this group: its weights are never read
    if (zero_inactive && tid < T * 2) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      *(u32x4*)(H + (size_t)(tid >> 1) * d_ff + c0 + (tid & 1) * 8) = z;
    }
    return;
  }

  // wave w takes the 32-wide K slices [s_lo, s_hi) of d / 32
  const int nsub_all = d / 32;
  const int s_lo = (wave * nsub_all) / 4;
  const int s_hi = ((wave + 1) * nsub_all) / 4;
  const int kbase = s_lo * 32 + 8 * (lane >> 4);
  const int row = c0 + (lane & 15);
  const int tok = lane & 15;
  const uint16_t* pg = Wg + (size_t)row * d + kbase;
  const uint16_t* pu = Wu + (size_t)row * d + kbase;
  const uint16_t* px = (tok < T) ? X + (size_t)tok * d + kbase : nullptr;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  f32x4 acc_g = {0.f, 0.f, 0.f, 0.f}, acc_u = {0.f, 0.f, 0.f, 0.f};
  const int nsub = s_hi - s_lo;
  int s = 0;
  for (; s + kUnroll <= nsub; s += kUnroll) {
    u32x4 ag[kUnroll], au[kUnroll], bx[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      ag[u] = ld16(pg + 32 * (s + u));
      au[u] = ld16(pu + 32 * (s + u));
      bx[u] = px ? ld16(px + 32 * (s + u)) : zero;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const bf16x8 b = __builtin_bit_cast(bf16x8, bx[u]);
      acc_g = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ag[u]), b, acc_g, 0, 0, 0);
      acc_u = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, au[u]), b, acc_u, 0, 0, 0);
    }
  }
  for (; s < nsub; ++s) {
    const bf16x8 b = __builtin_bit_cast(bf16x8, px ? ld16(px + 32 * s) : zero);
    acc_g = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ld16(pg + 32 * s)), b, acc_g, 0, 0, 0);
    acc_u = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ld16(pu + 32 * s)), b, acc_u, 0, 0, 0);
  }

#pragma unroll
  for (int j = 0; j < 4; ++j) {
    s_red[wave][lane][j] = acc_g[j];
    s_red[wave][lane][4 + j] = acc_u[j];
  }
  __syncthreads();
  if (wave != 0 || tok >= T) return;
  // lane holds rows (channels) 4*(lane/16) + j and column (token) lane % 16
  // A token that skips this group still gets +0.0 here: the down GEMV reads
  // every channel of a group that some token executes.
  const bool act = mask[(size_t)tok * ng + g] != 0;
  float h[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float gs = s_red[0][lane][j] + s_red[1][lane][j] + s_red[2][lane][j] + s_red[3][lane][j];
    const float us = s_red[0][lane][4 + j] + s_red[1][lane][4 + j] + s_red[2][lane][4 + j] +
                     s_red[3][lane][4 + j];
    h[j] = act ? silu_mul(gs, us) : 0.0f;
  }
  u32x2 v = {pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
  *(u32x2*)(H + (size_t)tok * d_ff + c0 + 4 * (lane >> 4)) = v;
}

__global__ __launch_bounds__(256) void decode_down_kernel(
    const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wd,
    const uint8_t* __restrict__ mask, int T, int d, int d_ff, int G, uint16_t* __restrict__ Y) {
  constexpr int kMaxChunks = 2048;  // d_ff / 32 limit
  __shared__ uint16_t s_chunks[kMaxChunks];
  __shared__ int s_wave_cnt[4];
  __shared__ float s_red[4][64][4];
  const int ng = d_ff / G;
  const int n0 = blockIdx.x * 16;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // chunks (32 channels) whose group some token executes
  const int nchunks = d_ff / 32;
  int nch = 0;
  for (int b0 = 0; b0 < nchunks; b0 += 256) {
    const int ch = b0 + tid;
    bool any = false;
    if (ch < nchunks) {
      const int glo = (ch * 32) / G;
      const int ghi = (ch * 32 + 31) / G;
      for (int t = 0; t < T && !any; ++t)
        for (int g = glo; g <= ghi; ++g) any |= mask[(size_t)t * ng + g] != 0;
    }
    const uint64_t bal = __ballot(any);
    if (lane == 0) s_wave_cnt[wave] = __popcll(bal);
    __syncthreads();
    int base = nch;
    for (int w = 0; w < wave; ++w) base += s_wave_cnt[w];
    if (any) {
      const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      s_chunks[base + rank] = (uint16_t)ch;
    }
    for (int w = 0; w < 4; ++w) nch += s_wave_cnt[w];
    __syncthreads();
  }

  const int koff = 8 * (lane >> 4);
  const int tok = lane & 15;
  const uint16_t* pw = Wd + (size_t)(n0 + (lane & 15)) * d_ff + koff;
  const uint16_t* ph = (tok < T) ? H + (size_t)tok * d_ff + koff : nullptr;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int i = wave;
  for (; i + 4 * (kUnroll - 1) < nch; i += 4 * kUnroll) {
    u32x4 a[kUnroll], b[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int k = (int)s_chunks[i + 4 * u] * 32;
      a[u] = ld16(pw + k);
      b[u] = ph ? ld16(ph + k) : zero;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[u]),
                                                    __builtin_bit_cast(bf16x8, b[u]), acc, 0, 0, 0);
  }
  for (; i < nch; i += 4) {
    const int k = (int)s_chunks[i] * 32;
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ld16(pw + k)),
                                                  __builtin_bit_cast(bf16x8, ph ? ld16(ph + k) : zero),
                                                  acc, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) s_red[wave][lane][j] = acc[j];
  __syncthreads();
  if (wave != 0 || tok >= T) return;
  float y[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    y[j] = s_red[0][lane][j] + s_red[1][lane][j] + s_red[2][lane][j] + s_red[3][lane][j];
  u32x2 v = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
  *(u32x2*)(Y + (size_t)tok * d + n0 + 4 * (lane >> 4)) = v;
}

}  // namespace

hipError_t launch_decode_gate_up_bf16(const uint16_t* X, const uint16_t* Wg, const uint16_t* Wu,
                                      const uint8_t* mask, int T, int d, int d_ff, int G,
                                      uint16_t* H, bool zero_inactive, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_gate_up_kernel, dim3(d_ff / 16), dim3(256), 0, stream, X, Wg, Wu, mask,
                     T, d, d_ff, G, H, zero_inactive ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_decode_down_bf16(const uint16_t* H, const uint16_t* Wd, const uint8_t* mask,
                                   int T, int d, int d_ff, int G, uint16_t* Y, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_down_kernel, dim3(d / 16), dim3(256), 0, stream, H, Wd, mask, T, d,
                     d_ff, G, Y);
  return hipGetLastError();
}

}  // namespace wide
