// Prefill down projection Y = H_masked . Wdown^T on the K axis (the pruned
// axis of the down projection: WIDE paper App. B, "Implementation of GEMM-K").
//
// The pages' GEMM-K runs each active K-group of a reordered token tile as its
// own pipeline and scatters the partial outputs with atomic adds into a
// zero-initialised buffer. On MI355X a measured fp32 global atomic add
// sustains about 1.3 TB/s of payload whatever the footprint, and that design
// issues one atomic per (active token, group, output column): about 15 GB at
// the Llama3.1-8B prefill shape. So this kernel keeps the pages' skipping
// predicates but owns its output tile instead:
//   * a workgroup owns Y[256 tokens (natural order), 256 output columns] and
//     accumulates over the groups in registers; every output has one writer,
//     no atomics, no zero-initialised buffer and a fixed summation order;
//   * K-blocks (64 channels) whose groups are inactive for every token of the
//     tile are skipped whole (copies, barriers and MFMAs): the K-block list is
//     built once per workgroup from the packed mask bits;
//   * H is loaded only for active (token, group) pairs; inactive pairs load
//     zeros, so H needs no initialisation at masked channels.
// Same data movement as the gate/up kernel: 16-byte loads one K-step ahead,
// two XOR-swizzled LDS stages, v_mfma_f32_32x32x16_bf16 on 4 waves (2 x 2),
// each wave 128 output columns x 128 tokens.
#include "common.h"

namespace wide {

namespace {

constexpr int kTile = 256;
constexpr int kMaxSteps = 1024;  // d_ff / 64 limit (d_ff <= 65536)

__global__ __launch_bounds__(256, 1) void down_bf16_kernel(
    const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wd,
    const uint32_t* __restrict__ maskbits, int T, int d, int d_ff, int G, uint16_t* __restrict__ Y,
    int ntt, int nnt, int words) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kTile * 64];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kTile * 64];
  __shared__ uint16_t s_steps[kMaxSteps];
  __shared__ int s_wave_cnt[4];

  const int total = ntt * nnt;
  const int per_xcd = (total + 7) / 8;
  const int L = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (L >= total) return;
  const int t0 = (L / nnt) * kTile;
  const int n0 = (L % nnt) * kTile;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int w0 = t0 / 32;  // first mask word of this token tile

  // K-block admission: keep the 64-channel blocks with any active token.
  const int ksteps = d_ff / 64;
  int nst = 0;
  for (int s0 = 0; s0 < ksteps; s0 += 256) {
    const int s = s0 + tid;
    bool any = false;
    if (s < ksteps) {
      const int glo = (s * 64) / G;
      const int ghi = (s * 64 + 63) / G;
      uint32_t acc = 0;
      for (int g = glo; g <= ghi; ++g) {
        const uint32_t* mw = maskbits + (size_t)g * words;
#pragma unroll
        for (int wi = 0; wi < 8; ++wi)
          if (w0 + wi < words) acc |= mw[w0 + wi];
      }
      any = acc != 0;
    }
    const uint64_t bal = __ballot(any);
    if (lane == 0) s_wave_cnt[wave] = __popcll(bal);
    __syncthreads();
    int base = nst;
    for (int w = 0; w < wave; ++w) base += s_wave_cnt[w];
    if (any) {
      const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      s_steps[base + rank] = (uint16_t)s;
    }
    for (int w = 0; w < 4; ++w) nst += s_wave_cnt[w];
    __syncthreads();
  }

  const int kc = tid & 7;
  const int rsub = tid >> 3;  // this thread stages rows rsub + 32*i, i = 0..7
  // Row i of a thread is 32*i rows below row 0, so one base per operand does.
  const uint16_t* pa0 = Wd + (size_t)(n0 + rsub) * d_ff + kc * 8;
  const uint16_t* pb0 = H + (size_t)(t0 + rsub) * d_ff + kc * 8;
  const size_t rstride = (size_t)32 * d_ff;
  const int a_rows = d - n0 - rsub;  // row i valid iff 32*i < a_rows
  const int b_rows = T - t0 - rsub;

  u32x4 ra[8], rb[8];
  auto load_step = [&](int k0) {
    // mask bits of this thread's 8 token rows for the group of its chunk
    const int gq = (k0 + kc * 8) / G;
    const uint32_t* mw = maskbits + (size_t)gq * words + w0;
    uint32_t bits[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) bits[i] = (w0 + i < words) ? mw[i] : 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ra[i] = (32 * i < a_rows) ? *(const u32x4*)(pa0 + i * rstride + k0) : u32x4{0u, 0u, 0u, 0u};
      const bool on = 32 * i < b_rows && ((bits[i] >> rsub) & 1u);
      rb[i] = on ? *(const u32x4*)(pb0 + i * rstride + k0) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_step = [&](int s) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = rsub + 32 * i;
      *(u32x4*)(&sA[s][swz(r, kc) * 8]) = ra[i];
      *(u32x4*)(&sB[s][swz(r, kc) * 8]) = rb[i];
    }
  };

  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int lrow = lane & 31;
  const int lhalf = lane >> 5;

  f32x16 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.0f;

  if (nst > 0) {
    load_step(s_steps[0] * 64);
    store_step(0);
  }
  __syncthreads();
  for (int it = 0; it < nst; ++it) {
    const int cur = it & 1;
    if (it + 1 < nst) load_step(s_steps[it + 1] * 64);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int chunk = kk * 2 + lhalf;
      bf16x8 a[4], b[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int row = wm * 128 + mi * 32 + lrow;
        a[mi] = __builtin_bit_cast(bf16x8, *(const u32x4*)(&sA[cur][swz(row, chunk) * 8]));
      }
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int row = wn * 128 + ni * 32 + lrow;
        b[ni] = __builtin_bit_cast(bf16x8, *(const u32x4*)(&sB[cur][swz(row, chunk) * 8]));
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
    if (it + 1 < nst) store_step(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds token (lane & 31) of each N fragment and output
  // columns 8*(j/4) + 4*(lane/32) + (j%4) of each M fragment.
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    const int t = t0 + wn * 128 + ni * 32 + lrow;
    if (t >= T) continue;
    uint16_t* yrow = Y + (size_t)t * d;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int nb = n0 + wm * 128 + mi * 32;
      if (nb >= d) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = 4 * q;
        u32x2 v = {pack_bf16x2(acc[mi][ni][j], acc[mi][ni][j + 1]),
                   pack_bf16x2(acc[mi][ni][j + 2], acc[mi][ni][j + 3])};
        *(u32x2*)(yrow + nb + 8 * q + 4 * lhalf) = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_down_bf16(const uint16_t* H, const uint16_t* Wd, const uint32_t* maskbits, int T,
                            int d, int d_ff, int G, uint16_t* Y, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int ntt = (T + kTile - 1) / kTile;
  const int nnt = (d + kTile - 1) / kTile;
  const int words = (T + 31) / 32;
  const int total = ntt * nnt;
  const int per_xcd = (total + 7) / 8;
  hipLaunchKernelGGL(down_bf16_kernel, dim3(per_xcd * 8), dim3(256), 0, stream, H, Wd, maskbits, T,
                     d, d_ff, G, Y, ntt, nnt, words);
  return hipGetLastError();
}

}  // namespace wide
