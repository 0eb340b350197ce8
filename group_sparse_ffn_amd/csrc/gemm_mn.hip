// Prefill gate/up projection over reordered tokens (WIDE paper App. B,
// "Implementation of GEMM-MN": each workgroup owns one output tile whose
// N coordinate selects a routing group; admission, predicated computation and
// a scatter epilogue).
//
// Workgroup tile: CW channels of one group (CW gate rows + CW up rows = the
// MFMA M side, 2*CW <= 256) x 256 tokens taken from the group's reordered
// token list (the MFMA N side), K = d in steps of 64. Skipping, as in the
// pages' three levels, re-derived for gfx950:
//   level 0: a workgroup whose 256-token tile starts at or past the group's
//            active count exits before touching memory;
//   level 1: token rows past the active count are never loaded (zeros go to
//            LDS instead);
//   level 2: 32-token MFMA fragments that lie wholly past the count are not
//            multiplied.
// The epilogue computes silu(gate) * up in fp32, rounds once to bf16 (RNE) and
// scatters each token's row segment to H[token, channels].
//
// Data movement: 16-byte global loads into registers one K-step ahead, two
// LDS stages (XOR-swizzled 128-byte rows), one barrier per K-step,
// v_mfma_f32_32x32x16_bf16 on 4 waves. The gate and up rows of the same
// channels are interleaved in LDS so that each lane holds both accumulators of
// a (channel, token) pair and the epilogue needs no data exchange.
#include "common.h"

namespace wide {

namespace {

template <int CW>
struct MnCfg {
  static constexpr int kRows = 2 * CW;               // gate + up rows in the tile
  static constexpr int kWM = (CW == 128) ? 2 : 1;    // waves along M
  static constexpr int kWN = 4 / kWM;                // waves along N (tokens)
  static constexpr int kRowsPerWave = kRows / kWM;   // gate half + up half
  static constexpr int kFM = kRowsPerWave / 32;      // 32-row MFMA fragments per wave
  static constexpr int kFN = 256 / kWN / 32;         // 32-token fragments per wave
  static constexpr int kAChunks = kRows * 8 / 256;   // 16-byte A chunks per thread per step
};

constexpr int kTokTile = 256;

template <int CW>
__global__ __launch_bounds__(256, 1) void gate_up_bf16_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wg,
    const uint16_t* __restrict__ Wu, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ counts, int T, int d, int d_ff, int G, uint16_t* __restrict__ H,
    int zero_inactive, int ntok_tiles, int nct, int total) {
  using C = MnCfg<CW>;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][C::kRows * 64];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kTokTile * 64];

  // XCD-aware order: consecutive workgroup ids go to different XCDs, so give
  // each XCD a contiguous range of (channel block, token tile) pairs; the
  // tiles of one channel block then share their weight rows in one L2.
  const int per_xcd = (total + 7) / 8;
  const int L = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (L >= total) return;
  const int blk = L / ntok_tiles;
  const int tile0 = (L % ntok_tiles) * kTokTile;
  const int g = blk / nct;
  const int ct = blk % nct;
  const int count = counts[g];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int32_t* __restrict__ prow = perm + (size_t)g * T + tile0;
  const int ch0 = g * G + ct * CW;  // first channel of this tile

  if (tile0 >= count) {
    // level 0: nothing active here. Only when H must hold exact zeros at
    // masked channels do the inactive tokens of this tile get written.
    if (!zero_inactive) return;
    const int r = tid;
    if (tile0 + r < T) {
      u32x4* dst = (u32x4*)(H + (size_t)prow[r] * d_ff + ch0);
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int c = 0; c < CW / 8; ++c) dst[c] = z;
    }
    return;
  }

  const int kc = tid & 7;  // this thread's 16-byte chunk within a 64-wide K step

  // A (weight) rows this thread stages: LDS row r -> gate/up row of channel.
  // Element offsets (they fit in 32 bits: d_ff*d and T*d stay below 2^31).
  int oa[C::kAChunks];
  bool agate[C::kAChunks];
#pragma unroll
  for (int i = 0; i < C::kAChunks; ++i) {
    const int r = (tid + 256 * i) >> 3;
    const int wmi = r / C::kRowsPerWave;
    const int within = r % C::kRowsPerWave;
    constexpr int half = C::kRowsPerWave / 2;
    agate[i] = within < half;
    const int ch = ch0 + wmi * half + (agate[i] ? within : within - half);
    oa[i] = ch * d + kc * 8;
  }
  // B (token) rows this thread stages; level 1: rows past the count get -1.
  int ob[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (tid >> 3) + 32 * i;
    ob[i] = (tile0 + r < count) ? prow[r] * d + kc * 8 : -1;
  }

  u32x4 ra[C::kAChunks];
  u32x4 rb[8];
  auto load_step = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::kAChunks; ++i)
      ra[i] = *(const u32x4*)((agate[i] ? Wg : Wu) + oa[i] + k0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      rb[i] = (ob[i] >= 0) ? *(const u32x4*)(X + ob[i] + k0) : u32x4{0u, 0u, 0u, 0u};
  };
  auto store_step = [&](int s) {
#pragma unroll
    for (int i = 0; i < C::kAChunks; ++i) {
      const int r = (tid + 256 * i) >> 3;
      *(u32x4*)(&sA[s][swz(r, kc) * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (tid >> 3) + 32 * i;
      *(u32x4*)(&sB[s][swz(r, kc) * 8]) = rb[i];
    }
  };

  const int wm = wave / C::kWN;
  const int wn = wave % C::kWN;
  // level 2: fragments of this wave that hold at least one active token
  const int wtok0 = tile0 + wn * C::kFN * 32;
  int nact = (count - wtok0 + 31) / 32;
  nact = nact < 0 ? 0 : (nact > C::kFN ? C::kFN : nact);

  f32x16 acc[C::kFM][C::kFN];
#pragma unroll
  for (int mi = 0; mi < C::kFM; ++mi)
#pragma unroll
    for (int ni = 0; ni < C::kFN; ++ni)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.0f;

  const int nsteps = d / 64;
  load_step(0);
  store_step(0);
  __syncthreads();
  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
  for (int step = 0; step < nsteps; ++step) {
    const int cur = step & 1;
    if (step + 1 < nsteps) load_step((step + 1) * 64);
    if (nact > 0) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int chunk = kk * 2 + lhalf;
        bf16x8 a[C::kFM], b[C::kFN];
#pragma unroll
        for (int mi = 0; mi < C::kFM; ++mi) {
          const int row = wm * C::kRowsPerWave + mi * 32 + lrow;
          a[mi] = __builtin_bit_cast(bf16x8, *(const u32x4*)(&sA[cur][swz(row, chunk) * 8]));
        }
#pragma unroll
        for (int ni = 0; ni < C::kFN; ++ni) {
          const int row = wn * C::kFN * 32 + ni * 32 + lrow;
          b[ni] = __builtin_bit_cast(bf16x8, *(const u32x4*)(&sB[cur][swz(row, chunk) * 8]));
        }
#pragma unroll
        for (int ni = 0; ni < C::kFN; ++ni) {
          if (ni < nact) {
#pragma unroll
            for (int mi = 0; mi < C::kFM; ++mi)
              acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
          }
        }
      }
    }
    if (step + 1 < nsteps) store_step(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds token (lane & 31) of each N fragment and, per M
  // fragment, rows 8*(j/4) + 4*(lane/32) + (j%4) for j = 0..15.
  constexpr int half = C::kRowsPerWave / 2;
#pragma unroll
  for (int ni = 0; ni < C::kFN; ++ni) {
    const int i = wtok0 + ni * 32 + lrow;  // position in the group's token list
    if (i >= T) continue;
    const bool act = i < count;
    if (!act && !zero_inactive) continue;
    uint16_t* hrow = H + (size_t)prow[i - tile0] * d_ff + ch0 + wm * half;
    if constexpr (C::kFM >= 2) {
#pragma unroll
      for (int p = 0; p < C::kFM / 2; ++p) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float h[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int j = 4 * q + jj;
            h[jj] = act ? silu_mul(acc[p][ni][j], acc[p + C::kFM / 2][ni][j]) : 0.0f;
          }
          u32x2 v = {pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
          *(u32x2*)(hrow + p * 32 + 8 * q + 4 * lhalf) = v;
        }
      }
    } else {
      // CW == 16: one fragment holds gate rows 0..15 (j < 8) and up rows 16..31 (j >= 8).
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float h[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = 4 * q + jj;
          h[jj] = act ? silu_mul(acc[0][ni][j], acc[0][ni][j + 8]) : 0.0f;
        }
        u32x2 v = {pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
        *(u32x2*)(hrow + 8 * q + 4 * lhalf) = v;
      }
    }
  }
}

template <int CW>
hipError_t launch_cw(const uint16_t* X, const uint16_t* Wg, const uint16_t* Wu, const int32_t* perm,
                     const int32_t* counts, int T, int d, int d_ff, int G, uint16_t* H,
                     bool zero_inactive, hipStream_t stream) {
  const int ng = d_ff / G;
  const int nct = G / CW;
  const int ntok_tiles = (T + kTokTile - 1) / kTokTile;
  const long long total = (long long)ng * nct * ntok_tiles;
  const int per_xcd = (int)((total + 7) / 8);
  hipLaunchKernelGGL(gate_up_bf16_kernel<CW>, dim3(per_xcd * 8), dim3(256), 0, stream, X, Wg, Wu,
                     perm, counts, T, d, d_ff, G, H, zero_inactive ? 1 : 0, ntok_tiles, nct,
                     (int)total);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_bf16(const uint16_t* X, const uint16_t* Wg, const uint16_t* Wu,
                               const int32_t* perm, const int32_t* counts, int T, int d, int d_ff,
                               int G, uint16_t* H, bool zero_inactive, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (G % 128 == 0)
    return launch_cw<128>(X, Wg, Wu, perm, counts, T, d, d_ff, G, H, zero_inactive, stream);
  if (G % 64 == 0)
    return launch_cw<64>(X, Wg, Wu, perm, counts, T, d, d_ff, G, H, zero_inactive, stream);
  if (G % 32 == 0)
    return launch_cw<32>(X, Wg, Wu, perm, counts, T, d, d_ff, G, H, zero_inactive, stream);
  return launch_cw<16>(X, Wg, Wu, perm, counts, T, d, d_ff, G, H, zero_inactive, stream);
}

}  // namespace wide
