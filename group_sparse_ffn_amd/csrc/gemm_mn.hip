// Prefill gate/up projection over reordered tokens (WIDE paper App. B,
// "Implementation of GEMM-MN": each workgroup owns one output tile whose
// N coordinate selects a routing group; admission, predicated computation and
// a scatter epilogue).
//
// Workgroup tile: CW = min(G, 128) channels of one group and 256 positions of
// the group's reordered token list. The MFMA A side holds the CW gate rows and
// the CW up rows of those channels (per wave: its gate half first, then the
// up half of the same channels, so one lane holds both accumulators of a
// (channel, token) pair); the MFMA B side holds the gathered token rows of X.
// The three skipping levels of the pages, re-derived for gfx950:
//   level 0: a workgroup whose 256-position tile starts at or past the group's
//            active count does no MFMA work at all;
//   level 1: token rows past the active count are never fetched: their copies
//            use an out-of-range buffer offset, which writes zeros to LDS
//            without touching memory;
//   level 2: 32-token MFMA fragments that lie wholly past the count are not
//            multiplied.
// Epilogue: silu(gate) * up in fp32, rounded once to bf16 (RNE), staged
// through LDS and scattered as 16-byte row segments to H[token, channels].
// With zero_inactive, every (token, channel) of the group that the token skips
// is also written as +0.0 (an H returned to the caller, or a down projection
// that cannot skip those copies); otherwise only active pairs are written.
#include "mfma_core.h"

namespace wide {

namespace {

constexpr int kTokTile = 256;

template <int CW>
struct MnShape {
  static constexpr int TP = 2 * CW;
  static constexpr int WP = (TP >= 256) ? 2 : 1;
  static constexpr int WQ = 8 / WP;
  using S = core::Shape<TP, kTokTile, WP, WQ>;
  static constexpr int PBLK = S::PBLOCKS, QBLK = S::QBLOCKS;
  static constexpr int NBLK = PBLK + QBLK;
  static constexpr int MAXB = (NBLK + 7) / 8;  // copy blocks per wave (upper bound)
  static constexpr int HALF = S::PW / 2;       // channels per wave
};

// The body is a device function template called from one plain kernel per
// channel width (a kernel template that passes a local lambda to the mainloop
// loses its host launch stub with this toolchain).
template <int CW>
__device__ __forceinline__ void gate_up_body(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wg,
    const uint16_t* __restrict__ Wu, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ counts, int T, int d, int d_ff, int G, uint16_t* __restrict__ H,
    int zero_inactive, int ntok_tiles, int nct, int total, uint8_t* sA, uint8_t* sB,
    int* s_tok) {
  using C = MnShape<CW>;
  using S = typename C::S;

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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ch0 = g * G + ct * CW;  // first channel of this tile
  const int32_t* __restrict__ prow = perm + (size_t)g * T + tile0;
  const int nrows = min(kTokTile, T - tile0);  // positions that exist
  const int nact = max(0, min(nrows, count - tile0));  // active positions

  if (tid < kTokTile) s_tok[tid] = tid < nrows ? prow[tid] : 0;
  __syncthreads();

  // Zeros for the positions of this tile whose token skips the group.
  if (zero_inactive) {
    constexpr int kChunks = CW / 8;  // 16-byte chunks per row segment
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int e = nact * kChunks + tid; e < nrows * kChunks; e += 512) {
      const int r = e / kChunks, c = e % kChunks;
      *(u32x4*)(H + (size_t)s_tok[r] * d_ff + ch0 + c * 8) = z;
    }
  }
  if (nact == 0) return;  // level 0

  // ---- copies: blocks [0, PBLK) are weight rows, [PBLK, NBLK) token rows.
  // Wave w issues blocks w, w+8, ...; lane offsets are fixed per block.
  uint32_t voff[C::MAXB];
#pragma unroll
  for (int i = 0; i < C::MAXB; ++i) {
    const int b = wave + 8 * i;
    const int chunk = core::copy_chunk(b, lane);
    if (b < C::PBLK) {
      // LDS row r -> (wave wp = r / PW, half) -> channel row of Wg or Wu
      const int r = 8 * b + (lane >> 3);
      const int within = r % S::PW;
      const int chan = ch0 + (r / S::PW) * C::HALF + (within % C::HALF);
      voff[i] = (uint32_t)(chan * d + chunk * 8) * 2u;
    } else if (b < C::NBLK) {
      const int r = 8 * (b - C::PBLK) + (lane >> 3);
      voff[i] = r < nact ? (uint32_t)(s_tok[r] * d + chunk * 8) * 2u : 0x80000000u;
    } else {
      voff[i] = 0;
    }
  }
  const uint32_t x_bytes = (uint32_t)T * (uint32_t)d * 2u;
  auto issue = [&](int s, uint8_t* stage) {
    const int k0 = s * core::kBK;
    // token rows: out-of-range offsets fill zeros (level 1)
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(X + k0), 0, (int)(x_bytes - 2u * k0), 0x00020000);
#pragma unroll
    for (int i = 0; i < C::MAXB; ++i) {
      const int b = wave + 8 * i;
      if (b < C::PBLK) {
        const int r0 = 8 * b;
        const bool gate = (r0 % S::PW) < C::HALF;
        const uint16_t* base = (gate ? Wg : Wu) + k0;
        __builtin_amdgcn_global_load_lds((const void*)((const char*)base + voff[i]),
                                         (void*)(stage + b * 1024), 16, 0, 0);
      } else if (b < C::NBLK) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (void*)(stage + b * 1024), 16, voff[i], 0, 0,
                                                 0);
      }
    }
  };

  const int wp = wave / S::WQ;
  const int wq = wave % S::WQ;
  // level 2: this wave's 32-token fragments that hold an active position
  const int nq = max(0, min(S::FQ, (nact - wq * S::QW + 31) / 32));
  core::Frags<S> f;
  core::mainloop<S>(f, sA, sB, d / core::kBK, wp, wq, lane, nq, issue);
  __syncthreads();  // every wave is done with the stages: reuse them for the epilogue

  // ---- epilogue: silu(gate) * up -> bf16, staged as [256 positions][CW] in LDS.
  constexpr int kRowB = CW * 2;      // bytes per staged row
  constexpr int kCpr = CW / 8;       // 16-byte chunks per staged row
  uint8_t* stg = sA;                 // 256 * kRowB <= 64 KB fits in one stage
  const int lrow = lane & 31, lhalf = lane >> 5;
#pragma unroll
  for (int j = 0; j < S::FQ; ++j) {
    const int r = wq * S::QW + j * 32 + lrow;  // position in the tile
    if constexpr (S::FP >= 2) {
#pragma unroll
      for (int i = 0; i < S::FP / 2; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            h[e] = silu_mul(f.acc[i][j][4 * q + e], f.acc[i + S::FP / 2][j][4 * q + e]);
          const int cl = wp * C::HALF + i * 32 + 8 * q + 4 * lhalf;  // channel within tile
          const int c = cl >> 3, hh = (cl >> 2) & 1;
          const u32x2 v = {pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
          *(u32x2*)(stg + r * kRowB + ((c ^ (r % kCpr)) << 4) + hh * 8) = v;
        }
      }
    } else {
      // CW == 16: one fragment holds gate rows 0..15 (e < 8) and up rows 16..31 (e >= 8)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = silu_mul(f.acc[0][j][4 * q + e], f.acc[0][j][4 * q + e + 8]);
        const int cl = 8 * q + 4 * lhalf;
        const int c = cl >> 3, hh = (cl >> 2) & 1;
        const u32x2 v = {pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
        *(u32x2*)(stg + r * kRowB + ((c ^ (r % kCpr)) << 4) + hh * 8) = v;
      }
    }
  }
  __syncthreads();
  // active positions: 16-byte segments to H[token, ch0 .. ch0 + CW)
  for (int e = tid; e < nact * kCpr; e += 512) {
    const int r = e / kCpr, c = e % kCpr;
    const u32x4 v = *(const u32x4*)(stg + r * kRowB + ((c ^ (r % kCpr)) << 4));
    *(u32x4*)(H + (size_t)s_tok[r] * d_ff + ch0 + c * 8) = v;
  }
}

#define WIDE_GATE_UP_KERNEL(CW)                                                               \
  __global__ __launch_bounds__(512, 1) void gate_up_bf16_kernel_##CW(                             \
      const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wg,                            \
      const uint16_t* __restrict__ Wu, const int32_t* __restrict__ perm,                          \
      const int32_t* __restrict__ counts, int T, int d, int d_ff, int G,                          \
      uint16_t* __restrict__ H, int zero_inactive, int ntok_tiles, int nct, int total) {          \
    __shared__ __attribute__((aligned(1024))) uint8_t sA[MnShape<CW>::S::STAGE];                  \
    __shared__ __attribute__((aligned(1024))) uint8_t sB[MnShape<CW>::S::STAGE];                  \
    __shared__ int s_tok[kTokTile];                                                               \
    gate_up_body<CW>(X, Wg, Wu, perm, counts, T, d, d_ff, G, H, zero_inactive, ntok_tiles, nct,   \
                     total, sA, sB, s_tok);                                                       \
  }
WIDE_GATE_UP_KERNEL(128)
WIDE_GATE_UP_KERNEL(64)
WIDE_GATE_UP_KERNEL(32)
WIDE_GATE_UP_KERNEL(16)
#undef WIDE_GATE_UP_KERNEL

template <int CW>
hipError_t launch_cw(const uint16_t* X, const uint16_t* Wg, const uint16_t* Wu, const int32_t* perm,
                     const int32_t* counts, int T, int d, int d_ff, int G, uint16_t* H,
                     bool zero_inactive, hipStream_t stream) {
  const int ng = d_ff / G;
  const int nct = G / CW;
  const int ntok_tiles = (T + kTokTile - 1) / kTokTile;
  const long long total = (long long)ng * nct * ntok_tiles;
  const int per_xcd = (int)((total + 7) / 8);
  auto kernel = CW == 128 ? gate_up_bf16_kernel_128
                : CW == 64  ? gate_up_bf16_kernel_64
                : CW == 32  ? gate_up_bf16_kernel_32
                            : gate_up_bf16_kernel_16;
  hipLaunchKernelGGL(kernel, dim3(per_xcd * 8), dim3(512), 0, stream, X, Wg, Wu, perm, counts, T, d,
                     d_ff, G, H, zero_inactive ? 1 : 0, ntok_tiles, nct, (int)total);
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
