// Prefill down projection Y = H_masked . Wdown^T on the K axis (the pruned
// axis of the down projection: WIDE paper App. B, "Implementation of GEMM-K").
//
// The pages' GEMM-K runs each active K-group of a reordered token tile as its
// own pipeline and scatters the partial outputs with atomic adds into a
// zero-initialised buffer. On MI355X an fp32 global atomic add sustains about
// 1.0-1.3 TB/s of payload whatever the footprint (one lane-operation per clock
// per L2 channel), and that design issues one atomic per (active token, group,
// output column): about 15 GB at the Llama3.1-8B prefill shape, over 10 ms.
// So this kernel keeps the pages' group-level skipping but owns its outputs:
//   * a workgroup owns Y[256 tokens (natural order), 256 output columns] (or
//     128 x 128 when 256-tiles would leave CUs idle) and
//     accumulates over the K axis in registers; every output has one writer,
//     no atomics, no zero-initialised buffer and a fixed summation order;
//   * 64-channel K-blocks whose groups are inactive for every token of the
//     tile are skipped whole (copies, barriers and MFMAs); the list of live
//     K-blocks is built once per workgroup from the packed mask bits;
//   * the copy of an H row segment whose (token, group) is inactive uses an
//     out-of-range buffer offset, which zero-fills LDS without touching
//     memory (level-1 skipping of A packets): inactive pairs contribute
//     exactly 0 whatever H holds there, and cost no HBM traffic. The tile's
//     mask bits (256 tokens x ngroups) sit in an LDS table built once per
//     workgroup; with more than kDownMaxGroups groups the table does not fit
//     and each lane reads its mask words from global memory instead, one
//     stage ahead, so the stage's own wait covers those loads too.
// Last round. With 256 x 256 tiles the grid is whole rounds of one tile per
// CU plus a remainder of r tiles (Qwen3-14B T = 4096: 320 tiles = 256 + 64);
// given a partial-sum buffer, the r remainder tiles are each split into
// s = 256 / r parts along their list of live K-blocks, so the last round has
// a CU for every part, each a 1/s of a tile. The parts write fp32 partial
// sums in their accumulator layout (1 KB coalesced stores) and a second
// kernel adds the s parts in order and rounds once to bf16.
// The same kernel is the K-axis masked GEMM C = (mask-expanded A) . B^T.
// Operands: MFMA A side = Wdown rows (output columns), B side = H rows
// (tokens); the shared 8-wave mainloop streams both through LDS with
// register-bypassing copies. Rows past d or T are zero-filled by
// out-of-range buffer copies. The epilogue rounds once to bf16 (RNE) and
// writes 16-byte row segments through an LDS staging tile.
#include "mfma_core.h"

namespace wide {

namespace {

constexpr int kMaxSteps = 1024;  // d_ff / 64 limit (d_ff <= 65536)
constexpr int kCopyWaves = 4;

// Tile shapes: kTile tokens x kTile output columns. 256 for large problems;
// 128 when 256-tiles would leave CUs idle (four times the workgroups).
template <int kTile>
struct DownShape {
  using DS = core::Shape<kTile, kTile, 2, 4>;
  static constexpr int kCB = DS::PBLOCKS / kCopyWaves;  // blocks per operand per copying wave
  static constexpr int kWords = kTile / 32;            // mask words per token tile
  static_assert(DS::PBLOCKS == DS::QBLOCKS && 8 * kCopyWaves == 32, "mask word i covers block i");
  static_assert(kCB == kWords, "block i of a copying wave holds mask word i");
  // epilogue staging rows of [kTile tokens][kTile columns] bf16 per LDS stage
  static constexpr int kRowB = kTile * 2;
  static constexpr int kStgRows = DS::STAGE / kRowB;
  static_assert(2 * kStgRows >= kTile, "epilogue staging fits the two stages");
};

// Tile order: super-row r holds token tiles [SM r, SM r + SM), its column q
// the output tiles [SN q, SN q + SN); listed super-row by super-row, column
// by column, then token tile by token tile, each XCD taking a contiguous
// range. The 32 tiles that run together on an XCD then share the H rows of 8
// token tiles and the Wd rows of 4 output tiles, where the row-major order
// streamed every output tile's Wd rows through each XCD's L2 every round.
// Measured against row-major (one process, two repetitions): Llama3.1-8B
// down 1.492-1.496 -> 1.474-1.476 ms, Qwen3-14B 0.584-0.588 -> 0.567-0.569,
// Llama3.2-3B G = 128 0.337-0.338 -> 0.332; 4 x 8 gained about half as much.
// Returns (token tile, output tile) of list index L; a bijection on
// [0, ntt * nnt), shared with the split-tile sum.
__device__ __forceinline__ int2 down_tile(int L, int ntt, int nnt) {
  constexpr int SM = 8, SN = 4;
  const int r = L / (SM * nnt);
  const int mr = min(SM, ntt - r * SM);
  int ii = L - r * SM * nnt;
  const int q = ii / (mr * SN);
  ii -= q * mr * SN;
  const int nq = min(SN, nnt - q * SN);
  return make_int2(r * SM + ii / nq, q * SN + ii % nq);
}

template <int kTile>
__device__ __forceinline__ void down_body(
    const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wd,
    const uint32_t* __restrict__ maskbits, int T, int d, int d_ff, int G, uint16_t* __restrict__ Y,
    int ntt, int nnt, int words, float* __restrict__ part, int nrem, int nsplit, uint8_t* sA,
    uint8_t* sB, uint16_t* s_steps, uint32_t* s_mw, int* s_wave_cnt) {
  using SH = DownShape<kTile>;
  using DS = typename SH::DS;
  constexpr int kCB = SH::kCB;
  constexpr int kW = SH::kWords;

  // whole tiles first (XCD-aware: each XCD a contiguous range), then the
  // nsplit parts of each of the last nrem tiles
  const int nfull = ntt * nnt - nrem;
  const int per_xcd = (nfull + 7) / 8;
  int L, spart = 0;
  if ((int)blockIdx.x < 8 * per_xcd) {
    L = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (L >= nfull) return;
  } else {
    const int u = (int)blockIdx.x - 8 * per_xcd;
    if (u >= nrem * nsplit) return;
    L = nfull + u / nsplit;
    spart = u % nsplit;
  }
  const bool split = L >= nfull;
  const int2 tn = down_tile(L, ntt, nnt);
  const int t0 = tn.x * kTile;
  const int n0 = tn.y * kTile;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w0 = t0 / 32;  // first mask word of this token tile
  const int ng = d_ff / G;
  const bool table = ng <= kDownMaxGroups;

  // the tile's mask words, group-major (zero past the last word). All of a
  // thread's loads are issued before the first store: indexes are clamped
  // into the bit rows and words past the last one are masked to zero, so no
  // load sits in a divergent branch.
  if (table) {
    constexpr int kTab = kDownMaxGroups * kW / 512;
    uint32_t v[kTab];
#pragma unroll
    for (int i = 0; i < kTab; ++i) {
      if (512 * i >= ng * kW) break;
      const int e = min(tid + 512 * i, ng * kW - 1);
      const int g = e / kW, wi = e % kW;
      v[i] = maskbits[(size_t)g * words + min(w0 + wi, words - 1)] &
             (w0 + wi < words ? 0xFFFFFFFFu : 0u);
    }
#pragma unroll
    for (int i = 0; i < kTab; ++i) {
      if (512 * i >= ng * kW) break;
      if (tid + 512 * i < ng * kW) s_mw[tid + 512 * i] = v[i];
    }
    __syncthreads();
  }

  // K-block admission: keep the 64-channel blocks with any active token.
  const int ksteps = d_ff / 64;
  int nst = 0;
  for (int s0 = 0; s0 < ksteps; s0 += 512) {
    const int s = s0 + tid;
    bool any = false;
    if (s < ksteps) {
      const int glo = (s * 64) / G;
      const int ghi = (s * 64 + 63) / G;
      uint32_t acc = 0;
      for (int g = glo; g <= ghi; ++g) {
        if (table) {
#pragma unroll
          for (int wi = 0; wi < kW; ++wi) acc |= s_mw[g * kW + wi];
        } else {
          const uint32_t* mw = maskbits + (size_t)g * words;
#pragma unroll
          for (int wi = 0; wi < kW; ++wi)
            acc |= mw[min(w0 + wi, words - 1)] & (w0 + wi < words ? 0xFFFFFFFFu : 0u);
        }
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
    for (int w = 0; w < 8; ++w) nst += s_wave_cnt[w];
    __syncthreads();
  }

  // a part of a split tile runs its share of the live K-blocks
  const int kb0 = split ? (spart * nst) / nsplit : 0;
  if (split) nst = ((spart + 1) * nst) / nsplit - kb0;
  const uint16_t* steps = s_steps + kb0;

  // Copies: only waves 0..kCopyWaves-1 issue them, so each SIMD runs one
  // copying and one MFMA-only wave, and the MFMA-only wave keeps the matrix
  // core busy while the other waits to issue its copies. Copying wave w
  // fills 1 KB blocks w, w+4, ..., w+28 of the Wdown rows and the same blocks
  // of the H rows; rows past d or T get an out-of-range offset (zeros). The
  // lane's 16-byte chunk is the same in all its blocks.
  const bool copier = wave < kCopyWaves;
  const int chunk = core::copy_chunk(wave, lane);
  uint32_t voff_p[kCB], voff_q[kCB];
#pragma unroll
  for (int i = 0; i < kCB; ++i) {
    const int b = wave + kCopyWaves * i;
    const int r = 8 * b + (lane >> 3);
    voff_p[i] = (n0 + r < d) ? (uint32_t)((n0 + r) * d_ff + chunk * 8) * 2u : 0x80000000u;
    voff_q[i] = (t0 + r < T) ? (uint32_t)((t0 + r) * d_ff + chunk * 8) * 2u : 0x80000000u;
  }
  // block i of a copying wave holds tile rows rw + 32 i (rw = 8 * wave +
  // lane / 8 < 32): mask word i of the tile, bit rw
  const int rw = 8 * wave + (lane >> 3);
  const uint32_t w_bytes = (uint32_t)d * (uint32_t)d_ff * 2u;
  const uint32_t h_bytes = (uint32_t)T * (uint32_t)d_ff * 2u;
  // H copy offsets of the next stage to issue, with inactive (token, group)
  // pairs turned into out-of-range offsets; computed by prepare() while the
  // MFMAs of an earlier stage run.
  uint32_t vq_next[kCB];
  // Without the LDS table: this lane's 8 mask words of the tile for the next
  // stage to prepare, loaded by the prepare() of the stage before (or before
  // the mainloop for stage 0). Words past the last one read as zero (the
  // index is clamped, so no load sits in a branch).
  uint32_t mwv[kCB];
  auto fetch = [&](int s) {
    const int k0 = (int)steps[s] * 64;
    const uint32_t* mw = maskbits + (size_t)((k0 + chunk * 8) / G) * words;
#pragma unroll
    for (int i = 0; i < kCB; ++i)
      mwv[i] = mw[min(w0 + i, words - 1)] & (w0 + i < words ? 0xFFFFFFFFu : 0u);
  };
  auto prepare = [&](int s) {
    if (!copier) return;
    const uint32_t sh = rw & 31;
    if (table) {
      const int k0 = (int)steps[s] * 64;
      const uint32_t* mw = s_mw + ((k0 + chunk * 8) / G) * kW;  // this lane's group
#pragma unroll
      for (int i = 0; i < kCB; ++i)
        vq_next[i] = ((mw[i] >> sh) & 1u) ? voff_q[i] : 0x80000000u;
    } else {
#pragma unroll
      for (int i = 0; i < kCB; ++i)
        vq_next[i] = ((mwv[i] >> sh) & 1u) ? voff_q[i] : 0x80000000u;
      if (s + 1 < nst) fetch(s + 1);
    }
  };
  if (copier && !table && nst > 0) fetch(0);
  auto issue = [&](int s, uint8_t* stage) {
    if (!copier) return;
    const int k0 = (int)steps[s] * 64;
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Wd + k0), 0, (int)(w_bytes - 2u * k0), 0x00020000);
    const __amdgpu_buffer_rsrc_t hr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(H + k0), 0, (int)(h_bytes - 2u * k0), 0x00020000);
#pragma unroll
    for (int i = 0; i < kCB; ++i) {
      const int b = wave + kCopyWaves * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (void*)(stage + b * 1024), 16, voff_p[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(hr, (void*)(stage + DS::PBYTES + b * 1024), 16,
                                               vq_next[i], 0, 0, 0);
    }
  };

  const int wp = wave / DS::WQ;
  const int wq = wave % DS::WQ;
  core::Frags<DS> f;
  core::mainloop<DS>(f, sA, sB, nst, wp, wq, lane, DS::FQ, issue, prepare);
  if (split) {
    // fp32 partial sums in accumulator order: [wave][i][j][q][lane] f32x4
    float* out = part + ((size_t)(L - nfull) * nsplit + spart) * (kTile * kTile);
#pragma unroll
    for (int i = 0; i < DS::FP; ++i)
#pragma unroll
      for (int j = 0; j < DS::FQ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = {f.acc[i][j][4 * q], f.acc[i][j][4 * q + 1], f.acc[i][j][4 * q + 2],
                           f.acc[i][j][4 * q + 3]};
          *(f32x4*)(out + ((((size_t)wave * DS::FP + i) * DS::FQ + j) * 4 + q) * 256 + 4 * lane) = v;
        }
    return;
  }
  __syncthreads();  // every wave is done with the stages: reuse them for the epilogue

  // Epilogue: staged as [kTile tokens][kTile columns] bf16 (kTile * 2-byte
  // rows, chunk c of row r at c ^ (r % chunks-per-row)); the first kStgRows
  // token rows in sA, the rest in sB.
  constexpr int kRowB = SH::kRowB;
  constexpr int kCpr = kTile / 8;  // 16-byte chunks per staged row
  constexpr int kStg = SH::kStgRows;
  auto srow = [&](int r) -> uint8_t* { return r < kStg ? sA + r * kRowB : sB + (r - kStg) * kRowB; };
  const int lrow = lane & 31, lhalf = lane >> 5;
#pragma unroll
  for (int j = 0; j < DS::FQ; ++j) {
    const int r = wq * DS::QW + j * 32 + lrow;
    uint8_t* row = srow(r);
#pragma unroll
    for (int i = 0; i < DS::FP; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = wp * DS::PW + i * 32 + 8 * q + 4 * lhalf;
        const int c = nl >> 3, hh = (nl >> 2) & 1;
        const u32x2 v = {pack_bf16x2(f.acc[i][j][4 * q], f.acc[i][j][4 * q + 1]),
                         pack_bf16x2(f.acc[i][j][4 * q + 2], f.acc[i][j][4 * q + 3])};
        *(u32x2*)(row + ((c ^ (r % kCpr)) << 4) + hh * 8) = v;
      }
    }
  }
  __syncthreads();
  const int nrows = min(kTile, T - t0);
  const int ncch = min(kTile, d - n0) / 8;  // 16-byte column chunks that exist
  for (int e = tid; e < nrows * kCpr; e += 512) {
    const int r = e / kCpr, c = e % kCpr;
    if (c >= ncch) continue;
    const u32x4 v = *(const u32x4*)(srow(r) + ((c ^ (r % kCpr)) << 4));
    *(u32x4*)(Y + (size_t)(t0 + r) * d + n0 + c * 8) = v;
  }
}

// One plain kernel per tile size (a kernel template that passes a local lambda
// to the mainloop loses its host launch stub with this toolchain).
#define WIDE_DOWN_KERNEL(NAME, TILE)                                                          \
  __global__ __launch_bounds__(512, 1) void NAME(                                             \
      const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wd,                        \
      const uint32_t* __restrict__ maskbits, int T, int d, int d_ff, int G,                   \
      uint16_t* __restrict__ Y, int ntt, int nnt, int words, float* __restrict__ part,        \
      int nrem, int nsplit) {                                                                 \
    using DSx = DownShape<TILE>::DS;                                                          \
    __shared__ __attribute__((aligned(1024))) uint8_t sA[DSx::STAGE];                         \
    __shared__ __attribute__((aligned(1024))) uint8_t sB[DSx::STAGE];                         \
    __shared__ uint16_t s_steps[kMaxSteps];                                                   \
    __shared__ __attribute__((aligned(16))) uint32_t s_mw[kDownMaxGroups * (TILE / 32)];     \
    __shared__ int s_wave_cnt[8];                                                             \
    down_body<TILE>(H, Wd, maskbits, T, d, d_ff, G, Y, ntt, nnt, words, part, nrem, nsplit,   \
                    sA, sB, s_steps, s_mw, s_wave_cnt);                                       \
  }
WIDE_DOWN_KERNEL(down_bf16_kernel, 256)
WIDE_DOWN_KERNEL(down_bf16_kernel_t128, 128)
#undef WIDE_DOWN_KERNEL

// Y of the split tiles: the nsplit parts' partial sums added in order, one
// rounding to bf16. Thread e handles f32x4 e of the accumulator layout of
// 256 x 256 tiles (8 waves x 4 x 2 fragments x 4 quads x 64 lanes).
__global__ __launch_bounds__(256) void down_split_reduce_kernel(
    const float* __restrict__ part, int nfull, int nrem, int nsplit, int ntt, int nnt, int T,
    int d, uint16_t* __restrict__ Y) {
  using DS = DownShape<256>::DS;
  constexpr int kPer = 256 * 256 / 4;  // f32x4 per tile
  const int e = (int)blockIdx.x * 256 + (int)threadIdx.x;
  if (e >= nrem * kPer) return;
  const int q = e / kPer, w = e % kPer;
  const int lane = w & 63, qd = (w >> 6) & 3, j = (w >> 8) % DS::FQ,
            i = (w >> 8) / DS::FQ % DS::FP, wave = (w >> 8) / (DS::FQ * DS::FP);
  const int wp = wave / DS::WQ, wq = wave % DS::WQ;
  const int r = wq * DS::QW + j * 32 + (lane & 31);                   // token in the tile
  const int n = wp * DS::PW + i * 32 + 8 * qd + 4 * (lane >> 5);      // first of 4 columns
  const int L = nfull + q;
  const int2 tn = down_tile(L, ntt, nnt);
  const int t = tn.x * 256 + r, c = tn.y * 256 + n;
  if (t >= T || c >= d) return;
  f32x4 y = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < nsplit; ++sp) y += *(const f32x4*)(part + ((size_t)q * nsplit + sp) * (4 * kPer) + 4 * w);
  const u32x2 v = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
  *(u32x2*)(Y + (size_t)t * d + c) = v;
}

}  // namespace

hipError_t launch_down_bf16(const uint16_t* H, const uint16_t* Wd, const uint32_t* maskbits, int T,
                            int d, int d_ff, int G, uint16_t* Y, float* part, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int tile = down_tile(T, d);
  const int ntt = (T + tile - 1) / tile;
  const int nnt = (d + tile - 1) / tile;
  const int words = (T + 31) / 32;
  const DownSplit ds = part != nullptr ? down_split(T, d, d_ff) : DownSplit{0, 1};
  const int nrem = ds.nsplit > 1 ? ds.nrem : 0;
  const int nfull = ntt * nnt - nrem;
  const int grid = (nfull + 7) / 8 * 8 + nrem * ds.nsplit;
  hipLaunchKernelGGL(tile == 256 ? down_bf16_kernel : down_bf16_kernel_t128, dim3(grid), dim3(512),
                     0, stream, H, Wd, maskbits, T, d, d_ff, G, Y, ntt, nnt, words, part, nrem,
                     ds.nsplit);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nrem == 0) return e;
  const int n4 = nrem * (256 * 256 / 4);
  hipLaunchKernelGGL(down_split_reduce_kernel, dim3((n4 + 255) / 256), dim3(256), 0, stream, part,
                     nfull, nrem, ds.nsplit, ntt, nnt, T, d, Y);
  return hipGetLastError();
}

}  // namespace wide
