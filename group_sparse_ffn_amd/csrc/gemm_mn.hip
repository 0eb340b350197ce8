// N-axis group-masked GEMM over reordered rows (WIDE paper App. B,
// "Implementation of GEMM-MN": each workgroup owns one output tile whose N
// coordinate selects a routing group; admission, predicated computation and a
// scatter epilogue). One body serves two epilogues:
//   * SwiGLU (the FFN gate/up projection): the MFMA A side holds CW gate rows
//     and CW up rows of one channel block (per wave: its gate half first, then
//     the up half of the same channels, so one lane holds both accumulators of
//     a (channel, row) pair); the epilogue forms silu(gate) * up;
//   * plain, C = A . B^T with N-axis pruning (an attention W_q projection, or
//     the M-axis / dynamic-depth case as a single group): the A side holds the
//     CW rows of B of one channel block.
// The MFMA B side holds 256 positions of the group's reordered row list,
// gathered from A (X for the FFN). The three skipping levels of the pages,
// re-derived for gfx950:
//   level 0: a workgroup whose 256-position tile starts at or past the group's
//            active count does no MFMA work at all;
//   level 1: rows past the active count are never fetched: their copies use an
//            out-of-range buffer offset, which writes zeros to LDS without
//            touching memory;
//   level 2: 32-row MFMA fragments that lie wholly past the count are not
//            multiplied.
// Tile order. A tile is (channel block, token tile); a group's tiles are
// full (TT active positions), at most one boundary tile (fewer), and tiles
// past its count (only zeros to write, and only with zero_inactive). Every
// workgroup scans the active counts and takes, on its XCD (workgroup ids go
// to the XCDs in turn), first an eighth of all full tiles in the sparse
// super-tile order below (the tiles that run at the same time on one XCD
// share the weight rows of two blocks in its L2, and row lists in token
// order share activation rows), then an eighth of the boundary tiles, then an eighth of
// the tiles past the counts. The last round of the grid is then filled by
// the short boundary tiles, workgroups with no work are dispatched after all
// of the real ones, and skewed counts spread evenly over the XCDs.
// The epilogue rounds once to bf16 (RNE), stages the tile through LDS and
// scatters 16-byte row segments to C[row, channels]. With zero_inactive,
// every (row, channel) of the group that the row skips is also written as
// +0.0 (always for the plain GEMM; for the FFN when H is returned); otherwise
// only active pairs are written.
#include "mfma_core.h"

namespace wide {

namespace {

constexpr int kCopyWaves = 4;

// TT: positions of the reordered row list per tile, 256 or 128 (with channel
// blocks of 64 or more); mn_token_tile (SwiGLU) and plain_mn_tile choose.
template <int CW, bool SWIGLU, int TT = 256>
struct MnShape {
  // a 16-channel plain block is padded to one 32-row fragment (zero rows)
  static constexpr int TP = SWIGLU ? 2 * CW : (CW < 32 ? 32 : CW);
  static constexpr int WP = (TP >= 256 || TT == 128) ? 2 : 1;
  static constexpr int WQ = 8 / WP;
  static constexpr int kTokTile = TT;
  using S = core::Shape<TP, TT, WP, WQ>;
  static constexpr int PBLK = S::PBLOCKS, QBLK = S::QBLOCKS;
  static constexpr int NBLK = PBLK + QBLK;
  // Only waves 0..kCopyWaves-1 issue copies: each SIMD then runs one copying
  // and one MFMA-only wave, and the MFMA-only wave keeps the matrix core
  // busy while the other waits to issue its copies.
  static constexpr int MAXB = (NBLK + kCopyWaves - 1) / kCopyWaves;  // copy blocks per copying wave
  static constexpr int HALF = S::PW / 2;       // SwiGLU: channels per wave
  // epilogue staging: [256 positions][CW] bf16, split over the two stages
  static constexpr int ROWB = CW * 2;
  static constexpr int STG_ROWS = S::STAGE / ROWB;  // staged rows per LDS stage
  static_assert(2 * STG_ROWS >= TT, "epilogue staging fits the two stages");
};

// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts within
// each 16-lane row, then the row totals carried by row broadcasts).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

// Tile order of the dense-masked form (every tile full, no counts to scan):
// super-row r holds channel blocks [8r, 8r + 8), its column q the token tiles
// [4q, 4q + 4); tiles are listed super-row by super-row, column by column,
// then block by block and tile by tile, and each XCD takes a contiguous
// eighth of that list. The 32 workgroups that run together on one XCD then
// share the weight rows of 8 blocks and the activation rows of 4 token tiles
// (about a third of the fabric traffic of 32 tiles of one block). Measured
// against the block-major order: Llama3.2-3B T = 8192 gate/up 0.738 -> 0.658
// ms at G = 16 and 0.737 -> 0.650 ms at G = 32; at the Llama3.1-8B prefill
// shape 3.19 -> 3.01 ms. The same 8 x 4 order for the sparse tiles (whose row
// lists are in token order) halves their fabric traffic but measured 1.662 ->
// 1.706 ms at the Llama3.1-8B shape; they use the narrower super-tiles below.
constexpr int kSuperBlocks = 8, kSuperTiles = 4;

// The sparse tiles' full tiles go in super-tiles of 2 blocks x 16 token tiles
// (super-row r: blocks 2r, 2r + 1; column q: their full tiles 16q .. 16q + 15),
// listed super-row by super-row, column by column, block by block, tile by
// tile, each XCD taking a contiguous eighth of that list. Measured against
// block-major (32 tiles of one block per XCD round): Llama3.1-8B gate/up
// 1.695 -> 1.656 ms, Llama3.2-3B T = 2048 0.147 -> 0.142 ms, G = 64 0.478 ->
// 0.487 ms, the other shapes within noise; 4 x 8 measured 1.666 ms and the
// 8 x 4 of the dense form 1.706 ms.
constexpr int kSparseSuperBlocks = 2, kSparseSuperTiles = 16;

// Full tiles of a block with f full tiles that fall in sparse super-tile
// column q.
__device__ __forceinline__ int in_column(int f, int q) {
  return min(max(f - kSparseSuperTiles * q, 0), kSparseSuperTiles);
}

// This workgroup's tile in the order above (blk, tile index and the group's
// active count), or false when it has none. Every wave computes it on its
// own, with no barrier: lane l scans a contiguous run of blocks (boundary and
// past-count tiles) and of sparse super-rows (full tiles), the run that holds
// the wanted index is found by a ballot, and its lane's answer is read by
// every lane.
template <int TT>
__device__ __forceinline__ bool ordered_tile(const int32_t* __restrict__ counts, int nblk, int nct,
                                             int ntok_tiles, bool with_zero, int& blk, int& tile,
                                             int& count) {
  constexpr int SM = kSparseSuperBlocks, SN = kSparseSuperTiles;
  const int lane = (int)(threadIdx.x & 63);
  const int per = (nblk + 63) / 64;
  const int b0 = lane * per;
  int sb = 0, sz = 0;
  for (int k = 0; k < per && b0 + k < nblk; ++k) {
    const int c = counts[(b0 + k) / nct];
    const int f = c / TT, b = c % TT != 0;
    sb += b;
    sz += ntok_tiles - f - b;
  }
  const int nsr = (nblk + SM - 1) / SM;
  const int rper = (nsr + 63) / 64;
  const int r0 = lane * rper;
  int sf = 0;
  for (int k = 0; k < rper && r0 + k < nsr; ++k)
#pragma unroll
    for (int m = 0; m < SM; ++m) {
      const int b = (r0 + k) * SM + m;
      if (b < nblk) sf += counts[b / nct] / TT;
    }
  const int pf = wave_incl_scan(sf), pb = wave_incl_scan(sb), pz = wave_incl_scan(sz);
  const int F = __builtin_amdgcn_readlane(pf, 63);
  const int B = __builtin_amdgcn_readlane(pb, 63);
  const int Z = __builtin_amdgcn_readlane(pz, 63);
  const int x = (int)(blockIdx.x % 8), j = (int)(blockIdx.x / 8);
  const int fx = (F + 7) / 8, bx = (B + 7) / 8, zx = (Z + 7) / 8;
  const int nf = min(max(F - x * fx, 0), fx);
  const int nb = min(max(B - x * bx, 0), bx);
  const int nz = with_zero ? min(max(Z - x * zx, 0), zx) : 0;
  int cls, i;
  if (j < nf) {
    cls = 0;
    i = x * fx + j;
  } else if (j < nf + nb) {
    cls = 1;
    i = x * bx + (j - nf);
  } else if (j < nf + nb + nz) {
    cls = 2;
    i = x * zx + (j - nf - nb);
  } else {
    return false;
  }
  const int mine = cls == 0 ? sf : cls == 1 ? sb : sz;
  int acc = (cls == 0 ? pf : cls == 1 ? pb : pz) - mine;  // tiles of the class before this run
  const uint64_t own = __ballot(i >= acc && i < acc + mine);
  if (own == 0) return false;  // (never: the runs cover the class)
  const int owner = (int)__builtin_ctzll(own);
  int rb = 0, rt = 0, rc = 0;
  if (lane == owner) {
    if (cls == 0) {
      for (int k = 0; k < rper && r0 + k < nsr; ++k) {
        const int r = r0 + k;
        int f[SM], c[SM], tot = 0;
#pragma unroll
        for (int m = 0; m < SM; ++m) {
          const int b = r * SM + m;
          c[m] = b < nblk ? counts[b / nct] : 0;
          f[m] = c[m] / TT;
          tot += f[m];
        }
        if (i < acc + tot) {
          int ii = i - acc;
          for (int q = 0; q * SN < ntok_tiles; ++q) {
            int cq = 0;
#pragma unroll
            for (int m = 0; m < SM; ++m) cq += in_column(f[m], q);
            if (ii < cq) {
#pragma unroll
              for (int m = 0; m < SM; ++m) {
                const int n = in_column(f[m], q);
                if (ii >= 0 && ii < n) {
                  rb = r * SM + m;
                  rt = q * SN + ii;
                  rc = c[m];
                }
                ii -= n;
              }
              break;
            }
            ii -= cq;
          }
          break;
        }
        acc += tot;
      }
    } else {
      for (int k = 0; k < per && b0 + k < nblk; ++k) {
        const int c = counts[(b0 + k) / nct];
        const int f = c / TT, b = c % TT != 0;
        const int n = cls == 1 ? b : ntok_tiles - f - b;
        if (i < acc + n) {
          rb = b0 + k;
          rt = cls == 1 ? f : f + b + (i - acc);
          rc = c;
          break;
        }
        acc += n;
      }
    }
  }
  blk = __builtin_amdgcn_readlane(rb, owner);
  tile = __builtin_amdgcn_readlane(rt, owner);
  count = __builtin_amdgcn_readlane(rc, owner);
  return true;
}

// The body is a device function template called from one plain kernel per
// (channel width, epilogue): a kernel template that passes a local lambda to
// the mainloop loses its host launch stub with this toolchain.
//   A [M, K] rows, gathered through perm; B and (SwiGLU) B2 [N, K]; C [M, N].
//   Group g's row list is perm[g*M .. g*M + M), its active prefix counts[g].
//
// DENSE (SwiGLU only, for groups narrower than 64 channels, where a group's
// own tile would give the MFMA an A side of 16 or 32 rows and its row lists
// skip almost nothing under random masks): tiles are 128-channel blocks of
// every group over natural-order rows (no gather, no reorder); every product
// is computed, and the store writes silu(gate) * up where the row executes
// the channel's group (bit of maskbits [ngroups, words]) and +0.0 elsewhere.
template <int CW, bool SWIGLU, int TT, bool DENSE = false>
__device__ __forceinline__ void mn_body(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
    const uint16_t* __restrict__ B2, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ counts, int M, int K, int N, int G, uint16_t* __restrict__ C,
    int zero_inactive, int ntok_tiles, int nct, int total, uint8_t* sA, uint8_t* sB,
    int* s_tok, const uint32_t* __restrict__ maskbits = nullptr, int words = 0) {
  using SH = MnShape<CW, SWIGLU, TT>;
  using S = typename SH::S;
  constexpr int kTokTile = TT;
  static_assert(!DENSE || SWIGLU, "the dense form is the gate/up projection's");

  int blk, tile, count;
  if constexpr (DENSE) {
    // XCD-aware: each XCD a contiguous range of the (channel block, token
    // tile) pairs in super-tile order (every tile is full here)
    const int per_xcd = (total + 7) / 8;
    const int L = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (L >= total) return;
    const int nblk = total / ntok_tiles;
    const int r = L / (kSuperBlocks * ntok_tiles);         // earlier super-rows are whole
    const int mr = min(kSuperBlocks, nblk - r * kSuperBlocks);  // blocks in this one
    int ii = L - r * kSuperBlocks * ntok_tiles;
    const int q = ii / (mr * kSuperTiles);                 // earlier columns are whole
    ii -= q * mr * kSuperTiles;
    const int nq = min(kSuperTiles, ntok_tiles - q * kSuperTiles);
    blk = r * kSuperBlocks + ii / nq;
    tile = q * kSuperTiles + ii % nq;
    count = M;
  } else {
    if (!ordered_tile<TT>(counts, total / ntok_tiles, nct, ntok_tiles, zero_inactive != 0, blk,
                          tile, count))
      return;
  }
  const int tile0 = tile * kTokTile;
  const int g = DENSE ? 0 : blk / nct;
  const int ct = DENSE ? blk : blk % nct;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ch0 = g * G + ct * CW;  // first channel of this tile
  const int nrows = min(kTokTile, M - tile0);          // positions that exist
  const int nact = max(0, min(nrows, count - tile0));  // active positions
  if (nact == 0 && !zero_inactive) return;  // level 0, nothing to clear

  if constexpr (DENSE) {
    if (tid < kTokTile) s_tok[tid] = tid < nrows ? tile0 + tid : 0;
  } else {
    const int32_t* __restrict__ prow = perm + (size_t)g * M + tile0;
    if (tid < kTokTile) s_tok[tid] = tid < nrows ? prow[tid] : 0;
  }
  __syncthreads();

  // Zeros for the positions of this tile whose row skips the group.
  if (!DENSE && zero_inactive) {
    constexpr int kChunks = CW / 8;  // 16-byte chunks per row segment
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int e = nact * kChunks + tid; e < nrows * kChunks; e += 512) {
      const int r = e / kChunks, c = e % kChunks;
      *(u32x4*)(C + (size_t)s_tok[r] * N + ch0 + c * 8) = z;
    }
  }
  if (nact == 0) return;  // level 0

  // ---- copies: blocks [0, PBLK) are weight rows, [PBLK, NBLK) gathered rows.
  // Copying wave w issues blocks w, w + kCopyWaves, ...; lane offsets are
  // fixed per block.
  const bool copier = wave < kCopyWaves;
  uint32_t voff[SH::MAXB];
#pragma unroll
  for (int i = 0; i < SH::MAXB; ++i) {
    const int b = wave + kCopyWaves * i;
    const int chunk = core::copy_chunk(b, lane);
    if (b < SH::PBLK) {
      const int r = 8 * b + (lane >> 3);
      if constexpr (SWIGLU) {
        // LDS row r -> (wave wp = r / PW, half) -> channel row of B (gate) or B2 (up)
        const int within = r % S::PW;
        const int chan = ch0 + (r / S::PW) * SH::HALF + (within % SH::HALF);
        voff[i] = (uint32_t)(chan * K + chunk * 8) * 2u;
      } else {
        // padding rows of a 16-channel block read zeros
        voff[i] = r < CW ? (uint32_t)((ch0 + r) * K + chunk * 8) * 2u : 0x80000000u;
      }
    } else if (b < SH::NBLK) {
      const int r = 8 * (b - SH::PBLK) + (lane >> 3);
      voff[i] = r < nact ? (uint32_t)(s_tok[r] * K + chunk * 8) * 2u : 0x80000000u;
    } else {
      voff[i] = 0;
    }
  }
  const uint32_t a_bytes = (uint32_t)M * (uint32_t)K * 2u;
  const uint32_t b_bytes = (uint32_t)N * (uint32_t)K * 2u;
  auto issue = [&](int s, uint8_t* stage) {
    if (!copier) return;
    const int k0 = s * core::kBK;
    // gathered rows: out-of-range offsets fill zeros (level 1)
    const __amdgpu_buffer_rsrc_t ar =
        __builtin_amdgcn_make_buffer_rsrc((void*)(A + k0), 0, (int)(a_bytes - 2u * k0), 0x00020000);
#pragma unroll
    for (int i = 0; i < SH::MAXB; ++i) {
      const int b = wave + kCopyWaves * i;
      if (b < SH::PBLK) {
        if constexpr (SWIGLU) {
          const int r0 = 8 * b;
          const bool gate = (r0 % S::PW) < SH::HALF;
          const uint16_t* base = (gate ? B : B2) + k0;
          __builtin_amdgcn_global_load_lds((const void*)((const char*)base + voff[i]),
                                           (void*)(stage + b * 1024), 16, 0, 0);
        } else {
          const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
              (void*)(B + k0), 0, (int)(b_bytes - 2u * k0), 0x00020000);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(br, (void*)(stage + b * 1024), 16, voff[i], 0,
                                                   0, 0);
        }
      } else if (b < SH::NBLK) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (void*)(stage + b * 1024), 16, voff[i], 0, 0,
                                                 0);
      }
    }
  };

  const int wp = wave / S::WQ;
  const int wq = wave % S::WQ;
  // level 2: this wave's 32-row fragments that hold an active position
  const int nq = max(0, min(S::FQ, (nact - wq * S::QW + 31) / 32));
  core::Frags<S> f;
  // a wave whose fragments are all active (every full tile) runs the MFMA
  // loop with the fragment count a constant, so it has no branch (1% faster)
  if (nq == S::FQ)
    core::mainloop<S>(f, sA, sB, K / core::kBK, wp, wq, lane, S::FQ, issue);
  else
    core::mainloop<S>(f, sA, sB, K / core::kBK, wp, wq, lane, nq, issue);
  __syncthreads();  // every wave is done with the stages: reuse them for the epilogue

  // ---- epilogue: bf16 values staged as [256 positions][CW]; position r sits
  // in row r % STG_ROWS of stage r / STG_ROWS, chunk c at c ^ (r % kCpr).
  constexpr int kRowB = SH::ROWB;
  constexpr int kCpr = CW / 8;  // 16-byte chunks per staged row
  auto srow = [&](int r) -> uint8_t* {
    return (r < SH::STG_ROWS ? sA + r * kRowB : sB + (r - SH::STG_ROWS) * kRowB);
  };
  const int lrow = lane & 31, lhalf = lane >> 5;
  auto put4 = [&](int r, int cl, const float (&h)[4]) {
    const int c = cl >> 3, hh = (cl >> 2) & 1;
    const u32x2 v = {pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
    *(u32x2*)(srow(r) + ((c ^ (r % kCpr)) << 4) + hh * 8) = v;
  };
#pragma unroll
  for (int j = 0; j < S::FQ; ++j) {
    const int r = wq * S::QW + j * 32 + lrow;  // position in the tile
    if constexpr (SWIGLU && S::FP >= 2) {
#pragma unroll
      for (int i = 0; i < S::FP / 2; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            h[e] = silu_mul(f.acc[i][j][4 * q + e], f.acc[i + S::FP / 2][j][4 * q + e]);
          put4(r, wp * SH::HALF + i * 32 + 8 * q + 4 * lhalf, h);
        }
      }
    } else if constexpr (SWIGLU) {
      // CW == 16: one fragment holds gate rows 0..15 (e < 8) and up rows 16..31 (e >= 8)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          h[e] = silu_mul(f.acc[0][j][4 * q + e], f.acc[0][j][4 * q + e + 8]);
        put4(r, 8 * q + 4 * lhalf, h);
      }
    } else {
#pragma unroll
      for (int i = 0; i < S::FP; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int cl = wp * S::PW + i * 32 + 8 * q + 4 * lhalf;
          if (cl < CW) {  // skip the padding rows of a 16-channel block
            float h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = f.acc[i][j][4 * q + e];
            put4(r, cl, h);
          }
        }
      }
    }
  }
  __syncthreads();
  // active positions: 16-byte segments to C[row, ch0 .. ch0 + CW)
  for (int e = tid; e < nact * kCpr; e += 512) {
    const int r = e / kCpr, c = e % kCpr;
    u32x4 v = *(const u32x4*)(srow(r) + ((c ^ (r % kCpr)) << 4));
    if constexpr (DENSE) {
      // a 16-byte segment (8 channels) lies in one group: G is a multiple of 16
      const int t = s_tok[r];
      const uint32_t bit = (maskbits[(size_t)((ch0 + c * 8) / G) * words + (t >> 5)] >> (t & 31)) & 1u;
      const uint32_t m = 0u - bit;
      v &= u32x4{m, m, m, m};
    }
    *(u32x4*)(C + (size_t)s_tok[r] * N + ch0 + c * 8) = v;
  }
}

#define WIDE_MN_KERNEL(NAME, CW, SWIGLU, TT)                                                  \
  __global__ __launch_bounds__(512, 1) void NAME(                                             \
      const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,                         \
      const uint16_t* __restrict__ B2, const int32_t* __restrict__ perm,                      \
      const int32_t* __restrict__ counts, int M, int K, int N, int G,                         \
      uint16_t* __restrict__ C, int zero_inactive, int ntok_tiles, int nct, int total) {      \
    __shared__ __attribute__((aligned(1024))) uint8_t sA[MnShape<CW, SWIGLU, TT>::S::STAGE];  \
    __shared__ __attribute__((aligned(1024))) uint8_t sB[MnShape<CW, SWIGLU, TT>::S::STAGE];  \
    __shared__ int s_tok[TT];                                                                 \
    mn_body<CW, SWIGLU, TT>(A, B, B2, perm, counts, M, K, N, G, C, zero_inactive, ntok_tiles, \
                            nct, total, sA, sB, s_tok);                                       \
  }
WIDE_MN_KERNEL(gate_up_bf16_kernel_128, 128, true, 256)
WIDE_MN_KERNEL(gate_up_bf16_kernel_32, 32, true, 256)
WIDE_MN_KERNEL(gate_up_bf16_kernel_16, 16, true, 256)
WIDE_MN_KERNEL(gate_up_bf16_kernel_128_t128, 128, true, 128)
WIDE_MN_KERNEL(gate_up_bf16_kernel_64_t128, 64, true, 128)
WIDE_MN_KERNEL(gemm_mn_bf16_kernel_256, 256, false, 256)
WIDE_MN_KERNEL(gemm_mn_bf16_kernel_32, 32, false, 256)
WIDE_MN_KERNEL(gemm_mn_bf16_kernel_16, 16, false, 256)
WIDE_MN_KERNEL(gemm_mn_bf16_kernel_128_t128, 128, false, 128)
WIDE_MN_KERNEL(gemm_mn_bf16_kernel_64_t128, 64, false, 128)
#undef WIDE_MN_KERNEL

__global__ __launch_bounds__(512, 1) void gate_up_dense_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
    const uint16_t* __restrict__ B2, const uint32_t* __restrict__ maskbits, int words, int M,
    int K, int N, int G, uint16_t* __restrict__ C, int ntok_tiles, int total) {
  using SH = MnShape<128, true, 256>;
  __shared__ __attribute__((aligned(1024))) uint8_t sA[SH::S::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t sB[SH::S::STAGE];
  __shared__ int s_tok[256];
  mn_body<128, true, 256, true>(A, B, B2, nullptr, nullptr, M, K, N, G, C, 1, ntok_tiles, 1, total,
                                sA, sB, s_tok, maskbits, words);
}

typedef void (*MnKernel)(const uint16_t*, const uint16_t*, const uint16_t*, const int32_t*,
                         const int32_t*, int, int, int, int, uint16_t*, int, int, int, int);

// Token tile of the SwiGLU gate/up. 64-channel blocks (a 128-row A side)
// take 128 positions: measured at 50% top-k masks on the Llama3.2-3B shape,
// G = 64, 0.246 against 0.265 ms at T = 4096, 0.481 against 0.496 at 8192 and
// 0.99 against 1.06 at 16384. 128-channel blocks take 128 positions only when
// the 256-position grid (before level-0 exits) has fewer than 256 tiles;
// otherwise 256 (the Llama3.1-8B and Qwen3-14B shapes: 1.68 against 2.10 and
// 0.71 against 0.91 ms with 128 positions; whether 64-channel blocks of 128
// positions gain at mid sizes depends on how the active tiles fill the last
// round: 0.132 against 0.143 ms at T = 2048 on the 3B shape, 0.184 against
// 0.164 at T = 3072). Blocks under 64 channels take 256 positions.
int mn_token_tile(int M, int N, int G, int CW) {
  if (CW < 64) return 256;
  if (CW == 64) return 128;
  const long long t256 = (long long)(N / G) * (G / CW) * ((M + 255) / 256);
  return t256 < 256 ? 128 : 256;
}

// Tile of the plain GEMM (channel block cw x token tile tt). Measured on
// MI355X over square shapes 2048-8192 and the Llama3.1-8B W_q shapes, 50%
// masks, every shape timed with each tile in one process (outputs bit-equal):
//   * 256 x 256 wins wherever G allows it and the full grid has at least one
//     such tile per CU (4096^3 N axis G = 512: 97.9 us against 117.8 for
//     128 x 128), even when half its tiles are idle;
//   * otherwise 128-position tiles win at every size: a 128-channel block with
//     128 positions against 256 positions, 120 against 137 us at 4096^3 and
//     703 against 762 us at 8192^3 (G = 128); at 3072^3 on the M axis 53
//     against 62-75 us for the 256-wide tiles;
//   * where the full grid of 128 x 128 tiles is at most one tile per CU (about
//     half of them active at 50% masks), 64-channel blocks double the
//     workgroups: 2048^3 M axis 36.4 against 37.8 (43.9 with 256 x 128), N axis
//     37.2 against 40.0 us.
void plain_mn_tile(int M, int N, int G, int* cw, int* tt) {
  const long long rows128 = (M + 127) / 128, rows256 = (M + 255) / 256;
  const int ncu = 256;  // MI355X compute units
  if (G % 256 == 0 && (long long)(N / 256) * rows256 >= ncu) {
    *cw = 256;
    *tt = 256;
  } else if (G % 64 == 0) {
    *cw = G % 128 == 0 && (long long)(N / 128) * rows128 > ncu ? 128 : 64;
    *tt = 128;
  } else {
    *cw = G % 32 == 0 ? 32 : 16;
    *tt = 256;
  }
}

hipError_t launch_mn(MnKernel kernel, int CW, int TT, const uint16_t* A, const uint16_t* B,
                     const uint16_t* B2, const int32_t* perm, const int32_t* counts, int M, int K,
                     int N, int G, uint16_t* C, bool zero_inactive, hipStream_t stream) {
  const int ng = N / G;
  const int nct = G / CW;
  const int ntok_tiles = (M + TT - 1) / TT;
  const long long total = (long long)ng * nct * ntok_tiles;
  // per XCD at most an eighth (rounded up) of each of the three tile classes
  const int per_xcd = (int)((total + 7) / 8) + 2;
  hipLaunchKernelGGL(kernel, dim3(per_xcd * 8), dim3(512), 0, stream, A, B, B2, perm, counts, M, K,
                     N, G, C, zero_inactive ? 1 : 0, ntok_tiles, nct, (int)total);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_bf16(const uint16_t* X, const uint16_t* Wg, const uint16_t* Wu,
                               const int32_t* perm, const int32_t* counts,
                               const uint32_t* maskbits, int T, int d, int d_ff, int G,
                               uint16_t* H, bool zero_inactive, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (gate_up_dense(G, d_ff)) {
    const int ntok_tiles = (T + 255) / 256;
    const int total = (d_ff / 128) * ntok_tiles;
    hipLaunchKernelGGL(gate_up_dense_bf16_kernel, dim3((total + 7) / 8 * 8), dim3(512), 0, stream, X,
                       Wg, Wu, maskbits, (T + 31) / 32, T, d, d_ff, G, H, ntok_tiles, total);
    return hipGetLastError();
  }
  const int cw = G % 128 == 0 ? 128 : G % 64 == 0 ? 64 : G % 32 == 0 ? 32 : 16;
  const int tt = mn_token_tile(T, d_ff, G, cw);
  MnKernel k = tt == 128 ? (cw == 128 ? gate_up_bf16_kernel_128_t128 : gate_up_bf16_kernel_64_t128)
               : cw == 128 ? gate_up_bf16_kernel_128
               : cw == 32  ? gate_up_bf16_kernel_32
                           : gate_up_bf16_kernel_16;
  return launch_mn(k, cw, tt, X, Wg, Wu, perm, counts, T, d, d_ff, G, H, zero_inactive, stream);
}

hipError_t launch_gemm_mn_bf16(const uint16_t* A, const uint16_t* B, const int32_t* perm,
                               const int32_t* counts, int M, int K, int N, int G, uint16_t* C,
                               hipStream_t stream) {
  if (M == 0) return hipSuccess;
  int cw, tt;
  plain_mn_tile(M, N, G, &cw, &tt);
  MnKernel k = cw == 256   ? gemm_mn_bf16_kernel_256
               : cw == 128 ? gemm_mn_bf16_kernel_128_t128
               : cw == 64  ? gemm_mn_bf16_kernel_64_t128
               : cw == 32  ? gemm_mn_bf16_kernel_32
                           : gemm_mn_bf16_kernel_16;
  return launch_mn(k, cw, tt, A, B, nullptr, perm, counts, M, K, N, G, C, true, stream);
}

}  // namespace wide
