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
//   * a workgroup owns Y[256 tokens (natural order), 256 output columns] and
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
// The same kernel is the K-axis masked GEMM C = (mask-expanded A) . B^T.
// Operands: MFMA A side = Wdown rows (output columns), B side = H rows
// (tokens); the shared 8-wave mainloop streams both through LDS with
// register-bypassing copies. Rows past d or T are zero-filled by
// out-of-range buffer copies. The epilogue rounds once to bf16 (RNE) and
// writes 16-byte row segments through an LDS staging tile.
#include "mfma_core.h"

namespace wide {

namespace {

constexpr int kTile = 256;
constexpr int kMaxSteps = 1024;  // d_ff / 64 limit (d_ff <= 65536)
using DS = core::Shape<kTile, kTile, 2, 4>;
constexpr int kCopyWaves = 4;
constexpr int kCB = DS::PBLOCKS / kCopyWaves;  // blocks per operand per copying wave
static_assert(DS::PBLOCKS == DS::QBLOCKS && 8 * kCopyWaves == 32, "mask word i covers block i");

__global__ __launch_bounds__(512, 1) void down_bf16_kernel(
    const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wd,
    const uint32_t* __restrict__ maskbits, int T, int d, int d_ff, int G, uint16_t* __restrict__ Y,
    int ntt, int nnt, int words) {
  __shared__ __attribute__((aligned(1024))) uint8_t sA[DS::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t sB[DS::STAGE];
  __shared__ uint16_t s_steps[kMaxSteps];
  __shared__ __attribute__((aligned(16))) uint32_t s_mw[kDownMaxGroups * 8];  // [group][8 words]: the tile's mask bits
  __shared__ int s_wave_cnt[8];

  const int total = ntt * nnt;
  const int per_xcd = (total + 7) / 8;
  const int L = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (L >= total) return;
  const int t0 = (L / nnt) * kTile;
  const int n0 = (L % nnt) * kTile;
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
    constexpr int kTab = kDownMaxGroups * 8 / 512;
    uint32_t v[kTab];
#pragma unroll
    for (int i = 0; i < kTab; ++i) {
      if (512 * i >= ng * 8) break;
      const int e = min(tid + 512 * i, ng * 8 - 1);
      const int g = e >> 3, wi = e & 7;
      v[i] = maskbits[(size_t)g * words + min(w0 + wi, words - 1)] &
             (w0 + wi < words ? 0xFFFFFFFFu : 0u);
    }
#pragma unroll
    for (int i = 0; i < kTab; ++i) {
      if (512 * i >= ng * 8) break;
      if (tid + 512 * i < ng * 8) s_mw[tid + 512 * i] = v[i];
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
          for (int wi = 0; wi < 8; ++wi) acc |= s_mw[g * 8 + wi];
        } else {
          const uint32_t* mw = maskbits + (size_t)g * words;
#pragma unroll
          for (int wi = 0; wi < 8; ++wi)
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
    const int k0 = (int)s_steps[s] * 64;
    const uint32_t* mw = maskbits + (size_t)((k0 + chunk * 8) / G) * words;
#pragma unroll
    for (int i = 0; i < kCB; ++i)
      mwv[i] = mw[min(w0 + i, words - 1)] & (w0 + i < words ? 0xFFFFFFFFu : 0u);
  };
  auto prepare = [&](int s) {
    if (!copier) return;
    const uint32_t sh = rw & 31;
    if (table) {
      const int k0 = (int)s_steps[s] * 64;
      const uint32_t* mw = s_mw + ((k0 + chunk * 8) / G) * 8;  // this lane's group
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
    const int k0 = (int)s_steps[s] * 64;
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
  __syncthreads();  // every wave is done with the stages: reuse them for the epilogue

  // Epilogue: staged as [256 tokens][256 columns] bf16 (512-byte rows, chunk
  // c of row r at c ^ (r & 31)); token rows 0..127 in sA, 128..255 in sB.
  const int lrow = lane & 31, lhalf = lane >> 5;
#pragma unroll
  for (int j = 0; j < DS::FQ; ++j) {
    const int r = wq * DS::QW + j * 32 + lrow;
    uint8_t* row = (r < 128 ? sA : sB) + (r & 127) * 512;
#pragma unroll
    for (int i = 0; i < DS::FP; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = wp * DS::PW + i * 32 + 8 * q + 4 * lhalf;
        const int c = nl >> 3, hh = (nl >> 2) & 1;
        const u32x2 v = {pack_bf16x2(f.acc[i][j][4 * q], f.acc[i][j][4 * q + 1]),
                         pack_bf16x2(f.acc[i][j][4 * q + 2], f.acc[i][j][4 * q + 3])};
        *(u32x2*)(row + ((c ^ (r & 31)) << 4) + hh * 8) = v;
      }
    }
  }
  __syncthreads();
  const int nrows = min(kTile, T - t0);
  const int ncch = min(kTile, d - n0) / 8;  // 16-byte column chunks that exist
  for (int e = tid; e < nrows * 32; e += 512) {
    const int r = e >> 5, c = e & 31;
    if (c >= ncch) continue;
    const uint8_t* row = (r < 128 ? sA : sB) + (r & 127) * 512;
    const u32x4 v = *(const u32x4*)(row + ((c ^ (r & 31)) << 4));
    *(u32x4*)(Y + (size_t)(t0 + r) * d + n0 + c * 8) = v;
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
  hipLaunchKernelGGL(down_bf16_kernel, dim3(per_xcd * 8), dim3(512), 0, stream, H, Wd, maskbits, T,
                     d, d_ff, G, Y, ntt, nnt, words);
  return hipGetLastError();
}

}  // namespace wide
