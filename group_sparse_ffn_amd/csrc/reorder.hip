// Mask reorder: per-group stable partition of the tokens into an active
// prefix and an inactive tail (ai.info summary, "How the speedups are
// obtained"; WIDE paper Sec. 1, tile-aligned prefixes).
//
// One workgroup of 1024 threads (16 waves of 64) per group. Pass 1 counts the
// active tokens of the column; pass 2 walks the column in chunks of 1024
// tokens: a 64-bit wave ballot gives each lane its rank among the wave's
// active lanes (mbcnt), an LDS scan over the 16 wave totals gives each wave
// its base, and running totals carry the bases across chunks. Active tokens
// go to perm[g][run_act + rank], inactive ones to perm[g][count + run_in +
// rank']. The same ballots, written out as 32-bit words, are the packed mask
// bits [ngroups, ceil(T/32)] that the down kernel predicates on.
#include "common.h"

namespace wide {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ uint32_t lane_rank(uint64_t ballot) {
  // number of set bits of `ballot` in lanes below this one
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(ballot >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)ballot, 0u));
}

__global__ __launch_bounds__(kThreads) void reorder_kernel(const uint8_t* __restrict__ mask, int T,
                                                            int ng, int tile,
                                                            int32_t* __restrict__ perm,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ padded,
                                                            uint32_t* __restrict__ maskbits,
                                                            int words) {
  __shared__ int s_act[kWaves];
  __shared__ int s_val[kWaves];
  __shared__ int s_count;
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // pass 1: popcount of the column
  int local = 0;
  for (int t = tid; t < T; t += kThreads) local += mask[(size_t)t * ng + g] != 0;
  for (int off = 32; off > 0; off >>= 1) local += __shfl_xor(local, off, 64);
  if (lane == 0) s_act[wave] = local;
  __syncthreads();
  if (tid == 0) {
    int c = 0;
    for (int w = 0; w < kWaves; ++w) c += s_act[w];
    s_count = c;
  }
  __syncthreads();
  const int count = s_count;

  // pass 2: place
  int32_t* __restrict__ prow = perm + (size_t)g * T;
  int run_act = 0, run_in = 0;
  for (int t0 = 0; t0 < T; t0 += kThreads) {
    const int t = t0 + tid;
    const bool valid = t < T;
    const bool act = valid && mask[(size_t)t * ng + g] != 0;
    const uint64_t b_act = __ballot(act);
    const uint64_t b_val = __ballot(valid);
    __syncthreads();  // previous chunk's readers of s_act/s_val are done
    if (lane == 0) {
      s_act[wave] = __popcll(b_act);
      s_val[wave] = __popcll(b_val);
    }
    __syncthreads();
    int base_act = 0, base_val = 0, tot_act = 0, tot_val = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int a = s_act[w], v = s_val[w];
      if (w < wave) {
        base_act += a;
        base_val += v;
      }
      tot_act += a;
      tot_val += v;
    }
    if (valid) {
      const int ra = (int)lane_rank(b_act);
      const int rv = (int)lane_rank(b_val);  // == lane for valid lanes
      if (act) {
        prow[run_act + base_act + ra] = t;
      } else {
        const int base_in = base_val - base_act;
        prow[count + run_in + base_in + (rv - ra)] = t;
      }
    }
    if (maskbits != nullptr && lane < 2) {
      const int tw = t0 + wave * 64;  // first token of this wave, a multiple of 64
      const int word = tw / 32 + lane;
      if (tw < T && word < words)
        maskbits[(size_t)g * words + word] = (uint32_t)(b_act >> (32 * lane));
    }
    run_act += tot_act;
    run_in += tot_val - tot_act;
  }
  if (tid == 0) {
    counts[g] = count;
    padded[g] = (int)(((long long)count + tile - 1) / tile) * tile;
  }
}

// Packed mask bits alone (the K-axis GEMM needs no row lists): thread (w, g)
// gathers bit b of word w of group g from mask[32w + b, g]; consecutive lanes
// take consecutive groups, so each of the 32 byte reads is coalesced.
__global__ __launch_bounds__(256) void pack_mask_bits_kernel(const uint8_t* __restrict__ mask,
                                                             int T, int ng, int words,
                                                             uint32_t* __restrict__ maskbits) {
  const unsigned idx = blockIdx.x * 256u + threadIdx.x;
  if (idx >= (unsigned)ng * (unsigned)words) return;
  const int g = (int)(idx % (unsigned)ng);
  const int w = (int)(idx / (unsigned)ng);
  const int t0 = 32 * w;
  const int n = min(32, T - t0);
  // Rows past T are clamped to the last row (so every load is in bounds and
  // none is predicated: the 32 loads are all issued before the first is used)
  // and their bits are cleared afterwards.
  uint8_t v[32];
#pragma unroll
  for (int b = 0; b < 32; ++b) v[b] = mask[(size_t)min(t0 + b, T - 1) * ng + g];
  uint32_t bits = 0;
#pragma unroll
  for (int b = 0; b < 32; ++b) bits |= (v[b] != 0 ? 1u : 0u) << b;
  if (n < 32) bits &= (1u << n) - 1u;
  maskbits[(size_t)g * words + w] = bits;
}

// Reorder from packed mask bits (the path inside wide_ffn_forward and
// wide_gemm_mn, where the bits are made by the packing kernel above from
// coalesced reads of the mask rows; the column reads of reorder_kernel touch a
// cache line per token). A workgroup of 256 threads owns one group and one
// chunk of 64 64-token words (4096 tokens) of its contiguous bit row: it counts
// the whole row and the words before its chunk, scans the chunk's word
// popcounts in one wave, and each wave places a word's 64 tokens at once
// (lane l: token 64 w + l; rank among the word's actives = popcount of the
// bits below l).
constexpr int kBitsThreads = 256;
constexpr int kBitsWaves = kBitsThreads / 64;
constexpr int kBitsChunk = 64;  // 64-token words per workgroup

__global__ __launch_bounds__(kBitsThreads) void reorder_bits_kernel(
    const uint32_t* __restrict__ maskbits, int T, int ng, int tile, int words,
    int32_t* __restrict__ perm, int32_t* __restrict__ counts, int32_t* __restrict__ padded) {
  __shared__ int s_sum[2][kBitsWaves];
  __shared__ int s_base[kBitsChunk];
  __shared__ uint64_t s_bits[kBitsChunk];
  const int g = blockIdx.x;
  const int c0 = (int)blockIdx.y * kBitsChunk;  // first word of this chunk
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const uint32_t* __restrict__ mb = maskbits + (size_t)g * words;
  const int nw64 = (words + 1) / 2;
  auto word64 = [&](int w) -> uint64_t {
    const uint64_t lo = mb[2 * w];
    const uint64_t hi = 2 * w + 1 < words ? mb[2 * w + 1] : 0u;
    return lo | (hi << 32);
  };

  // the row's count and the actives before this chunk
  int all = 0, before = 0;
  for (int w = tid; w < nw64; w += kBitsThreads) {
    const int pc = __popcll(word64(w));
    all += pc;
    before += w < c0 ? pc : 0;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    all += __shfl_xor(all, off, 64);
    before += __shfl_xor(before, off, 64);
  }
  if (lane == 0) {
    s_sum[0][wave] = all;
    s_sum[1][wave] = before;
  }
  // the chunk's words and their exclusive popcount scan (wave 0)
  if (wave == 0) {
    const int w = c0 + lane;
    const uint64_t bits = w < nw64 ? word64(w) : 0ull;
    const int pc = __popcll(bits);
    int incl = pc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    s_base[lane] = incl - pc;
    s_bits[lane] = bits;
  }
  __syncthreads();
  int count = 0, base0 = 0;
#pragma unroll
  for (int w = 0; w < kBitsWaves; ++w) {
    count += s_sum[0][w];
    base0 += s_sum[1][w];
  }
  int32_t* __restrict__ prow = perm + (size_t)g * T;
  const int nwc = min(kBitsChunk, nw64 - c0);
  for (int j = wave; j < nwc; j += kBitsWaves) {
    const uint64_t b = s_bits[j];
    const int base = base0 + s_base[j];
    const int t = 64 * (c0 + j) + lane;
    const int below = __popcll(b & ((1ull << lane) - 1ull));
    if (t < T) {
      const int pos = ((b >> lane) & 1ull) ? base + below : count + (t - base - below);
      prow[pos] = t;
    }
  }
  if (blockIdx.y == 0 && tid == 0) {
    counts[g] = count;
    padded[g] = (int)(((long long)count + tile - 1) / tile) * tile;
  }
}

}  // namespace

hipError_t launch_reorder_from_bits(const uint32_t* maskbits, int T, int ng, int tile,
                                    int32_t* perm, int32_t* counts, int32_t* padded,
                                    hipStream_t stream) {
  const int words = (T + 31) / 32;
  const int nw64 = (words + 1) / 2;
  const int nchunks = nw64 > 0 ? (nw64 + kBitsChunk - 1) / kBitsChunk : 1;
  hipLaunchKernelGGL(reorder_bits_kernel, dim3(ng, nchunks), dim3(kBitsThreads), 0, stream,
                     maskbits, T, ng, tile, words, perm, counts, padded);
  return hipGetLastError();
}

hipError_t launch_pack_mask_bits(const uint8_t* mask, int T, int ng, uint32_t* maskbits,
                                 hipStream_t stream) {
  const int words = (T + 31) / 32;
  const long long n = (long long)ng * words;
  if (n == 0) return hipSuccess;
  if (n > 0xFFFFFF00LL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_mask_bits_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     mask, T, ng, words, maskbits);
  return hipGetLastError();
}

hipError_t launch_reorder(const uint8_t* mask, int T, int ng, int tile, int32_t* perm,
                          int32_t* counts, int32_t* padded, uint32_t* maskbits,
                          hipStream_t stream) {
  const int words = (T + 31) / 32;
  hipLaunchKernelGGL(reorder_kernel, dim3(ng), dim3(kThreads), 0, stream, mask, T, ng, tile, perm,
                     counts, padded, maskbits, words);
  return hipGetLastError();
}

}  // namespace wide
