// Head-group-pruned attention for one decoding step (one new query per
// sequence at position T - 1, attending to the T cached keys; WIDE paper
// App. B, "Implementation of Attention": for decoding the routing is checked
// directly, without mask reordering, and the split online softmax follows the
// same predicated organisation; ai.info summary, "What gets pruned").
//
// The step streams the K/V cache of the kept groups, so it is bound by HBM:
//   * one workgroup per (128-key split, KV group); a group the token skips
//     exits at once and its K/V are never read (level-0 skipping);
//   * 16 lanes cover one 256-byte key row (16 bytes each), so a wave load
//     reads 4 whole rows; all K and V loads of a wave are issued before the
//     first is used;
//   * the group's HPG query heads share every K/V row (GQA packing): each
//     lane forms partial dot products for all of them over its 8 dims, and a
//     16-lane butterfly completes them;
//   * the split's softmax statistics (max, sum) and unnormalized O go to an
//     fp32 workspace; a second kernel merges the splits of each kept head in
//     a fixed order and rounds O once to bf16.
#include "common.h"

namespace wide {

namespace {

constexpr int kDcDh = 128;
constexpr int kDcKeys = 128;  // keys per split (4 waves x 32)
constexpr int kDcNI = kDcKeys / 16;  // key rows per lane
constexpr int kDcThreads = 256;

__device__ __forceinline__ u32x4 dc_ld(const uint16_t* p) { return *(const u32x4*)p; }

typedef __bf16 dc_bf16x2 __attribute__((ext_vector_type(2)));
// sum of the products of the eight bf16 pairs of a and b plus acc, in fp32
// (four v_dot2_f32_bf16; the pairs are built from whole-vector casts)
__device__ __forceinline__ float dot8_bf16(const u32x4& a, const u32x4& b, float acc) {
  const bf16x8 av = __builtin_bit_cast(bf16x8, a), bv = __builtin_bit_cast(bf16x8, b);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const dc_bf16x2 x = {av[2 * e], av[2 * e + 1]}, y = {bv[2 * e], bv[2 * e + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(x, y, acc, false);
  }
  return acc;
}

// partial record of one (split, head): m, l, then dh floats of O
constexpr int kDcRec = kDcDh + 2;

// Sum over the 16 lanes of each DPP row, left in every lane of the row: four
// row rotations (row_ror 8, 4, 2, 1) instead of LDS-crossbar shuffles.
__device__ __forceinline__ float row_sum16(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false));
  return v;
}

constexpr int kDcSlots = 16;  // 4 waves x 4 lane rows: partial (max, sum, O) slots in LDS

template <int HPG>
__global__ __launch_bounds__(kDcThreads) void attention_decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint8_t* __restrict__ mask, int T, int Hk,
    float scale_log2, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t s_q[HPG][kDcDh];
  __shared__ float s_m[kDcSlots][HPG], s_l[kDcSlots][HPG];
  __shared__ float s_o[kDcSlots][HPG][kDcDh];
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  if (mask[g] == 0) return;  // the token skips this head group
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = wave * 4 + (lane >> 4);  // this lane's row of 16 lanes
  const int Hq = Hk * HPG;
  const size_t ld = (size_t)Hk * kDcDh;
  for (int e = tid; e < HPG * kDcDh; e += kDcThreads)
    s_q[e / kDcDh][e % kDcDh] = q[(size_t)(g * HPG + e / kDcDh) * kDcDh + e % kDcDh];

  // lane: dims 8 (lane % 16) .. + 7 of key kDcKeys/4 * wave + 4 i + lane / 16
  const int d0 = 8 * (lane & 15);
  const int kbase = split * kDcKeys + (kDcKeys / 4) * wave + (lane >> 4);
  u32x4 kv[kDcNI], vv[kDcNI];
#pragma unroll
  for (int i = 0; i < kDcNI; ++i) {
    const int key = min(kbase + 4 * i, T - 1);  // keys past T are masked below
    kv[i] = dc_ld(K + (size_t)key * ld + (size_t)g * kDcDh + d0);
  }
#pragma unroll
  for (int i = 0; i < kDcNI; ++i) {
    const int key = min(kbase + 4 * i, T - 1);
    vv[i] = dc_ld(V + (size_t)key * ld + (size_t)g * kDcDh + d0);
  }
  __syncthreads();  // s_q ready
  u32x4 qr[HPG];  // this lane's 8 dims of every head's query (bf16, as given)
#pragma unroll
  for (int h = 0; h < HPG; ++h) qr[h] = *(const u32x4*)&s_q[h][d0];

  // scores (base 2); every lane of a row ends with its key's full dot
  float sc[kDcNI][HPG];
#pragma unroll
  for (int i = 0; i < kDcNI; ++i) {
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
      const float a = row_sum16(dot8_bf16(kv[i], qr[h], 0.0f));
      sc[i][h] = kbase + 4 * i < T ? a * scale_log2 : -INFINITY;
    }
  }
  // split max per head: in-lane over this row's keys, then over the 16 rows in LDS
  if ((lane & 15) == 0) {
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < kDcNI; ++i) m = fmaxf(m, sc[i][h]);
      s_m[slot][h] = m;
    }
  }
  __syncthreads();
  float mh[HPG];
#pragma unroll
  for (int h = 0; h < HPG; ++h) {
    float m = -INFINITY;
#pragma unroll
    for (int r = 0; r < kDcSlots; ++r) m = fmaxf(m, s_m[r][h]);
    mh[h] = m;  // finite: every split holds a key < T
  }
  float acc[HPG][8], lsum[HPG];
#pragma unroll
  for (int h = 0; h < HPG; ++h) {
    lsum[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
  }
#pragma unroll
  for (int i = 0; i < kDcNI; ++i) {
    const bf16x8 vb = __builtin_bit_cast(bf16x8, vv[i]);
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
      const float p = __builtin_amdgcn_exp2f(sc[i][h] - mh[h]);  // 0 for masked keys
      lsum[h] += p;  // (the same in every lane of the row)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, (float)vb[e], acc[h][e]);
    }
  }
  // partials of this row of lanes: O over its dims, the sum once per row
#pragma unroll
  for (int h = 0; h < HPG; ++h) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s_o[slot][h][d0 + e] = acc[h][e];
    if ((lane & 15) == 0) s_l[slot][h] = lsum[h];
  }
  __syncthreads();
  // record (m, l, O) of every head of the group for this split (slots summed in order)
  for (int e = tid; e < HPG * kDcDh; e += kDcThreads) {
    const int h = e / kDcDh, d = e % kDcDh;
    float o = 0.0f;
#pragma unroll
    for (int r = 0; r < kDcSlots; ++r) o += s_o[r][h][d];
    float* rec = part + ((size_t)split * Hq + g * HPG + h) * kDcRec;
    rec[2 + d] = o;
    if (d == 0) {
      float l = 0.0f;
#pragma unroll
      for (int r = 0; r < kDcSlots; ++r) l += s_l[r][h];
      rec[0] = mh[h];
      rec[1] = l;
    }
  }
}

// O[h] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the splits. One
// workgroup of 8 x dh threads per query head: slice z takes splits z, z + 8,
// ..., sixteen records at a time (their loads issued together) with a running
// maximum, and the 8 slices are merged in LDS in slice order.
constexpr int kDcSlices = 8;

__device__ __forceinline__ void merge_step(float mv, float lv, float ov, float& M, float& num,
                                           float& den) {
  const float Mn = fmaxf(M, mv);
  const float base = Mn == -INFINITY ? 0.0f : Mn;  // nothing seen yet: weights exp2(-inf) = 0
  const float a = __builtin_amdgcn_exp2f(M - base), w = __builtin_amdgcn_exp2f(mv - base);
  num = fmaf(w, ov, num * a);
  den = fmaf(w, lv, den * a);
  M = Mn;
}

__global__ __launch_bounds__(kDcSlices * kDcDh) void attention_decode_merge_kernel(
    const float* __restrict__ part, const uint8_t* __restrict__ mask, int nsplit, int Hq, int HPG,
    uint16_t* __restrict__ O, int zero_inactive) {
  __shared__ float s_M[kDcSlices][kDcDh], s_num[kDcSlices][kDcDh], s_den[kDcSlices][kDcDh];
  const int h = blockIdx.x;
  const int d = threadIdx.x % kDcDh, z = threadIdx.x / kDcDh;
  if (mask[h / HPG] == 0) {
    if (zero_inactive && z == 0) O[(size_t)h * kDcDh + d] = 0;
    return;
  }
  float M = -INFINITY, num = 0.0f, den = 0.0f;
  for (int s0 = z; s0 < nsplit; s0 += 16 * kDcSlices) {
    float mv[16], lv[16], ov[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int sp = s0 + kDcSlices * u;
      const float* rec = part + ((size_t)min(sp, nsplit - 1) * Hq + h) * kDcRec;
      mv[u] = sp < nsplit ? rec[0] : -INFINITY;
      lv[u] = rec[1];
      ov[u] = rec[2 + d];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) merge_step(mv[u], lv[u], ov[u], M, num, den);
  }
  s_M[z][d] = M;
  s_num[z][d] = num;
  s_den[z][d] = den;
  __syncthreads();
  if (z != 0) return;
  M = -INFINITY;
  num = den = 0.0f;
#pragma unroll
  for (int k = 0; k < kDcSlices; ++k) merge_step(s_M[k][d], s_den[k][d], s_num[k][d], M, num, den);
  O[(size_t)h * kDcDh + d] = f32_to_bf16_bits(num / den);
}

}  // namespace

int64_t attention_decode_splits(int64_t T) { return (T + kDcKeys - 1) / kDcKeys; }
size_t attention_decode_part_floats(int64_t T, int64_t Hq) {
  return (size_t)(attention_decode_splits(T) * Hq * kDcRec);
}

hipError_t launch_attention_decode_bf16(const uint16_t* q, const uint16_t* K, const uint16_t* V,
                                        const uint8_t* mask, int T, int Hq, int Hk, int dh,
                                        uint16_t* O, bool zero_inactive, float* part,
                                        hipStream_t stream) {
  if (dh != kDcDh || Hk <= 0 || Hq % Hk != 0) return hipErrorInvalidValue;
  const int hpg = Hq / Hk;
  const int nsplit = (int)attention_decode_splits(T);
  if (T > 0) {
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)dh);
    const dim3 grid(nsplit, Hk), block(kDcThreads);
    switch (hpg) {
      case 1:
        hipLaunchKernelGGL(attention_decode_split_kernel<1>, grid, block, 0, stream, q, K, V, mask,
                           T, Hk, scale_log2, part);
        break;
      case 2:
        hipLaunchKernelGGL(attention_decode_split_kernel<2>, grid, block, 0, stream, q, K, V, mask,
                           T, Hk, scale_log2, part);
        break;
      case 4:
        hipLaunchKernelGGL(attention_decode_split_kernel<4>, grid, block, 0, stream, q, K, V, mask,
                           T, Hk, scale_log2, part);
        break;
      case 8:
        hipLaunchKernelGGL(attention_decode_split_kernel<8>, grid, block, 0, stream, q, K, V, mask,
                           T, Hk, scale_log2, part);
        break;
      default:
        return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(attention_decode_merge_kernel, dim3(Hq), dim3(kDcSlices * kDcDh), 0, stream,
                     part, mask, nsplit, Hq, hpg, O, zero_inactive ? 1 : 0);
  return hipGetLastError();
}

}  // namespace wide
