// Head-group-pruned causal attention, prefill (WIDE paper App. B,
// "Implementation of Attention"; ai.info summary, "What gets pruned": the
// attention unit is a GQA-aligned group of H_q/H_k query heads, and each token
// keeps or skips each group).
//
// A workgroup owns one query head and one tile of 128 of its group's tokens in
// reordered order (the group's active tokens first, ascending). The head fixes
// its KV head, which is also its routing group. The stages:
//   * admission: tiles past the group's active prefix exit (or, when the caller
//     asks for zeros at skipped pairs, write them);
//   * Q prologue: each wave gathers the rows of its 32 queries into MFMA
//     operand registers once;
//   * dense K/V mainloop over the key tiles the tile's last (largest) position
//     needs, with the FlashAttention online softmax; K and V are the same for
//     every query, only the query side is predicated;
//   * scatter epilogue: output rows go back to their tokens.
// Readings (the pages give the organisation, not the formulas): causal over
// one sequence (key j is valid for query t when j <= t) and a scale of
// 1/sqrt(dh). A query with no valid key in a key tile gets P = 0 there and
// keeps its running maximum and sum.
//
// gfx950 design:
//   * Both products run on v_mfma_f32_32x32x16_bf16, transposed: S^T = K Q^T
//     puts one query per lane (lane % 32), so the softmax reductions over keys
//     are in-lane plus one exchange with lane ^ 32, and the rescale of the O^T
//     accumulator is per lane.
//   * Lane l of the K operand reads key row pi(l % 32), pi swapping bits 2 and
//     3. The accumulator element e of lane l then holds key
//     16 (e / 8) + 8 (l / 32) + e % 8 of its 32-key block, so the eight values
//     of one MFMA k-step are eight consecutive keys: P^T feeds O^T += V^T P^T
//     straight from registers as the B operand.
//   * V^T (per KV head, [dh, keys], zero past T) is built once per call by a
//     transpose kernel, so the A operand of O^T reads 16 contiguous bytes.
//   * K and V^T tiles (64 keys) go global -> LDS with register-bypassing
//     copies, double buffered: the copies of tile k+1 are in flight during
//     the MFMAs of tile k. 16-byte chunks are XOR-swizzled by row so that 16
//     lanes reading one chunk column hit distinct banks (each copying lane
//     fetches the chunk that the swizzle puts at its position).
//   * Level-2 skipping: a wave with no active query, or past its own last key
//     tile, skips its MFMAs but joins every barrier.
#include "common.h"

namespace wide {

namespace {

constexpr int kAtBQ = 128;   // queries per workgroup (4 waves x 32)
// keys per tile (a multiple of 32). 32-key tiles (160 registers, 32 KB of
// LDS: three workgroups per CU) measured 1.70 against 1.65 ms at the
// Llama3.1-8B shape, so 64 it is.
constexpr int kAtBK = 64;
constexpr int kAtNB = kAtBK / 32;  // 32-key MFMA blocks per tile
constexpr int kAtTpadAlign = 64;   // V^T rows are padded to multiples of 64 keys
constexpr int kAtDh = 128;   // head dimension
constexpr int kAtThreads = 256;
constexpr int kKBytes = kAtBK * kAtDh * 2;  // K tile [keys][128]: 256 B rows
constexpr int kVBytes = kAtDh * kAtBK * 2;  // V^T tile [128][keys]: kVRow B rows
constexpr int kVRow = kAtBK * 2;
constexpr int kVChunks = kVRow / 16;        // 16-byte chunks per V^T row
constexpr int kStage = kKBytes + kVBytes;
// workgroups per CU: the LDS of two stages and the registers allow three with
// 32-key tiles, two with 64-key tiles
constexpr int kAtMinBlocks = kAtBK == 32 ? 3 : 2;
static_assert(kAtBK % 32 == 0 && kAtTpadAlign % kAtBK == 0, "key tiles");
static_assert(2 * kStage >= 128 * 256, "the epilogue stages 128 rows of 256 bytes in the slots");

__device__ __forceinline__ int kswz(int row) { return row & 15; }
// V^T rows of 8 chunks (64 keys): 16 consecutive rows read one chunk column
// on distinct banks with (row & 7) ^ ((row >> 3) & 1); rows of 4 chunks (32
// keys) with (row >> 2) & 3 (rows r and r + 4 share a 256-byte bank line)
__device__ __forceinline__ int vswz(int row) {
  return kVChunks == 8 ? (row & 7) ^ ((row >> 3) & 1) : (row >> 2) & 3;
}
// key row read by MFMA row i of a 32-key block: bits 2 and 3 of i swapped
__device__ __forceinline__ int key_of_row(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

__device__ __forceinline__ u32x4 at_ld(const uint16_t* p) { return *(const u32x4*)p; }


__global__ __launch_bounds__(kAtThreads, kAtMinBlocks) void attention_prefill_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ Vt, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ counts, int T, int Tpad, int Hq, int Hk, float scale_log2,
    uint16_t* __restrict__ O, int zero_inactive) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kStage];
  const int h = blockIdx.y;
  const int g = h / (Hq / Hk);  // KV head = routing group
  const int count = counts[g];
  const int nact = (count + kAtBQ - 1) / kAtBQ;
  const int bx = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int32_t* __restrict__ prow = perm + (size_t)g * T;
  const size_t ldq = (size_t)Hq * kAtDh, ldk = (size_t)Hk * kAtDh;
  uint16_t* __restrict__ obase = O + (size_t)h * kAtDh;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  if (bx >= nact) {
    // admission: no active query here. The tile's rows are tokens that skip
    // the group (the partition's suffix); +0.0 for them if asked.
    if (!zero_inactive) return;
    const int r0 = bx * kAtBQ;
    const int r1 = min(T, r0 + kAtBQ);
    for (int e = tid; e < (r1 - r0) * 16; e += kAtThreads) {
      const int tok = prow[r0 + e / 16];
      *(u32x4*)(obase + (size_t)tok * ldq + (e % 16) * 8) = zero4;
    }
    return;
  }
  const int tile = nact - 1 - bx;  // the tiles with the latest positions start first
  const int r0 = tile * kAtBQ;
  const int nrow = min(kAtBQ, count - r0);  // >= 1
  const int nkt = prow[r0 + nrow - 1] / kAtBK + 1;

  // this lane's query: column q of the wave's 32
  const int q = lane & 31, hh = lane >> 5;
  const int wrow = wave * 32 + q;
  const int qpos = wrow < nrow ? prow[r0 + wrow] : -1;  // -1: no valid key anywhere
  const int wave_rows = min(32, nrow - wave * 32);
  const int wave_nkt = wave_rows > 0 ? prow[r0 + wave * 32 + wave_rows - 1] / kAtBK + 1 : 0;
  // key tiles below this one are valid for every kept query of the wave (the
  // wave's first row has its smallest position); only later tiles need the
  // causal compare
  const int wave_full = wave_rows > 0 ? (prow[r0 + wave * 32] + 1) / kAtBK : 0;

  // Q prologue: the B operand of S^T = K Q^T, k-step kk holds dims 16 kk + 8 hh .. + 7
  bf16x8 qf[kAtDh / 16];
  {
    const int tok = qpos >= 0 ? qpos : prow[r0];
    const uint16_t* pq = Q + (size_t)tok * ldq + (size_t)h * kAtDh + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < kAtDh / 16; ++kk) qf[kk] = __builtin_bit_cast(bf16x8, at_ld(pq + 16 * kk));
  }

  f32x16 o[kAtDh / 32];
#pragma unroll
  for (int j = 0; j < kAtDh / 32; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[j][e] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  // copies: register-bypassing global -> LDS copies of 1 KB per instruction
  // (lane l writes 16 bytes at l * 16). K slot: kAtBK key rows of 256 bytes,
  // 4 rows per copy; V^T slot: 128 dim rows of kVRow bytes. Each lane fetches
  // the logical chunk that the swizzle puts at its physical position. The
  // four waves share a tile's copies.
  const uint16_t* kbase = K + (size_t)g * kAtDh;
  const uint16_t* vbase = Vt + (size_t)g * kAtDh * Tpad;
  auto issue_k = [&](int kt, int slot) {
    uint8_t* sk = smem + slot * kStage;
#pragma unroll
    for (int i = 0; i < kKBytes / 4096; ++i) {
      const int blk = wave + 4 * i;
      const int row = 4 * blk + (lane >> 4);
      const int key = min(kt * kAtBK + row, T - 1);  // rows past T: never valid keys
      const int c = (lane & 15) ^ kswz(row);
      __builtin_amdgcn_global_load_lds((const void*)(kbase + (size_t)key * ldk + c * 8),
                                       (void*)(sk + blk * 1024), 16, 0, 0);
    }
  };
  auto issue_v = [&](int kt, int slot) {
    uint8_t* sv = smem + slot * kStage + kKBytes;
#pragma unroll
    for (int i = 0; i < kVBytes / 4096; ++i) {
      const int blk = wave + 4 * i;
      const int row = (64 / kVChunks) * blk + lane / kVChunks;
      const int c = (lane % kVChunks) ^ vswz(row);
      __builtin_amdgcn_global_load_lds((const void*)(vbase + (size_t)row * Tpad + kt * kAtBK + c * 8),
                                       (void*)(sv + blk * 1024), 16, 0, 0);
    }
  };

  const int krow0 = key_of_row(q);
  // S^T of key tile in K slot `slot` (its 32-key blocks)
  auto s_mfma = [&](f32x16 (&s)[kAtNB], int slot) {
    const uint8_t* sk = smem + slot * kStage;
#pragma unroll
    for (int b = 0; b < kAtNB; ++b) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[b][e] = 0.0f;
      const int krow = 32 * b + krow0;
      const uint8_t* pk = sk + krow * 256;
      const int sw = kswz(krow);
#pragma unroll
      for (int kk = 0; kk < kAtDh / 16; ++kk) {
        const bf16x8 a = *(const bf16x8*)(pk + (((2 * kk + hh) ^ sw) << 4));
        s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[b], 0, 0, 0);
      }
    }
  };
  // online softmax of tile kt's scores s: P (bf16 MFMA operands) and the
  // rescale factor of O; the running max and sum are updated
  auto mask_diag = [&](f32x16 (&s)[kAtNB], int kt) {
    // element e of block b is key kt*kAtBK + 32 b + 16 (e / 8) + 8 hh + e % 8.
    // Keys past a query's position get -inf (only on the wave's diagonal
    // tiles). The maximum is taken on the raw scores (the scale is positive,
    // so the order is the same) and the scale and the subtraction of the
    // maximum meet in one fma inside exp2: p = 2^(s c - m c), c = log2(e) /
    // sqrt(dh).
    if (kt >= wave_full) {
#pragma unroll
      for (int b = 0; b < kAtNB; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kt * kAtBK + 32 * b + 16 * (e >> 3) + 8 * hh + (e & 7);
          s[b][e] = key <= qpos ? s[b][e] : -INFINITY;
        }
    }
  };
  auto softmax_p = [&](f32x16 (&s)[kAtNB], bf16x8 (&pf)[kAtNB][2], float& alpha) {
    // the row maximum as a tree (a chain of dependent maxima otherwise)
    float mx[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      mx[e] = s[0][e];
#pragma unroll
      for (int b = 1; b < kAtNB; ++b) mx[e] = fmaxf(mx[e], s[b][e]);
    }
#pragma unroll
    for (int w = 8; w >= 1; w /= 2)
#pragma unroll
      for (int e = 0; e < w; ++e) mx[e] = fmaxf(mx[e], mx[e + w]);
    const float mt = fmaxf(mx[0], __shfl_xor(mx[0], 32));
    const float m_new = fmaxf(m_run, mt);  // raw-score units
    // While no key is valid the running max is -inf: the exponent base 0
    // then gives exp2(-inf) = 0 for every P and for alpha, never NaN (O and l
    // stay zero). A key that is not valid gets P = 0 the same way.
    const float mc = (m_new == -INFINITY ? 0.0f : m_new) * scale_log2;
    // exactly 1 when the maximum did not move (the fma would leave m c's
    // rounding error in the exponent)
    alpha = m_run == m_new ? 1.0f : __builtin_amdgcn_exp2f(fmaf(m_run, scale_log2, -mc));
    float psum = 0.0f;
#pragma unroll
    for (int b = 0; b < kAtNB; ++b)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[b][8 * c + 2 * i], scale_log2, -mc));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[b][8 * c + 2 * i + 1], scale_log2, -mc));
          psum += p0 + p1;
          w[i] = pack_bf16x2(p0, p1);
        }
        const u32x4 wv = {w[0], w[1], w[2], w[3]};
        pf[b][c] = __builtin_bit_cast(bf16x8, wv);
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
  };
  // O^T = alpha O^T + V^T P^T with the V^T tile in V slot `slot`; the
  // running max of most queries stops moving after the first tiles, so the
  // rescale runs only when some lane's max changed
  auto o_update = [&](const bf16x8 (&pf)[kAtNB][2], float alpha, int slot) {
    if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
      for (int j = 0; j < kAtDh / 32; ++j) o[j] *= alpha;
    }
    // O^T += V^T P^T: A = V^T rows (dims), B = P^T (k-step (b, c): keys 32 b + 16 c + 8 hh ..)
    const uint8_t* sv = smem + slot * kStage + kKBytes;
#pragma unroll
    for (int j = 0; j < kAtDh / 32; ++j) {
      const int vrow = 32 * j + q;
      const uint8_t* pv = sv + vrow * kVRow;
      const int sw = vswz(vrow);
#pragma unroll
      for (int b = 0; b < kAtNB; ++b)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bf16x8 a = *(const bf16x8*)(pv + (((4 * b + 2 * c + hh) ^ sw) << 4));
          o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[b][c], o[j], 0, 0, 0);
        }
    }
  };

  // K/V mainloop: tile i lives in slot i % 2; after the barrier that ends
  // iteration i, tile i + 2 is requested into that slot (used an iteration
  // later, after the next end-of-iteration wait and barrier). Tile indices
  // past the last are clamped (a valid tile reloaded into a free slot), so
  // no copy sits under a condition.
  const int last = nkt - 1;
  issue_k(0, 0);
  issue_v(0, 0);
  issue_k(min(1, last), 1);
  issue_v(min(1, last), 1);
  __builtin_amdgcn_s_waitcnt(WIDE_VMCNT(0));  // this wave's copies have landed
  __syncthreads();
  for (int i = 0; i < nkt; ++i) {
    if (i < wave_nkt) {
      f32x16 sc[kAtNB];
      bf16x8 pf[kAtNB][2];
      float alpha;
      s_mfma(sc, i & 1);
      mask_diag(sc, i);
      softmax_p(sc, pf, alpha);
      o_update(pf, alpha, i & 1);
    }
    __builtin_amdgcn_s_waitcnt(WIDE_VMCNT(0));  // tile i + 1 (requested after barrier i - 1)
    __syncthreads();
    issue_k(min(i + 2, last), i & 1);
    issue_v(min(i + 2, last), i & 1);
  }
  __builtin_amdgcn_s_waitcnt(WIDE_VMCNT(0));  // no copy outlives the loop
  __syncthreads();  // the epilogue reuses the slots

  // epilogue: O = O^T / l, staged in LDS as [row][dims] (16-byte chunks
  // swizzled by row), then whole 256-byte rows go to their tokens
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (wave_rows > 0) {
#pragma unroll
    for (int j = 0; j < kAtDh / 32; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // dims 32 j + 8 r + 4 hh .. + 3 of row wrow
        const u32x2 v = {pack_bf16x2(o[j][4 * r] * inv, o[j][4 * r + 1] * inv),
                         pack_bf16x2(o[j][4 * r + 2] * inv, o[j][4 * r + 3] * inv)};
        const int chunk = 4 * j + r;
        *(u32x2*)(smem + wrow * 256 + ((chunk ^ kswz(wrow)) << 4) + 8 * hh) = v;
      }
  }
  __syncthreads();
  for (int e = tid; e < kAtBQ * 16; e += kAtThreads) {
    const int row = e / 16, c = e % 16;
    if (r0 + row >= T) break;  // rows only grow with e
    const int tok = prow[r0 + row];
    if (row < nrow)
      *(u32x4*)(obase + (size_t)tok * ldq + c * 8) =
          *(const u32x4*)(smem + row * 256 + ((c ^ kswz(row)) << 4));
    else if (zero_inactive)
      *(u32x4*)(obase + (size_t)tok * ldq + c * 8) = zero4;
  }
}

// V [T, Hk * dh] -> V^T [Hk, dh, Tpad] (zeros past T), one workgroup per
// (64 tokens, KV head) through LDS so both sides move whole rows.
__global__ __launch_bounds__(256) void attention_vt_kernel(const uint16_t* __restrict__ V, int T,
                                                           int Tpad, int Hk,
                                                           uint16_t* __restrict__ Vt) {
  __shared__ uint16_t s[64][kAtDh + 8];
  const int t0 = blockIdx.x * 64;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const size_t ldk = (size_t)Hk * kAtDh;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = i * 256 + tid;
    const int t = idx / 16, c = idx % 16;
    const u32x4 v = at_ld(V + (size_t)min(t0 + t, T - 1) * ldk + (size_t)g * kAtDh + c * 8);
    const u32x4 w = t0 + t < T ? v : zero4;
    uint32_t* d = (uint32_t*)&s[t][c * 8];
    d[0] = w[0];
    d[1] = w[1];
    d[2] = w[2];
    d[3] = w[3];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = i * 256 + tid;
    const int dim = idx / 8, c = idx % 8;  // 8 tokens 8c .. 8c+7 of dim `dim`
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = (uint32_t)s[8 * c + 2 * k][dim] | ((uint32_t)s[8 * c + 2 * k + 1][dim] << 16);
    const u32x4 v = {w[0], w[1], w[2], w[3]};
    *(u32x4*)(Vt + ((size_t)g * kAtDh + dim) * Tpad + t0 + 8 * c) = v;
  }
}

}  // namespace

int64_t attention_tpad(int64_t T) { return (T + kAtTpadAlign - 1) / kAtTpadAlign * kAtTpadAlign; }

hipError_t launch_attention_prefill_bf16(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                                         const int32_t* perm, const int32_t* counts, int T, int Hq,
                                         int Hk, int dh, uint16_t* O, bool zero_inactive,
                                         uint16_t* Vt, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (dh != kAtDh || Hk <= 0 || Hq % Hk != 0) return hipErrorInvalidValue;
  const int Tpad = (int)attention_tpad(T);  // T * Hq * dh < 2^31 is checked by the caller
  hipLaunchKernelGGL(attention_vt_kernel, dim3(Tpad / 64, Hk), dim3(256), 0, stream, V, T, Tpad, Hk,
                     Vt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)dh);
  hipLaunchKernelGGL(attention_prefill_kernel, dim3((T + kAtBQ - 1) / kAtBQ, Hq), dim3(kAtThreads),
                     0, stream, Q, K, Vt, perm, counts, T, Tpad, Hq, Hk, scale_log2, O,
                     zero_inactive ? 1 : 0);
  return hipGetLastError();
}

}  // namespace wide
