// Shared bf16 MFMA mainloop of the prefill kernels (gate/up and down).
//
// A workgroup of 8 waves computes acc += P . Q^T for a tile of TP rows of P
// (the MFMA A operand) and TQ rows of Q (the MFMA B operand), reducing over K
// in stages of 64. Both operands are bf16 rows with K contiguous.
//
// Data movement, designed for gfx950:
//   * global -> LDS copies that bypass registers (16 bytes per lane); one
//     1 KB copy instruction fills 8 LDS rows of 128 bytes;
//   * two LDS stages; the copies of stage s+2 are issued right after the
//     barrier of stage s, so they overlap the MFMAs of stage s+1;
//   * 16-byte chunk c of LDS row r is stored at chunk c ^ swz(r), which keeps
//     the 16 lanes that read one MFMA fragment row-group on distinct banks;
//   * fragments are read one MFMA k-step ahead of their use, and the barrier
//     sits before the last k-step of a stage so the fragments of the next
//     stage are read while the last MFMAs of this one run. The P fragments of
//     the next k-step are read in one burst at the start of a k-step (two
//     register sets); each Q fragment is read again right after its last
//     MFMA of the current k-step (one set), which spreads the LDS reads over
//     the k-step (dense probe: 2-5% faster than reading both in one burst);
//   * v_mfma_f32_32x32x16_bf16, fp32 accumulation in registers.
//
// Output fragment layout (per wave, fragment (i, j)): lane l holds Q row
// (j*32 + l%32) and P rows i*32 + 8*(e/4) + 4*(l/32) + e%4 for e = 0..15, i.e.
// four runs of four consecutive P rows.
#pragma once

#include "common.h"

namespace wide {
namespace core {

constexpr int kBK = 64;         // K per LDS stage
constexpr int kRowBytes = 128;  // one LDS row holds 64 bf16 of K

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }


template <int TP_, int TQ_, int WP_, int WQ_>
struct Shape {
  static constexpr int TP = TP_, TQ = TQ_, WP = WP_, WQ = WQ_;
  static constexpr int NW = WP * WQ;
  static_assert(NW == 8, "the mainloop runs 8 waves");
  static constexpr int PW = TP / WP, QW = TQ / WQ;  // rows per wave
  static constexpr int FP = PW / 32, FQ = QW / 32;  // 32-row fragments per wave
  static_assert(FP >= 1 && FQ >= 1 && PW % 32 == 0 && QW % 32 == 0, "fragment shape");
  static constexpr int PBYTES = TP * kRowBytes;
  static constexpr int STAGE = (TP + TQ) * kRowBytes;
  static constexpr int PBLOCKS = TP / 8, QBLOCKS = TQ / 8;  // 1 KB copy blocks per stage
};

// The copy lane mapping: lane l of a copy into 1 KB block b writes LDS row
// 8b + l/8 at physical chunk l%8, which holds logical chunk (l%8) ^ swz(row).
// Returns the logical chunk (0..7) lane l must fetch for a block b.
__device__ __forceinline__ int copy_chunk(int b, int lane) {
  const int row = 8 * b + (lane >> 3);
  return (lane & 7) ^ swz(row);
}

// Accumulators and fragment registers of one wave.
template <class S>
struct Frags {
  f32x16 acc[S::FP][S::FQ];
  bf16x8 fa[2][S::FP];
  bf16x8 fb[S::FQ];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < S::FP; ++i)
#pragma unroll
      for (int j = 0; j < S::FQ; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  }

  // P fragments of MFMA k-step kk (0..3) of the stage held at `stage`, into `set`.
  __device__ __forceinline__ void load_p(const uint8_t* stage, int kk, int set, int pbase, int sw,
                                         int lhalf) {
    const int off = ((kk * 2 + lhalf) ^ sw) << 4;
#pragma unroll
    for (int i = 0; i < S::FP; ++i)
      fa[set][i] = *(const bf16x8*)(stage + pbase + i * 32 * kRowBytes + off);
  }

  // Q fragment j of MFMA k-step kk of the stage held at `stage`.
  __device__ __forceinline__ void load_q(const uint8_t* stage, int kk, int j, int qbase, int sw,
                                         int lhalf) {
    const int off = ((kk * 2 + lhalf) ^ sw) << 4;
    fb[j] = *(const bf16x8*)(stage + S::PBYTES + qbase + j * 32 * kRowBytes + off);
  }

  // MFMAs of one k-step with P set `set`; Q fragments j >= nq are skipped
  // (their rows are inactive). When `next` is set, Q fragment j of k-step nkk
  // of the stage at `next` is read right after its last MFMA here.
  __device__ __forceinline__ void step(int set, int nq, const uint8_t* next, int nkk, int qbase,
                                       int sw, int lhalf) {
#pragma unroll
    for (int j = 0; j < S::FQ; ++j) {
      if (j < nq) {
#pragma unroll
        for (int i = 0; i < S::FP; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][i], fb[j], acc[i][j], 0, 0, 0);
        if (next != nullptr) load_q(next, nkk, j, qbase, sw, lhalf);
      }
    }
  }
};

// Runs the mainloop over `nst` stages. issue(s, stage_ptr) enqueues this
// wave's copies of stage s into the LDS stage at stage_ptr (waves may issue
// different numbers of copies; every wait drains this wave's copies). sA/sB are the two LDS stages. nq is the
// number of this wave's Q fragments that hold at least one active row (level-2
// skipping); a wave with nq == 0 still joins every barrier.
// prepare(s) is called for stage s at least one k-step before issue(s) (for
// stages >= 2 during the first k-step of stage s-2, while MFMAs run), so
// per-stage copy offsets can be computed off the critical path.
template <class S, class Issue, class Prepare>
__device__ __forceinline__ void mainloop(Frags<S>& f, uint8_t* sA, uint8_t* sB, int nst, int wp,
                                         int wq, int lane, int nq, Issue&& issue,
                                         Prepare&& prepare) {
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int sw = swz(lrow);  // fragment bases are multiples of 32 rows
  const int pbase = (wp * S::PW + lrow) * kRowBytes;
  const int qbase = (wq * S::QW + lrow) * kRowBytes;
  f.zero();
  if (nst <= 0) return;
  prepare(0);
  issue(0, sA);
  if (nst > 1) {
    prepare(1);
    issue(1, sB);
  }
  __builtin_amdgcn_s_waitcnt(WIDE_VMCNT(0));
  __syncthreads();
  f.load_p(sA, 0, 0, pbase, sw, lhalf);
#pragma unroll
  for (int j = 0; j < S::FQ; ++j)
    if (j < nq) f.load_q(sA, 0, j, qbase, sw, lhalf);
  for (int s = 0; s < nst; ++s) {
    uint8_t* cur = (s & 1) ? sB : sA;
    uint8_t* nxt = (s & 1) ? sA : sB;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int set = kk & 1;
      if (kk < 3) {
        f.load_p(cur, kk + 1, set ^ 1, pbase, sw, lhalf);
        if (kk == 0 && s + 2 < nst) prepare(s + 2);
        f.step(set, nq, cur, kk + 1, qbase, sw, lhalf);
      } else {
        // stage s+1 must have landed (each wave waits for its own copies)
        // and be visible to all waves; after the barrier every wave has read
        // its last fragments of stage s, so its buffer can be refilled.
        __builtin_amdgcn_s_waitcnt(WIDE_VMCNT(0));
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        if (s + 2 < nst) issue(s + 2, cur);
        const bool more = s + 1 < nst;
        if (more) f.load_p(nxt, 0, set ^ 1, pbase, sw, lhalf);
        f.step(set, nq, more ? nxt : nullptr, 0, qbase, sw, lhalf);
      }
    }
  }
}

template <class S, class Issue>
__device__ __forceinline__ void mainloop(Frags<S>& f, uint8_t* sA, uint8_t* sB, int nst, int wp,
                                         int wq, int lane, int nq, Issue&& issue) {
  mainloop(f, sA, sB, nst, wp, wq, lane, nq, issue, [](int) {});
}

}  // namespace core
}  // namespace wide
