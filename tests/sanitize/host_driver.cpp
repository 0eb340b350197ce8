// Sanitizer driver for the host side of libwide.so (test infrastructure):
// csrc/wide_api.cpp (argument validation, workspace layout, dispatch) is
// compiled for the host only, with AddressSanitizer and UndefinedBehavior-
// Sanitizer, and linked against the stand-in launchers below instead of the
// HIP kernels. Every "device" buffer is a host allocation of exactly the size
// the header documents (the workspace: exactly the size the library asks
// for). Each stand-in reads the first and last element of every input and
// writes every byte the real kernel writes, so a workspace carve that
// overlaps or overruns its allocation, or an output sized wrong, aborts under
// AddressSanitizer; a signed overflow in the size arithmetic aborts under
// UndefinedBehaviorSanitizer. Exits non-zero on a wrong status.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "common.h"
#include "wide.h"

extern "C" const char* hipGetErrorString(hipError_t) { return "stand-in"; }
extern "C" int c_caller_bad_enums(void* p);  // c_caller.c

namespace {
int g_launches = 0;
volatile uint8_t g_sink;
void rd(const void* p, size_t n) {  // touch the first and last byte
  if (n == 0) return;
  const uint8_t* b = static_cast<const uint8_t*>(p);
  g_sink = b[0];
  g_sink = b[n - 1];
}
void wr(void* p, size_t n) {
  if (n) memset(p, 0xA5, n);
}
size_t words(int T) { return (size_t)((T + 31) / 32); }
}  // namespace

namespace wide {
hipError_t launch_reorder(const uint8_t* mask, int T, int ng, int, int32_t* perm, int32_t* counts,
                          int32_t* padded, uint32_t* maskbits, hipStream_t) {
  ++g_launches;
  rd(mask, (size_t)T * ng);
  wr(perm, (size_t)ng * T * 4);
  wr(counts, (size_t)ng * 4);
  wr(padded, (size_t)ng * 4);
  if (maskbits) wr(maskbits, ng * words(T) * 4);
  return hipSuccess;
}
hipError_t launch_reorder_from_bits(const uint32_t* maskbits, int T, int ng, int, int32_t* perm,
                                    int32_t* counts, int32_t* padded, hipStream_t) {
  ++g_launches;
  rd(maskbits, ng * words(T) * 4);
  wr(perm, (size_t)ng * T * 4);
  wr(counts, (size_t)ng * 4);
  wr(padded, (size_t)ng * 4);
  return hipSuccess;
}
hipError_t launch_pack_mask_bits(const uint8_t* mask, int T, int ng, uint32_t* maskbits, hipStream_t) {
  ++g_launches;
  rd(mask, (size_t)T * ng);
  wr(maskbits, ng * words(T) * 4);
  return hipSuccess;
}
int64_t attention_tpad(int64_t T) { return (T + 63) / 64 * 64; }
hipError_t launch_attention_prefill_bf16(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                                         const int32_t* perm, const int32_t* counts, int T, int Hq,
                                         int Hk, int dh, uint16_t* O, bool, uint16_t* Vt,
                                         hipStream_t) {
  ++g_launches;
  rd(Q, (size_t)T * Hq * dh * 2);
  rd(K, (size_t)T * Hk * dh * 2);
  rd(V, (size_t)T * Hk * dh * 2);
  rd(perm, (size_t)Hk * T * 4);
  rd(counts, (size_t)Hk * 4);
  wr(Vt, (size_t)Hk * dh * attention_tpad(T) * 2);
  wr(O, (size_t)T * Hq * dh * 2);
  return hipSuccess;
}
int64_t attention_decode_splits(int64_t T) { return (T + 127) / 128; }
size_t attention_decode_part_floats(int64_t T, int64_t Hq) {
  return (size_t)(attention_decode_splits(T) * Hq * (128 + 2));
}
hipError_t launch_attention_decode_bf16(const uint16_t* q, const uint16_t* K, const uint16_t* V,
                                        const uint8_t* mask, int T, int Hq, int Hk, int dh,
                                        uint16_t* O, bool, float* part, hipStream_t) {
  ++g_launches;
  rd(q, (size_t)Hq * dh * 2);
  rd(K, (size_t)T * Hk * dh * 2);
  rd(V, (size_t)T * Hk * dh * 2);
  rd(mask, (size_t)Hk);
  wr(part, attention_decode_part_floats(T, Hq) * 4);
  wr(O, (size_t)Hq * dh * 2);
  return hipSuccess;
}
hipError_t launch_gate_up_bf16(const uint16_t* X, const uint16_t* Wg, const uint16_t* Wu,
                               const int32_t* perm, const int32_t* counts,
                               const uint32_t* maskbits, int T, int d, int d_ff, int G,
                               uint16_t* H, bool, hipStream_t) {
  ++g_launches;
  rd(X, (size_t)T * d * 2);
  rd(Wg, (size_t)d_ff * d * 2);
  rd(Wu, (size_t)d_ff * d * 2);
  if (gate_up_dense(G, d_ff)) {
    rd(maskbits, (size_t)(d_ff / G) * words(T) * 4);
  } else {
    rd(perm, (size_t)(d_ff / G) * T * 4);
    rd(counts, (size_t)(d_ff / G) * 4);
  }
  wr(H, (size_t)T * d_ff * 2);
  return hipSuccess;
}
hipError_t launch_gemm_mn_bf16(const uint16_t* A, const uint16_t* B, const int32_t* perm,
                               const int32_t* counts, int M, int K, int N, int G, uint16_t* C,
                               hipStream_t) {
  ++g_launches;
  rd(A, (size_t)M * K * 2);
  rd(B, (size_t)N * K * 2);
  rd(perm, (size_t)(N / G) * M * 4);
  rd(counts, (size_t)(N / G) * 4);
  wr(C, (size_t)M * N * 2);
  return hipSuccess;
}
hipError_t launch_down_bf16(const uint16_t* H, const uint16_t* Wd, const uint32_t* maskbits, int T,
                            int d, int d_ff, int G, uint16_t* Y, float* part, hipStream_t) {
  ++g_launches;
  rd(H, (size_t)T * d_ff * 2);
  rd(Wd, (size_t)d * d_ff * 2);
  rd(maskbits, (size_t)(d_ff / G) * words(T) * 4);
  if (part) wr(part, down_split_bytes(T, d, d_ff));
  wr(Y, (size_t)T * d * 2);
  return hipSuccess;
}
hipError_t launch_decode_pack_bf16(const uint16_t* W, int rows, int cols, uint16_t* out, hipStream_t) {
  ++g_launches;
  rd(W, (size_t)rows * cols * 2);
  wr(out, (size_t)rows * cols * 2);
  return hipSuccess;
}
hipError_t launch_decode_gate_up_bf16(const uint16_t* X, const uint16_t* Wg, const uint16_t* Wu,
                                      const uint16_t* Wg_op, const uint16_t* Wu_op,
                                      const uint8_t* mask, int T, int d, int d_ff, int G,
                                      uint16_t* H, bool, hipStream_t) {
  ++g_launches;
  rd(X, (size_t)T * d * 2);
  rd(Wg, (size_t)d_ff * d * 2);
  rd(Wu, (size_t)d_ff * d * 2);
  if (Wg_op) rd(Wg_op, (size_t)d_ff * d * 2);
  if (Wu_op) rd(Wu_op, (size_t)d_ff * d * 2);
  rd(mask, (size_t)T * (d_ff / G));
  wr(H, (size_t)T * d_ff * 2);
  return hipSuccess;
}
hipError_t launch_decode_down_bf16(const uint16_t* H, const uint16_t* Wd, const uint16_t* Wd_op,
                                   const uint8_t* mask, int T, int d, int d_ff, int G, uint16_t* Y,
                                   float* part, hipStream_t) {
  ++g_launches;
  rd(H, (size_t)T * d_ff * 2);
  rd(Wd, (size_t)d * d_ff * 2);
  if (Wd_op) rd(Wd_op, (size_t)d * d_ff * 2);
  rd(mask, (size_t)T * (d_ff / G));
  wr(part, (size_t)kDecodeDownSplit * T * d * 4);
  wr(Y, (size_t)T * d * 2);
  return hipSuccess;
}
hipError_t launch_router_bf16(const uint16_t* X, const uint16_t* W1, const uint16_t* W2, int T,
                              int D, int r, int ng, int, uint8_t* mask, float* logits,
                              uint32_t* maskbits, float* zpart, hipStream_t) {
  ++g_launches;
  rd(X, (size_t)T * D * 2);
  rd(W1, (size_t)r * D * 2);
  rd(W2, (size_t)2 * ng * r * 2);
  if (T <= kRouterSmallT) wr(zpart, router_zpart_bytes(T, r));
  if (mask) wr(mask, (size_t)T * ng);
  if (logits) wr(logits, (size_t)T * ng * 2 * 4);
  if (maskbits) wr(maskbits, (size_t)ng * words(T) * 4);
  return hipSuccess;
}
// the scratch array of wide_ffn_forward_noalloc: an exact-size host buffer
hipError_t noalloc_scratch(hipStream_t, void** out) {
  static void* p = aligned_alloc(256, WIDE_NOALLOC_SCRATCH_BYTES);
  *out = p;
  return hipSuccess;
}
hipError_t launch_gate_up_f32(const float* X, const float* Wg, const float* Wu, const int32_t* perm,
                              const int32_t* counts, int T, int d, int d_ff, int G, float* H, bool,
                              hipStream_t) {
  ++g_launches;
  rd(X, (size_t)T * d * 4);
  rd(Wg, (size_t)d_ff * d * 4);
  rd(Wu, (size_t)d_ff * d * 4);
  rd(perm, (size_t)(d_ff / G) * T * 4);
  rd(counts, (size_t)(d_ff / G) * 4);
  wr(H, (size_t)T * d_ff * 4);
  return hipSuccess;
}
hipError_t launch_down_f32(const float* H, const float* Wd, const uint32_t* maskbits, int T, int d,
                           int d_ff, int G, float* Y, hipStream_t) {
  ++g_launches;
  rd(H, (size_t)T * d_ff * 4);
  rd(Wd, (size_t)d * d_ff * 4);
  rd(maskbits, (size_t)(d_ff / G) * words(T) * 4);
  wr(Y, (size_t)T * d * 4);
  return hipSuccess;
}
}  // namespace wide

namespace {
int fails = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "%s:%d: failed: %s (%s)\n", __FILE__, __LINE__, #cond, \
              wide_last_error());                                           \
      ++fails;                                                              \
    }                                                                       \
  } while (0)

// A host buffer of exactly n bytes (256-byte aligned start, as the device
// allocator gives; the allocation ends at the last byte, so an access past
// it is an overflow).
struct Buf {
  void* p = nullptr;
  size_t n = 0;
  explicit Buf(size_t bytes) : n(bytes) {
    p = aligned_alloc(256, (bytes + 255) / 256 * 256);
    memset(p, 0, (bytes + 255) / 256 * 256);
  }
  ~Buf() { free(p); }
  Buf(const Buf&) = delete;
  Buf& operator=(const Buf&) = delete;
};

// Workspace of exactly `need` bytes, 256-byte aligned: the last 256-byte
// block is allocated in full, so a one-byte overrun of the carve past `need`
// rounded down would stay unseen; the sizes here are multiples of 256.
void ffn_case(int T, int d, int d_ff, int G, wide_dtype_t dt, bool with_h, uint32_t flags) {
  const size_t e = dt == WIDE_BF16 ? 2 : 4;
  Buf X((size_t)T * d * e), Wg((size_t)d_ff * d * e), Wu((size_t)d_ff * d * e),
      Wd((size_t)d * d_ff * e), mask((size_t)T * (d_ff / G)), Y((size_t)T * d * e),
      H((size_t)T * d_ff * e);
  const size_t need = wide_ffn_workspace_size_for(T, d, d_ff, G, dt, with_h ? 1 : 0);
  EXPECT(need % 256 == 0);
  Buf ws(need);
  const int before = g_launches;
  EXPECT(wide_ffn_forward(X.p, Wg.p, Wu.p, Wd.p, (const uint8_t*)mask.p, T, d, d_ff, G, dt, Y.p,
                          with_h ? H.p : nullptr, ws.p, need, flags, nullptr) == WIDE_OK);
  EXPECT(T == 0 || g_launches > before);
  EXPECT(wide_ffn_forward(X.p, Wg.p, Wu.p, Wd.p, (const uint8_t*)mask.p, T, d, d_ff, G, dt, Y.p,
                          with_h ? H.p : nullptr, ws.p, need - 1, flags,
                          nullptr) == (T == 0 && need == 0 ? WIDE_OK : WIDE_ERR_WORKSPACE) ||
         need == 0);
  const bool dec = T <= wide_decode_max_t() && dt == WIDE_BF16 && !(flags & WIDE_FLAG_FORCE_PREFILL);
  const int stages[3] = {dec ? WIDE_STAGE_DECODE_GATE_UP : WIDE_STAGE_REORDER,
                         dec ? WIDE_STAGE_DECODE_DOWN : WIDE_STAGE_GATE_UP,
                         dec ? -1 : WIDE_STAGE_DOWN};
  for (int s : stages)
    if (s >= 0)
      EXPECT(wide_ffn_stage((wide_stage_t)s, X.p, Wg.p, Wu.p, Wd.p, (const uint8_t*)mask.p, T, d,
                            d_ff, G, dt, Y.p, with_h ? H.p : nullptr, ws.p, need, flags,
                            nullptr) == WIDE_OK);
  if (with_h) {
    const size_t small = wide_ffn_workspace_size_for(T, d, d_ff, G, dt, 1);
    EXPECT(wide_ffn_forward_noalloc(X.p, Wg.p, Wu.p, Wd.p, (const uint8_t*)mask.p, T, d, d_ff, G,
                                    dt, Y.p, H.p, flags, nullptr) ==
           (small <= WIDE_NOALLOC_SCRATCH_BYTES ? WIDE_OK : WIDE_ERR_WORKSPACE));
  } else {
    EXPECT(wide_ffn_forward_noalloc(X.p, Wg.p, Wu.p, Wd.p, (const uint8_t*)mask.p, T, d, d_ff, G,
                                    dt, Y.p, nullptr, flags, nullptr) ==
           (T == 0 ? WIDE_OK : WIDE_ERR_NULL));
  }
  if (dt == WIDE_BF16 && T <= WIDE_DECODE_T_LIMIT && d_ff % 64 == 0) {
    const size_t pn = wide_decode_weights_size(d, d_ff);
    Buf prep(pn);
    EXPECT(wide_decode_prepare_weights(Wg.p, Wu.p, Wd.p, d, d_ff, prep.p, pn, nullptr) == WIDE_OK);
    EXPECT(wide_ffn_decode_prepared(X.p, Wg.p, Wu.p, Wd.p, prep.p, pn, (const uint8_t*)mask.p, T, d,
                                    d_ff, G, Y.p, with_h ? H.p : nullptr, ws.p, need,
                                    nullptr) == WIDE_OK);
    EXPECT(wide_ffn_decode_prepared(X.p, Wg.p, Wu.p, Wd.p, prep.p, pn - 1, (const uint8_t*)mask.p,
                                    T, d, d_ff, G, Y.p, with_h ? H.p : nullptr, ws.p, need,
                                    nullptr) == WIDE_ERR_WORKSPACE);
  }
}

void gemm_case(int M, int N, int K, int G, bool kaxis) {
  Buf A((size_t)M * K * 2), B((size_t)N * K * 2), C((size_t)M * N * 2),
      mask((size_t)M * ((kaxis ? K : N) / G));
  const size_t need = wide_gemm_workspace_size(M, (kaxis ? K : N) / G);
  Buf ws(need);
  auto fn = kaxis ? wide_gemm_k : wide_gemm_mn;
  EXPECT(fn(A.p, B.p, (const uint8_t*)mask.p, M, N, K, G, WIDE_BF16, C.p, ws.p, need, nullptr) ==
         WIDE_OK);
  if (M > 0)
    EXPECT(fn(A.p, B.p, (const uint8_t*)mask.p, M, N, K, G, WIDE_BF16, C.p, ws.p, need - 1,
              nullptr) == WIDE_ERR_WORKSPACE);
  EXPECT(fn(A.p, B.p, (const uint8_t*)mask.p, M, N, K, G + 1, WIDE_BF16, C.p, ws.p, need,
            nullptr) != WIDE_OK);
}

void attention_case(int T, int Hq, int Hk) {
  const int dh = 128;
  Buf Q((size_t)T * Hq * dh * 2), K((size_t)T * Hk * dh * 2), V((size_t)T * Hk * dh * 2),
      O((size_t)T * Hq * dh * 2), mask((size_t)T * Hk);
  const size_t need = wide_attention_workspace_size(T, Hk, dh);
  Buf ws(need);
  EXPECT(wide_attention_prefill(Q.p, K.p, V.p, (const uint8_t*)mask.p, T, Hq, Hk, dh, WIDE_BF16,
                                O.p, WIDE_ATTN_ZERO_INACTIVE, ws.p, need, nullptr) == WIDE_OK);
  EXPECT(wide_attention_prefill(Q.p, K.p, V.p, (const uint8_t*)mask.p, T, Hq, Hk, 64, WIDE_BF16,
                                O.p, 0, ws.p, need, nullptr) == WIDE_ERR_UNSUPPORTED);
  if (T < 1) return;
  const size_t nd = wide_attention_decode_workspace_size(T, Hq, dh);
  Buf wd(nd), q((size_t)Hq * dh * 2), od((size_t)Hq * dh * 2), md((size_t)Hk);
  EXPECT(wide_attention_decode(q.p, K.p, V.p, (const uint8_t*)md.p, T, Hq, Hk, dh, WIDE_BF16, od.p,
                               0, wd.p, nd, nullptr) == WIDE_OK);
  EXPECT(wide_attention_decode(q.p, K.p, V.p, (const uint8_t*)md.p, T, Hq, Hk, dh, WIDE_BF16, od.p,
                               0, wd.p, nd - 1, nullptr) == WIDE_ERR_WORKSPACE);
}

void router_reorder_case(int T, int D, int r, int ng, bool mask_out) {
  Buf X((size_t)T * D * 2), W1((size_t)r * D * 2), W2((size_t)2 * ng * r * 2), mask((size_t)T * ng),
      perm((size_t)ng * T * 4), counts((size_t)ng * 4), padded((size_t)ng * 4);
  const size_t need = wide_router_reorder_workspace_size(T, ng);
  Buf ws(need);
  EXPECT(wide_router_reorder(X.p, W1.p, W2.p, T, D, r, ng, WIDE_ACT_SILU, WIDE_BF16, 7,
                             mask_out ? (uint8_t*)mask.p : nullptr, nullptr, (int32_t*)perm.p,
                             (int32_t*)counts.p, (int32_t*)padded.p, ws.p, need,
                             nullptr) == WIDE_OK);
  if (need > 0)
    EXPECT(wide_router_reorder(X.p, W1.p, W2.p, T, D, r, ng, WIDE_ACT_SILU, WIDE_BF16, 7, nullptr,
                               nullptr, (int32_t*)perm.p, (int32_t*)counts.p, (int32_t*)padded.p,
                               ws.p, need - 1, nullptr) == WIDE_ERR_WORKSPACE);
}

void router_case(int T, int D, int r, int ng, bool logits) {
  Buf X((size_t)T * D * 2), W1((size_t)r * D * 2), W2((size_t)2 * ng * r * 2), mask((size_t)T * ng),
      lg((size_t)T * ng * 2 * 4);
  const size_t need = wide_router_workspace_size(T, r);
  Buf ws(need);
  EXPECT(wide_router_forward(X.p, W1.p, W2.p, T, D, r, ng, WIDE_ACT_SILU, WIDE_BF16,
                             (uint8_t*)mask.p, logits ? (float*)lg.p : nullptr,
                             need ? ws.p : nullptr, need, nullptr) == WIDE_OK);
  if (need > 0)
    EXPECT(wide_router_forward(X.p, W1.p, W2.p, T, D, r, ng, WIDE_ACT_SILU, WIDE_BF16,
                               (uint8_t*)mask.p, nullptr, ws.p, need - 1,
                               nullptr) == WIDE_ERR_WORKSPACE);
  EXPECT(wide_router_forward(X.p, W1.p, W2.p, T, D, 24, ng, WIDE_ACT_SILU, WIDE_BF16,
                             (uint8_t*)mask.p, nullptr, ws.p, need, nullptr) == WIDE_ERR_UNSUPPORTED);
}
}  // namespace

int main() {
  // prefill (reorder, gate/up, down), decode, fp32, ragged and edge sizes
  const wide_dtype_t bf = WIDE_BF16, f32 = WIDE_F32;
  for (int with_h = 0; with_h < 2; ++with_h) {
    ffn_case(300, 256, 1024, 64, bf, with_h, 0);
    ffn_case(33, 128, 1536, 48, bf, with_h, 0);
    ffn_case(17, 192, 512, 16, bf, with_h, 0);
    ffn_case(5, 256, 1024, 128, bf, with_h, 0);            // decode
    ffn_case(16, 256, 1024, 128, bf, with_h, 0);           // decode, largest T
    ffn_case(1, 512, 2048, 32, bf, with_h, 0);             // decode, one token
    ffn_case(7, 256, 1024, 64, bf, with_h, WIDE_FLAG_FORCE_PREFILL);
    ffn_case(40, 64, 256, 64, f32, with_h, 0);
    ffn_case(3, 64, 320, 64, f32, with_h, 0);              // fp32 never takes the decode path
    ffn_case(0, 64, 128, 64, bf, with_h, 0);
  }
  // prefill whose workspace (without H) nearly fills the scratch array
  // (32.4 of its 33.6 MB)
  EXPECT(wide_ffn_workspace_size_for(122880, 64, 1024, 16, bf, 1) > (30u << 20));
  ffn_case(122880, 64, 1024, 16, bf, true, 0);
  gemm_case(300, 1024, 256, 256, false);
  gemm_case(300, 256, 1024, 256, true);
  gemm_case(77, 64, 128, 64, false);  // one group: dynamic depth
  gemm_case(0, 64, 128, 64, true);
  attention_case(200, 8, 2);
  attention_case(1, 4, 4);
  attention_case(0, 4, 1);
  router_case(100, 256, 32, 7, true);
  router_case(1, 512, 16, 40, false);
  router_case(0, 64, 64, 3, false);
  router_case(16, 4096, 64, 112, true);
  router_case(17, 4096, 32, 112, false);
  router_reorder_case(1000, 256, 32, 37, true);
  router_reorder_case(33, 64, 16, 1, false);
  router_reorder_case(0, 64, 16, 5, false);
  router_reorder_case(16, 256, 64, 9, true);
  router_reorder_case(1, 4096, 32, 112, false);
  // rejected arguments: nothing launched, a message set
  const int before = g_launches;
  std::vector<uint8_t> small(4096);
  void* p = small.data();
  EXPECT(wide_ffn_forward(p, p, p, p, (const uint8_t*)p, 64, 96, 1024, 64, WIDE_BF16, p, nullptr, p,
                          1u << 30, 0, nullptr) == WIDE_ERR_UNSUPPORTED);
  EXPECT(wide_ffn_forward(p, p, p, p, (const uint8_t*)p, 1 << 20, 4096, 4096, 128, WIDE_BF16, p,
                          nullptr, p, 1u << 30, 0, nullptr) == WIDE_ERR_UNSUPPORTED);
  EXPECT(wide_ffn_forward(p, p, p, p, (const uint8_t*)p, INT32_MAX, 65536, 65536, 16, WIDE_BF16,
                          p, nullptr, p, 1u << 30, 0, nullptr) == WIDE_ERR_UNSUPPORTED);
  EXPECT(wide_reorder_masks((const uint8_t*)p, 1 << 30, 8, 4, (int32_t*)p, (int32_t*)p,
                            (int32_t*)p, nullptr) == WIDE_ERR_SHAPE);
  EXPECT(wide_ffn_workspace_size(INT32_MAX, 65536, 65536, 16, WIDE_BF16) > 0);
  EXPECT(wide_gemm_workspace_size(INT32_MAX, 4096) > 0);
  EXPECT(wide_attention_workspace_size(INT32_MAX, 64, 128) > 0);
  EXPECT(wide_attention_decode_workspace_size(INT32_MAX, 64, 128) > 0);
  EXPECT(g_launches == before);
  // enum arguments outside their enumerators, passed from C
  EXPECT(c_caller_bad_enums(p) == 0);
  {
    // reorder, standalone, with exact-size outputs
    const int T = 1025, ng = 5;
    Buf mask((size_t)T * ng), perm((size_t)ng * T * 4), counts(ng * 4), padded(ng * 4);
    EXPECT(wide_reorder_masks((const uint8_t*)mask.p, T, ng, 7, (int32_t*)perm.p,
                              (int32_t*)counts.p, (int32_t*)padded.p, nullptr) == WIDE_OK);
  }
  if (fails) return 1;
  printf("host sanitizer driver: ok (%d stand-in launches)\n", g_launches);
  return 0;
}
