// C ABI of libwide.so: argument validation, workspace layout, path dispatch
// and kernel launches. Everything is enqueued on the caller's stream; no call
// allocates, frees, synchronises or reads device memory on the host.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "common.h"
#include "wide.h"

#define WIDE_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

wide_status_t fail(wide_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

wide_status_t ok() {
  g_last_error.clear();
  return WIDE_OK;
}

wide_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return WIDE_OK;
  return fail(WIDE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// An enum argument as the int the C caller passed. C lets a caller pass any
// int for an enum parameter; reading a value outside the enumerators as a C++
// enum is undefined, so every entry point reads its enum arguments through
// this and validates the int.
template <class E>
int32_t raw(const E& e) {  // by reference: no enum-typed load
  static_assert(sizeof(E) == sizeof(int32_t), "C enums are int-sized on this ABI");
  int32_t v;
  memcpy(&v, &e, sizeof v);
  return v;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t elt_size(int32_t dt) { return dt == WIDE_BF16 ? 2 : 4; }

// Workspace layout (each region 256-byte aligned):
//   perm     int32  [ngroups, T]
//   counts   int32  [ngroups]
//   padded   int32  [ngroups]
//   maskbits uint32 [ngroups, ceil(T/32)]
//   part     fp32   [kDecodeDownSplit, T, d]   (T <= WIDE_DECODE_T_LIMIT only:
//                   the decode down GEMV's partial sums)
//   dpart    fp32   down_split_bytes(T, d, d_ff) (the prefill down
//                   projection's split last-round tiles; often empty)
//   H        dtype  [T, d_ff]   (only when the caller passes no H_out; last, so
//                   the other offsets do not depend on it)
struct Layout {
  size_t perm, counts, padded, maskbits, h, part, dpart, total;
};

Layout layout(int64_t T, int64_t d, int64_t d_ff, int64_t G, int32_t dt, bool with_h) {
  const int64_t ng = d_ff / G;
  const int64_t words = (T + 31) / 32;
  Layout L{};
  size_t off = 0;
  L.perm = off;
  off = round_up(off + (size_t)(ng * T) * 4, 256);
  L.counts = off;
  off = round_up(off + (size_t)ng * 4, 256);
  L.padded = off;
  off = round_up(off + (size_t)ng * 4, 256);
  L.maskbits = off;
  off = round_up(off + (size_t)(ng * words) * 4, 256);
  L.part = off;
  if (T <= WIDE_DECODE_T_LIMIT) off = round_up(off + (size_t)(wide::kDecodeDownSplit * T * d) * 4, 256);
  L.dpart = off;
  off = round_up(off + wide::down_split_bytes((int)T, (int)d, (int)d_ff), 256);
  L.h = off;
  if (with_h) off = round_up(off + (size_t)(T * d_ff) * elt_size(dt), 256);
  L.total = off;
  return L;
}

int decode_max_t_value() {
  static const int v = [] {
    const char* s = std::getenv("WIDE_DECODE_MAX_T");
    if (s == nullptr || *s == '\0') return (int)WIDE_DECODE_T_LIMIT;
    char* end = nullptr;
    long x = std::strtol(s, &end, 10);
    if (end == s || x < 0) return (int)WIDE_DECODE_T_LIMIT;
    return (int)(x > WIDE_DECODE_T_LIMIT ? WIDE_DECODE_T_LIMIT : x);
  }();
  return v;
}

struct Args {
  const void* X;
  const void* Wg;
  const void* Wu;
  const void* Wd;
  const uint8_t* mask;
  int32_t T, d, d_ff, G;
  int32_t dt;  // wide_dtype_t value as passed (validated before use)
  void* Y;
  void* H_out;
  void* ws;
  size_t ws_bytes;
  uint32_t flags;
  hipStream_t stream;
  const void* prep = nullptr;  // operand-order weights for the decode MFMA kernels, or NULL
};

// Operand-order weight copy (wide_decode_prepare_weights): Wgate, Wup, Wdown
// regions of d * d_ff bf16 each, 256-byte aligned.
size_t prep_region(int64_t d, int64_t d_ff) { return round_up((size_t)(d * d_ff) * 2, 256); }

// Host-side checks of the arguments (all but the workspace) shared by
// wide_ffn_forward, wide_ffn_stage, wide_ffn_decode_prepared and
// wide_ffn_forward_noalloc. Sets *decode to the path the call takes.
wide_status_t validate_args(const Args& a, bool* decode) {
  if (!a.Wg || !a.Wu || !a.Wd) return fail(WIDE_ERR_NULL, "Wgate, Wup and Wdown must be non-NULL");
  // X, mask and Y have T rows: with T == 0 they may be NULL (nothing is read or written).
  if (a.T != 0 && (!a.X || !a.mask || !a.Y))
    return fail(WIDE_ERR_NULL, "X, mask and Y must be non-NULL when T > 0");
  if (a.dt != WIDE_F32 && a.dt != WIDE_BF16) return fail(WIDE_ERR_DTYPE, "unknown dtype %d", a.dt);
  if (a.T < 0 || a.d <= 0 || a.d_ff <= 0 || a.G <= 0)
    return fail(WIDE_ERR_SHAPE, "need T >= 0 and d, d_ff, G >= 1 (T=%d d=%d d_ff=%d G=%d)", a.T, a.d,
                a.d_ff, a.G);
  if (a.d_ff % a.G != 0) return fail(WIDE_ERR_SHAPE, "d_ff=%d is not a multiple of G=%d", a.d_ff, a.G);
  if (a.d % 64 != 0 || a.d_ff % 64 != 0 || a.G % 16 != 0)
    return fail(WIDE_ERR_UNSUPPORTED, "kernels need d %% 64 == 0, d_ff %% 64 == 0, G %% 16 == 0 (d=%d d_ff=%d G=%d)",
                a.d, a.d_ff, a.G);
  if (a.d_ff > 65536) return fail(WIDE_ERR_UNSUPPORTED, "kernels need d_ff <= 65536 (d_ff=%d)", a.d_ff);
  // The bf16 kernels address each operand with 32-bit byte offsets into a
  // buffer of at most 2^31 - 1 bytes.
  if ((int64_t)a.T * a.d_ff >= (1ll << 30) || (int64_t)a.T * a.d >= (1ll << 30) ||
      (int64_t)a.d * a.d_ff >= (1ll << 30))
    return fail(WIDE_ERR_UNSUPPORTED, "T*d_ff, T*d and d*d_ff must stay below 2^30");
  if (!aligned16(a.X) || !aligned16(a.Wg) || !aligned16(a.Wu) || !aligned16(a.Wd) ||
      !aligned16(a.Y) || (a.H_out && !aligned16(a.H_out)))
    return fail(WIDE_ERR_ALIGN, "X, W*, Y and H_out must be 16-byte aligned");
  if ((a.flags & WIDE_FLAG_FORCE_PREFILL) && (a.flags & WIDE_FLAG_FORCE_DECODE))
    return fail(WIDE_ERR_SHAPE, "FORCE_PREFILL and FORCE_DECODE are exclusive");
  if (a.flags & ~(WIDE_FLAG_FORCE_PREFILL | WIDE_FLAG_FORCE_DECODE))
    return fail(WIDE_ERR_SHAPE, "unknown flag bits 0x%x", a.flags);
  bool dec = a.dt == WIDE_BF16 && a.T <= decode_max_t_value();
  if (a.flags & WIDE_FLAG_FORCE_PREFILL) dec = false;
  if (a.flags & WIDE_FLAG_FORCE_DECODE) {
    if (a.dt != WIDE_BF16 || a.T > WIDE_DECODE_T_LIMIT)
      return fail(WIDE_ERR_UNSUPPORTED, "the decode path needs bf16 and T <= %d", WIDE_DECODE_T_LIMIT);
    dec = true;
  }
  *decode = dec;
  return WIDE_OK;
}

// The workspace argument against the layout of a validated call.
wide_status_t check_workspace(const Args& a) {
  const Layout L = layout(a.T, a.d, a.d_ff, a.G, a.dt, a.H_out == nullptr);
  if (!a.ws) return fail(WIDE_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", L.total);
  if ((reinterpret_cast<uintptr_t>(a.ws) & 255u) != 0)
    return fail(WIDE_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (a.ws_bytes < L.total)
    return fail(WIDE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", a.ws_bytes, L.total);
  return WIDE_OK;
}

wide_status_t validate(const Args& a, bool* decode) {
  const wide_status_t st = validate_args(a, decode);
  return st != WIDE_OK ? st : check_workspace(a);
}

// Per-group row lists (and the packed mask bits) from the mask [T, ng]. Up to
// kOneLaunchRows rows one kernel reads each group's mask column and places
// its rows; beyond that the column reads (a cache line per row) cost more
// than packing the bits from coalesced row reads first and partitioning each
// group's contiguous bit row in a second kernel. Measured on the masked
// N-axis GEMM (50% masks, graph replay): 2048^3 37.9 -> 34.5 us (N axis) and
// 36.9 -> 33.9 us (M axis), 3072^3 M axis 58 -> 53 us, 4096^3 unchanged.
constexpr int kOneLaunchRows = 4096;
hipError_t reorder_rows(const uint8_t* mask, int T, int ng, int tile, int32_t* perm,
                        int32_t* counts, int32_t* padded, uint32_t* maskbits, hipStream_t s) {
  if (T <= kOneLaunchRows)
    return wide::launch_reorder(mask, T, ng, tile, perm, counts, padded, maskbits, s);
  hipError_t e = wide::launch_pack_mask_bits(mask, T, ng, maskbits, s);
  if (e != hipSuccess) return e;
  return wide::launch_reorder_from_bits(maskbits, T, ng, tile, perm, counts, padded, s);
}

wide_status_t run_stage(int32_t stage, const Args& a) {
  const Layout L = layout(a.T, a.d, a.d_ff, a.G, a.dt, a.H_out == nullptr);
  char* ws = static_cast<char*>(a.ws);
  int32_t* perm = reinterpret_cast<int32_t*>(ws + L.perm);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* padded = reinterpret_cast<int32_t*>(ws + L.padded);
  uint32_t* maskbits = reinterpret_cast<uint32_t*>(ws + L.maskbits);
  float* part = reinterpret_cast<float*>(ws + L.part);
  void* H = a.H_out ? a.H_out : static_cast<void*>(ws + L.h);
  const bool zero_h = a.H_out != nullptr;
  const int ng = a.d_ff / a.G;
  hipError_t e = hipSuccess;
  switch (stage) {
    case WIDE_STAGE_REORDER:
      // the dense-masked gate/up (narrow groups, bf16) and the down read
      // only the bits
      if (a.dt == WIDE_BF16 && wide::gate_up_dense(a.G, a.d_ff)) {
        e = wide::launch_pack_mask_bits(a.mask, a.T, ng, maskbits, a.stream);
        return hip_status(e, "mask pack launch");
      }
      e = reorder_rows(a.mask, a.T, ng, WIDE_TOKEN_TILE, perm, counts, padded, maskbits, a.stream);
      return hip_status(e, "mask reorder launch");
    case WIDE_STAGE_GATE_UP:
      if (a.dt == WIDE_BF16)
        // zeros at skipped pairs only when H is returned: the down kernel
        // never reads H at an inactive (token, group)
        e = wide::launch_gate_up_bf16((const uint16_t*)a.X, (const uint16_t*)a.Wg,
                                      (const uint16_t*)a.Wu, perm, counts, maskbits, a.T, a.d,
                                      a.d_ff, a.G, (uint16_t*)H, zero_h, a.stream);
      else
        e = wide::launch_gate_up_f32((const float*)a.X, (const float*)a.Wg, (const float*)a.Wu,
                                     perm, counts, a.T, a.d, a.d_ff, a.G, (float*)H, zero_h,
                                     a.stream);
      return hip_status(e, "gate/up launch");
    case WIDE_STAGE_DOWN:
      if (a.dt == WIDE_BF16)
        e = wide::launch_down_bf16((const uint16_t*)H, (const uint16_t*)a.Wd, maskbits, a.T, a.d,
                                   a.d_ff, a.G, (uint16_t*)a.Y,
                                   reinterpret_cast<float*>(ws + L.dpart), a.stream);
      else
        e = wide::launch_down_f32((const float*)H, (const float*)a.Wd, maskbits, a.T, a.d, a.d_ff,
                                  a.G, (float*)a.Y, a.stream);
      return hip_status(e, "down launch");
    case WIDE_STAGE_DECODE_GATE_UP: {
      const char* pp = static_cast<const char*>(a.prep);
      const size_t R = prep_region(a.d, a.d_ff);
      e = wide::launch_decode_gate_up_bf16(
          (const uint16_t*)a.X, (const uint16_t*)a.Wg, (const uint16_t*)a.Wu,
          pp ? (const uint16_t*)pp : nullptr, pp ? (const uint16_t*)(pp + R) : nullptr, a.mask,
          a.T, a.d, a.d_ff, a.G, (uint16_t*)H, zero_h, a.stream);
      return hip_status(e, "decode gate/up launch");
    }
    case WIDE_STAGE_DECODE_DOWN: {
      const char* pp = static_cast<const char*>(a.prep);
      const size_t R = prep_region(a.d, a.d_ff);
      e = wide::launch_decode_down_bf16((const uint16_t*)H, (const uint16_t*)a.Wd,
                                        pp ? (const uint16_t*)(pp + 2 * R) : nullptr, a.mask, a.T,
                                        a.d, a.d_ff, a.G, (uint16_t*)a.Y, part, a.stream);
      return hip_status(e, "decode down launch");
    }
  }
  return fail(WIDE_ERR_SHAPE, "unknown stage %d", (int)stage);
}

}  // namespace

WIDE_API wide_status_t wide_reorder_masks(const uint8_t* mask, int32_t T, int32_t ngroups,
                                          int32_t tile, int32_t* perm, int32_t* counts,
                                          int32_t* padded, void* stream) {
  if (!counts || !padded) return fail(WIDE_ERR_NULL, "counts and padded must be non-NULL");
  if (T != 0 && (!mask || !perm))
    return fail(WIDE_ERR_NULL, "mask and perm must be non-NULL when T > 0");
  if (T < 0 || ngroups < 1 || tile < 1)
    return fail(WIDE_ERR_SHAPE, "need T >= 0, ngroups >= 1, tile >= 1 (T=%d ngroups=%d tile=%d)", T,
                ngroups, tile);
  if ((int64_t)T * ngroups > INT32_MAX)
    return fail(WIDE_ERR_SHAPE, "T*ngroups must stay below 2^31");
  const hipError_t e = wide::launch_reorder(mask, T, ngroups, tile, perm, counts, padded, nullptr,
                                            static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_status(e, "mask reorder launch");
  return ok();
}

namespace {
size_t ffn_workspace_size(int32_t T, int32_t d, int32_t d_ff, int32_t G, int32_t dt, bool with_h) {
  if (T < 0 || d <= 0 || d_ff <= 0 || G <= 0 || d_ff % G != 0) return 0;
  if (dt != WIDE_F32 && dt != WIDE_BF16) return 0;
  return layout(T, d, d_ff, G, dt, with_h).total;
}
}  // namespace

WIDE_API size_t wide_ffn_workspace_size_for(int32_t T, int32_t d, int32_t d_ff, int32_t G,
                                            wide_dtype_t dtype, int32_t h_out_given) {
  return ffn_workspace_size(T, d, d_ff, G, raw(dtype), h_out_given == 0);
}

WIDE_API size_t wide_ffn_workspace_size(int32_t T, int32_t d, int32_t d_ff, int32_t G,
                                        wide_dtype_t dtype) {
  return ffn_workspace_size(T, d, d_ff, G, raw(dtype), true);
}

WIDE_API wide_status_t wide_ffn_forward(const void* X, const void* Wgate, const void* Wup,
                                        const void* Wdown, const uint8_t* mask, int32_t T,
                                        int32_t d, int32_t d_ff, int32_t G, wide_dtype_t dtype,
                                        void* Y, void* H_out, void* workspace,
                                        size_t workspace_bytes, uint32_t flags, void* stream) {
  const Args a{X, Wgate, Wup, Wdown, mask, T, d, d_ff, G, raw(dtype), Y, H_out, workspace,
               workspace_bytes, flags, static_cast<hipStream_t>(stream)};
  bool dec = false;
  wide_status_t st = validate(a, &dec);
  if (st != WIDE_OK) return st;
  if (T == 0) return ok();
  const int32_t prefill[] = {WIDE_STAGE_REORDER, WIDE_STAGE_GATE_UP, WIDE_STAGE_DOWN};
  const int32_t decode[] = {WIDE_STAGE_DECODE_GATE_UP, WIDE_STAGE_DECODE_DOWN};
  const int32_t* stages = dec ? decode : prefill;
  const int n = dec ? 2 : 3;
  for (int i = 0; i < n; ++i) {
    st = run_stage(stages[i], a);
    if (st != WIDE_OK) return st;
  }
  return ok();
}

WIDE_API wide_status_t wide_ffn_stage(wide_stage_t stage, const void* X, const void* Wgate,
                                      const void* Wup, const void* Wdown, const uint8_t* mask,
                                      int32_t T, int32_t d, int32_t d_ff, int32_t G,
                                      wide_dtype_t dtype, void* Y, void* H_out, void* workspace,
                                      size_t workspace_bytes, uint32_t flags, void* stream) {
  const Args a{X, Wgate, Wup, Wdown, mask, T, d, d_ff, G, raw(dtype), Y, H_out, workspace,
               workspace_bytes, flags, static_cast<hipStream_t>(stream)};
  const int32_t sg = raw(stage);
  bool dec = false;
  wide_status_t st = validate(a, &dec);
  if (st != WIDE_OK) return st;
  const bool is_dec_stage = sg == WIDE_STAGE_DECODE_GATE_UP || sg == WIDE_STAGE_DECODE_DOWN;
  if (sg < WIDE_STAGE_REORDER || sg > WIDE_STAGE_DECODE_DOWN)
    return fail(WIDE_ERR_SHAPE, "unknown stage %d", sg);
  if (is_dec_stage != dec)
    return fail(WIDE_ERR_UNSUPPORTED, "stage %d is not on the %s path these arguments take", sg,
                dec ? "decode" : "prefill");
  if (T == 0) return ok();
  st = run_stage(sg, a);
  if (st != WIDE_OK) return st;
  return ok();
}

WIDE_API size_t wide_decode_weights_size(int32_t d, int32_t d_ff) {
  if (d <= 0 || d_ff <= 0 || d % 64 != 0 || d_ff % 64 != 0 || (int64_t)d * d_ff >= (1ll << 30))
    return 0;
  return 3 * prep_region(d, d_ff);
}

WIDE_API wide_status_t wide_decode_prepare_weights(const void* Wgate, const void* Wup,
                                                   const void* Wdown, int32_t d, int32_t d_ff,
                                                   void* prepared, size_t prepared_bytes,
                                                   void* stream) {
  if (!Wgate || !Wup || !Wdown || !prepared)
    return fail(WIDE_ERR_NULL, "Wgate, Wup, Wdown and prepared must be non-NULL");
  const size_t need = wide_decode_weights_size(d, d_ff);
  if (need == 0)
    return fail(WIDE_ERR_SHAPE, "need d, d_ff >= 64, multiples of 64, d*d_ff < 2^30 (d=%d d_ff=%d)",
                d, d_ff);
  if (!aligned16(Wgate) || !aligned16(Wup) || !aligned16(Wdown))
    return fail(WIDE_ERR_ALIGN, "Wgate, Wup and Wdown must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(prepared) & 255u) != 0)
    return fail(WIDE_ERR_ALIGN, "prepared must be 256-byte aligned");
  if (prepared_bytes < need)
    return fail(WIDE_ERR_WORKSPACE, "prepared has %zu bytes, needs %zu", prepared_bytes, need);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* out = static_cast<char*>(prepared);
  const size_t R = prep_region(d, d_ff);
  hipError_t e = wide::launch_decode_pack_bf16((const uint16_t*)Wgate, d_ff, d, (uint16_t*)out, s);
  if (e == hipSuccess)
    e = wide::launch_decode_pack_bf16((const uint16_t*)Wup, d_ff, d, (uint16_t*)(out + R), s);
  if (e == hipSuccess)
    e = wide::launch_decode_pack_bf16((const uint16_t*)Wdown, d, d_ff, (uint16_t*)(out + 2 * R), s);
  if (e != hipSuccess) return hip_status(e, "weight packing launch");
  return ok();
}

WIDE_API wide_status_t wide_ffn_decode_prepared(const void* X, const void* Wgate, const void* Wup,
                                                const void* Wdown, const void* prepared,
                                                size_t prepared_bytes, const uint8_t* mask,
                                                int32_t T, int32_t d,
                                                int32_t d_ff, int32_t G, void* Y, void* H_out,
                                                void* workspace, size_t workspace_bytes,
                                                void* stream) {
  Args a{X, Wgate, Wup, Wdown, mask, T, d, d_ff, G, WIDE_BF16, Y, H_out, workspace,
         workspace_bytes, WIDE_FLAG_FORCE_DECODE, static_cast<hipStream_t>(stream)};
  bool dec = false;
  wide_status_t st = validate(a, &dec);
  if (st != WIDE_OK) return st;
  if (!prepared) return fail(WIDE_ERR_NULL, "prepared must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(prepared) & 255u) != 0)
    return fail(WIDE_ERR_ALIGN, "prepared must be 256-byte aligned");
  const size_t need = wide_decode_weights_size(d, d_ff);
  if (prepared_bytes < need)
    return fail(WIDE_ERR_WORKSPACE, "prepared has %zu bytes, needs %zu", prepared_bytes, need);
  a.prep = prepared;
  if (T == 0) return ok();
  st = run_stage(WIDE_STAGE_DECODE_GATE_UP, a);
  if (st != WIDE_OK) return st;
  st = run_stage(WIDE_STAGE_DECODE_DOWN, a);
  if (st != WIDE_OK) return st;
  return ok();
}

// ---------------------------------------------------------------- no-allocation entry point

WIDE_API wide_status_t wide_ffn_forward_noalloc(const void* X, const void* Wgate, const void* Wup,
                                                const void* Wdown, const uint8_t* mask, int32_t T,
                                                int32_t d, int32_t d_ff, int32_t G,
                                                wide_dtype_t dtype, void* Y, void* H_out,
                                                uint32_t flags, void* stream) {
  Args a{X, Wgate, Wup, Wdown, mask, T, d, d_ff, G, raw(dtype), Y, H_out, nullptr,
         (size_t)WIDE_NOALLOC_SCRATCH_BYTES, flags, static_cast<hipStream_t>(stream)};
  bool dec = false;
  wide_status_t st = validate_args(a, &dec);
  if (st != WIDE_OK) return st;
  if (T != 0 && H_out == nullptr)
    return fail(WIDE_ERR_NULL, "H_out is required: the scratch array holds no H");
  const size_t need = layout(T, d, d_ff, G, a.dt, false).total;
  if (need > (size_t)WIDE_NOALLOC_SCRATCH_BYTES)
    return fail(WIDE_ERR_WORKSPACE,
                "this call needs %zu bytes of scratch; the no-allocation entry point holds %zu "
                "(WIDE_NOALLOC_SCRATCH_BYTES)", need, (size_t)WIDE_NOALLOC_SCRATCH_BYTES);
  if (T == 0) return ok();
  const hipError_t e = wide::noalloc_scratch(a.stream, &a.ws);
  if (e != hipSuccess) return hip_status(e, "scratch array of the stream's device");
  st = check_workspace(a);
  if (st != WIDE_OK) return st;
  const int32_t prefill[] = {WIDE_STAGE_REORDER, WIDE_STAGE_GATE_UP, WIDE_STAGE_DOWN};
  const int32_t decode[] = {WIDE_STAGE_DECODE_GATE_UP, WIDE_STAGE_DECODE_DOWN};
  const int32_t* stages = dec ? decode : prefill;
  for (int i = 0; i < (dec ? 2 : 3); ++i) {
    st = run_stage(stages[i], a);
    if (st != WIDE_OK) return st;
  }
  return ok();
}

// ---------------------------------------------------------------- masked GEMMs

namespace {

// Workspace of the masked GEMMs (each region 256-byte aligned):
//   perm     int32  [ngroups, M]   (N axis)
//   counts   int32  [ngroups]      (N axis)
//   padded   int32  [ngroups]      (N axis)
//   maskbits uint32 [ngroups, ceil(M/32)]   (K axis)
struct GemmLayout {
  size_t perm, counts, padded, maskbits, total;
};

GemmLayout gemm_layout(int64_t M, int64_t ng) {
  GemmLayout L{};
  size_t off = 0;
  L.perm = off;
  off = round_up(off + (size_t)(ng * M) * 4, 256);
  L.counts = off;
  off = round_up(off + (size_t)ng * 4, 256);
  L.padded = off;
  off = round_up(off + (size_t)ng * 4, 256);
  L.maskbits = off;
  off = round_up(off + (size_t)(ng * ((M + 31) / 32)) * 4, 256);
  L.total = off;
  return L;
}

// routed = N (N axis) or K (K axis).
wide_status_t validate_gemm(const void* A, const void* B, const uint8_t* mask, int32_t M, int32_t N,
                            int32_t K, int32_t G, int32_t routed, int32_t dt, const void* C,
                            const void* ws, size_t ws_bytes) {
  if (!B) return fail(WIDE_ERR_NULL, "B must be non-NULL");
  if (M != 0 && (!A || !mask || !C))
    return fail(WIDE_ERR_NULL, "A, mask and C must be non-NULL when M > 0");
  if (dt != WIDE_F32 && dt != WIDE_BF16) return fail(WIDE_ERR_DTYPE, "unknown dtype %d", dt);
  if (M < 0 || N <= 0 || K <= 0 || G <= 0)
    return fail(WIDE_ERR_SHAPE, "need M >= 0 and N, K, G >= 1 (M=%d N=%d K=%d G=%d)", M, N, K, G);
  if (routed % G != 0)
    return fail(WIDE_ERR_SHAPE, "the routed axis (%d) is not a multiple of G=%d", routed, G);
  if (dt != WIDE_BF16) return fail(WIDE_ERR_UNSUPPORTED, "the masked GEMMs run bf16 only");
  if (K % 64 != 0 || G % 16 != 0 || N % 8 != 0)
    return fail(WIDE_ERR_UNSUPPORTED, "kernels need K %% 64 == 0, G %% 16 == 0, N %% 8 == 0 (N=%d K=%d G=%d)",
                N, K, G);
  if (K > 65536) return fail(WIDE_ERR_UNSUPPORTED, "kernels need K <= 65536 (K=%d)", K);
  if ((int64_t)M * K >= (1ll << 30) || (int64_t)N * K >= (1ll << 30) || (int64_t)M * N >= (1ll << 30))
    return fail(WIDE_ERR_UNSUPPORTED, "M*K, N*K and M*N must stay below 2^30");
  if (!aligned16(A) || !aligned16(B) || !aligned16(C))
    return fail(WIDE_ERR_ALIGN, "A, B and C must be 16-byte aligned");
  const GemmLayout L = gemm_layout(M, routed / G);
  if (!ws) return fail(WIDE_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", L.total);
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(WIDE_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (ws_bytes < L.total)
    return fail(WIDE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, L.total);
  return WIDE_OK;
}

}  // namespace

WIDE_API size_t wide_gemm_workspace_size(int32_t M, int32_t ngroups) {
  if (M < 0 || ngroups < 1) return 0;
  return gemm_layout(M, ngroups).total;
}

WIDE_API wide_status_t wide_gemm_mn(const void* A, const void* B, const uint8_t* mask, int32_t M,
                                    int32_t N, int32_t K, int32_t G, wide_dtype_t dtype, void* C,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  wide_status_t st =
      validate_gemm(A, B, mask, M, N, K, G, N, raw(dtype), C, workspace, workspace_bytes);
  if (st != WIDE_OK) return st;
  if (M == 0) return ok();
  const int ng = N / G;
  const GemmLayout L = gemm_layout(M, ng);
  char* ws = static_cast<char*>(workspace);
  int32_t* perm = reinterpret_cast<int32_t*>(ws + L.perm);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* padded = reinterpret_cast<int32_t*>(ws + L.padded);
  uint32_t* maskbits = reinterpret_cast<uint32_t*>(ws + L.maskbits);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = reorder_rows(mask, M, ng, WIDE_TOKEN_TILE, perm, counts, padded, maskbits, s);
  if (e != hipSuccess) return hip_status(e, "mask reorder launch");
  e = wide::launch_gemm_mn_bf16((const uint16_t*)A, (const uint16_t*)B, perm, counts, M, K, N, G,
                                (uint16_t*)C, s);
  if (e != hipSuccess) return hip_status(e, "GEMM-MN launch");
  return ok();
}

WIDE_API wide_status_t wide_gemm_k(const void* A, const void* B, const uint8_t* mask, int32_t M,
                                   int32_t N, int32_t K, int32_t G, wide_dtype_t dtype, void* C,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  wide_status_t st =
      validate_gemm(A, B, mask, M, N, K, G, K, raw(dtype), C, workspace, workspace_bytes);
  if (st != WIDE_OK) return st;
  if (M == 0) return ok();
  const int ng = K / G;
  const GemmLayout L = gemm_layout(M, ng);
  uint32_t* maskbits = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + L.maskbits);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = wide::launch_pack_mask_bits(mask, M, ng, maskbits, s);
  if (e != hipSuccess) return hip_status(e, "mask pack launch");
  // (no partial-sum space in this workspace: no split last round)
  e = wide::launch_down_bf16((const uint16_t*)A, (const uint16_t*)B, maskbits, M, N, K, G,
                             (uint16_t*)C, nullptr, s);
  if (e != hipSuccess) return hip_status(e, "GEMM-K launch");
  return ok();
}

namespace {

// Workspace of the attention: the reorder of the [T, Hk] mask (the masked
// GEMMs' layout) followed by the transposed V copy [Hk, dh, Tpad] bf16.
constexpr int kAttnTile = 128;

struct AttnLayout {
  GemmLayout g;
  size_t vt, total;
};

AttnLayout attn_layout(int64_t T, int64_t Hk, int64_t dh) {
  AttnLayout L{};
  L.g = gemm_layout(T, Hk);
  L.vt = L.g.total;
  L.total = round_up(L.vt + (size_t)(Hk * dh) * (size_t)wide::attention_tpad(T) * 2, 256);
  return L;
}

}  // namespace

WIDE_API size_t wide_attention_workspace_size(int32_t T, int32_t Hk, int32_t dh) {
  if (T < 0 || Hk < 1 || dh < 1) return 0;
  return attn_layout(T, Hk, dh).total;
}

WIDE_API wide_status_t wide_attention_prefill(const void* Q, const void* K, const void* V,
                                              const uint8_t* mask, int32_t T, int32_t Hq,
                                              int32_t Hk, int32_t dh, wide_dtype_t dtype, void* O,
                                              uint32_t flags, void* workspace,
                                              size_t workspace_bytes, void* stream) {
  const int32_t dt = raw(dtype);
  if (T != 0 && (!Q || !K || !V || !mask || !O))
    return fail(WIDE_ERR_NULL, "Q, K, V, mask and O must be non-NULL when T > 0");
  if (dt != WIDE_F32 && dt != WIDE_BF16) return fail(WIDE_ERR_DTYPE, "unknown dtype %d", dt);
  if (T < 0 || Hq < 1 || Hk < 1 || dh < 1 || Hq % Hk != 0)
    return fail(WIDE_ERR_SHAPE, "need T >= 0, Hq, Hk, dh >= 1 and Hk dividing Hq (T=%d Hq=%d Hk=%d dh=%d)",
                T, Hq, Hk, dh);
  if ((flags & ~WIDE_ATTN_ZERO_INACTIVE) != 0) return fail(WIDE_ERR_SHAPE, "unknown flags 0x%x", flags);
  if (dt != WIDE_BF16) return fail(WIDE_ERR_UNSUPPORTED, "the attention kernel runs bf16 only");
  if (dh != 128) return fail(WIDE_ERR_UNSUPPORTED, "the attention kernel needs dh == 128 (dh=%d)", dh);
  if ((int64_t)T * Hq * dh >= (1ll << 31))
    return fail(WIDE_ERR_UNSUPPORTED, "T*Hq*dh must stay below 2^31");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O))
    return fail(WIDE_ERR_ALIGN, "Q, K, V and O must be 16-byte aligned");
  const AttnLayout L = attn_layout(T, Hk, dh);
  if (!workspace) return fail(WIDE_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", L.total);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(WIDE_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(WIDE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);
  if (T == 0) return ok();
  char* ws = static_cast<char*>(workspace);
  int32_t* perm = reinterpret_cast<int32_t*>(ws + L.g.perm);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.g.counts);
  int32_t* padded = reinterpret_cast<int32_t*>(ws + L.g.padded);
  uint32_t* maskbits = reinterpret_cast<uint32_t*>(ws + L.g.maskbits);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = reorder_rows(mask, T, Hk, kAttnTile, perm, counts, padded, maskbits, s);
  if (e != hipSuccess) return hip_status(e, "mask reorder launch");
  e = wide::launch_attention_prefill_bf16(
      (const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)V, perm, counts, T, Hq, Hk, dh,
      (uint16_t*)O, (flags & WIDE_ATTN_ZERO_INACTIVE) != 0,
      reinterpret_cast<uint16_t*>(ws + L.vt), s);
  if (e != hipSuccess) return hip_status(e, "attention launch");
  return ok();
}

WIDE_API size_t wide_attention_decode_workspace_size(int32_t T, int32_t Hq, int32_t dh) {
  if (T < 1 || Hq < 1 || dh != 128) return 0;
  return round_up(wide::attention_decode_part_floats(T, Hq) * 4, 256);
}

WIDE_API wide_status_t wide_attention_decode(const void* q, const void* K, const void* V,
                                             const uint8_t* mask, int32_t T, int32_t Hq,
                                             int32_t Hk, int32_t dh, wide_dtype_t dtype, void* O,
                                             uint32_t flags, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  const int32_t dt = raw(dtype);
  if (!q || !K || !V || !mask || !O) return fail(WIDE_ERR_NULL, "q, K, V, mask and O must be non-NULL");
  if (dt != WIDE_F32 && dt != WIDE_BF16) return fail(WIDE_ERR_DTYPE, "unknown dtype %d", dt);
  if (T < 1 || Hq < 1 || Hk < 1 || dh < 1 || Hq % Hk != 0)
    return fail(WIDE_ERR_SHAPE, "need T >= 1, Hq, Hk, dh >= 1 and Hk dividing Hq (T=%d Hq=%d Hk=%d dh=%d)",
                T, Hq, Hk, dh);
  if ((flags & ~WIDE_ATTN_ZERO_INACTIVE) != 0) return fail(WIDE_ERR_SHAPE, "unknown flags 0x%x", flags);
  if (dt != WIDE_BF16) return fail(WIDE_ERR_UNSUPPORTED, "the attention kernel runs bf16 only");
  const int hpg = Hq / Hk;
  if (dh != 128 || (hpg != 1 && hpg != 2 && hpg != 4 && hpg != 8))
    return fail(WIDE_ERR_UNSUPPORTED, "the decode kernel needs dh == 128 and Hq/Hk in {1, 2, 4, 8} (dh=%d Hq/Hk=%d)",
                dh, hpg);
  if ((int64_t)T * Hk * dh >= (1ll << 31)) return fail(WIDE_ERR_UNSUPPORTED, "T*Hk*dh must stay below 2^31");
  if (!aligned16(q) || !aligned16(K) || !aligned16(V) || !aligned16(O))
    return fail(WIDE_ERR_ALIGN, "q, K, V and O must be 16-byte aligned");
  const size_t need = wide_attention_decode_workspace_size(T, Hq, dh);
  if (!workspace) return fail(WIDE_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(WIDE_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(WIDE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  const hipError_t e = wide::launch_attention_decode_bf16(
      (const uint16_t*)q, (const uint16_t*)K, (const uint16_t*)V, mask, T, Hq, Hk, dh, (uint16_t*)O,
      (flags & WIDE_ATTN_ZERO_INACTIVE) != 0, static_cast<float*>(workspace),
      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_status(e, "attention decode launch");
  return ok();
}

namespace {

// Host checks shared by the router entry points (everything but the outputs).
wide_status_t validate_router(const void* X, const void* W1, const void* W2, int32_t T, int32_t D,
                              int32_t r, int32_t ngroups, int32_t ac, int32_t dt) {
  if (!W1 || !W2) return fail(WIDE_ERR_NULL, "W1 and W2 must be non-NULL");
  if (T != 0 && !X) return fail(WIDE_ERR_NULL, "X must be non-NULL when T > 0");
  if (dt != WIDE_F32 && dt != WIDE_BF16) return fail(WIDE_ERR_DTYPE, "unknown dtype %d", dt);
  if (T < 0 || D <= 0 || r <= 0 || ngroups <= 0)
    return fail(WIDE_ERR_SHAPE, "need T >= 0 and D, r, ngroups >= 1 (T=%d D=%d r=%d ngroups=%d)", T, D,
                r, ngroups);
  if (ac != WIDE_ACT_IDENTITY && ac != WIDE_ACT_RELU && ac != WIDE_ACT_SILU)
    return fail(WIDE_ERR_SHAPE, "unknown activation %d", ac);
  if (dt != WIDE_BF16) return fail(WIDE_ERR_UNSUPPORTED, "the router kernel runs bf16 only");
  if (D % 32 != 0 || (r != 16 && r != 32 && r != 64))
    return fail(WIDE_ERR_UNSUPPORTED, "the router kernel needs D %% 32 == 0 and r in {16, 32, 64} (D=%d r=%d)",
                D, r);
  if ((int64_t)T * D >= (1ll << 31) || (int64_t)T * ngroups >= (1ll << 31))
    return fail(WIDE_ERR_UNSUPPORTED, "T*D and T*ngroups must stay below 2^31");
  if (!aligned16(X) || !aligned16(W1) || !aligned16(W2))
    return fail(WIDE_ERR_ALIGN, "X, W1 and W2 must be 16-byte aligned");
  return WIDE_OK;
}

size_t router_bits_bytes(int64_t T, int64_t ngroups) {
  return round_up((size_t)(ngroups * ((T + 31) / 32)) * 4, 256);
}

}  // namespace

WIDE_API size_t wide_router_workspace_size(int32_t T, int32_t r) {
  if (T < 0 || (r != 16 && r != 32 && r != 64)) return 0;
  return wide::router_zpart_bytes(T, r);
}

WIDE_API wide_status_t wide_router_forward(const void* X, const void* W1, const void* W2,
                                           int32_t T, int32_t D, int32_t r, int32_t ngroups,
                                           wide_act_t act, wide_dtype_t dtype, uint8_t* mask,
                                           float* logits, void* workspace, size_t workspace_bytes,
                                           void* stream) {
  const int32_t ac = raw(act);
  wide_status_t st = validate_router(X, W1, W2, T, D, r, ngroups, ac, raw(dtype));
  if (st != WIDE_OK) return st;
  if (T != 0 && !mask) return fail(WIDE_ERR_NULL, "mask must be non-NULL when T > 0");
  if ((reinterpret_cast<uintptr_t>(logits) & 7u) != 0)
    return fail(WIDE_ERR_ALIGN, "logits must be 8-byte aligned");
  const size_t need = wide::router_zpart_bytes(T, r);
  if (need > 0) {
    if (!workspace) return fail(WIDE_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(WIDE_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
      return fail(WIDE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  }
  if (T == 0) return ok();
  const hipError_t e = wide::launch_router_bf16(
      (const uint16_t*)X, (const uint16_t*)W1, (const uint16_t*)W2, T, D, r, ngroups, ac, mask,
      logits, nullptr, need > 0 ? static_cast<float*>(workspace) : nullptr,
      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_status(e, "router launch");
  return ok();
}

// [bits][partial sums of the first map for T <= 16, sized for r = 64]
WIDE_API size_t wide_router_reorder_workspace_size(int32_t T, int32_t ngroups) {
  if (T < 0 || ngroups < 1) return 0;
  return router_bits_bytes(T, ngroups) + wide::router_zpart_bytes(T, 64);
}

WIDE_API wide_status_t wide_router_reorder(const void* X, const void* W1, const void* W2,
                                           int32_t T, int32_t D, int32_t r, int32_t ngroups,
                                           wide_act_t act, wide_dtype_t dtype, int32_t tile,
                                           uint8_t* mask, float* logits, int32_t* perm,
                                           int32_t* counts, int32_t* padded, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  const int32_t ac = raw(act);
  wide_status_t st = validate_router(X, W1, W2, T, D, r, ngroups, ac, raw(dtype));
  if (st != WIDE_OK) return st;
  if (!counts || !padded) return fail(WIDE_ERR_NULL, "counts and padded must be non-NULL");
  if (T != 0 && !perm) return fail(WIDE_ERR_NULL, "perm must be non-NULL when T > 0");
  if (tile < 1) return fail(WIDE_ERR_SHAPE, "need tile >= 1 (tile=%d)", tile);
  if ((reinterpret_cast<uintptr_t>(logits) & 7u) != 0)
    return fail(WIDE_ERR_ALIGN, "logits must be 8-byte aligned");
  const size_t need = router_bits_bytes(T, ngroups) + wide::router_zpart_bytes(T, 64);
  if (!workspace) return fail(WIDE_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(WIDE_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(WIDE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* maskbits = static_cast<uint32_t*>(workspace);
  float* zpart = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                          router_bits_bytes(T, ngroups));
  hipError_t e = hipSuccess;
  if (T > 0) {
    e = wide::launch_router_bf16((const uint16_t*)X, (const uint16_t*)W1, (const uint16_t*)W2, T, D,
                                 r, ngroups, ac, mask, logits, maskbits, zpart, s);
    if (e != hipSuccess) return hip_status(e, "router launch");
  }
  // T == 0: the partition still writes counts = padded = 0
  e = wide::launch_reorder_from_bits(maskbits, T, ngroups, tile, perm, counts, padded, s);
  if (e != hipSuccess) return hip_status(e, "mask reorder launch");
  return ok();
}

WIDE_API const char* wide_status_string(wide_status_t status) {
  switch (raw(status)) {
    case WIDE_OK: return "ok";
    case WIDE_ERR_NULL: return "null pointer argument";
    case WIDE_ERR_SHAPE: return "invalid size or argument";
    case WIDE_ERR_DTYPE: return "unknown dtype";
    case WIDE_ERR_ALIGN: return "misaligned pointer";
    case WIDE_ERR_WORKSPACE: return "workspace missing or too small";
    case WIDE_ERR_UNSUPPORTED: return "unsupported by these kernels";
    case WIDE_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

WIDE_API const char* wide_last_error(void) { return g_last_error.c_str(); }

WIDE_API int32_t wide_decode_max_t(void) { return decode_max_t_value(); }
