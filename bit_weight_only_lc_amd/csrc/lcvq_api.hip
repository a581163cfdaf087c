// C ABI of the LC-VQ library: argument checks, workspace carving and kernel launch order.
// Declarations and the contract of every call are in include/lcvq.h.
#include "lcvq.h"
#include "lcvq_internal.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <vector>

using namespace lcvq;

namespace {

constexpr size_t kAlign = 256;
constexpr size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool d_ok(int d) { return d == 4 || d == 8 || d == 16; }
inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }
inline lcvq_status_t from_hip(hipError_t e) { return e == hipSuccess ? LCVQ_OK : LCVQ_ERR_HIP; }

// Launch limits. A HIP grid holds at most 2^32 - 1 work-items per dimension. The largest
// grids of a layer call are the products (one 512-thread workgroup per 256 x 256 tile,
// rounded up to a multiple of 8) and the row prologues (256-thread blocks, one per row
// or per few rows, after at most 65535 quantizer blocks); the transposed-code kernel
// has a (K / 256) x (N / 64) grid. These limits keep every one of them inside the range.
constexpr int64_t kMaxRows = (int64_t(1) << 24) - (int64_t(1) << 17);   // M
constexpr int64_t kMaxDim = int64_t(1) << 21;                           // N, K
constexpr int64_t kMaxTiles = (int64_t(1) << 23) - 8;                   // per product
constexpr int64_t kMaxBlocks256 = (int64_t(1) << 24) - 1;              // 256-thread grids
// Decode: one 1024- or 512-thread workgroup per 16 or 32 output rows, and the
// layout kernel's one 256-thread block per four 1 KiB tiles.
constexpr int64_t kMaxDecodeRows = int64_t(1) << 26;                    // N, sum over a batch
constexpr int64_t kMaxDecodeWeights = int64_t(1) << 36;                 // N * K

inline int64_t tiles(int64_t P, int64_t Q) { return ((P + 255) / 256) * ((Q + 255) / 256); }

// PTQ initialisation: K a multiple of 64 up to 16384 (the sweep keeps a workgroup's 16
// rows of codes in LDS); N a multiple of 16 up to 2^20.
constexpr int64_t kPtqMaxK = 16384;
inline bool ptq_shape_ok(int64_t N, int64_t K) {
  return N >= 16 && (N % 16) == 0 && N <= (int64_t(1) << 20) && K >= 64 && (K % 64) == 0 &&
         K <= kPtqMaxK;
}

// Linear-layer shapes: M rows of activations, weight [N, K].
inline bool layer_shape_ok(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || M > kMaxRows) return false;
  if (N < 64 || K < 64 || (N % 64) || (K % 64)) return false;
  if (N > kMaxDim || K > kMaxDim) return false;
  if (N * K >= (int64_t(1) << 40)) return false;
  if (tiles(M, N) > kMaxTiles || tiles(K, N) > kMaxTiles || tiles(K, M) > kMaxTiles)
    return false;
  return true;
}

// Decode products: K a multiple of 64 (the canonical packed layout); the decode layout of
// lcvq_gemv2b_shuffle is made of whole 256-column blocks, so it also needs K % 256 == 0.
inline bool decode_shape_ok(int64_t N, int64_t K) {
  return N >= 16 && (N % 16) == 0 && K >= 64 && (K % 64) == 0 && N <= kMaxDecodeRows &&
         K <= INT32_MAX && N * K <= kMaxDecodeWeights;
}
inline bool decode_layout_shape_ok(int64_t N, int64_t K) {
  return decode_shape_ok(N, K) && (K % 256) == 0;
}

// Blocked R16 code words for `rows` operand rows and a contraction of length `kc`.
inline size_t r16_bytes(int64_t rows, int64_t kc) {
  return (size_t)((rows + 255) / 256) * 256 * (size_t)(kc / 16) * 4;
}

struct FwdWs {
  size_t xs, beta, r16, xs_lo, split, total;
};
inline FwdWs fwd_ws(int64_t M, int64_t N, int64_t K, bool f32) {
  FwdWs w;
  w.xs = 0;
  w.beta = w.xs + up((size_t)M * K * 2);
  w.r16 = w.beta + up((size_t)M * 4);
  w.xs_lo = w.r16 + up(r16_bytes(N, K));
  w.split = w.xs_lo + (f32 ? up((size_t)M * K * 2) : 0);
  w.total = w.split + up(gemm_fwd_split_bytes(M, N, K));   // split partials of few-tile shapes
  return w;
}

struct BwdWs {
  size_t r, r16t, partials, dy_hi, dy_lo, x_hi, x_lo, split, total;
};
inline BwdWs bwd_ws(int64_t M, int64_t N, int64_t K, int d, bool f32) {
  BwdWs w;
  w.r = 0;
  w.r16t = w.r + up((size_t)M * 4);
  w.partials = w.r16t + up(r16_bytes(K, N));
  const size_t prows = (size_t)dw_partial_rows(M, N, K);
  w.dy_hi = w.partials + up(prows * (size_t)(d * d + d) * 4);
  const size_t dyb = f32 ? up((size_t)M * N * 2) : 0, xb = f32 ? up((size_t)M * K * 2) : 0;
  w.dy_lo = w.dy_hi + dyb;
  w.x_hi = w.dy_lo + dyb;
  w.x_lo = w.x_hi + xb;
  w.split = w.x_lo + xb;
  w.total = w.split + up(dw_split_bytes(M, N, K));   // dW's split partials
  return w;
}

struct GemvWs {
  size_t xq, rowinfo, total;
};
constexpr GemvWs gemv_ws(int64_t K) {
  const size_t nkb = (size_t)((K + 255) / 256);       // the last block may be partial
  GemvWs w{0, 0, 0};
  w.rowinfo = up(nkb * 4 * 2 * 1024);
  w.total = w.rowinfo + up(nkb * 16 * 8);
  return w;
}

// The decode product without a caller workspace (lcvq_gemv2b_noalloc): its X' limbs and
// block scales live in a file-scope device array of fixed size, enough for K up to
// kNoAllocMaxK. Every GPU the library runs on holds one copy until the process ends.
constexpr int64_t kNoAllocMaxK = 65536;
constexpr size_t kScratchBytes = gemv_ws(kNoAllocMaxK).total;   // 2,129,920 bytes

struct ProfSlot {
  int id = 0;
  hipEvent_t start = nullptr, stop = nullptr;
};
thread_local ProfSlot g_prof;

}  // namespace

// Device-side scratch of lcvq_gemv2b_noalloc. In host code `scratch` names a host-side
// stand-in, not device memory: kernels get the address that hipGetSymbolAddress returns
// for the current device (scratch_ptr below), never the symbol itself.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
// Address of this device's copy of `scratch`, looked up once per device with that
// device current and kept for later calls.
lcvq_status_t scratch_ptr(uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return LCVQ_ERR_HIP;
  static std::mutex mu;
  static std::vector<void*> ptrs;
  std::lock_guard<std::mutex> lock(mu);
  if ((size_t)dev >= ptrs.size()) ptrs.resize((size_t)dev + 1, nullptr);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LCVQ_ERR_HIP;
    ptrs[dev] = p;
  }
  *out = static_cast<uint8_t*>(ptrs[dev]);
  return LCVQ_OK;
}
}  // namespace

bool lcvq::take_profile(int id, hipEvent_t* start, hipEvent_t* stop) {
  if (g_prof.id != id || !g_prof.start || !g_prof.stop) return false;
  *start = g_prof.start;
  *stop = g_prof.stop;
  g_prof = ProfSlot();
  return true;
}

extern "C" {

lcvq_status_t lcvq_profile_next(int kernel_id, void* start_event, void* stop_event) {
  if (kernel_id < PROF_QUANTIZE || kernel_id > PROF_LAST) return LCVQ_ERR_SHAPE;
  g_prof.id = (start_event && stop_event) ? kernel_id : 0;
  g_prof.start = static_cast<hipEvent_t>(start_event);
  g_prof.stop = static_cast<hipEvent_t>(stop_event);
  return LCVQ_OK;
}

const char* lcvq_status_string(lcvq_status_t s) {
  switch (s) {
    case LCVQ_OK: return "ok";
    case LCVQ_ERR_NULL: return "a required pointer is NULL";
    case LCVQ_ERR_SHAPE: return "shape outside the supported limits";
    case LCVQ_ERR_D: return "d must be 4, 8 or 16";
    case LCVQ_ERR_DTYPE: return "unknown dtype";
    case LCVQ_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case LCVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case LCVQ_ERR_HIP: return "kernel launch failed";
    case LCVQ_ERR_VALUE: return "a scalar argument is out of range";
    case LCVQ_ERR_SCRATCH: return "shape larger than the no-allocation scratch serves";
  }
  return "unknown status";
}

lcvq_status_t lcvq_quantize(const float* Wp, int64_t N, int64_t K, uint8_t* z_u8,
                            uint8_t* packed, uint8_t* mask, void* stream) {
  if (!Wp) return LCVQ_ERR_NULL;
  if (N < 1 || K < 16 || (K % 16) || N * K >= (int64_t(1) << 40)) return LCVQ_ERR_SHAPE;
  if (!aligned16(Wp) || !aligned16(z_u8) || !aligned16(packed) || !aligned16(mask))
    return LCVQ_ERR_ALIGN;
  if (!z_u8 && !packed && !mask) return LCVQ_OK;
  return from_hip(launch_quantize(Wp, N, K, z_u8, packed, mask, nullptr, nullptr, nullptr,
                                  nullptr, 4, as_stream(stream)));
}

lcvq_status_t lcvq_pack2b(const uint8_t* z_u8, int64_t N, int64_t K, uint8_t* packed,
                          void* stream) {
  if (!z_u8 || !packed) return LCVQ_ERR_NULL;
  if (N < 1 || K < 16 || (K % 16) || N * K >= (int64_t(1) << 40)) return LCVQ_ERR_SHAPE;
  if (!aligned16(z_u8) || !aligned16(packed)) return LCVQ_ERR_ALIGN;
  return from_hip(launch_pack2b(z_u8, N, K, packed, as_stream(stream)));
}

lcvq_status_t lcvq_unpack2b(const uint8_t* packed, int64_t N, int64_t K, uint8_t* z_u8,
                            void* stream) {
  if (!z_u8 || !packed) return LCVQ_ERR_NULL;
  if (N < 1 || K < 16 || (K % 16) || N * K >= (int64_t(1) << 40)) return LCVQ_ERR_SHAPE;
  if (!aligned16(z_u8) || !aligned16(packed)) return LCVQ_ERR_ALIGN;
  return from_hip(launch_unpack2b(packed, N, K, z_u8, as_stream(stream)));
}

size_t lcvq_linear_fwd_workspace_size(int64_t M, int64_t N, int64_t K, int d) {
  (void)d;
  if (!layer_shape_ok(M, N, K)) return 0;
  return fwd_ws(M, N, K, true).total;   // sized for float32 activations (the larger case)
}

lcvq_status_t lcvq_linear_fwd(const void* X, lcvq_dtype_t xdt, int64_t M, int64_t N,
                              int64_t K, int d, const float* Wp, const float* A,
                              const float* B, void* Y, uint8_t* packed_out,
                              uint8_t* mask_out, float* What_out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!X || !Wp || !A || !B || !Y || !packed_out || !mask_out) return LCVQ_ERR_NULL;
  if (xdt != LCVQ_F32 && xdt != LCVQ_BF16) return LCVQ_ERR_DTYPE;
  if (!d_ok(d)) return LCVQ_ERR_D;
  if (!layer_shape_ok(M, N, K)) return LCVQ_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(Wp) || !aligned16(A) || !aligned16(B) || !aligned16(Y) ||
      !aligned16(packed_out) || !aligned16(mask_out) || !aligned16(What_out) ||
      !aligned16(workspace))
    return LCVQ_ERR_ALIGN;
  const bool f32 = xdt == LCVQ_F32;
  const FwdWs w = fwd_ws(M, N, K, f32);
  if (!workspace || workspace_bytes < w.total) return LCVQ_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint16_t* xs = reinterpret_cast<uint16_t*>(ws + w.xs);
  uint16_t* xs_lo = f32 ? reinterpret_cast<uint16_t*>(ws + w.xs_lo) : nullptr;
  float* beta = reinterpret_cast<float*>(ws + w.beta);
  uint32_t* r16 = reinterpret_cast<uint32_t*>(ws + w.r16);
  hipError_t e;
  if (M + 65536 <= kMaxBlocks256) {                // quantizer and prologue in one launch
    e = launch_fwd_prep(Wp, N, K, packed_out, mask_out, r16, What_out, X, f32, M, A, B, d, xs,
                        xs_lo, beta, s);
  } else {
    e = launch_quantize(Wp, N, K, nullptr, packed_out, mask_out, r16, What_out, A, B, d, s);
    if (e == hipSuccess) e = launch_fwd_prologue(X, f32, M, K, A, B, d, xs, xs_lo, beta, s);
  }
  if (e != hipSuccess) return LCVQ_ERR_HIP;
  void* split = gemm_fwd_split_bytes(M, N, K) ? static_cast<void*>(ws + w.split) : nullptr;
  return from_hip(launch_gemm_fwd(xs, xs_lo, r16, beta, (int)M, (int)N, (int)K, d, Y, f32, split,
                                  s));
}

size_t lcvq_linear_bwd_workspace_size(int64_t M, int64_t N, int64_t K, int d) {
  if (!layer_shape_ok(M, N, K) || !d_ok(d)) return 0;
  // sized for float32 activations (the larger case)
  return bwd_ws(M, N, K, d, true).total;
}

}  // extern "C"

namespace {
lcvq_status_t linear_bwd_impl(const void* dY, const void* X, lcvq_dtype_t dt, int64_t M,
                              int64_t N, int64_t K, int d, const uint8_t* packed,
                              const uint8_t* mask, const float* Wp, float alpha,
                              const float* A, const float* B, void* dX, float* dWp, float* dA,
                              float* dB, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (!dY || !X || !packed || !mask || !A || !B || !dWp || !dA || !dB) return LCVQ_ERR_NULL;
  if (dt != LCVQ_F32 && dt != LCVQ_BF16) return LCVQ_ERR_DTYPE;
  if (!d_ok(d)) return LCVQ_ERR_D;
  if (!layer_shape_ok(M, N, K)) return LCVQ_ERR_SHAPE;
  if (!aligned16(dY) || !aligned16(X) || !aligned16(packed) || !aligned16(mask) ||
      !aligned16(A) || !aligned16(B) || !aligned16(dX) || !aligned16(dWp) || !aligned16(dA) ||
      !aligned16(dB) || !aligned16(workspace))
    return LCVQ_ERR_ALIGN;
  const bool f32 = dt == LCVQ_F32;
  const BwdWs w = bwd_ws(M, N, K, d, f32);
  if (!workspace || workspace_bytes < w.total) return LCVQ_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* r = reinterpret_cast<float*>(ws + w.r);
  uint32_t* r16t = reinterpret_cast<uint32_t*>(ws + w.r16t);
  float* partials = reinterpret_cast<float*>(ws + w.partials);
  uint16_t* dy_hi = f32 ? reinterpret_cast<uint16_t*>(ws + w.dy_hi) : nullptr;
  uint16_t* dy_lo = f32 ? reinterpret_cast<uint16_t*>(ws + w.dy_lo) : nullptr;
  uint16_t* x_hi = f32 ? reinterpret_cast<uint16_t*>(ws + w.x_hi) : nullptr;
  uint16_t* x_lo = f32 ? reinterpret_cast<uint16_t*>(ws + w.x_lo) : nullptr;
  // prologue and the transposed codes (read by dW's epilogue and by dX) in one launch
  const int64_t rblocks = ((K + 255) / 256) * (N / 64);
  const bool merged = M + rblocks <= kMaxBlocks256;
  hipError_t e = merged ? launch_bwd_prep(dY, X, f32, M, N, K, r, dy_hi, dy_lo, x_hi, x_lo,
                                          packed, r16t, s)
                        : launch_bwd_prologue(dY, X, f32, M, N, K, r, dy_hi, dy_lo, x_hi,
                                              x_lo, s);
  if (e == hipSuccess && !merged) e = launch_codes_to_r16t(packed, N, K, r16t, s);
  if (e != hipSuccess) return LCVQ_ERR_HIP;
  const uint16_t* dyb = f32 ? dy_hi : static_cast<const uint16_t*>(dY);
  const uint16_t* xb = f32 ? x_hi : static_cast<const uint16_t*>(X);
  // dW first; with dX wanted, the dX product then also reduces dW's dA/dB partials
  // (saving the reduction's own launch), otherwise a small kernel does.
  void* split = dw_split_bytes(M, N, K) ? static_cast<void*>(ws + w.split) : nullptr;
  e = launch_gemm_dw(xb, x_lo, dyb, dy_lo, r16t, mask, A, (int)M, (int)N, (int)K, d, dWp,
                     partials, dA, dB, Wp, alpha, !dX, split, s);
  if (e != hipSuccess) return LCVQ_ERR_HIP;
  if (dX) {
    e = launch_gemm_dx(r16t, dyb, dy_lo, r, A, B, (int)M, (int)N, (int)K, d, dX, f32, partials,
                       dA, dB, s);
    if (e != hipSuccess) return LCVQ_ERR_HIP;
  }
  return LCVQ_OK;
}
}  // namespace

extern "C" {

lcvq_status_t lcvq_linear_bwd(const void* dY, const void* X, lcvq_dtype_t dt, int64_t M,
                              int64_t N, int64_t K, int d, const uint8_t* packed,
                              const uint8_t* mask, const float* A, const float* B,
                              void* dX, float* dWp, float* dA, float* dB, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return linear_bwd_impl(dY, X, dt, M, N, K, d, packed, mask, nullptr, 0.f, A, B, dX, dWp, dA,
                         dB, workspace, workspace_bytes, stream);
}

lcvq_status_t lcvq_linear_bwd_dge(const void* dY, const void* X, lcvq_dtype_t dt, int64_t M,
                                  int64_t N, int64_t K, int d, const uint8_t* packed,
                                  const uint8_t* mask, const float* Wp, float alpha,
                                  const float* A, const float* B, void* dX, float* dWp,
                                  float* dA, float* dB, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!Wp) return LCVQ_ERR_NULL;
  if (!aligned16(Wp)) return LCVQ_ERR_ALIGN;
  if (!(alpha > 0.f) || !(alpha <= 1000.f)) return LCVQ_ERR_VALUE;   // also rejects NaN
  return linear_bwd_impl(dY, X, dt, M, N, K, d, packed, mask, Wp, alpha, A, B, dX, dWp, dA,
                         dB, workspace, workspace_bytes, stream);
}

size_t lcvq_gemv2b_workspace_size(int64_t M, int64_t N, int64_t K, int d) {
  (void)d;
  if (M < 1 || M > 16 || !decode_shape_ok(N, K)) return 0;
  return gemv_ws(K).total;
}

}  // extern "C"

// lcvq_gemv2b and lcvq_gemv2b_shuffled: the codes in the canonical packed layout or in
// the decode layout written by lcvq_gemv2b_shuffle.
static lcvq_status_t gemv2b_impl(const void* X, int64_t M, int64_t N, int64_t K, int d,
                                 const uint8_t* packed, int shuffled, const void* A16,
                                 const void* B16, void* Y, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!X || !packed || !A16 || !B16 || !Y) return LCVQ_ERR_NULL;
  if (!d_ok(d)) return LCVQ_ERR_D;
  if (M < 1 || M > 16 || !decode_shape_ok(N, K)) return LCVQ_ERR_SHAPE;
  if (shuffled && !decode_layout_shape_ok(N, K)) return LCVQ_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(packed) || !aligned16(A16) || !aligned16(B16) ||
      !aligned16(Y) || !aligned16(workspace))
    return LCVQ_ERR_ALIGN;
  const GemvWs w = gemv_ws(K);
  if (!workspace || workspace_bytes < w.total) return LCVQ_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int8_t* xq = reinterpret_cast<int8_t*>(ws + w.xq);
  float* rowinfo = reinterpret_cast<float*>(ws + w.rowinfo);
  return from_hip(launch_gemv(static_cast<const uint16_t*>(X), (int)M, (int)N, (int)K,
                              static_cast<const uint16_t*>(A16),
                              static_cast<const uint16_t*>(B16), d, packed, shuffled,
                              static_cast<uint16_t*>(Y), xq, rowinfo, s));
}

extern "C" {

lcvq_status_t lcvq_gemv2b(const void* X, int64_t M, int64_t N, int64_t K, int d,
                          const uint8_t* packed, const void* A16, const void* B16, void* Y,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return gemv2b_impl(X, M, N, K, d, packed, 0, A16, B16, Y, workspace, workspace_bytes, stream);
}

lcvq_status_t lcvq_gemv2b_shuffled(const void* X, int64_t M, int64_t N, int64_t K, int d,
                                   const uint8_t* codes, const void* A16, const void* B16,
                                   void* Y, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  return gemv2b_impl(X, M, N, K, d, codes, 1, A16, B16, Y, workspace, workspace_bytes, stream);
}

lcvq_status_t lcvq_gemv2b_noalloc(const void* X, int64_t M, int64_t N, int64_t K, int d,
                                  const uint8_t* packed, const void* A16, const void* B16,
                                  void* Y, void* stream) {
  if (!X || !packed || !A16 || !B16 || !Y) return LCVQ_ERR_NULL;
  if (!d_ok(d)) return LCVQ_ERR_D;
  if (M < 1 || M > 16 || !decode_shape_ok(N, K)) return LCVQ_ERR_SHAPE;
  if (K > kNoAllocMaxK) return LCVQ_ERR_SCRATCH;
  static_assert(gemv_ws(kNoAllocMaxK).total <= kScratchBytes, "scratch covers the largest K");
  uint8_t* ws = nullptr;
  const lcvq_status_t st = scratch_ptr(&ws);
  if (st != LCVQ_OK) return st;
  return gemv2b_impl(X, M, N, K, d, packed, 0, A16, B16, Y, ws, kScratchBytes, stream);
}

lcvq_status_t lcvq_hessian(const void* X, int64_t M, int64_t K, float* H, void* stream) {
  if (!X || !H) return LCVQ_ERR_NULL;
  if (M < 1 || M > kMaxRows || K < 64 || (K % 64) || K > kPtqMaxK) return LCVQ_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(H)) return LCVQ_ERR_ALIGN;
  return from_hip(launch_gram(static_cast<const uint16_t*>(X), (int)M, (int)K, H,
                              as_stream(stream)));
}

size_t lcvq_ptq_workspace_size(int64_t N, int64_t K) {
  if (!ptq_shape_ok(N, K)) return 0;
  return ptq_workspace_bytes(N, K);
}

lcvq_status_t lcvq_ptq_init(const float* H, const float* W0, int64_t N, int64_t K, float damp,
                            int iters, uint8_t* packed_out, float* sb_out, float* obj_out,
                            float* U_out, float* D_out, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!H || !W0 || !packed_out || !sb_out) return LCVQ_ERR_NULL;
  if (!ptq_shape_ok(N, K)) return LCVQ_ERR_SHAPE;
  if (!(damp > 0.f) || !(damp <= 1.f) || iters < 1 || iters > 64) return LCVQ_ERR_VALUE;
  if (!aligned16(H) || !aligned16(W0) || !aligned16(packed_out) || !aligned16(sb_out) ||
      !aligned16(obj_out) || !aligned16(U_out) || !aligned16(D_out) || !aligned16(workspace))
    return LCVQ_ERR_ALIGN;
  if (!workspace || workspace_bytes < ptq_workspace_bytes(N, K)) return LCVQ_ERR_WORKSPACE;
  return from_hip(launch_ptq_init(H, W0, (int)N, (int)K, damp, iters, packed_out, sb_out,
                                  obj_out, U_out, D_out, workspace, as_stream(stream)));
}

lcvq_status_t lcvq_read_probe(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink) return LCVQ_ERR_NULL;
  if (bytes < 16 || (bytes % 16) || bytes > (int64_t(1) << 40)) return LCVQ_ERR_SHAPE;
  if (!aligned16(buf) || !aligned16(sink)) return LCVQ_ERR_ALIGN;
  return from_hip(launch_read_probe(buf, bytes, sink, as_stream(stream)));
}

lcvq_status_t lcvq_mfma_probe(int64_t iters, uint32_t* sink, void* stream) {
  if (!sink) return LCVQ_ERR_NULL;
  if (iters < 2 || iters > (int64_t(1) << 24) || (iters % 2)) return LCVQ_ERR_SHAPE;
  if (!aligned16(sink)) return LCVQ_ERR_ALIGN;
  return from_hip(launch_mfma_probe((int)iters, sink, as_stream(stream)));
}

lcvq_status_t lcvq_gemv2b_shuffle(const uint8_t* packed, int64_t N, int64_t K, uint8_t* codes,
                                  void* stream) {
  if (!packed || !codes) return LCVQ_ERR_NULL;
  if (!decode_layout_shape_ok(N, K)) return LCVQ_ERR_SHAPE;
  if (!aligned16(packed) || !aligned16(codes)) return LCVQ_ERR_ALIGN;
  return from_hip(launch_gemv_shuffle(packed, N, K, codes, as_stream(stream)));
}

lcvq_status_t lcvq_gemv2b_batched(const void* X, int64_t M, int64_t K, int d,
                                  const lcvq_gemv2b_matrix* mats, int count, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!X || !mats) return LCVQ_ERR_NULL;
  if (!d_ok(d)) return LCVQ_ERR_D;
  if (count < 1 || count > GEMV_MAX_BATCH) return LCVQ_ERR_SHAPE;
  if (M < 1 || M > 16 || !decode_shape_ok(16, K)) return LCVQ_ERR_SHAPE;
  int64_t nmax = 0, groups = 0;
  for (int i = 0; i < count; ++i) {
    const lcvq_gemv2b_matrix& m = mats[i];
    if (!m.packed || !m.A16 || !m.B16 || !m.Y) return LCVQ_ERR_NULL;
    if (m.layout != 0 && m.layout != 1) return LCVQ_ERR_VALUE;
    if (!decode_shape_ok(m.N, K)) return LCVQ_ERR_SHAPE;
    if (m.layout == 1 && !decode_layout_shape_ok(m.N, K)) return LCVQ_ERR_SHAPE;
    if (!aligned16(m.packed) || !aligned16(m.A16) || !aligned16(m.B16) || !aligned16(m.Y))
      return LCVQ_ERR_ALIGN;
    nmax = m.N > nmax ? m.N : nmax;
    groups += m.N / 16;
  }
  if (groups * 16 > kMaxDecodeRows) return LCVQ_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(workspace)) return LCVQ_ERR_ALIGN;
  const GemvWs w = gemv_ws(K);
  if (!workspace || workspace_bytes < w.total) return LCVQ_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  if (gemv_fused_path((int)M, (int)K, groups * 16, d)) {
    GemvBatch b = {};
    b.count = count;
    for (int i = 0; i < count; ++i) {
      b.packed[i] = mats[i].packed;
      b.A16[i] = static_cast<const uint16_t*>(mats[i].A16);
      b.B16[i] = static_cast<const uint16_t*>(mats[i].B16);
      b.Y[i] = static_cast<uint16_t*>(mats[i].Y);
      b.N[i] = (int)mats[i].N;
      b.shuffled[i] = mats[i].layout;
    }
    return from_hip(launch_gemv_fused(static_cast<const uint16_t*>(X), (int)M, (int)K, d, b, s));
  }
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  for (int i = 0; i < count; ++i) {
    const hipError_t e = launch_gemv(static_cast<const uint16_t*>(X), (int)M, (int)mats[i].N,
                                     (int)K, static_cast<const uint16_t*>(mats[i].A16),
                                     static_cast<const uint16_t*>(mats[i].B16), d,
                                     mats[i].packed, mats[i].layout,
                                     static_cast<uint16_t*>(mats[i].Y),
                                     reinterpret_cast<int8_t*>(ws + w.xq),
                                     reinterpret_cast<float*>(ws + w.rowinfo), s);
    if (e != hipSuccess) return LCVQ_ERR_HIP;
  }
  return LCVQ_OK;
}

}  // extern "C"
