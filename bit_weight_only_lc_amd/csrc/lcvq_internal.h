// Internal launchers of the LC-VQ kernels (not part of the public ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lcvq {

// Kernel ids of the profiling hook (lcvq_profile_next).
enum { PROF_QUANTIZE = 1, PROF_FWD = 2, PROF_DX = 3, PROF_DW = 4, PROF_GEMV = 5, PROF_BWD_PREP = 6,
       PROF_GRAM = 7, PROF_PTQ_SWEEP = 8, PROF_READ_PROBE = 9,
       PROF_MFMA_PROBE = 10, PROF_PACK = 11, PROF_UNPACK = 12, PROF_LAST = 12 };
// True (once) if the calling thread armed timing for kernel `id`; returns the events.
bool take_profile(int id, hipEvent_t* start, hipEvent_t* stop);

}  // namespace lcvq

#include <hip/hip_ext.h>
// Launch through hipExtLaunchKernelGGL when timing is armed for this kernel id.
#define LCVQ_LAUNCH(ID, KERNEL, GRID, BLOCK, SHM, STREAM, ...)                            \
  do {                                                                                  \
    hipEvent_t lcvq_ev0_, lcvq_ev1_;                                                    \
    if (::lcvq::take_profile((ID), &lcvq_ev0_, &lcvq_ev1_))                             \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, SHM, STREAM, lcvq_ev0_, lcvq_ev1_, 0,    \
                            __VA_ARGS__);                                               \
    else                                                                                \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHM, STREAM, __VA_ARGS__);                \
  } while (0)

namespace lcvq {

hipError_t launch_quantize(const float* wp, int64_t N, int64_t K, uint8_t* z, uint8_t* packed,
                           uint8_t* mask, uint32_t* r16, float* what, const float* A,
                           const float* B, int d, hipStream_t s);
hipError_t launch_pack2b(const uint8_t* z, int64_t N, int64_t K, uint8_t* packed, hipStream_t s);
hipError_t launch_unpack2b(const uint8_t* packed, int64_t N, int64_t K, uint8_t* z, hipStream_t s);
hipError_t launch_codes_to_r16t(const uint8_t* packed, int64_t N, int64_t K, uint32_t* r16t,
                                hipStream_t s);
hipError_t launch_fwd_prologue(const void* X, bool x_f32, int64_t M, int64_t K, const float* A,
                               const float* B, int d, uint16_t* xs, uint16_t* xs_lo,
                               float* beta, hipStream_t s);
hipError_t launch_bwd_prologue(const void* dY, const void* X, bool f32, int64_t M, int64_t N,
                               int64_t K, float* r, uint16_t* dy_hi, uint16_t* dy_lo,
                               uint16_t* x_hi, uint16_t* x_lo, hipStream_t s);

// One launch each for the forward's quantizer + prologue and the backward's prologue +
// transposed codes (r16t may be NULL when dX is not wanted). Their grids are 256-thread
// blocks, so the callers use them only while the block count stays below 2^24 (2^32
// work-items); otherwise they launch the parts separately.
hipError_t launch_fwd_prep(const float* wp, int64_t N, int64_t K, uint8_t* packed, uint8_t* mask,
                           uint32_t* r16, float* what, const void* X, bool x_f32, int64_t M,
                           const float* A, const float* B, int d, uint16_t* xs,
                           uint16_t* xs_lo, float* beta, hipStream_t s);
hipError_t launch_bwd_prep(const void* dY, const void* X, bool f32, int64_t M, int64_t N,
                           int64_t K, float* r, uint16_t* dy_hi, uint16_t* dy_lo,
                           uint16_t* x_hi, uint16_t* x_lo, const uint8_t* packed,
                           uint32_t* r16t, hipStream_t s);

int gemm_tiles(int64_t P, int64_t Q);
// Launches with at most 128 tiles (of 256 x 256) split their contraction over up to four
// workgroups per tile: gemm_splits() of them (1: no split), and gemm_split_bytes() of
// workspace (0 without a split) for the forward (P = M, Q = N, R = K) and dW (P = K,
// Q = N, R = M) products.
int gemm_splits(int64_t P, int64_t Q, int64_t R);
size_t gemm_split_bytes(int64_t P, int64_t Q, int64_t R);
// The forward instead runs 128 x 256 tiles without a split where those fill more than half
// of the CUs (gemm_fwd_half_tiles); gemm_fwd_split_bytes is its workspace for partials.
bool gemm_fwd_half_tiles(int64_t M, int64_t N);
size_t gemm_fwd_split_bytes(int64_t M, int64_t N, int64_t K);
// Rows of dA/dB partials ([rows][d*d + d] floats) the dW product writes for M tokens and a
// weight [N, K]: one per tile, or DW_EPI_G per tile when its contraction is split.
int dw_partial_rows(int64_t M, int64_t N, int64_t K);
// Bytes of float32 partial tiles the dW product of this shape needs (few-tile split or the
// tail split of its last partial round; 0: none).
size_t dw_split_bytes(int64_t M, int64_t N, int64_t K);
// Products. `*_lo` operands are NULL for bf16 activations; for float32 activations
// they hold the low bf16 half of each value and add the cross terms in extra passes.
hipError_t launch_gemm_fwd(const uint16_t* xs, const uint16_t* xs_lo, const uint32_t* r16,
                           const float* beta, int M, int N, int K, int d, void* Y, bool y_f32,
                           void* split_ws, hipStream_t s);
// dX; with dw_partials (the dW product already enqueued) it also reduces them into dA, dB.
hipError_t launch_gemm_dx(const uint32_t* r16t, const uint16_t* dy, const uint16_t* dy_lo,
                          const float* r, const float* A, const float* B, int M, int N, int K,
                          int d, void* dX, bool f32, const float* dw_partials, float* dA,
                          float* dB, hipStream_t s);
// dW reads the codes as the transposed code words r16t (launch_codes_to_r16t's layout).
hipError_t launch_gemm_dw(const uint16_t* x, const uint16_t* x_lo, const uint16_t* dy,
                          const uint16_t* dy_lo, const uint32_t* r16t, const uint8_t* mask,
                          const float* A, int M, int N, int K, int d, float* dWp,
                          float* partials, float* dA, float* dB, const float* dge_wp,
                          float dge_alpha, bool reduce, void* split_ws, hipStream_t s);

// PTQ initialisation: H = X^T X (bf16 X [M][K], K a multiple of 64, float H [K][K]).
hipError_t launch_gram(const uint16_t* X, int M, int K, float* H, hipStream_t s);
// The rest of the initialisation (damped factorisation, alternation, packed output); the
// workspace is carved by ptq_workspace().
size_t ptq_workspace_bytes(int64_t N, int64_t K);
hipError_t launch_ptq_init(const float* H, const float* W0, int N, int K, float damp, int iters,
                           uint8_t* packed_out, float* sb_out, float* obj_out, float* U_out,
                           float* D_out, void* workspace, hipStream_t s);

// Matrices that share X for one fused decode launch (kernel argument, by value).
constexpr int GEMV_MAX_BATCH = 8;
struct GemvBatch {
  const uint8_t* packed[GEMV_MAX_BATCH];
  const uint16_t* A16[GEMV_MAX_BATCH];
  const uint16_t* B16[GEMV_MAX_BATCH];
  uint16_t* Y[GEMV_MAX_BATCH];
  int N[GEMV_MAX_BATCH];
  int shuffled[GEMV_MAX_BATCH];  // codes in the decode layout (lcvq_gemv2b_shuffle)
  int wg0[GEMV_MAX_BATCH];     // first workgroup of each matrix (set by the launcher)
  int count;
};
// True when the fused single-launch path serves M tokens at this K.
bool gemv_fused_path(int M, int K, int64_t rows, int d);
hipError_t launch_gemv_fused(const uint16_t* X, int M, int K, int d, GemvBatch b,
                             hipStream_t s);

// Decode product. Few tokens: one fused kernel (xq and rowinfo unused); otherwise a
// prologue writes X' limbs to xq and block scales to rowinfo, and the product reads them.
hipError_t launch_gemv(const uint16_t* X, int M, int N, int K, const uint16_t* A16,
                       const uint16_t* B16, int d, const uint8_t* packed, int shuffled,
                       uint16_t* Y, int8_t* xq, float* rowinfo, hipStream_t s);
// Measurement helper: stream `bytes` once in one launch (same-size read ceiling).
hipError_t launch_read_probe(const void* p, int64_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_mfma_probe(int iters, uint32_t* sink, hipStream_t s);
// Canonical packed codes [N][K/4] -> the decode layout read with shuffled = 1.
hipError_t launch_gemv_shuffle(const uint8_t* packed, int64_t N, int64_t K, uint8_t* out,
                               hipStream_t s);

}  // namespace lcvq
