/*
 * lcvq.h -- C ABI of the LC-VQ hot path on AMD Instinct MI355X (gfx950).
 *
 * LC-VQ reconstructs every d-vector of a weight matrix as c = A z + B, where the code
 * z = clamp(round(Wp), 0, 3) comes from float proxy weights Wp, and one d x d matrix A
 * and one d-vector B are shared by the whole matrix ("LC-QAT: Data-Efficient 2-Bit QAT
 * for LLMs via Linear-Constrained Vector Quantization", technical summary, Methodology 1
 * and 3). This library runs the quantizer, the forward product with the decoded weights,
 * the straight-through backward, 2-bit packing and the packed-weight decode product.
 *
 * Conventions for every call:
 *  - Tensor pointers are DEVICE pointers, allocated and owned by the caller. The library
 *    never allocates, frees or synchronizes; it validates arguments on the host, enqueues
 *    kernels on `stream` (a hipStream_t; NULL means the default stream) and returns.
 *  - Tensors are dense and row-major. A weight matrix is W[N, K] (N outputs, K inputs, as
 *    torch.nn.Linear stores it) and the layer computes Y = X W^T. The d-vectors run along
 *    K: vector (n, g) is W[n, g*d : (g+1)*d]. Decoding: What[n, g*d+i] = B[i] +
 *    sum_j A[i*d + j] * z[n, g*d+j] (A row-major, multiplying z as a column vector).
 *  - Rounding is round-half-to-even. The straight-through mask is 1 exactly where
 *    0 <= round(Wp) <= 3 (the clamp did nothing). NaN gives code 0, +inf code 3, -inf
 *    code 0, all with mask 0.
 *  - Packed codes: 4 per byte, code k = 4b + t in bits [2t, 2t+1] of byte b of its row.
 *    Mask: 8 per byte, bit k = 8c + t in bit t of byte c of its row.
 *  - All pointers must be 16-byte aligned. Outputs must not overlap inputs or each other.
 *  - Shape limits of the layer calls: d in {4, 8, 16}; 1 <= M <= 2^24 - 2^17; N and K
 *    multiples of 64 in [64, 2^21]; N * K < 2^40; and at most 2^23 - 8 tiles of 256 x 256
 *    in each of the products (M x N, K x N, K x M). These keep every kernel grid within
 *    HIP's 2^32 - 1 work-items. (lcvq_quantize / pack / unpack need only K a multiple
 *    of 16 and N * K < 2^40.) Shapes outside them return LCVQ_ERR_SHAPE.
 *  - Errors are returned synchronously from host-side checks, before anything is
 *    enqueued. LCVQ_ERR_HIP reports a failed launch; faults inside kernels surface at the
 *    caller's next synchronization, as with any HIP work.
 *  - Calls are re-entrant. State kept between calls: the per-thread profiling hook at
 *    the end of this file, and a process-wide record of the devices on which the decode
 *    kernels' dynamic LDS size has been requested (hipFuncSetAttribute, once per device
 *    and kernel; a failed request returns LCVQ_ERR_HIP and is not recorded).
 */
#ifndef LCVQ_H
#define LCVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LCVQ_OK = 0,
  LCVQ_ERR_NULL = 1,       /* a required pointer is NULL */
  LCVQ_ERR_SHAPE = 2,      /* M, N or K outside the limits above */
  LCVQ_ERR_D = 3,          /* d not in {4, 8, 16} */
  LCVQ_ERR_DTYPE = 4,      /* unknown dtype code */
  LCVQ_ERR_ALIGN = 5,      /* a pointer is not 16-byte aligned */
  LCVQ_ERR_WORKSPACE = 6,  /* workspace NULL or smaller than the *_workspace_size() */
  LCVQ_ERR_HIP = 7,        /* a kernel launch failed */
  LCVQ_ERR_VALUE = 8,      /* a scalar argument is out of range */
  LCVQ_ERR_SCRATCH = 9     /* shape beyond what lcvq_gemv2b_noalloc's fixed scratch holds */
} lcvq_status_t;

typedef enum { LCVQ_F32 = 0, LCVQ_BF16 = 1 } lcvq_dtype_t;

/* Text for a status code (static storage). */
const char* lcvq_status_string(lcvq_status_t s);

/*
 * Quantizer: z = clamp(round(Wp), 0, 3) and the straight-through mask
 * (LC-QAT summary: Methodology 1, rounding and clamping; Methodology 3, forward).
 *   Wp      float [N, K]            in
 *   z_u8    uint8 [N, K]   or NULL  out: one code per byte
 *   packed  uint8 [N, K/4] or NULL  out: 4 codes per byte
 *   mask    uint8 [N, K/8] or NULL  out: 8 mask bits per byte
 * Requires K % 16 == 0, N >= 1.
 */
lcvq_status_t lcvq_quantize(const float* Wp, int64_t N, int64_t K, uint8_t* z_u8,
                            uint8_t* packed, uint8_t* mask, void* stream);

/*
 * 2-bit packing of codes (values 0..3; higher bits are ignored) and its inverse.
 * The integer part is what a deployment keeps (decoupleQ, section 3.2).
 *   z_u8 uint8 [N, K] <-> packed uint8 [N, K/4]. Requires K % 16 == 0.
 */
lcvq_status_t lcvq_pack2b(const uint8_t* z_u8, int64_t N, int64_t K, uint8_t* packed,
                          void* stream);
lcvq_status_t lcvq_unpack2b(const uint8_t* packed, int64_t N, int64_t K, uint8_t* z_u8,
                            void* stream);

/*
 * Forward of one LC-VQ linear layer: quantize Wp, decode with A z + B, Y = X What^T
 * (LC-QAT summary, Methodology 3 forward; the product runs on 2-bit codes).
 *   X          [M, K] in xdt (LCVQ_BF16 or LCVQ_F32)
 *   Wp         float [N, K];  A float [d, d];  B float [d]
 *   Y          [M, N] in xdt                         out
 *   packed_out uint8 [N, K/4]                        out (required: the backward needs it)
 *   mask_out   uint8 [N, K/8]                        out (required)
 *   What_out   float [N, K] or NULL                  out: decoded weights in float32
 *   workspace  >= lcvq_linear_fwd_workspace_size(M, N, K, d) bytes, device memory
 * Numerics: the product runs on bf16 matrix cores with float32 accumulation; the
 * decoding matrix A is applied to X (X' = X (I kron A), rounded to bf16), the codes
 * enter exactly, and X B is added in float32. With LCVQ_F32 activations every bf16
 * operand is carried as a hi + lo pair (about 16 significant bits) over extra passes.
 * The workspace size covers both activation types.
 */
size_t lcvq_linear_fwd_workspace_size(int64_t M, int64_t N, int64_t K, int d);
lcvq_status_t lcvq_linear_fwd(const void* X, lcvq_dtype_t xdt, int64_t M, int64_t N,
                              int64_t K, int d, const float* Wp, const float* A,
                              const float* B, void* Y, uint8_t* packed_out,
                              uint8_t* mask_out, float* What_out, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * Straight-through backward of the same layer (gradients flow through the linear decode,
 * LC-QAT summary, Methodology 1; the rounding is passed straight through, masked where
 * the clamp was active):
 *   dX  = dY What                                              [M, K] in dt, or NULL
 *   G   = dY^T X  (never stored)
 *   dWp[n, g*d+j] = mask * sum_i A[i, j] G[n, g*d+i]           float [N, K]
 *   dA[i, j] = sum over vectors of G[n, g*d+i] z[n, g*d+j]     float [d, d]
 *   dB[i]    = sum over vectors of G[n, g*d+i]                 float [d]
 * Inputs: dY [M, N] and X [M, K] in dt; packed and mask as written by lcvq_linear_fwd.
 * All outputs are overwritten. dA and dB are reduced in a fixed order, so repeated
 * calls give identical bytes.
 */
size_t lcvq_linear_bwd_workspace_size(int64_t M, int64_t N, int64_t K, int d);
lcvq_status_t lcvq_linear_bwd(const void* dY, const void* X, lcvq_dtype_t dt, int64_t M,
                              int64_t N, int64_t K, int d, const uint8_t* packed,
                              const uint8_t* mask, const float* A, const float* B,
                              void* dX, float* dWp, float* dA, float* dB, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * The same backward with LC-QAT's differentiable gradient estimator in place of the
 * straight-through one (LC-QAT summary, Methodology 3 backward: the rounding's gradient
 * comes from a smooth, differentiable curve that approximates the discretization). The
 * summary does not give the curve; this library uses tanh-smoothed rounding,
 *   s(w) = floor(w) + 1/2 + tanh(alpha (f - 1/2)) / (2 tanh(alpha / 2)),  f = w - floor(w),
 * which passes through every integer, is steepest at the half-integers, tends to the
 * straight-through estimator as alpha -> 0 and to rounding as alpha grows. The forward
 * is unchanged (it rounds). Only dWp changes:
 *   dWp[n, k] = mask * s'(Wp[n, k]) * sum_i A[i, j] G[n, g*d+i]     (k = g*d + j)
 * with s'(w) = alpha (1 - tanh^2(alpha (f - 1/2))) / (2 tanh(alpha / 2)) (0 for non-finite
 * w). dX, dA and dB are those of lcvq_linear_bwd.
 *   Wp     float [N, K], the proxies the forward quantized (read once more, 4 B/weight)
 *   alpha  sharpness, 0 < alpha <= 1000 (LCVQ_ERR_VALUE otherwise)
 * Every other argument, the workspace and the errors are as for lcvq_linear_bwd.
 */
lcvq_status_t lcvq_linear_bwd_dge(const void* dY, const void* X, lcvq_dtype_t dt, int64_t M,
                                  int64_t N, int64_t K, int d, const uint8_t* packed,
                                  const uint8_t* mask, const float* Wp, float alpha,
                                  const float* A, const float* B, void* dX, float* dWp,
                                  float* dA, float* dB, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Decode product from the deployed artefact (packed codes plus half-precision A, B):
 * Y = X What^T for a few tokens (decoupleQ, section 3.2: one linear transform turns the
 * integer part back into weights; LC-QAT summary, Methodology 3).
 *   X   bfloat16 [M, K], 1 <= M <= 16;  packed uint8 [N, K/4]
 *   N a multiple of 16, at most 2^26; K a multiple of 64; N * K <= 2^36
 *   A16 float16 [d, d];  B16 float16 [d]
 *   Y   bfloat16 [M, N]                                          out
 *   workspace >= lcvq_gemv2b_workspace_size(M, N, K, d) bytes (0 for invalid shapes)
 * Numerics: X (I kron A) is formed in float32 and held as 16-bit fixed point per row;
 * the product with the codes is exact integer arithmetic, and partial sums are added
 * in a fixed order, so repeated calls give identical bytes. The workspace size depends
 * on K only today; N is part of the query so that it may grow with N later. Calls that
 * share one workspace must not run concurrently.
 */
size_t lcvq_gemv2b_workspace_size(int64_t M, int64_t N, int64_t K, int d);
lcvq_status_t lcvq_gemv2b(const void* X, int64_t M, int64_t N, int64_t K, int d,
                          const uint8_t* packed, const void* A16, const void* B16, void* Y,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * lcvq_gemv2b for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same product, the
 * same kernels and the same output bytes as lcvq_gemv2b, without a workspace argument.
 * Its scratch (X' limbs and block scales of the few-token path that writes them) is a
 * fixed device array in the library, 2,129,920 bytes per GPU, held from the first call
 * on that GPU until the process ends; its address is looked up once per device. The
 * call allocates and frees nothing.
 *   Arguments as for lcvq_gemv2b, less the workspace; K at most 65536.
 * Errors as for lcvq_gemv2b; LCVQ_ERR_SCRATCH for K > 65536; LCVQ_ERR_HIP if the
 * scratch address cannot be had. Every call on one GPU shares that GPU's scratch, which
 * keeps the last call's contents (no part of it needs to start at zero): calls that
 * overlap in time on one GPU (other streams, other host threads) race and must not be
 * made.
 */
lcvq_status_t lcvq_gemv2b_noalloc(const void* X, int64_t M, int64_t N, int64_t K, int d,
                                  const uint8_t* packed, const void* A16, const void* B16,
                                  void* Y, void* stream);

/*
 * Decode layout of the codes, for deployment: the same bytes as the canonical packed
 * [N, K/4] rearranged so that the decode product reads each 16-row x 256-column block as
 * one contiguous 1 KiB tile. Tile t = (n / 16) * (K / 256) + kb; within it, the 16 bytes
 * of row 16 (t / (K/256)) + j, columns 256 kb + 64 q .. +63, sit at byte 16 (16 q + j).
 * The layout is this library's own (the pages fix only what the integer part holds).
 *   packed  uint8 [N, K/4] canonical (2-bit fields, little-endian along K)         in
 *   codes   uint8, N * K / 4 bytes, must not overlap packed                          out
 *   N a multiple of 16, at most 2^26; K a multiple of 256; N * K <= 2^36; both pointers
 *   16-byte aligned
 * Errors: LCVQ_ERR_NULL, LCVQ_ERR_SHAPE, LCVQ_ERR_ALIGN, LCVQ_ERR_HIP.
 */
lcvq_status_t lcvq_gemv2b_shuffle(const uint8_t* packed, int64_t N, int64_t K, uint8_t* codes,
                                  void* stream);

/*
 * lcvq_gemv2b with the codes in the decode layout (lcvq_gemv2b_shuffle). Arguments,
 * errors and numerics as for lcvq_gemv2b, except that K must be a multiple of 256 (the
 * layout is made of whole 256-column blocks); the output is byte for byte the same as
 * lcvq_gemv2b's on the canonical codes.
 */
lcvq_status_t lcvq_gemv2b_shuffled(const void* X, int64_t M, int64_t N, int64_t K, int d,
                                   const uint8_t* codes, const void* A16, const void* B16,
                                   void* Y, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * Decode product of several matrices that share the input X (and K), for instance the
 * q, k and v projections, or gate and up, of one transformer layer; each matrix has its
 * own codes and its own A, B (LC-QAT summary, Methodology 1: A and B are shared within
 * one weight matrix). Every output equals what lcvq_gemv2b gives for that matrix, byte
 * for byte. With M <= 2 and K <= 16384, or M <= 4 and K <= 8192, all of them run in
 * one launch; likewise for up to 8192 rows in all (4096 with M <= 4) with M >= 3, where
 * the one-launch kernel's bound on its activation work, M * ceil(K / 256) * d <= 1792
 * (K <= 16384 for M <= 4, K <= 4096 beyond), holds; otherwise each matrix is computed as
 * lcvq_gemv2b computes it, one after the other, on `stream`.
 *   X       bfloat16 [M, K], 1 <= M <= 16, K a multiple of 64 (of 256 if any matrix is
 *           in the decode layout)
 *   mats    host array of `count` descriptors, 1 <= count <= 8; mats[i].N a multiple of
 *           16, the N summed over the matrices at most 2^26, each N * K <= 2^36; packed
 *           (N * K / 4 bytes: canonical [N, K/4] for layout 0, the decode layout of
 *           lcvq_gemv2b_shuffle for layout 1), A16 float16 [d, d], B16 float16 [d] and the
 *           output Y bfloat16 [M, N] are device pointers; outputs must not overlap
 *           anything
 *   workspace >= lcvq_gemv2b_workspace_size(M, largest N, K, d) bytes
 * Errors as for lcvq_gemv2b; LCVQ_ERR_SHAPE also for count outside 1..8 and for a matrix
 * in the decode layout with K not a multiple of 256, LCVQ_ERR_VALUE for a layout other
 * than 0 or 1.
 */
typedef struct {
  const uint8_t* packed;
  const void* A16;
  const void* B16;
  void* Y;
  int64_t N;
  int32_t layout;              /* 0: canonical packed; 1: decode layout */
} lcvq_gemv2b_matrix;
lcvq_status_t lcvq_gemv2b_batched(const void* X, int64_t M, int64_t K, int d,
                                  const lcvq_gemv2b_matrix* mats, int count, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Gram matrix of calibration activations for the PTQ initialisation: H = X^T X
 * (decoupleQ, section 3.1: H = X^T X of the layer input over a small calibration set).
 *   X  bfloat16 [M, K], 1 <= M <= 2^24 - 2^17, K a multiple of 64 up to 16384
 *   H  float [K, K]                                                    out, overwritten
 * Products of bf16 values are exact; sums are float32 on the matrix cores. H is exactly
 * symmetric (each off-diagonal pair is written from one sum).
 * Errors: LCVQ_ERR_NULL, LCVQ_ERR_SHAPE, LCVQ_ERR_ALIGN, LCVQ_ERR_HIP.
 */
lcvq_status_t lcvq_hessian(const void* X, int64_t M, int64_t K, float* H, void* stream);

/*
 * PTQ initialisation of one matrix with a per-tensor code, A = s I and B = b 1 (the
 * starting point LC-QAT takes from post-training quantization: LC-QAT summary,
 * Methodology 2; the problem and its alternating solver: decoupleQ, sections 3.1-3.3,
 * eq. (5)-(11), with decoupleQ's integers {-2..1} as codes {0..3}, z = b + 2 s).
 * It minimises
 *   g(c; s, b) = 1/2 sum_n (s c_n + b 1 - w0_n)^T Hd (s c_n + b 1 - w0_n)
 * over codes c in {0..3}^[N, K] and floats s, b, with Hd = H + damp * mean(diag H) I.
 * Start: s = (max W0 - min W0) / 3, b = min W0. Then `iters` times:
 *  1. integer step at the current (s, b): for every row, element by element in index
 *     order, round half to even and clip to {0..3} the element's value, then re-solve the
 *     later elements of the row without constraints (decoupleQ eq. (11)); computed as
 *     t_k = (q_k - b e_k) / s - sum_{i<k} U_ik c_i with Hd = U D U^T (U unit upper), q =
 *     U^T w0, e = U^T 1. These codes replace the current ones unless they raise g at this
 *     (s, b) (on the first iteration they always do);
 *  2. (s, b) step: the least-squares (s, b) of the current codes (eq. (7) set to zero);
 *     kept unchanged if that system is singular or gives s = 0.
 * The objective therefore never increases.
 *   H          float [K, K], symmetric (lcvq_hessian's output)                       in
 *   W0         float [N, K], the weight to initialise (N outputs, K inputs)          in
 *   N          a multiple of 16 up to 2^20;  K a multiple of 64 up to 16384
 *   damp       0 < damp <= 1 (LCVQ_ERR_VALUE otherwise);  iters in 1..64
 *   packed_out uint8 [N, K/4], the codes in the canonical packed layout              out
 *   sb_out     float [2]: s, b (both NaN if Hd's factorisation met a pivot <= 0)     out
 *   obj_out    float [2 * iters] or NULL: g after each step                          out
 *   U_out      float [K, K] or NULL: U (unit upper triangular), row-major            out
 *   D_out      float [K] or NULL: D                                                  out
 *   workspace  >= lcvq_ptq_workspace_size(N, K) bytes (0 for invalid shapes)
 * Numerics: float32 factorisation and sums (double for the workgroup and final sums);
 * the sweep's sums over earlier codes run on the bf16 matrix cores with U split into bf16
 * hi + lo halves (about 16 significant bits) and the codes exact. A code decided from a
 * value within a few 1e-5 of a half-integer may differ from a float64 computation.
 */
size_t lcvq_ptq_workspace_size(int64_t N, int64_t K);
lcvq_status_t lcvq_ptq_init(const float* H, const float* W0, int64_t N, int64_t K, float damp,
                            int iters, uint8_t* packed_out, float* sb_out, float* obj_out,
                            float* U_out, float* D_out, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * Measurement helper, no step of the method: one launch that reads `bytes` of device
 * memory once (16-byte non-temporal loads, as the decode kernels read codes) and writes
 * one word per workgroup into `sink` (uint32 [1024], device). Timed with the profiling
 * hook (kernel id 9), it is the same-size read ceiling the decode product is compared to.
 *   bytes a multiple of 16, 16 <= bytes <= 2^40; buf and sink 16-byte aligned.
 * Errors: LCVQ_ERR_NULL, LCVQ_ERR_SHAPE, LCVQ_ERR_ALIGN, LCVQ_ERR_HIP.
 */
lcvq_status_t lcvq_read_probe(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

/*
 * Measurement helper, no step of the method: the matrix-core issue ceiling the products are
 * compared to. One launch of 256 workgroups of 8 waves (2 per SIMD, as the products run);
 * each wave issues `iters` rounds of 8 independent 32x32x16 bf16 MFMAs (the products' 4 x 2
 * accumulator blocks) on pseudo-random operands in [-1, -0.5] U [0.5, 1) that alternate
 * between two sets every round, so that operand bits toggle as when data streams through.
 * It performs iters * 2^29 floating-point operations and writes one word per workgroup into
 * `sink` (uint32 [1024], device). Timed with the profiling hook (kernel id 10).
 *   iters even, 2 <= iters <= 2^24; sink 16-byte aligned.
 * Errors: LCVQ_ERR_NULL, LCVQ_ERR_SHAPE, LCVQ_ERR_ALIGN, LCVQ_ERR_HIP.
 */
lcvq_status_t lcvq_mfma_probe(int64_t iters, uint32_t* sink, void* stream);

/*
 * Profiling hook (changes no result). Arms a one-shot timing of the next launch of one
 * kernel by calls made from this host thread: the kernel is launched with
 * hipExtLaunchKernel between `start_event` and `stop_event` (hipEvent_t handles created
 * by the caller with timing enabled); a product split into several launches (few-tile
 * forward and dW, a dW whose last round of tiles is split, the decode product's two-launch
 * path) gets the events recorded on the stream around all of them. kernel_id: 1 quantizer, 2 forward product,
 * 3 dX product, 4 dW product (with the straight-through epilogue), 5 decode product (where
 * it takes two launches, the X' prologue and the product, the events bracket both),
 * 6 backward prologue (r = dY 1 and the transposed codes, lcvq_linear_bwd), 7 Gram
 * product (lcvq_hessian), 8 PTQ integer step (lcvq_ptq_init; each call times the first),
 * 9 read probe (lcvq_read_probe), 10 MFMA probe (lcvq_mfma_probe), 11 packer
 * (lcvq_pack2b), 12 unpacker (lcvq_unpack2b).
 * Passing NULL events disarms. Returns LCVQ_ERR_SHAPE for an unknown kernel_id.
 */
lcvq_status_t lcvq_profile_next(int kernel_id, void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif
#endif /* LCVQ_H */
