// PTQ initialisation of a per-tensor LC code (A = s I, B = b 1) on gfx950.
//
// LC-QAT starts training from a post-training quantization found by column-wise rounding
// with sequential error compensation ("LC-QAT: Data-Efficient 2-Bit QAT for LLMs via
// Linear-Constrained Vector Quantization", technical summary, Methodology 2). decoupleQ
// (sections 3.1-3.3) states the layer problem and its solver: minimise
//   g(c; s, b) = 1/2 sum_n (s c_n + b 1 - w0_n)^T H (s c_n + b 1 - w0_n),  H = X^T X,
// over codes c_n in {0..3}^K (decoupleQ's {-2..1} shifted by 2) and floats (s, b), by
// alternating a closed-form (s, b) step (eq. (7) differentiated) and an integer step that
// rounds and clips element k, then re-solves the later elements without constraints
// (eq. (11)). With H damped (H + delta I, delta = damp * mean diag H) and factored as
// H = U D U^T (U unit upper triangular), eq. (11)'s minimiser gives element k the value
//   t_k = (q_k - b e_k) / s - sum_{i<k} U_ik c_i,   q = U^T w0,  e = U^T 1,
// so the integer step is one triangular sweep per row, and with a = U^T c the sums of the
// (s, b) normal equations are sum D a^2, sum D a e, sum D a q, N sum D e^2, sum D e q, and
// the objective of the sweep's codes at the (s, b) it used is s^2 / 2 sum D (t - c)^2.
//
// Kernels, in launch order:
//   k_ptq_delta     delta from the diagonal of H; state reset
//   k_ptq_reverse   A' = J (H + delta I) J, J the index reversal (lower triangle)
//   k_chol_diag / k_chol_panel / k_chol_update   blocked lower Cholesky A' = L L^T,
//                   64 columns per step (U D U^T of H in reversed index order)
//   k_ptq_udu_out   U, D from L; U^T as bf16 hi + lo, U's 64 x 64 diagonal blocks in fp32
//   k_ptq_rowsum_e  e = U^T 1
//   k_ptq_q         Q = W0 U (fp32), with per-tile sums of D e q, D q^2 and min / max of W0
//   k_ptq_start     the initial (s, b) from the weight's range; the constant sums
//   per iteration:  k_ptq_sweep (codes of 16 rows per workgroup, sums) and k_ptq_solve
//   k_ptq_final     packed codes, s, b out
#include <math.h>

#include <algorithm>

#include "lcvq_device.h"
#include "lcvq_internal.h"

namespace lcvq {

constexpr int PB = 64;            // factorisation and sweep column block
constexpr int SWR = 16;           // rows of W0 per sweep workgroup
constexpr int PTQ_MAX_K = 16384;
constexpr int PTQ_MAX_ITERS = 64;

struct PtqState {
  double s, b, g;                 // current (s, b) and the objective of the current codes
  double S1, S2, T1;              // sums of the current codes
  double S3, T2, W;               // sums that do not depend on the codes
  float delta;
  int cur;                        // which code buffer holds the current codes
  int bad;                        // a pivot of the factorisation was not positive
  int pad;
};

// ------------------------------------------------------------------ damping, reversal
__global__ __launch_bounds__(256) void k_ptq_delta(const float* __restrict__ H, int K, float damp,
                                                   PtqState* st) {
  __shared__ double red[256];
  double sum = 0.0;
  for (int i = threadIdx.x; i < K; i += 256) sum += (double)H[(int64_t)i * K + i];
  red[threadIdx.x] = sum;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    st->delta = (float)(damp * red[0] / K);
    st->bad = 0;
    st->cur = 0;
  }
}

// Row i' of A' = J (H + delta I) J: A'[i'][j'] = H[K-1-i'][K-1-j'] (+ delta), j' <= i'.
__global__ __launch_bounds__(256) void k_ptq_reverse(const float* __restrict__ H, int K,
                                                     const PtqState* st, float* __restrict__ A) {
  const int ip = blockIdx.x;
  const float* src = H + (int64_t)(K - 1 - ip) * K;
  float* dst = A + (int64_t)ip * K;
  const float delta = st->delta;
  for (int jp = threadIdx.x; jp <= ip; jp += 256) {
    float v = src[K - 1 - jp];
    if (jp == ip) v += delta;
    dst[jp] = v;
  }
}

// ------------------------------------------------------------------ blocked Cholesky
// Step j0: the diagonal block (already updated by the earlier steps) is factored by one
// wave, row t of the block in lane t's registers. For column c the pivot is lane c's entry
// c; the column is scaled (lanes t < c hold 0 there), and every later entry k > c of the
// row subtracts the row's entry c times lane k's scaled entry c, broadcast with readlane
// in groups of eight (so that few broadcast values are live at once). Entries above the
// diagonal (k > t) take the same updates unmasked: no lane reads them before step c = k
// sets them to 0, and they are written back as 0. A pivot that is not positive is
// recorded in the state and replaced by 1 so that the rest stays finite; the outputs are
// then flagged.
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
// Thread t < 64 (one wave) holds row j0 + t of the block.
// colbuf: 64 floats of LDS, 16-byte aligned, through which each column of L reaches the
// wave (the lanes read it back as broadcast 16-byte reads).
__device__ __forceinline__ void chol_diag_body(float* __restrict__ A, int K, int j0,
                                               PtqState* st, int t, float* colbuf) {
  float* row = A + (int64_t)(j0 + t) * K + j0;
  float x[PB];
#pragma unroll
  for (int v = 0; v < PB / 4; ++v) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(row + 4 * v);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * v + e] = 4 * v + e <= t ? a[e] : 0.f;   // lower part
  }
  bool bad = false;
#pragma unroll
  for (int c = 0; c < PB; ++c) {
    const float piv = lane_value(x[c], c);
    bad |= !(piv > 0.f);
    const float d = piv > 0.f ? sqrtf(piv) : 1.f;
    const float sc = x[c] / d;
    x[c] = t == c ? d : (t > c ? sc : 0.f);
    // Column c of L (lane k holds L[k][c]) to all lanes: written to LDS once and read back
    // as broadcast 16-byte reads. The wave's LDS operations complete in order, so the
    // reads see this column, and the next column's write follows them.
    colbuf[t] = x[c];
    // The next pivot's column first, with its one entry of column c taken straight from
    // lane c + 1: the next column's square root and division then need not wait for the
    // LDS round trip, and run under this column's other updates (the same multiply-add
    // as through LDS).
    if (c + 1 < PB) x[c + 1] = __builtin_fmaf(-x[c], lane_value(x[c], c + 1), x[c + 1]);
    __builtin_amdgcn_sched_barrier(0);
    constexpr int Q = PB / 4;
    f32x4 l[Q];
#pragma unroll
    for (int q = (c + 2) >> 2; q < Q; ++q) l[q] = *reinterpret_cast<const f32x4*>(colbuf + 4 * q);
    __builtin_amdgcn_sched_barrier(0);           // all of the column's reads in flight first
#pragma unroll
    for (int q = (c + 2) >> 2; q < Q; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * q + e > c + 1) x[4 * q + e] = __builtin_fmaf(-x[c], l[q][e], x[4 * q + e]);
    // Materialise the row after each column: otherwise the compiler sinks every update
    // of an entry to where the entry is next used, which keeps all earlier broadcasts
    // live (in SGPRs, spilled).
#pragma unroll
    for (int k = c + 1; k < PB; ++k) asm volatile("" : "+v"(x[k]));
  }
  // the upper part of the block (never read by the later steps) is written as zeros
#pragma unroll
  for (int v = 0; v < PB / 4; ++v) {
    f32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = 4 * v + e <= t ? x[4 * v + e] : 0.f;
    *reinterpret_cast<f32x4*>(row + 4 * v) = o;
  }
  if (bad && t == 0) st->bad = 1;
}
__global__ __launch_bounds__(PB) void k_chol_diag(float* __restrict__ A, int K, int j0,
                                                  PtqState* st) {
  __shared__ __attribute__((aligned(16))) float colbuf[PB];
  chol_diag_body(A, K, j0, st, threadIdx.x, colbuf);
}

// Rows i >= j0 + 64 of the panel: x L11^T = a, forward substitution with the factored
// diagonal block L11 (from LDS). One row per wave, lane c holding column c: column u is
// solved by lane u and broadcast to the wave (readlane), and every lane then subtracts its
// term x_u L11[c][u]. Each column's sum takes its terms in the order u = 0, 1, ... and
// ends with the same division, exactly as a sequential solve of the row; the chain of one
// row is 64 steps of a division, a broadcast and a multiply-add.
constexpr int PANEL_ROWS = 16;                   // rows (waves) per workgroup
__global__ __launch_bounds__(PANEL_ROWS * 64) void k_chol_panel(float* __restrict__ A, int K,
                                                                int j0) {
  __shared__ float L[PB][PB + 1];
  const int t = threadIdx.x;
  for (int x = t; x < PB * PB; x += PANEL_ROWS * 64) {
    const int i = x / PB, k = x % PB;
    L[i][k] = k <= i ? A[(int64_t)(j0 + i) * K + j0 + k] : 0.f;
  }
  __syncthreads();
  const int lane = t & 63;
  const int i = j0 + PB + blockIdx.x * PANEL_ROWS + (t >> 6);
  if (i >= K) return;                            // uniform within the wave
  float* row = A + (int64_t)i * K + j0;
  float v = row[lane];
  float Lr[PB];                                  // this lane's row of L11 (zeros above it)
#pragma unroll
  for (int u = 0; u < PB; ++u) Lr[u] = L[lane][u];
  const float dg = L[lane][lane];
  float res = 0.f;
#pragma unroll
  for (int u = 0; u < PB; ++u) {
    const float xa = v / dg;                     // final in lane u: x_u
    const float xu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, xa), u));
    res = lane == u ? xu : res;
    v -= xu * Lr[u];                             // lanes c > u: their next term
  }
  row[lane] = res;
}

// Trailing update A[i][k] -= sum_c L[i][j0+c] L[k][j0+c] for j0 + 64 <= k <= i, on
// 64 x 64 tiles of the lower triangle; each thread updates a 4 x 4 patch. Workgroup 0
// updates tile (0, 0), the next step's diagonal block, and then factors it (its first
// wave, after a barrier): the look-ahead that keeps the serial factor of step s + 1 off the
// critical path while the other workgroups finish step s's update.
__global__ __launch_bounds__(256) void k_chol_update(float* __restrict__ A, int K, int j0,
                                                     PtqState* st) {
  __shared__ float Li[PB][PB + 4];
  __shared__ float Lk[PB][PB + 4];
  __shared__ __attribute__((aligned(16))) float colbuf[PB];
  const int j1 = j0 + PB;
  int t = blockIdx.x, ti = 0;                     // lower tile t -> (ti, tk), tk <= ti
  while (t > ti) {
    t -= ti + 1;
    ++ti;
  }
  const int tk = t;
  const int i0 = j1 + ti * PB, k0 = j1 + tk * PB;
  const int tid = threadIdx.x;
  for (int x = tid; x < PB * PB / 4; x += 256) {
    const int r = x / (PB / 4), c4 = (x % (PB / 4)) * 4;
    const f32x4 a = *reinterpret_cast<const f32x4*>(A + (int64_t)(i0 + r) * K + j0 + c4);
    const f32x4 b = *reinterpret_cast<const f32x4*>(A + (int64_t)(k0 + r) * K + j0 + c4);
    Li[r][c4] = a[0]; Li[r][c4 + 1] = a[1]; Li[r][c4 + 2] = a[2]; Li[r][c4 + 3] = a[3];
    Lk[r][c4] = b[0]; Lk[r][c4 + 1] = b[1]; Lk[r][c4 + 2] = b[2]; Lk[r][c4 + 3] = b[3];
  }
  __syncthreads();
  const int ri = (tid / 16) * 4, rk = (tid % 16) * 4;
  float acc[4][4] = {};
#pragma unroll 8
  for (int c = 0; c < PB; ++c) {
    float a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) { a[u] = Li[ri + u][c]; b[u] = Lk[rk + u][c]; }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[u][v] += a[u] * b[v];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = i0 + ri + u, k = k0 + rk + v;
      if (k <= i) A[(int64_t)i * K + k] -= acc[u][v];
    }
  if (blockIdx.x == 0) {                          // uniform per workgroup
    __syncthreads();                              // the tile's updated entries
    if (tid < PB) chol_diag_body(A, K, j1, st, tid, colbuf);
  }
}

// ------------------------------------------------------------------ U, D from L
// In reversed indices A' = L L^T; with i = K-1-i', U_ij = L[K-1-i][K-1-j] / L[K-1-j][K-1-j]
// for i <= j and D_j = L[K-1-j][K-1-j]^2. Tile (jb, ib) of U^T (rows j, columns i) goes
// through LDS so that both the reads of L and the writes of U^T are row runs.
__global__ __launch_bounds__(256) void k_ptq_udu_out(const float* __restrict__ L, int K,
                                                    float* __restrict__ Ut32,
                                                    uint16_t* __restrict__ Ut_hi,
                                                    uint16_t* __restrict__ Ut_lo,
                                                    float* __restrict__ Udiag,
                                                    float* __restrict__ D,
                                                    float* __restrict__ U_out,
                                                    float* __restrict__ D_out) {
  __shared__ float T[PB][PB + 1];
  __shared__ float dg[PB];
  const int jb = blockIdx.x, ib = blockIdx.y;    // Ut rows j in jb, columns i in ib
  const int tid = threadIdx.x;
  if (tid < PB) {
    const int jp = K - 1 - (jb * PB + tid);
    dg[tid] = L[(int64_t)jp * K + jp];
  }
  // T[j][i] = L[K-1-i][K-1-j] for i <= j: read rows i' = K-1-i of L, columns j' = K-1-j.
  for (int x = tid; x < PB * PB; x += 256) {
    const int il = x / PB, jl = x % PB;          // consecutive threads: consecutive j
    const int i = ib * PB + il, j = jb * PB + jl;
    T[jl][il] = i <= j ? L[(int64_t)(K - 1 - i) * K + (K - 1 - j)] : 0.f;
  }
  __syncthreads();
  for (int x = tid; x < PB * PB; x += 256) {
    const int jl = x / PB, il = x % PB;          // consecutive threads: consecutive i
    const int i = ib * PB + il, j = jb * PB + jl;
    const float u = i < j ? T[jl][il] / dg[jl] : (i == j ? 1.f : 0.f);
    const int64_t o = (int64_t)j * K + i;
    Ut32[o] = u;
    const __bf16 hi = (__bf16)u;
    const __bf16 lo = (__bf16)(u - (float)hi);
    Ut_hi[o] = __builtin_bit_cast(uint16_t, hi);
    Ut_lo[o] = __builtin_bit_cast(uint16_t, lo);
    if (ib == jb) Udiag[((int64_t)jb * PB + il) * PB + jl] = u;   // [block][i][j]
    if (U_out) U_out[(int64_t)i * K + j] = u;
  }
  if (ib == jb && tid < PB) {
    const float d = dg[tid] * dg[tid];
    D[jb * PB + tid] = d;
    if (D_out) D_out[jb * PB + tid] = d;
  }
}

// e_j = sum_{i <= j} U_ij: one workgroup per row j of U^T.
__global__ __launch_bounds__(256) void k_ptq_rowsum_e(const float* __restrict__ Ut32, int K,
                                                      float* __restrict__ e) {
  __shared__ float red[256];
  const int j = blockIdx.x;
  float s = 0.f;
  for (int i = threadIdx.x; i <= j; i += 256) s += Ut32[(int64_t)j * K + i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) e[j] = red[0];
}

// ------------------------------------------------------------------ Q = W0 U
// Q[n][j] = sum_{i <= j} W0[n][i] U_ij = sum_i W0[n][i] Ut[j][i], on 64 x 64 tiles
// (rows n, columns j), contraction staged 16 at a time in LDS; each thread a 4 x 4 patch.
// Each workgroup also adds sum D_j e_j Q[n][j] and sum D_j Q[n][j]^2 over its tile (in
// fixed order) and the min / max of its W0 rows, for the start of the alternation.
constexpr int QT = 64, QC = 16;
__global__ __launch_bounds__(256) void k_ptq_q(const float* __restrict__ W0,
                                               const float* __restrict__ Ut32,
                                               const float* __restrict__ D,
                                               const float* __restrict__ e, int N, int K,
                                               float* __restrict__ Q,
                                               double* __restrict__ part) {
  __shared__ float Aw[QC][QT + 4];                // [c][n]
  __shared__ float Bu[QC][QT + 4];                // [c][j]
  __shared__ double red[256][4];
  const int jb = blockIdx.x, nb = blockIdx.y;
  const int tid = threadIdx.x;
  const int rn = (tid / 16) * 4, rj = (tid % 16) * 4;
  float acc[4][4] = {};
  const int iend = (jb + 1) * QT;                 // U_ij = 0 for i > j
  for (int i0 = 0; i0 < iend; i0 += QC) {
    // 64 rows x 16 columns of each operand: thread -> (row tid / 4, 4 columns)
    {
      const int r = tid / 4, c4 = (tid % 4) * 4;
      const int nr = min(nb * QT + r, N - 1);     // rows past N: a valid row, not stored
      const f32x4 a = *reinterpret_cast<const f32x4*>(W0 + (int64_t)nr * K + i0 + c4);
      const f32x4 b = *reinterpret_cast<const f32x4*>(Ut32 + (int64_t)(jb * QT + r) * K + i0 + c4);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        Aw[c4 + u][r] = a[u];
        Bu[c4 + u][r] = b[u];
      }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < QC; ++c) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&Aw[c][rn]);
      const f32x4 b = *reinterpret_cast<const f32x4*>(&Bu[c][rj]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] += a[u] * b[v];
    }
    __syncthreads();
  }
  double seq = 0.0, sqq = 0.0;
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int n = nb * QT + rn + u;
    if (n >= N) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = jb * QT + rj + v;
      const float q = acc[u][v];
      Q[(int64_t)n * K + j] = q;
      seq += (double)D[j] * e[j] * q;
      sqq += (double)D[j] * q * q;
      const float w = W0[(int64_t)n * K + j];
      mn = fminf(mn, w);
      mx = fmaxf(mx, w);
    }
  }
  red[tid][0] = seq;
  red[tid][1] = sqq;
  red[tid][2] = mn;
  red[tid][3] = mx;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (tid < w) {
      red[tid][0] += red[tid + w][0];
      red[tid][1] += red[tid + w][1];
      red[tid][2] = fmin(red[tid][2], red[tid + w][2]);
      red[tid][3] = fmax(red[tid][3], red[tid + w][3]);
    }
    __syncthreads();
  }
  if (tid < 4) part[((int64_t)nb * gridDim.x + jb) * 4 + tid] = red[0][tid];
}

// The initial (s, b) = ((max - min) / 3, min) of W0 (s = 1 for a constant matrix) and the
// code-independent sums S3 = N sum D e^2, T2 = sum D e q, W = sum D q^2.
__global__ __launch_bounds__(256) void k_ptq_start(const double* __restrict__ part, int nparts,
                                                   const float* __restrict__ D,
                                                   const float* __restrict__ e, int N, int K,
                                                   PtqState* st) {
  __shared__ double red[256][5];
  const int tid = threadIdx.x;
  double t2 = 0.0, w = 0.0, mn = INFINITY, mx = -INFINITY, s3 = 0.0;
  for (int p = tid; p < nparts; p += 256) {
    t2 += part[p * 4 + 0];
    w += part[p * 4 + 1];
    mn = fmin(mn, part[p * 4 + 2]);
    mx = fmax(mx, part[p * 4 + 3]);
  }
  for (int j = tid; j < K; j += 256) s3 += (double)D[j] * e[j] * e[j];
  red[tid][0] = t2; red[tid][1] = w; red[tid][2] = mn; red[tid][3] = mx; red[tid][4] = s3;
  __syncthreads();
  for (int k = 128; k >= 1; k >>= 1) {
    if (tid < k) {
      red[tid][0] += red[tid + k][0];
      red[tid][1] += red[tid + k][1];
      red[tid][2] = fmin(red[tid][2], red[tid + k][2]);
      red[tid][3] = fmax(red[tid][3], red[tid + k][3]);
      red[tid][4] += red[tid + k][4];
    }
    __syncthreads();
  }
  if (tid == 0) {
    st->T2 = red[0][0];
    st->W = red[0][1];
    st->S3 = (double)N * red[0][4];
    const double lo = red[0][2], hi = red[0][3];
    st->s = hi > lo ? (hi - lo) / 3.0 : 1.0;
    st->b = lo;
    st->g = INFINITY;
    st->S1 = st->S2 = st->T1 = 0.0;
  }
}

// ------------------------------------------------------------------ the integer step
// One workgroup sweeps 16 rows of W0 over K, 64 columns at a time. For a column block:
//  1. its feedback from all earlier codes, F[r][j] = sum_{i < j0} c_ri U_ij, on the bf16
//     matrix cores: codes (exact) times U^T's hi and lo halves (summed in two float32
//     accumulators, added at the end); a feedback wave covers 16 of the block's columns;
//  2. the walk over the block's columns in order, 4 lanes per row, each lane holding 16
//     columns' running value t = (q - b e) / s - F - (feedback inside the block): the
//     owner of column k broadcasts t_k, every lane rounds it the same way
//     (c = clip(rint(t), 0, 3)), and the four lanes update their later columns with
//     U's diagonal block (fp32, LDS). The owner accumulates the sums of a = U^T c.
// The walk of block b (wave 0) runs while waves 1-3 form block b + 1's feedback from the
// blocks before b (wave 1 two of the four 16-column tiles, waves 2 and 3 one each); after
// a barrier they add block b's own codes (two steps) and write it.
// F and the diagonal block are double-buffered. The feedback steps run in ascending order
// either way, so F is the same as one pass over i < j0 would give.
// The codes of the workgroup's rows stay in LDS (2 bits each) for the later blocks'
// feedback, and go out packed (canonical layout) at the end.
__device__ __forceinline__ bf16x8 codes8_bf16(uint32_t two_bytes) {
  // 8 codes (2 bits each, little-endian) -> 8 bf16 values 0, 1, 2, 3 (exact), two per
  // dword by a byte-table lookup (v_perm_b32): the low bytes of bf16 0, 1, 2, 3 are
  // 00 80 00 40 (table LO, byte c) and the high bytes 00 3F 40 40 (table HI, byte 4 + c).
  constexpr uint32_t LO = 0x40008000u, HI = 0x40403F00u;
  u32x4 o;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t c0 = (two_bytes >> (4 * p)) & 3u, c1 = (two_bytes >> (4 * p + 2)) & 3u;
    const uint32_t sel = (c0 | (c1 << 16)) * 0x0101u + 0x04000400u;   // c0, 4+c0, c1, 4+c1
    o[p] = __builtin_amdgcn_perm(HI, LO, sel);
  }
  return __builtin_bit_cast(bf16x8, o);
}

constexpr int SW_WAVES = 4;                 // wave 0 walks, waves 1-3 form the feedback
__global__ __launch_bounds__(SW_WAVES * 64) void k_ptq_sweep(const float* __restrict__ Q,
                                                   const float* __restrict__ e,
                                                   const float* __restrict__ D,
                                                   const uint16_t* __restrict__ Ut_hi,
                                                   const uint16_t* __restrict__ Ut_lo,
                                                   const float* __restrict__ Udiag, int N,
                                                   int K, uint8_t* __restrict__ codes0,
                                                   uint8_t* __restrict__ codes1,
                                                   double* __restrict__ part,
                                                   const PtqState* __restrict__ st) {
  __shared__ __attribute__((aligned(16))) uint8_t cl[SWR * (PTQ_MAX_K / 4)];   // 64 KiB
  __shared__ float F[2][SWR][PB + 4];
  __shared__ __attribute__((aligned(16))) float Ub[2][PB][PB];
  __shared__ double red[64][4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * SWR;
  const int KB = K / 4;                            // packed bytes per row
  const float s = (float)st->s, b = (float)st->b;
  const float inv_s = 1.f / s;
  uint8_t* out = st->cur ? codes0 : codes1;        // the candidate buffer
  // walk lanes (wave 0): row r = lane / 4, columns 16 sub .. 16 sub + 15 of each block
  const int r = lane >> 2, sub = lane & 3;
  // feedback waves: tiles ft0 (and 3 for wave 1) of 16 columns of the block
  const int ft0 = wave - 1;
  float sG = 0.f, sS1 = 0.f, sS2 = 0.f, sT1 = 0.f;
  const int nb = K / PB;

  // Feedback of the codes i in [ia, ib) on columns j1 + 16 ft .. + 15, accumulated in
  // order into acc (U^T hi) and accl (U^T lo). Steps of 32 rows in groups of FG: all of a
  // group's loads are issued before its matrix-core products.
  auto feedback = [&](int ft, int j1, int ia, int ib, f32x4& acc, f32x4& accl) {
    const int jc = j1 + 16 * ft + (lane & 15);                   // B column of this lane
    const uint16_t* bh = Ut_hi + (int64_t)jc * K + 8 * (lane >> 4);
    const uint16_t* bl = Ut_lo + (int64_t)jc * K + 8 * (lane >> 4);
    const uint8_t* ca = cl + (lane & 15) * KB + 2 * (lane >> 4);
    constexpr int FG = 8;
    int i0 = ia;
    for (; i0 + 32 * FG <= ib; i0 += 32 * FG) {
      bf16x8 h[FG], l[FG];
      uint32_t cw[FG];
#pragma unroll
      for (int u = 0; u < FG; ++u) {
        h[u] = *reinterpret_cast<const bf16x8*>(bh + i0 + 32 * u);
        l[u] = *reinterpret_cast<const bf16x8*>(bl + i0 + 32 * u);
        cw[u] = *reinterpret_cast<const uint16_t*>(ca + (i0 + 32 * u) / 4);
      }
#pragma unroll
      for (int u = 0; u < FG; ++u) {
        const bf16x8 a = codes8_bf16(cw[u]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, h[u], acc, 0, 0, 0);
        accl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, l[u], accl, 0, 0, 0);
      }
    }
    for (; i0 < ib; i0 += 64) {                                  // ia, ib multiples of 64
      bf16x8 h[2], l[2];
      uint32_t cw[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        h[u] = *reinterpret_cast<const bf16x8*>(bh + i0 + 32 * u);
        l[u] = *reinterpret_cast<const bf16x8*>(bl + i0 + 32 * u);
        cw[u] = *reinterpret_cast<const uint16_t*>(ca + (i0 + 32 * u) / 4);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 a = codes8_bf16(cw[u]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, h[u], acc, 0, 0, 0);
        accl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, l[u], accl, 0, 0, 0);
      }
    }
  };
  auto load_diag = [&](int blk, int buf) {                       // waves 1-3
    const float* ud = Udiag + (int64_t)blk * PB * PB;
    for (int x = tid - 64; x < PB * PB / 4; x += (SW_WAVES - 1) * 64)
      reinterpret_cast<f32x4*>(&Ub[buf][0][0])[x] = reinterpret_cast<const f32x4*>(ud)[x];
  };

  // block 0: no earlier codes
  if (wave > 0) {
    for (int x = tid - 64; x < SWR * (PB + 4); x += (SW_WAVES - 1) * 64) (&F[0][0][0])[x] = 0.f;
    load_diag(0, 0);
  }
  __syncthreads();
  for (int blk = 0; blk < nb; ++blk) {
    const int j0 = blk * PB, cur = blk & 1;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, accl = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc3 = {0.f, 0.f, 0.f, 0.f}, accl3 = {0.f, 0.f, 0.f, 0.f};   // wave 1: tile 3
    if (wave == 0) {
      // the ordered walk over this block's columns
      const int n = n0 + r;
      const int jl0 = 16 * sub;
      float t[16], qv[16], ev[16], dv[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int j = j0 + jl0 + u;
        qv[u] = Q[(int64_t)n * K + j];
        ev[u] = e[j];
        dv[u] = D[j];
        t[u] = (qv[u] - b * ev[u]) * inv_s - F[cur][r][jl0 + u];
      }
      uint32_t packed = 0;                         // this lane's 16 codes, 2 bits each
#pragma unroll
      for (int k = 0; k < PB; ++k) {
        const int owner = k >> 4, uk = k & 15;
        const float tk = __shfl(t[uk], (lane & ~3) | owner);
        const float rr = __builtin_rintf(tk);
        const float c = fminf(fmaxf(rr, 0.f), 3.f);
        if (sub == owner) {
          // a_k = c_k + sum_{i<k} U_ik c_i = c_k + (q_k - b e_k) / s - t_k
          const float a = c + ((qv[uk] - b * ev[uk]) * inv_s - tk);
          const float d = dv[uk];
          sG += d * (tk - c) * (tk - c);
          sS1 += d * a * a;
          sS2 += d * a * ev[uk];
          sT1 += d * a * qv[uk];
          packed |= (uint32_t)c << (2 * uk);
        }
        // later columns of this lane: t_j -= U_kj c. U_kj is 0 for j < k and 1 for
        // j = k, whose values have been used already, so no column test is needed.
#pragma unroll
        for (int u = 0; u < 16; ++u) t[u] -= Ub[cur][k][jl0 + u] * c;
      }
      *reinterpret_cast<uint32_t*>(cl + r * KB + (j0 + jl0) / 4) = packed;
    } else if (blk + 1 < nb) {
      // the next block's feedback from the blocks before this one, and its diagonal block
      feedback(ft0, j0 + PB, 0, j0, acc, accl);
      if (wave == 1) feedback(3, j0 + PB, 0, j0, acc3, accl3);
      load_diag(blk + 1, cur ^ 1);
    }
    __syncthreads();
    if (wave > 0 && blk + 1 < nb) {
      // this block's codes (written by the walk) on the next block's columns
      feedback(ft0, j0 + PB, j0, j0 + PB, acc, accl);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] += accl[v];
      // D layout: lane l holds rows 4 (l / 16) + v, column l % 16
#pragma unroll
      for (int v = 0; v < 4; ++v) F[cur ^ 1][4 * (lane >> 4) + v][16 * ft0 + (lane & 15)] = acc[v];
      if (wave == 1) {
        feedback(3, j0 + PB, j0, j0 + PB, acc3, accl3);
#pragma unroll
        for (int v = 0; v < 4; ++v) F[cur ^ 1][4 * (lane >> 4) + v][48 + (lane & 15)] = acc3[v] + accl3[v];
      }
    }
    __syncthreads();
  }
  // 3. the codes out (canonical packed rows), and this workgroup's sums
  for (int x = tid; x < SWR * KB / 16; x += SW_WAVES * 64) {
    const int rr = x / (KB / 16), c16 = (x % (KB / 16)) * 16;
    *reinterpret_cast<uint4*>(out + (int64_t)(n0 + rr) * KB + c16) =
        *reinterpret_cast<const uint4*>(cl + rr * KB + c16);
  }
  if (wave == 0) {
    red[lane][0] = sG; red[lane][1] = sS1; red[lane][2] = sS2; red[lane][3] = sT1;
  }
  __syncthreads();
  if (tid < 4) {
    double sum = 0.0;
    for (int l = 0; l < 64; ++l) sum += red[l][tid];
    part[(int64_t)blockIdx.x * 4 + tid] = sum;
  }
}

// ------------------------------------------------------------------ the (s, b) step
// Adds the sweep workgroups' sums in a fixed order. The sweep's codes become the current
// ones if they do not raise the objective at the (s, b) they were computed with (always
// on the first iteration); then (s, b) solves the normal equations of the current codes
// unless they are singular or give s = 0. obj[2 it] and obj[2 it + 1] receive the
// objective after each of the two steps.
__global__ __launch_bounds__(256) void k_ptq_solve(const double* __restrict__ part, int nparts,
                                                   int it, PtqState* st, float* __restrict__ obj) {
  __shared__ double red[256][4];
  const int tid = threadIdx.x;
  double a[4] = {0.0, 0.0, 0.0, 0.0};
  for (int p = tid; p < nparts; p += 256)
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] += part[p * 4 + k];
#pragma unroll
  for (int k = 0; k < 4; ++k) red[tid][k] = a[k];
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (tid < w)
#pragma unroll
      for (int k = 0; k < 4; ++k) red[tid][k] += red[tid + w][k];
    __syncthreads();
  }
  if (tid != 0) return;
  const double s = st->s;
  const double g_new = 0.5 * s * s * red[0][0];
  if (it == 0 || g_new <= st->g) {
    st->cur ^= 1;
    st->S1 = red[0][1];
    st->S2 = red[0][2];
    st->T1 = red[0][3];
    st->g = g_new;
  }
  if (obj) obj[2 * it] = (float)st->g;
  const double S1 = st->S1, S2 = st->S2, S3 = st->S3, T1 = st->T1, T2 = st->T2;
  const double det = S1 * S3 - S2 * S2;
  if (fabs(det) > 1e-12 * fabs(S1 * S3) && isfinite(det)) {
    const double sn = (T1 * S3 - S2 * T2) / det;
    const double bn = (S1 * T2 - S2 * T1) / det;
    if (sn != 0.0 && isfinite(sn) && isfinite(bn)) {
      st->s = sn;
      st->b = bn;
    }
  }
  const double sv = st->s, bv = st->b;
  st->g = 0.5 * (sv * sv * S1 + 2.0 * sv * bv * S2 - 2.0 * sv * T1 + bv * bv * S3 -
                 2.0 * bv * T2 + st->W);
  if (obj) obj[2 * it + 1] = (float)st->g;
}

// The current codes to the caller's packed output; s and b (NaN if a pivot failed).
__global__ __launch_bounds__(256) void k_ptq_final(const uint8_t* __restrict__ codes0,
                                                   const uint8_t* __restrict__ codes1,
                                                   int64_t nbytes, const PtqState* st,
                                                   uint8_t* __restrict__ packed_out,
                                                   float* __restrict__ sb_out) {
  const uint8_t* src = st->cur ? codes1 : codes0;
  for (int64_t x = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 16; x < nbytes;
       x += (int64_t)gridDim.x * 256 * 16)
    *reinterpret_cast<uint4*>(packed_out + x) = *reinterpret_cast<const uint4*>(src + x);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    sb_out[0] = st->bad ? NAN : (float)st->s;
    sb_out[1] = st->bad ? NAN : (float)st->b;
  }
}

// ------------------------------------------------------------------ host side
struct PtqWs {
  size_t A, Ut32, Ut_hi, Ut_lo, Udiag, D, e, Q, c0, c1, qpart, spart, state, total;
};
static size_t up256(size_t x) { return (x + 255) / 256 * 256; }
static PtqWs ptq_ws(int64_t N, int64_t K) {
  PtqWs w;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += up256(bytes); return at; };
  w.A = take((size_t)K * K * 4);
  w.Ut32 = take((size_t)K * K * 4);
  w.Ut_hi = take((size_t)K * K * 2);
  w.Ut_lo = take((size_t)K * K * 2);
  w.Udiag = take((size_t)K * PB * 4);
  w.D = take((size_t)K * 4);
  w.e = take((size_t)K * 4);
  w.Q = take((size_t)N * K * 4);
  w.c0 = take((size_t)N * K / 4);
  w.c1 = take((size_t)N * K / 4);
  w.qpart = take((size_t)(K / QT) * (N / QT + 1) * 4 * 8);
  w.spart = take((size_t)(N / SWR) * 4 * 8);
  w.state = take(sizeof(PtqState));
  w.total = o;
  return w;
}

size_t ptq_workspace_bytes(int64_t N, int64_t K) { return ptq_ws(N, K).total; }

hipError_t launch_ptq_init(const float* H, const float* W0, int N, int K, float damp, int iters,
                           uint8_t* packed_out, float* sb_out, float* obj_out, float* U_out,
                           float* D_out, void* workspace, hipStream_t s) {
  const PtqWs w = ptq_ws(N, K);
  uint8_t* base = static_cast<uint8_t*>(workspace);
  float* A = reinterpret_cast<float*>(base + w.A);
  float* Ut32 = reinterpret_cast<float*>(base + w.Ut32);
  uint16_t* Ut_hi = reinterpret_cast<uint16_t*>(base + w.Ut_hi);
  uint16_t* Ut_lo = reinterpret_cast<uint16_t*>(base + w.Ut_lo);
  float* Udiag = reinterpret_cast<float*>(base + w.Udiag);
  float* D = reinterpret_cast<float*>(base + w.D);
  float* e = reinterpret_cast<float*>(base + w.e);
  float* Q = reinterpret_cast<float*>(base + w.Q);
  uint8_t* c0 = base + w.c0;
  uint8_t* c1 = base + w.c1;
  double* qpart = reinterpret_cast<double*>(base + w.qpart);
  double* spart = reinterpret_cast<double*>(base + w.spart);
  PtqState* st = reinterpret_cast<PtqState*>(base + w.state);

  hipLaunchKernelGGL(k_ptq_delta, dim3(1), dim3(256), 0, s, H, K, damp, st);
  hipLaunchKernelGGL(k_ptq_reverse, dim3(K), dim3(256), 0, s, H, K, st, A);
  // The first diagonal block on its own; every later one is factored by the update of the
  // step before (its workgroup 0).
  hipLaunchKernelGGL(k_chol_diag, dim3(1), dim3(PB), 0, s, A, K, 0, st);
  for (int j0 = 0; j0 < K; j0 += PB) {
    const int rows = K - j0 - PB;
    if (rows > 0) {
      hipLaunchKernelGGL(k_chol_panel, dim3((rows + PANEL_ROWS - 1) / PANEL_ROWS),
                         dim3(PANEL_ROWS * 64), 0, s, A, K, j0);
      const int T = rows / PB;
      hipLaunchKernelGGL(k_chol_update, dim3(T * (T + 1) / 2), dim3(256), 0, s, A, K, j0, st);
    }
  }
  hipLaunchKernelGGL(k_ptq_udu_out, dim3(K / PB, K / PB), dim3(256), 0, s, A, K, Ut32, Ut_hi,
                     Ut_lo, Udiag, D, U_out, D_out);
  hipLaunchKernelGGL(k_ptq_rowsum_e, dim3(K), dim3(256), 0, s, Ut32, K, e);
  const dim3 qgrid(K / QT, (N + QT - 1) / QT);
  hipLaunchKernelGGL(k_ptq_q, qgrid, dim3(256), 0, s, W0, Ut32, D, e, N, K, Q, qpart);
  hipLaunchKernelGGL(k_ptq_start, dim3(1), dim3(256), 0, s, qpart, (int)(qgrid.x * qgrid.y), D,
                     e, N, K, st);
  const int nwg = N / SWR;
  for (int it = 0; it < iters; ++it) {
    LCVQ_LAUNCH(PROF_PTQ_SWEEP, k_ptq_sweep, dim3(nwg), dim3(SW_WAVES * 64), 0, s, Q, e, D, Ut_hi, Ut_lo,
                Udiag, N, K, c0, c1, spart, st);
    hipLaunchKernelGGL(k_ptq_solve, dim3(1), dim3(256), 0, s, spart, nwg, it, st, obj_out);
  }
  const int64_t nbytes = (int64_t)N * K / 4;
  hipLaunchKernelGGL(k_ptq_final, dim3((unsigned)std::min<int64_t>((nbytes / 16 + 255) / 256, 4096)),
                     dim3(256), 0, s, c0, c1, nbytes, st, packed_out, sb_out);
  return hipGetLastError();
}

}  // namespace lcvq
