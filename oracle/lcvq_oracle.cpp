// CPU oracle of the LC-VQ hot path in plain C++17 -- TEST INFRASTRUCTURE ONLY.
//
// Only the test suite, the smoke check of the entry module and the CPU-baseline leg of the
// benchmark load this library (through oracle/coracle.py). The GPU library never links or
// calls it, and the two share no code, headers, tables or constants.
//
// Every function is written from the definitions on the pages, in float64 arithmetic
// (the quantizer decides on the float32 proxy itself, which float64 holds exactly), as
// plain loops: no BLAS, no blocking, no reordering beyond the loop order that makes rows
// contiguous. OpenMP splits independent output rows between threads; every sum is taken
// in a fixed order, so results do not depend on the thread count.
//
// Sources (page titles; the same summary appears in three languages):
//  [LCQAT-M1] "LC-QAT: Data-Efficient 2-Bit QAT for LLMs via Linear-Constrained Vector
//             Quantization", technical summary, Methodology 1: a codeword is c = A z + B,
//             z in {0,1,2,3}^d, with A (d x d) and B (d) shared by one weight matrix;
//             rounding and clamping pick z, and gradients pass through the linear map.
//  [LCQAT-M2] same page, Methodology 2: initialisation from a layer-wise reconstruction
//             with column groups and sequential error compensation (LDLQ).
//  [LCQAT-M3] same page, Methodology 3: the forward rounds and clamps the proxy weights
//             and decodes them with A Wz + B before the matmul; the backward needs an
//             estimator for the rounding's gradient.
//  [DQ-3]     "decoupleQ" (Chinese article), section 3.1 eq. (3)-(5): uniform 2-bit
//             quantization W^ = clip(round((W0 - z)/s), -2, 1), W~ = W^ s + z, and the
//             layer objective || X W0 - X W~ ||^2; section 3.2 eq. (6)-(7): the same
//             objective through H = X^T X with (s, z) as free floats; section 3.3
//             eq. (8)-(11): alternate between (s, z) by least squares and the integer
//             part column by column, each column rounded and clipped and the columns
//             not yet fixed re-solved to absorb its error.
//
// Readings of what the pages leave open (the same as the GPU library's):
//  * W[N, K] is stored as torch.nn.Linear does (N outputs, K inputs); Y = X W^T;
//  * d-vectors run along K: vector (n, g) is W[n, g*d .. g*d+d-1];
//  * A multiplies z as a column vector: What[n, g*d+i] = B[i] + sum_j A[i*d+j] z[n, g*d+j];
//  * rounding is round half to even; the straight-through mask is 1 exactly where
//    0 <= round(Wp) <= 3; NaN -> code 0, +inf -> code 3, -inf -> code 0, all mask 0;
//  * packing is little-endian: code k = 4b + t in bits [2t, 2t+1] of byte b; mask bit
//    k = 8c + t in bit t of byte c.
#include <cfenv>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

extern "C" {

int oc_threads() {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

// ---------------------------------------------------------------- O1 quantize
// [LCQAT-M1], [LCQAT-M3]: z = clamp(round(Wp), 0, 3); m = 1 iff the clamp did nothing.
void oc_quantize(const float* wp, int64_t count, uint8_t* z, uint8_t* m) {
  std::fesetround(FE_TONEAREST);          // nearbyint: round half to even
  for (int64_t i = 0; i < count; ++i) {
    const double w = (double)wp[i];
    uint8_t code = 0, keep = 0;
    if (std::isnan(w)) {
      code = 0;
    } else if (std::isinf(w)) {
      code = w > 0 ? 3 : 0;
    } else {
      const double r = std::nearbyint(w);
      keep = (r >= 0.0 && r <= 3.0) ? 1 : 0;
      code = (uint8_t)(r < 0.0 ? 0.0 : (r > 3.0 ? 3.0 : r));
    }
    z[i] = code;
    m[i] = keep;
  }
}

// ---------------------------------------------------------------- O2 packing
void oc_pack2b(const uint8_t* z, int64_t rows, int64_t k, uint8_t* out) {
  const int64_t nb = k / 4;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b) {
      unsigned v = 0;
      for (int t = 0; t < 4; ++t) v |= (unsigned)(z[r * k + 4 * b + t] & 3u) << (2 * t);
      out[r * nb + b] = (uint8_t)v;
    }
}

void oc_unpack2b(const uint8_t* packed, int64_t rows, int64_t k, uint8_t* z) {
  const int64_t nb = k / 4;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b)
      for (int t = 0; t < 4; ++t) z[r * k + 4 * b + t] = (packed[r * nb + b] >> (2 * t)) & 3u;
}

void oc_pack_mask(const uint8_t* m, int64_t rows, int64_t k, uint8_t* out) {
  const int64_t nb = k / 8;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < nb; ++c) {
      unsigned v = 0;
      for (int t = 0; t < 8; ++t) v |= (unsigned)(m[r * k + 8 * c + t] & 1u) << t;
      out[r * nb + c] = (uint8_t)v;
    }
}

void oc_unpack_mask(const uint8_t* bits, int64_t rows, int64_t k, uint8_t* m) {
  const int64_t nb = k / 8;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < nb; ++c)
      for (int t = 0; t < 8; ++t) m[r * k + 8 * c + t] = (bits[r * nb + c] >> t) & 1u;
}

// ---------------------------------------------------------------- O3 reconstruct
// [LCQAT-M1]: c = A z + B for every d-vector along K.
void oc_reconstruct(const uint8_t* z, int64_t N, int64_t K, int d, const double* A,
                    const double* B, double* What) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t g = 0; g < K / d; ++g)
      for (int i = 0; i < d; ++i) {
        double c = B[i];
        for (int j = 0; j < d; ++j) c += A[i * d + j] * (double)z[n * K + g * d + j];
        What[n * K + g * d + i] = c;
      }
}

// ---------------------------------------------------------------- O4 forward
// [LCQAT-M3]: Y = X What^T. rows (nrows entries) selects the rows of X to compute; NULL
// means all M rows. Y is [nrows][N].
void oc_forward(const double* X, int64_t M, int64_t K, const double* What, int64_t N,
                const int64_t* rows, int64_t nrows, double* Y) {
  if (!rows) nrows = M;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const double* x = X + (rows ? rows[r] : r) * K;
    for (int64_t n = 0; n < N; ++n) {
      const double* w = What + n * K;
      double s = 0.0;
      for (int64_t k = 0; k < K; ++k) s += x[k] * w[k];
      Y[r * N + n] = s;
    }
  }
}

// ---------------------------------------------------------------- O5 backward
// Backpropagation through Y = X What^T and the linear decode ([LCQAT-M1]), with the
// rounding passed straight through where the clamp was inactive ([LCQAT-M3]):
//   dX = dY What;  G = dY^T X;  dWp[n, g*d+j] = m * sum_i A[i][j] G[n, g*d+i];
//   dA[i][j] = sum_(n,g) G[n, g*d+i] z[n, g*d+j];  dB[i] = sum_(n,g) G[n, g*d+i].

// dX rows: dX[r, :] = sum_n dY[rows[r], n] What[n, :]. rows NULL means all M rows.
void oc_backward_dx(const double* dY, int64_t M, int64_t N, const double* What, int64_t K,
                    const int64_t* rows, int64_t nrows, double* dX) {
  if (!rows) nrows = M;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const double* dy = dY + (rows ? rows[r] : r) * N;
    double* o = dX + r * K;
    for (int64_t k = 0; k < K; ++k) o[k] = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double a = dy[n];
      const double* w = What + n * K;
      for (int64_t k = 0; k < K; ++k) o[k] += a * w[k];
    }
  }
}

// Slope of the smooth rounding curve used by the DGE estimator (a reading of the pages:
// [LCQAT-M3] names a smooth, differentiable stand-in for rounding but gives no curve):
//   s(w) = floor(w) + 1/2 + tanh(alpha (f - 1/2)) / (2 tanh(alpha / 2)),  f = w - floor(w)
//   s'(w) = alpha (1 - tanh^2(alpha (f - 1/2))) / (2 tanh(alpha / 2)); 0 for non-finite w.
void oc_dge_slope(const double* wp, int64_t count, double alpha, double* out) {
  for (int64_t i = 0; i < count; ++i) {
    const double w = wp[i];
    if (!std::isfinite(w)) {
      out[i] = 0.0;
      continue;
    }
    const double t = std::tanh(alpha * ((w - std::floor(w)) - 0.5));
    out[i] = alpha * (1.0 - t * t) / (2.0 * std::tanh(alpha / 2.0));
  }
}

// dWp rows, and dA, dB summed over the vectors of those rows. rows (nrows entries)
// selects weight rows n; NULL means all N rows. dWp is [nrows][K]. With wp non-NULL the
// rounding's gradient is the DGE slope at wp (sharpness alpha), still masked; wp is the
// full [N][K] proxy matrix. For each row: G[n, :] = sum_m dY[m, n] X[m, :], then the
// d-vector formulas; dA and dB add the rows' sums in row order.
void oc_backward_dw(const double* dY, const double* X, int64_t M, int64_t N, int64_t K,
                    int d, const uint8_t* z, const uint8_t* m, const double* A,
                    const float* wp, double alpha, const int64_t* rows, int64_t nrows,
                    double* dWp, double* dA, double* dB) {
  if (!rows) nrows = N;
  const int64_t nv = K / d;
  std::vector<double> rowA((size_t)nrows * d * d), rowB((size_t)nrows * d);
#pragma omp parallel
  {
    std::vector<double> G((size_t)K), wrow((size_t)K), slope((size_t)K);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
      const int64_t n = rows ? rows[r] : r;
      for (int64_t k = 0; k < K; ++k) G[k] = 0.0;
      for (int64_t mm = 0; mm < M; ++mm) {
        const double a = dY[mm * N + n];
        const double* x = X + mm * K;
        for (int64_t k = 0; k < K; ++k) G[k] += a * x[k];
      }
      if (wp) {
        for (int64_t k = 0; k < K; ++k) wrow[k] = (double)wp[n * K + k];
        oc_dge_slope(wrow.data(), K, alpha, slope.data());
      }
      double* ra = rowA.data() + r * d * d;
      double* rb = rowB.data() + r * d;
      for (int i = 0; i < d * d; ++i) ra[i] = 0.0;
      for (int i = 0; i < d; ++i) rb[i] = 0.0;
      for (int64_t g = 0; g < nv; ++g) {
        const double* gv = G.data() + g * d;
        const uint8_t* zv = z + n * K + g * d;
        const uint8_t* mv = m + n * K + g * d;
        for (int j = 0; j < d; ++j) {
          double s = 0.0;
          for (int i = 0; i < d; ++i) s += A[i * d + j] * gv[i];
          double v = mv[j] ? s : 0.0;
          if (wp) v *= slope[g * d + j];
          dWp[r * K + g * d + j] = v;
        }
        for (int i = 0; i < d; ++i) {
          for (int j = 0; j < d; ++j) ra[i * d + j] += gv[i] * (double)zv[j];
          rb[i] += gv[i];
        }
      }
    }
  }
  for (int i = 0; i < d * d; ++i) dA[i] = 0.0;
  for (int i = 0; i < d; ++i) dB[i] = 0.0;
  for (int64_t r = 0; r < nrows; ++r) {
    for (int i = 0; i < d * d; ++i) dA[i] += rowA[r * d * d + i];
    for (int i = 0; i < d; ++i) dB[i] += rowB[r * d + i];
  }
}

// ---------------------------------------------------------------- O6 decode product
// The deployed artefact is the integer part plus the float part; one linear transform
// turns it back into weights ([DQ-3] section 3.2, [LCQAT-M3]): unpack, decode, multiply.
// rows selects weight rows n (NULL: all N); Y is [M][nrows].
void oc_gemv2b(const double* X, int64_t M, int64_t K, const uint8_t* packed, int64_t N,
               int d, const double* A, const double* B, const int64_t* rows, int64_t nrows,
               double* Y) {
  if (!rows) nrows = N;
#pragma omp parallel
  {
    std::vector<uint8_t> zr((size_t)K);
    std::vector<double> w((size_t)K);
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < nrows; ++r) {
      const int64_t n = rows ? rows[r] : r;
      oc_unpack2b(packed + n * (K / 4), 1, K, zr.data());
      for (int64_t g = 0; g < K / d; ++g)
        for (int i = 0; i < d; ++i) {
          double c = B[i];
          for (int j = 0; j < d; ++j) c += A[i * d + j] * (double)zr[g * d + j];
          w[g * d + i] = c;
        }
      for (int64_t mm = 0; mm < M; ++mm) {
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) s += X[mm * K + k] * w[k];
        Y[mm * nrows + r] = s;
      }
    }
  }
}

// ---------------------------------------------------------------- PTQ initialisation
// Layer-wise initialisation of a per-tensor code (A = s I, B = b 1: one scale and one
// offset per matrix), the starting point that [LCQAT-M2] takes from post-training
// quantization. The objective is [DQ-3] eq. (5)/(7) in this layout (W[N, K], X [M, K],
// layer output X W^T), summed over the N output rows:
//   g(c; s, b) = 1/2 sum_n (s c_n + b 1 - w0_n)^T H (s c_n + b 1 - w0_n),  c_n in {0..3}^K
// with H = X^T X damped as H + delta I, delta = damp * mean(diag(X^T X)) (a reading: the
// pages give no regularisation, and without one X^T X from fewer calibration tokens than
// inputs is singular and eq. (11)'s minimiser is not unique). LC's codes {0..3} are
// decoupleQ's {-2..1} shifted by 2, so s c + b is eq. (4) with z = b + 2 s.
// [DQ-3] section 3.3 alternates two steps:
//  * (s, b): with c fixed, g is an unconstrained quadratic in (s, b); its stationary point
//    solves [S1 S2; S2 S3] [s; b] = [T1; T2] with S1 = sum c^T H c, S2 = sum c^T H 1,
//    S3 = N 1^T H 1, T1 = sum c^T H w0, T2 = sum 1^T H w0 (eq. (7) differentiated);
//  * c: element by element in index order, round and clip element k of the current
//    continuous solution, then re-solve the elements after k without the integer and box
//    constraints (eq. (11)). Written with H = U D U^T (U unit upper triangular), the
//    continuous value of element k once elements 0..k-1 are fixed is
//      t_k = v_k + sum_{i<k} U_ik (v_i - c_i),   v = (w0 - b) / s,
//    (for fixed d_P = c_P - v_P the minimiser is d_F = -H_FF^-1 H_FP d_P, and with the
//    factorisation H_FF^-1 H_FP = U_FF^-T U_PF^T, whose first row gives the sum above),
//    and c_k = clip(round(t_k), 0, 3).

// H = X^T X, plain loops (row i of H in parallel).
void oc_hessian(const double* X, int64_t M, int64_t K, double* H) {
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t i = 0; i < K; ++i)
    for (int64_t j = 0; j < K; ++j) {
      double s = 0.0;
      for (int64_t m = 0; m < M; ++m) s += X[m * K + i] * X[m * K + j];
      H[i * K + j] = s;
    }
}

// The damped matrix: Hd = H + damp * mean(diag(H)) I.
void oc_damp(const double* H, int64_t K, double damp, double* Hd) {
  double tr = 0.0;
  for (int64_t i = 0; i < K; ++i) tr += H[i * K + i];
  const double delta = damp * tr / (double)K;
  for (int64_t i = 0; i < K * K; ++i) Hd[i] = H[i];
  for (int64_t i = 0; i < K; ++i) Hd[i * K + i] += delta;
}

// Hd = U diag(D) U^T with U unit upper triangular (the last index is eliminated first):
//   D_k = Hd_kk - sum_{j>k} U_kj^2 D_j;  U_ik = (Hd_ik - sum_{j>k} U_ij D_j U_kj) / D_k, i < k.
// Returns 0, or k + 1 if D_k <= 0 (Hd not positive definite).
int oc_udu(const double* Hd, int64_t K, double* U, double* D) {
  for (int64_t i = 0; i < K * K; ++i) U[i] = 0.0;
  for (int64_t k = K - 1; k >= 0; --k) {
    double d = Hd[k * K + k];
    for (int64_t j = k + 1; j < K; ++j) d -= U[k * K + j] * U[k * K + j] * D[j];
    if (!(d > 0.0)) return (int)(k + 1);
    D[k] = d;
    U[k * K + k] = 1.0;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < k; ++i) {
      double v = Hd[i * K + k];
      for (int64_t j = k + 1; j < K; ++j) v -= U[i * K + j] * D[j] * U[k * K + j];
      U[i * K + k] = v / d;
    }
  }
  return 0;
}

// g(c; s, b) computed straight from its definition with Hd (rows in parallel, added in
// row order).
double oc_ptq_objective(const double* W0, const uint8_t* c, int64_t N, int64_t K,
                        const double* Hd, double s, double b) {
  std::vector<double> rowg((size_t)N);
#pragma omp parallel
  {
    std::vector<double> r((size_t)K);
#pragma omp for schedule(dynamic, 4)
    for (int64_t n = 0; n < N; ++n) {
      for (int64_t k = 0; k < K; ++k) r[k] = s * (double)c[n * K + k] + b - W0[n * K + k];
      double acc = 0.0;
      for (int64_t i = 0; i < K; ++i) {
        double hr = 0.0;
        for (int64_t j = 0; j < K; ++j) hr += Hd[i * K + j] * r[j];
        acc += r[i] * hr;
      }
      rowg[n] = 0.5 * acc;
    }
  }
  double g = 0.0;
  for (int64_t n = 0; n < N; ++n) g += rowg[n];
  return g;
}

// The integer step for fixed (s, b): codes c [N][K]; t (optional, [N][K]) receives the
// continuous value t_k each element was rounded from.
void oc_ptq_sweep(const double* W0, int64_t N, int64_t K, const double* U, double s, double b,
                  uint8_t* c, double* t) {
  std::fesetround(FE_TONEAREST);
#pragma omp parallel
  {
    std::vector<double> v((size_t)K), e((size_t)K);
#pragma omp for schedule(dynamic, 4)
    for (int64_t n = 0; n < N; ++n) {
      for (int64_t k = 0; k < K; ++k) v[k] = (W0[n * K + k] - b) / s;
      for (int64_t k = 0; k < K; ++k) {
        double tk = v[k];
        for (int64_t i = 0; i < k; ++i) tk += U[i * K + k] * e[i];
        const double r = std::nearbyint(tk);
        const double q = r < 0.0 ? 0.0 : (r > 3.0 ? 3.0 : r);
        c[n * K + k] = (uint8_t)q;
        e[k] = v[k] - q;
        if (t) t[n * K + k] = tk;
      }
    }
  }
}

// The continuous values the integer step rounds, given the codes that were decided:
// t_k = v_k + sum_{i<k} U_ik (v_i - c_i), v = (w0 - b) / s, for codes c [N][K] from any
// source (used to check another implementation's decisions one by one).
void oc_ptq_targets(const double* W0, int64_t N, int64_t K, const double* U, double s,
                    double b, const uint8_t* c, double* t) {
#pragma omp parallel
  {
    std::vector<double> v((size_t)K), e((size_t)K);
#pragma omp for schedule(dynamic, 4)
    for (int64_t n = 0; n < N; ++n) {
      for (int64_t k = 0; k < K; ++k) v[k] = (W0[n * K + k] - b) / s;
      for (int64_t k = 0; k < K; ++k) {
        double tk = v[k];
        for (int64_t i = 0; i < k; ++i) tk += U[i * K + k] * e[i];
        t[n * K + k] = tk;
        e[k] = v[k] - (double)c[n * K + k];
      }
    }
  }
}

// The (s, b) step for fixed codes: the stationary point of g, computed from the sums of
// its normal equations (each a plain double loop over H). Leaves s, b unchanged and
// returns 1 when the system is singular or gives s = 0 (the next integer step divides by
// s); returns 0 otherwise.
int oc_ptq_solve_sb(const double* W0, const uint8_t* c, int64_t N, int64_t K, const double* Hd,
                    double* s, double* b) {
  std::vector<double> h1((size_t)K, 0.0);
  for (int64_t i = 0; i < K; ++i)
    for (int64_t j = 0; j < K; ++j) h1[i] += Hd[i * K + j];
  double one_h_one = 0.0;
  for (int64_t i = 0; i < K; ++i) one_h_one += h1[i];
  std::vector<double> rs((size_t)N * 4);
#pragma omp parallel
  {
    std::vector<double> hc((size_t)K);
#pragma omp for schedule(dynamic, 4)
    for (int64_t n = 0; n < N; ++n) {
      const uint8_t* cn = c + n * K;
      const double* wn = W0 + n * K;
      for (int64_t i = 0; i < K; ++i) {
        double v = 0.0;
        for (int64_t j = 0; j < K; ++j) v += Hd[i * K + j] * (double)cn[j];
        hc[i] = v;
      }
      double s1 = 0.0, s2 = 0.0, t1 = 0.0, t2 = 0.0;
      for (int64_t i = 0; i < K; ++i) {
        s1 += (double)cn[i] * hc[i];      // c^T H c
        s2 += hc[i];                      // 1^T H c
        t1 += hc[i] * wn[i];              // c^T H w0
        t2 += h1[i] * wn[i];              // 1^T H w0
      }
      rs[n * 4 + 0] = s1; rs[n * 4 + 1] = s2; rs[n * 4 + 2] = t1; rs[n * 4 + 3] = t2;
    }
  }
  double S1 = 0.0, S2 = 0.0, T1 = 0.0, T2 = 0.0;
  for (int64_t n = 0; n < N; ++n) {
    S1 += rs[n * 4 + 0]; S2 += rs[n * 4 + 1]; T1 += rs[n * 4 + 2]; T2 += rs[n * 4 + 3];
  }
  const double S3 = (double)N * one_h_one;
  const double det = S1 * S3 - S2 * S2;
  if (!(std::fabs(det) > 1e-12 * std::fabs(S1 * S3)) || !std::isfinite(det)) return 1;
  const double sn = (T1 * S3 - S2 * T2) / det;
  const double bn = (S1 * T2 - S2 * T1) / det;
  if (sn == 0.0 || !std::isfinite(sn) || !std::isfinite(bn)) return 1;
  *s = sn;
  *b = bn;
  return 0;
}

// The whole initialisation: start from the uniform grid over the weight's range (s =
// (max - min) / 3, b = min; s = 1 for a constant matrix), then `iters` alternations of
// the integer step and the (s, b) step. The integer step's codes replace the current
// ones only if they do not raise g at the current (s, b) (the first always does), so the
// objective never increases. obj (2 * iters values, optional): g after each step.
// H is X^T X; it is damped here. Returns 0, or the oc_udu failure index.
int oc_ptq_init(const double* W0, int64_t N, int64_t K, const double* H, double damp,
                int iters, uint8_t* codes, double* s_out, double* b_out, double* obj) {
  std::vector<double> Hd((size_t)K * K), U((size_t)K * K), D((size_t)K);
  oc_damp(H, K, damp, Hd.data());
  const int bad = oc_udu(Hd.data(), K, U.data(), D.data());
  if (bad) return bad;
  double lo = W0[0], hi = W0[0];
  for (int64_t i = 1; i < N * K; ++i) {
    lo = W0[i] < lo ? W0[i] : lo;
    hi = W0[i] > hi ? W0[i] : hi;
  }
  double s = hi > lo ? (hi - lo) / 3.0 : 1.0, b = lo;
  std::vector<uint8_t> cand((size_t)N * K);
  double gcur = 0.0;
  for (int it = 0; it < iters; ++it) {
    oc_ptq_sweep(W0, N, K, U.data(), s, b, cand.data(), nullptr);
    const double gc = oc_ptq_objective(W0, cand.data(), N, K, Hd.data(), s, b);
    if (it == 0 || gc <= gcur) {
      std::memcpy(codes, cand.data(), (size_t)N * K);
      gcur = gc;
    }
    if (obj) obj[2 * it] = gcur;
    oc_ptq_solve_sb(W0, codes, N, K, Hd.data(), &s, &b);
    gcur = oc_ptq_objective(W0, codes, N, K, Hd.data(), s, b);
    if (obj) obj[2 * it + 1] = gcur;
  }
  *s_out = s;
  *b_out = b;
  return 0;
}

}  // extern "C"
