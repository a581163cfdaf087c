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

}  // extern "C"
