// Decode product Y = X What^T from packed 2-bit codes (gfx950), for 1..16 tokens.
//
// Deployment keeps only the integer part (the codes) and the float part (A, B) and
// turns them back into weights with one linear transform (decoupleQ, section 3.2;
// LC-QAT summary, Methodology 3). The product is folded the same way as in training:
//   Y[m, n] = sum_k X'[m, k] z[n, k] + beta[m],   X' = X (I kron A),  beta = X (1 kron B)
// so the weight stream is consumed as raw codes. Reading the codes is the whole cost
// (2 bits per weight from HBM), so the kernel is built around cheap code expansion:
//   * codes go to the int8 matrix cores unchanged in value: (w >> 2t) & 0x03030303
//     turns 16 packed codes into 4 int8 lanes-words in 7 VALU operations;
//   * X' is held per (row, 256-column block) as 16-bit fixed point split into two int8
//     limbs, so each block is two exact int32 MFMA sums, scaled once per block.
// The order in which a lane's 16 codes reach the MFMA differs from their order in k;
// the prologue writes X' limbs in that same order.
#include "lcvq_device.h"
#include "lcvq_internal.h"

namespace lcvq {

constexpr int GK = 256;   // k per block (4 MFMA of k = 64)

// X' limbs layout: for block kb, MFMA step s (0..3), limb (0 = high, 1 = low):
//   1 KiB at ((kb*4 + s)*2 + limb) * 1024, lane l = 16*kq + m at byte 16*l; the lane's
//   dword t, byte b holds column 64*kq + 16*s + 4*b + t of the block.
// rowinfo[kb][m] = (2^-e, partial beta) with e the block's fixed-point exponent.
__global__ __launch_bounds__(256) void k_gemv_prologue(const uint16_t* __restrict__ X, int M,
                                                       int K, const uint16_t* __restrict__ A16,
                                                       const uint16_t* __restrict__ B16, int d,
                                                       int8_t* __restrict__ xq,
                                                       float2* __restrict__ rowinfo) {
  const int kb = blockIdx.x;
  const int t = threadIdx.x;
  const int m = t >> 4, kc = t & 15;
  float xp[16];
  float bsum = 0.f, amax = 0.f;
  if (m < M) {
    const uint4* src = reinterpret_cast<const uint4*>(X + (int64_t)m * K + kb * GK + kc * 16);
    const uint4 a = src[0], b = src[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float x[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) { x[2 * i] = bf16lo_to_f32(w[i]); x[2 * i + 1] = bf16hi_to_f32(w[i]); }
    for (int v0 = 0; v0 < 16; v0 += d) {
      for (int j = 0; j < d; ++j) {
        float s = 0.f;
        for (int i = 0; i < d; ++i)
          s = __builtin_fmaf(x[v0 + i], (float)__builtin_bit_cast(_Float16, A16[i * d + j]), s);
        xp[v0 + j] = s;
        amax = fmaxf(amax, fabsf(s));
      }
      for (int i = 0; i < d; ++i)
        bsum = __builtin_fmaf(x[v0 + i], (float)__builtin_bit_cast(_Float16, B16[i]), bsum);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) xp[i] = 0.f;
  }
  // reduce over the 16 threads of row m (consecutive lanes)
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) {
    amax = fmaxf(amax, __shfl_xor(amax, o));
    bsum += __shfl_xor(bsum, o);
  }
  int ex = 0;
  if (amax > 0.f) {
    int E;
    frexpf(amax, &E);          // amax = f * 2^E, f in [0.5, 1)
    ex = 14 - E;               // |X' * 2^ex| < 2^14
  }
  uint32_t hi[4] = {0, 0, 0, 0}, lo[4] = {0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int q = (int)__builtin_rintf(ldexpf(xp[u], ex));
    const int l = ((q + 128) & 255) - 128;
    const int h = (q - l) >> 8;
    const int tt = u & 3, bb = u >> 2;          // column 4*bb + tt -> dword tt, byte bb
    hi[tt] |= (uint32_t)(h & 255) << (8 * bb);
    lo[tt] |= (uint32_t)(l & 255) << (8 * bb);
  }
  if (m < M) {
    const int kq = kc >> 2, s = kc & 3;
    const int lane = 16 * kq + m;
    uint4* dh = reinterpret_cast<uint4*>(xq + ((int64_t)(kb * 4 + s) * 2 + 0) * 1024 + lane * 16);
    uint4* dl = reinterpret_cast<uint4*>(xq + ((int64_t)(kb * 4 + s) * 2 + 1) * 1024 + lane * 16);
    *dh = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    *dl = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
  if (kc == 0) rowinfo[kb * 16 + m] = m < M ? make_float2(ldexpf(1.f, -ex), bsum) : make_float2(0.f, 0.f);
}

// One workgroup = 4 waves on 16 output rows n; wave w takes blocks kb = w, w+4, ...
// and the four partial results are added in LDS in a fixed order.
__global__ __launch_bounds__(256) void k_gemv(const int8_t* __restrict__ xq,
                                              const float2* __restrict__ rowinfo,
                                              const uint8_t* __restrict__ packed, int M, int N,
                                              int K, uint16_t* __restrict__ Y) {
  __shared__ float red[4][64][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int nl = lane & 15, kq = lane >> 4;
  const int nkb = K / GK;
  const uint8_t* crow = packed + (int64_t)(n0 + nl) * (K >> 2) + kq * 16;
  const bool has_a = nl < M;                       // A-operand lane row m = lane % 16
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int kb = wave; kb < nkb; kb += 4) {
    const uint4 w = *reinterpret_cast<const uint4*>(crow + kb * 64);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    i32x4 ahi[4], alo[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (has_a) {
        ahi[s] = *reinterpret_cast<const i32x4*>(xq + ((int64_t)(kb * 4 + s) * 2 + 0) * 1024 + lane * 16);
        alo[s] = *reinterpret_cast<const i32x4*>(xq + ((int64_t)(kb * 4 + s) * 2 + 1) * 1024 + lane * 16);
      } else {
        ahi[s] = i32x4{0, 0, 0, 0};
        alo[s] = i32x4{0, 0, 0, 0};
      }
    }
    i32x4 chi = {0, 0, 0, 0}, clo = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      i32x4 bz;
      bz[0] = (int)(ws[s] & 0x03030303u);
      bz[1] = (int)((ws[s] >> 2) & 0x03030303u);
      bz[2] = (int)((ws[s] >> 4) & 0x03030303u);
      bz[3] = (int)((ws[s] >> 6) & 0x03030303u);
      chi = __builtin_amdgcn_mfma_i32_16x16x64_i8(ahi[s], bz, chi, 0, 0, 0);
      clo = __builtin_amdgcn_mfma_i32_16x16x64_i8(alo[s], bz, clo, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float2 ri = rowinfo[kb * 16 + 4 * kq + r];
      acc[r] = __builtin_fmaf((float)(chi[r] * 256 + clo[r]), ri.x, acc[r] + ri.y);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][lane][r] = acc[r];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = ((red[0][lane][r] + red[1][lane][r]) + red[2][lane][r]) + red[3][lane][r];
      const int m = 4 * kq + r;
      if (m < M) reinterpret_cast<__bf16*>(Y)[(int64_t)m * N + n0 + nl] = (__bf16)v;
    }
  }
}

hipError_t launch_gemv_prologue(const uint16_t* X, int M, int K, const uint16_t* A16,
                                const uint16_t* B16, int d, int8_t* xq, float* rowinfo,
                                hipStream_t s) {
  hipLaunchKernelGGL(k_gemv_prologue, dim3(K / GK), dim3(256), 0, s, X, M, K, A16, B16, d, xq,
                     reinterpret_cast<float2*>(rowinfo));
  return hipGetLastError();
}

hipError_t launch_gemv(const int8_t* xq, const float* rowinfo, const uint8_t* packed, int M,
                       int N, int K, uint16_t* Y, hipStream_t s) {
  LCVQ_LAUNCH(PROF_GEMV, k_gemv, dim3(N / 16), dim3(256), 0, s, xq,
                     reinterpret_cast<const float2*>(rowinfo), packed, M, N, K, Y);
  return hipGetLastError();
}

}  // namespace lcvq
