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
// rowinfo[kb][m] = (2^-e, partial beta) with e the block's fixed-point exponent; rows
// m >= M hold zeros.
// Thread t = 16*m + kc of block kb forms the 16 columns of (kq, s) = (kc >> 2, kc & 3).
template <int D>
__global__ __launch_bounds__(256) void k_gemv_prologue(const uint16_t* __restrict__ X, int M,
                                                       int K, const uint16_t* __restrict__ A16,
                                                       const uint16_t* __restrict__ B16,
                                                       int8_t* __restrict__ xq,
                                                       float2* __restrict__ rowinfo) {
  __shared__ float As[D * D];
  __shared__ float Bs[D];
  const int kb = blockIdx.x;
  const int t = threadIdx.x;
  const int m = t >> 4, kc = t & 15;
  uint4 a = make_uint4(0, 0, 0, 0), b = a;
  if (m < M) {
    const uint4* src = reinterpret_cast<const uint4*>(X + (int64_t)m * K + kb * GK + kc * 16);
    a = src[0];
    b = src[1];
  }
  if (t < D * D) As[t] = (float)__builtin_bit_cast(_Float16, A16[t]);
  if (t < D) Bs[t] = (float)__builtin_bit_cast(_Float16, B16[t]);
  __syncthreads();
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  float x[16], xp[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) { x[2 * i] = bf16lo_to_f32(w[i]); x[2 * i + 1] = bf16hi_to_f32(w[i]); }
  float bsum = 0.f, amax = 0.f;
#pragma unroll
  for (int v0 = 0; v0 < 16; v0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) s = __builtin_fmaf(x[v0 + i], As[i * D + j], s);
      xp[v0 + j] = s;
      amax = fmaxf(amax, fabsf(s));
    }
#pragma unroll
    for (int i = 0; i < D; ++i) bsum = __builtin_fmaf(x[v0 + i], Bs[i], bsum);
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

// One workgroup = GW waves on 16 output rows n; wave w takes the PF blocks
// kb = w + GW*u (u < PF). It issues the code loads of all of them first (one round trip
// to HBM for the whole share), then walks them with the X' limbs and block scales of the
// next block in flight while the current one runs on the matrix cores. The GW partial
// sums of a row are added in LDS in a fixed order.
constexpr int GW = 8;

struct GemvA {
  i32x4 hi[4], lo[4];
  f32x4 r0, r1;
};

__device__ __forceinline__ void gemv_load_a(GemvA& a, const i32x4* xa, const f32x4* ri, int kb,
                                            bool has_a) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (has_a) {
      a.hi[s] = xa[((kb * 4 + s) * 2 + 0) * 64];
      a.lo[s] = xa[((kb * 4 + s) * 2 + 1) * 64];
    } else {
      a.hi[s] = i32x4{0, 0, 0, 0};
      a.lo[s] = i32x4{0, 0, 0, 0};
    }
  }
  a.r0 = ri[kb * 8];                               // rows 4kq..4kq+3: (scale, beta) x 4
  a.r1 = ri[kb * 8 + 1];
}

__device__ __forceinline__ void gemv_block(f32x4& acc, const GemvA& a, const u32x4& cw) {
  i32x4 chi = {0, 0, 0, 0}, clo = {0, 0, 0, 0};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t w = cw[s];
    i32x4 bz;
    bz[0] = (int)(w & 0x03030303u);
    bz[1] = (int)((w >> 2) & 0x03030303u);
    bz[2] = (int)((w >> 4) & 0x03030303u);
    bz[3] = (int)((w >> 6) & 0x03030303u);
    chi = __builtin_amdgcn_mfma_i32_16x16x64_i8(a.hi[s], bz, chi, 0, 0, 0);
    clo = __builtin_amdgcn_mfma_i32_16x16x64_i8(a.lo[s], bz, clo, 0, 0, 0);
  }
  acc[0] = __builtin_fmaf((float)(chi[0] * 256 + clo[0]), a.r0[0], acc[0] + a.r0[1]);
  acc[1] = __builtin_fmaf((float)(chi[1] * 256 + clo[1]), a.r0[2], acc[1] + a.r0[3]);
  acc[2] = __builtin_fmaf((float)(chi[2] * 256 + clo[2]), a.r1[0], acc[2] + a.r1[1]);
  acc[3] = __builtin_fmaf((float)(chi[3] * 256 + clo[3]), a.r1[2], acc[3] + a.r1[3]);
}

template <int PF>
__global__ __launch_bounds__(GW * 64) void k_gemv(const int8_t* __restrict__ xq,
                                                  const float2* __restrict__ rowinfo,
                                                  const uint8_t* __restrict__ packed, int M,
                                                  int N, int K, uint16_t* __restrict__ Y) {
  __shared__ f32x4 red[GW][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * 16;
  const int nl = lane & 15, kq = lane >> 4;
  const int nkb = K / GK;
  const u32x4* crow =
      reinterpret_cast<const u32x4*>(packed + (int64_t)(n0 + nl) * (K >> 2) + kq * 16);
  const i32x4* xa = reinterpret_cast<const i32x4*>(xq) + lane;
  const f32x4* ri = reinterpret_cast<const f32x4*>(rowinfo) + 2 * kq;
  const bool has_a = nl < M;                       // A-operand lane row m = lane % 16
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int kb0 = wave; kb0 < nkb; kb0 += GW * PF) {
    u32x4 cw[PF];
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int kb = kb0 + GW * u;
      cw[u] = kb < nkb ? __builtin_nontemporal_load(crow + kb * 4) : u32x4{0, 0, 0, 0};
    }
    GemvA a[2];
    gemv_load_a(a[0], xa, ri, kb0, has_a);
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int kb = kb0 + GW * u;
      if (kb >= nkb) break;
      if (u + 1 < PF && kb + GW < nkb) gemv_load_a(a[(u + 1) & 1], xa, ri, kb + GW, has_a);
      gemv_block(acc, a[u & 1], cw[u]);
    }
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4 v = red[0][lane];
#pragma unroll
    for (int w = 1; w < GW; ++w) {
      const f32x4 o = red[w][lane];
      v[0] += o[0]; v[1] += o[1]; v[2] += o[2]; v[3] += o[3];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * kq + r;
      if (m < M) reinterpret_cast<__bf16*>(Y)[(int64_t)m * N + n0 + nl] = (__bf16)v[r];
    }
  }
}

hipError_t launch_gemv_prologue(const uint16_t* X, int M, int K, const uint16_t* A16,
                                const uint16_t* B16, int d, int8_t* xq, float* rowinfo,
                                hipStream_t s) {
  float2* ri = reinterpret_cast<float2*>(rowinfo);
  switch (d) {
    case 4: hipLaunchKernelGGL(k_gemv_prologue<4>, dim3(K / GK), dim3(256), 0, s, X, M, K, A16, B16, xq, ri); break;
    case 8: hipLaunchKernelGGL(k_gemv_prologue<8>, dim3(K / GK), dim3(256), 0, s, X, M, K, A16, B16, xq, ri); break;
    default: hipLaunchKernelGGL(k_gemv_prologue<16>, dim3(K / GK), dim3(256), 0, s, X, M, K, A16, B16, xq, ri); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemv(const int8_t* xq, const float* rowinfo, const uint8_t* packed, int M,
                       int N, int K, uint16_t* Y, hipStream_t s) {
  const int per_wave = (K / GK + GW - 1) / GW;     // blocks per wave
  const dim3 grid(N / 16), block(GW * 64);
  const float2* ri = reinterpret_cast<const float2*>(rowinfo);
  if (per_wave <= 1)
    LCVQ_LAUNCH(PROF_GEMV, k_gemv<1>, grid, block, 0, s, xq, ri, packed, M, N, K, Y);
  else if (per_wave <= 2)
    LCVQ_LAUNCH(PROF_GEMV, k_gemv<2>, grid, block, 0, s, xq, ri, packed, M, N, K, Y);
  else if (per_wave <= 4)
    LCVQ_LAUNCH(PROF_GEMV, k_gemv<4>, grid, block, 0, s, xq, ri, packed, M, N, K, Y);
  else
    LCVQ_LAUNCH(PROF_GEMV, k_gemv<8>, grid, block, 0, s, xq, ri, packed, M, N, K, Y);
  return hipGetLastError();
}

}  // namespace lcvq
