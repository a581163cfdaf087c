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
#include <algorithm>
#include <atomic>

#include "lcvq_device.h"
#include "lcvq_internal.h"

namespace lcvq {

constexpr int GK = 256;   // k per block (4 MFMA of k = 64)
constexpr int GWF = 8;    // waves per workgroup of the fused kernel
constexpr size_t GEMV_LDS_MAX = 160 * 1024;

// Blocks of 256 columns along K (a multiple of 64): the last one holds K - 256 (nkb - 1)
// = 64, 128, 192 or 256 columns. Columns past K contribute nothing: their X' is zero.
__host__ __device__ inline int gemv_blocks(int64_t K) { return (int)((K + GK - 1) / GK); }

// Dynamic LDS of the fused kernel: the dense X' limbs (nkb * 32 * M * 16 bytes), the block
// scales (nkb * 128) and A, B; at least the final reduction's area.
inline size_t gemv_fused_lds(int M, int K, int d, int rg) {
  const size_t nkb = gemv_blocks(K);
  const size_t base = nkb * (32 * M + 8) * 16 + (size_t)(d * d + d) * 4;
  return std::max<size_t>(base, (size_t)GWF * rg * 64 * 16);
}

// The fused path (X' formed in LDS by every workgroup) repeats the M * K * d multiply-adds
// of X' in every workgroup, under the code stream; the two-kernel path pays a second
// launch and the X' round trip through memory instead. Fused:
//  * base range: one or two tokens with K up to 64 blocks; three or four with K up to 32
//    blocks; one row group per workgroup, or two from 8192 rows on;
//  * extended range, where the X' work per workgroup, M * (K / 256) * d, is at most 1792,
//    the grid runs in one round of one workgroup per CU and the LDS fits: one row group
//    per workgroup up to 4096 rows (three or four tokens with K up to 64 blocks, five to
//    sixteen with K up to 16 blocks), two up to 8192 rows (five to sixteen tokens).
// (Measured one build against the other on one GPU, shapes 4096 x 4096, 1024 x 4096,
// 4096 x 2048, 8192 x 4096 and 4096 x 14336 at d = 4, 8, 16: within the bound the fused
// launch took 0.56-0.91x the two launches, beyond it 1.0-1.28x.)
constexpr int GEMV_FUSED_WORK = 1792;
inline bool gemv_fused_base(int M, int nkb) {
  return M <= 2 ? nkb <= 64 : (M <= 4 && nkb <= 32);
}
inline bool gemv_fused(int M, int K, int64_t rows, int d) {
  const int nkb = gemv_blocks(K);
  if (gemv_fused_base(M, nkb)) return true;
  if (M > 16 || M * nkb * d > GEMV_FUSED_WORK) return false;
  const bool two = rows > 16 * 256;
  if (rows > (two ? 2 : 1) * 16 * 256 || (two && M <= 4)) return false;
  if (gemv_fused_lds(M, K, d, two ? 2 : 1) > GEMV_LDS_MAX) return false;
  return M <= 4 ? nkb <= 64 : nkb <= 16;
}
// Row groups of 16 per workgroup: in the base range two from 8192 rows on, and four from
// 16384 rows on for one or two tokens with K up to 16 blocks (the 28672 rows of a batched
// gate + up call then take 448 workgroups, which are resident at once, instead of 896);
// in the extended range two beyond 4096 rows. Each keeps the grid to about one round.
inline int gemv_row_groups(int M, int K, int64_t rows) {
  const int nkb = gemv_blocks(K);
  if (!gemv_fused_base(M, nkb)) return rows > 16 * 256 ? 2 : 1;
  if (rows >= 4 * 16 * 256 && M <= 2 && nkb <= 16) return 4;
  return rows >= 2 * 16 * 256 ? 2 : 1;
}
bool gemv_fused_path(int M, int K, int64_t rows, int d) { return gemv_fused(M, K, rows, d); }

// X' limbs: each (block kb, MFMA step s, limb 0 = high / 1 = low, quarter kq, row m) is
// a 16-byte chunk whose dword t, byte b holds column 64*kq + 16*s + 4*b + t of the block.
// The two-kernel path keeps them in global memory in MFMA lane order, 1 KiB per
// (kb, s, limb) with lane l = 16*kq + m at byte 16*l; the fused path keeps only rows
// m < M, dense in LDS, chunk index ((kb*8 + 2s + limb)*4 + kq)*M + m.
// rowinfo[kb][m] = (2^-e, partial beta) with e the block's fixed-point exponent; rows
// m >= M hold zeros.

// X' for one (row m, 256-column block): 16 consecutive lanes (kc = 0..15) each take the
// 16 columns of (kq, s) = (kc >> 2, kc & 3), given as 32 bytes of bf16 X. The lanes form
// X' = X (I kron A) and X (1 kron B) in float32, agree on the block's exponent
// (|X' 2^e| < 2^14) and return the two int8 limbs in MFMA byte order (column 4b + t in
// dword t, byte b), the scale 2^-e and the block's partial beta.
// A lane move within rows of 16 lanes (DPP control CTRL; every source lane is valid).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}

template <int D>
__device__ __forceinline__ void xprime_chunk(uint4 a, uint4 b, const float* As, const float* Bs,
                                             uint32_t (&hi)[4], uint32_t (&lo)[4],
                                             float& scale, float& bsum) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  float x[16], xp[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) { x[2 * i] = bf16lo_to_f32(w[i]); x[2 * i + 1] = bf16hi_to_f32(w[i]); }
  float amax = 0.f;
  bsum = 0.f;
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
  // Max and sum over the 16 lanes, as the xor butterfly o = 8, 4, 2, 1 with DPP lane moves
  // instead of LDS permutes: rotating a row of 16 lanes by 8 is xor 8; after that step
  // lanes i and i ^ 8 hold the same value, so a rotation by 4 brings lane i the value of
  // lane i ^ 4; xor 2 and xor 1 are quad permutations. Every lane ends with the same sum,
  // bit for bit, as the butterfly gives.
  amax = fmaxf(amax, dpp_f32<0x128>(amax));        // row_ror:8
  bsum += dpp_f32<0x128>(bsum);
  amax = fmaxf(amax, dpp_f32<0x124>(amax));        // row_ror:4
  bsum += dpp_f32<0x124>(bsum);
  amax = fmaxf(amax, dpp_f32<0x4E>(amax));         // quad_perm [2, 3, 0, 1]
  bsum += dpp_f32<0x4E>(bsum);
  amax = fmaxf(amax, dpp_f32<0xB1>(amax));         // quad_perm [1, 0, 3, 2]
  bsum += dpp_f32<0xB1>(bsum);
  int ex = 0;
  if (amax > 0.f) {
    int E;
    frexpf(amax, &E);          // amax = f * 2^E, f in [0.5, 1)
    ex = 14 - E;               // |X' * 2^ex| < 2^14
  }
  // q = rint(X' 2^ex) split as q = 256 h + l, l in [-128, 127]. Adding 1.5 * 2^23 + 128
  // rounds X' 2^ex + 128 to an integer t = q + 128 in the float's low mantissa bits
  // (|t| < 2^22; the bits are 0x4B400000 + t): byte 1 of them is h = t >> 8 (mod 256) and
  // byte 0 is t mod 256 = l + 128, i.e. l with its top bit flipped. Column 4*bb + tt goes
  // to dword tt, byte bb; v_perm_b32 gathers the bytes, two columns per step.
  uint32_t fb[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) fb[u] = __float_as_uint(ldexpf(xp[u], ex) + 12583040.f);
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    // bytes k of columns tt, 4 + tt (low half) and 8 + tt, 12 + tt (high half)
    const uint32_t l01 = __builtin_amdgcn_perm(fb[4 + tt], fb[tt], 0x0c0c0400u);
    const uint32_t l23 = __builtin_amdgcn_perm(fb[12 + tt], fb[8 + tt], 0x0c0c0400u);
    const uint32_t h01 = __builtin_amdgcn_perm(fb[4 + tt], fb[tt], 0x0c0c0501u);
    const uint32_t h23 = __builtin_amdgcn_perm(fb[12 + tt], fb[8 + tt], 0x0c0c0501u);
    lo[tt] = __builtin_amdgcn_perm(l23, l01, 0x05040100u) ^ 0x80808080u;
    hi[tt] = __builtin_amdgcn_perm(h23, h01, 0x05040100u);
  }
  scale = ldexpf(1.f, -ex);
}

// Prologue of the two-kernel path: thread t = 16*m + kc of block kb.
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
  if (m < M && kb * GK + kc * 16 < K) {             // columns past K: X' = 0
    const uint4* src = reinterpret_cast<const uint4*>(X + (int64_t)m * K + kb * GK + kc * 16);
    a = src[0];
    b = src[1];
  }
  if (t < D * D) As[t] = (float)__builtin_bit_cast(_Float16, A16[t]);
  if (t < D) Bs[t] = (float)__builtin_bit_cast(_Float16, B16[t]);
  __syncthreads();
  uint32_t hi[4], lo[4];
  float scale, bsum;
  xprime_chunk<D>(a, b, As, Bs, hi, lo, scale, bsum);
  if (m < M) {
    const int kq = kc >> 2, s = kc & 3;
    const int64_t oh = ((int64_t)(kb * 4 + s) * 2 + 0) * 1024 + (16 * kq + m) * 16;
    const int64_t ol = ((int64_t)(kb * 4 + s) * 2 + 1) * 1024 + (16 * kq + m) * 16;
    *reinterpret_cast<uint4*>(xq + oh) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    *reinterpret_cast<uint4*>(xq + ol) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
  if (kc == 0) rowinfo[kb * 16 + m] = m < M ? make_float2(scale, bsum) : make_float2(0.f, 0.f);
}

// One workgroup = GW waves on RG groups of 16 output rows n, over the whole of K. Wave w
// takes the blocks kb = w + GW*u; it issues the code loads of all of them (for every row
// group) first, then walks them with the X' limbs and block scales of the next block in
// flight while the current one runs on the matrix cores. One X' fragment serves the RG
// row groups. The GW partial sums of a row are added in LDS in a fixed order. The grid
// is shaped so that every workgroup of a launch is resident at once (one round), which
// keeps each workgroup's chain to one HBM round trip plus the X' walk.
constexpr int GW = 16;

// Where a lane's 16 bytes of codes for (row group g of a workgroup, block kb) live, in
// 16-byte units: base + g * gstride + kb * kstride. Lane l = 16 kq + nl takes row
// n0 + 16 g + nl, codes 256 kb + 64 kq .. +63.
//   canonical packed [N][K/4]: the row's bytes 64 kb + 16 kq;
//   decode layout: one 1 KiB tile per (16-row group, 256-column block), tile index
//   (n / 16) * (K / 256) + kb, lane l's bytes at 16 l, i.e. in the order the lanes load.
// The layout choice is uniform, so the loads themselves carry no branch.
struct CodeAddr {
  const u32x4* base;
  int64_t gstride, kstride;
};
__device__ __forceinline__ CodeAddr code_addr(const uint8_t* packed, int shuffled, int n0, int K,
                                              int lane) {
  const int64_t nkb = K / GK, rowb = K >> 2;
  CodeAddr c;
  if (shuffled) {
    c.base = reinterpret_cast<const u32x4*>(packed + (int64_t)(n0 >> 4) * nkb * 1024) + lane;
    c.gstride = nkb * 64;
    c.kstride = 64;
  } else {
    c.base = reinterpret_cast<const u32x4*>(packed + (int64_t)(n0 + (lane & 15)) * rowb +
                                            (lane >> 4) * 16);
    c.gstride = rowb;
    c.kstride = 4;
  }
  return c;
}

// In a last block of fewer than 256 columns (canonical layout only; the decode layout needs
// K % 256 == 0), a lane whose 64 columns lie past K reads the row's first 64 columns of
// that block instead: a valid address, and its X' is zero. Returned in 16-byte units, to
// be subtracted from the lane's address.
__device__ __forceinline__ int code_tail_back(int kb, int nkb, int K, int lane) {
  const int kq = lane >> 4;
  return (kb == nkb - 1 && kb * GK + 64 * kq >= K) ? kq : 0;
}

// Canonical packed codes -> decode layout (see code_addr): one 1 KiB tile per wave.
__global__ __launch_bounds__(256) void k_gemv_shuffle(const uint8_t* __restrict__ packed,
                                                      int64_t N, int64_t K,
                                                      uint8_t* __restrict__ out) {
  const int64_t nkb = K / GK, tiles = (N / 16) * nkb;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= tiles) return;
  const int lane = threadIdx.x & 63;
  const int64_t r = t / nkb, kb = t - r * nkb;
  const uint4 v = *reinterpret_cast<const uint4*>(packed + (r * 16 + (lane & 15)) * (K >> 2) +
                                                  kb * 64 + (lane >> 4) * 16);
  *reinterpret_cast<uint4*>(out + t * 1024 + lane * 16) = v;
}

// Measurement helper: one launch that streams `bytes` (a multiple of 16) once, with the
// decode kernels' non-temporal 16-byte loads, and writes one word per workgroup to `sink`
// (so that the loads are kept). It gives the same-size read ceiling beside the decode
// product; it is no step of the method.
__global__ __launch_bounds__(256) void k_read_probe(const u32x4* __restrict__ p, int64_t n16,
                                                    uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * 256) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  acc = __reduce_xor_sync(~0ull, acc);   // wave-wide, then one store per wave-0 lane 0
  __shared__ uint32_t w[4];
  if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x & 1023] = w[0] ^ w[1] ^ w[2] ^ w[3];
}

hipError_t launch_read_probe(const void* p, int64_t bytes, uint32_t* sink, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  // four 16-byte loads per thread, and no more workgroups than four per CU's worth of
  // rounds would need
  int64_t blocks = (n16 + 1023) / 1024;
  if (blocks > 65536) blocks = 65536;
  LCVQ_LAUNCH(PROF_READ_PROBE, k_read_probe, dim3((unsigned)blocks), dim3(256), 0, s,
              static_cast<const u32x4*>(p), n16, sink);
  return hipGetLastError();
}

hipError_t launch_gemv_shuffle(const uint8_t* packed, int64_t N, int64_t K, uint8_t* out,
                               hipStream_t s) {
  const int64_t tiles = (N / 16) * (K / GK);
  hipLaunchKernelGGL(k_gemv_shuffle, dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0, s, packed,
                     N, K, out);
  return hipGetLastError();
}

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

template <int RG, int KSW>
__global__ __launch_bounds__(GW * 64) void k_gemv(const int8_t* __restrict__ xq,
                                                  const float2* __restrict__ rowinfo,
                                                  const uint8_t* __restrict__ packed,
                                                  int shuffled, int M, int N, int K,
                                                  uint16_t* __restrict__ Y) {
  __shared__ f32x4 red[GW][RG][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * 16 * RG;
  const int nl = lane & 15, kq = lane >> 4;
  const int nkb = gemv_blocks(K);
  const CodeAddr ca = code_addr(packed, shuffled, n0, K, lane);
  const i32x4* xa = reinterpret_cast<const i32x4*>(xq) + lane;
  const f32x4* ri = reinterpret_cast<const f32x4*>(rowinfo) + 2 * kq;
  const bool has_a = nl < M;                       // A-operand lane row m = lane % 16
  f32x4 acc[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kb0 = wave; kb0 < nkb; kb0 += GW * KSW) {
    u32x4 cw[KSW][RG];
#pragma unroll
    for (int u = 0; u < KSW; ++u) {
      const int kb = kb0 + GW * u;
#pragma unroll
      for (int g = 0; g < RG; ++g)
        cw[u][g] = (kb < nkb && n0 + 16 * g < N)
                       ? __builtin_nontemporal_load(ca.base + g * ca.gstride + kb * ca.kstride -
                                                    code_tail_back(kb, nkb, K, lane))
                       : u32x4{0, 0, 0, 0};
    }
    GemvA a[2];
    gemv_load_a(a[0], xa, ri, kb0, has_a);
#pragma unroll
    for (int u = 0; u < KSW; ++u) {
      const int kb = kb0 + GW * u;
      if (kb >= nkb) break;
      if (u + 1 < KSW && kb + GW < nkb) gemv_load_a(a[(u + 1) & 1], xa, ri, kb + GW, has_a);
#pragma unroll
      for (int g = 0; g < RG; ++g) gemv_block(acc[g], a[u & 1], cw[u][g]);
    }
  }
#pragma unroll
  for (int g = 0; g < RG; ++g) red[wave][g][lane] = acc[g];
  __syncthreads();
  if (wave < RG) {
    const int g = wave;
    f32x4 v = red[0][g][lane];
#pragma unroll
    for (int w = 1; w < GW; ++w) {
      const f32x4 o = red[w][g][lane];
      v[0] += o[0]; v[1] += o[1]; v[2] += o[2]; v[3] += o[3];
    }
    const int n = n0 + 16 * g + nl;
    if (n < N) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * kq + r;
        if (m < M) reinterpret_cast<__bf16*>(Y)[(int64_t)m * N + n] = (__bf16)v[r];
      }
    }
  }
}

// Fused path (the cases of gemv_fused): one launch. A workgroup of GWF waves covers
// RG groups of 16 rows n over the whole of K. It first issues the code loads of all its
// waves' blocks (they stream from HBM meanwhile), then forms X' of rows m < M for the
// whole of K in LDS (dense chunk order, M * K * 2 bytes, at most 64 KiB) plus the block
// scales, and then runs the int8 products with fragments read from LDS one step at a
// time. Forming X' per workgroup repeats M * K * d multiply-adds that a separate
// prologue would do once, but it overlaps the code stream and saves a kernel boundary
// and the X' round trip through memory.
// One launch can serve up to GEMV_MAX_BATCH matrices that share X (and K), each with its
// own codes, A, B and output: workgroups [wg0[i], wg0[i+1]) belong to matrix i.
// MT is the token count, or for MT = 8, 12 and 16 a bound on the run-time count Mrt
// (5..8, 9..12, 13..16), which then sets the LDS layout and the X' work.
template <int D, int RG, int KSW, int MT>
__global__ __launch_bounds__(GWF * 64) void k_gemv_fused(const uint16_t* __restrict__ X,
                                                         GemvBatch batch, int K, int Mrt) {
  extern __shared__ __attribute__((aligned(16))) uint8_t gsm[];
  const int M = MT <= 4 ? MT : Mrt;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  int mi = 0;
#pragma unroll
  for (int i = 1; i < GEMV_MAX_BATCH; ++i)
    if (i < batch.count && (int)blockIdx.x >= batch.wg0[i]) mi = i;
  const uint8_t* __restrict__ packed = batch.packed[mi];
  const int shuffled = batch.shuffled[mi];
  const uint16_t* __restrict__ A16 = batch.A16[mi];
  const uint16_t* __restrict__ B16 = batch.B16[mi];
  uint16_t* __restrict__ Y = batch.Y[mi];
  const int N = batch.N[mi];
  const int n0 = ((int)blockIdx.x - batch.wg0[mi]) * 16 * RG;
  const int nl = lane & 15, kq = lane >> 4;
  const int nkb = gemv_blocks(K);
  const int XB = nkb * 32 * M * 16;                // dense X' bytes
  float2* ris = reinterpret_cast<float2*>(gsm + XB);              // [nkb][16]
  float* As = reinterpret_cast<float*>(gsm + XB + nkb * 128);     // [D][D], then B [D]
  float* Bs = As + D * D;

  // 1. A, B and this thread's X chunks, before the codes: vector-memory loads complete in
  //    issue order, so a wait for X or A issued after the code loads would also wait for
  //    the whole code stream, and forming X' could not overlap it. Item i = (kb * M + m)
  //    * 16 + kc covers 16 columns; the 16 items of a (kb, m) are 16 consecutive lanes.
  //    The launch picks KSW >= nkb / GWF, so nkb * M * 16 <= XI * GWF * 64.
  //    All loads here are unconditional, from clamped addresses: a load merged with a
  //    default value across a branch, or counted differently on two paths, makes the
  //    compiler wait for it (and for everything issued before it) right there.
  constexpr int XI = (KSW * MT + 3) / 4;
  static_assert(XI * GWF * 64 >= GWF * KSW * MT * 16, "X items of nkb <= GWF * KSW blocks");
  const int nitems = nkb * M * 16;
  uint4 xv[XI][2];
#pragma unroll
  for (int j = 0; j < XI; ++j) {
    const int i = min(t + j * GWF * 64, nitems - 1);     // threads past the end: not used
    const int kc = i & 15, gm = i >> 4;
    const int m = gm % M, kb = gm / M;
    const int col = kb * GK + kc * 16;                   // past K: read column 0, X' = 0
    const uint4* src = reinterpret_cast<const uint4*>(X + (int64_t)m * K + (col < K ? col : 0));
    xv[j][0] = src[0];
    xv[j][1] = src[1];
  }
  const uint16_t a16 = A16[min(t, D * D - 1)];
  const uint16_t b16 = B16[min(t, D - 1)];
  __builtin_amdgcn_sched_barrier(0);

  // 2. the codes of this wave's blocks, for every row group. Blocks past the end of K are
  //    never used (the product loop stops first) and rows past N are not stored, so those
  //    loads read the last block or the first row group instead.
  const CodeAddr ca = code_addr(packed, shuffled, n0, K, lane);
  u32x4 cw[KSW][RG];
#pragma unroll
  for (int u = 0; u < KSW; ++u) {
    const int kb = min(wave + GWF * u, nkb - 1);
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      const int gc = n0 + 16 * g < N ? g : 0;
      cw[u][g] = __builtin_nontemporal_load(ca.base + gc * ca.gstride + kb * ca.kstride -
                                            code_tail_back(kb, nkb, K, lane));
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // 3. A, B, zero block scales for the rows m >= M, then X' of rows m < M
  if (t < D * D) As[t] = (float)__builtin_bit_cast(_Float16, a16);
  if (t < D) Bs[t] = (float)__builtin_bit_cast(_Float16, b16);
  for (int i = t; i < nkb * 16; i += GWF * 64)
    if ((i & 15) >= M) ris[i] = make_float2(0.f, 0.f);
  __syncthreads();
  // With two or more chunks per thread, d <= 8 and one row group per workgroup (two row
  // groups keep to 128 VGPRs), A and B are copied to registers once: read from LDS inside
  // the loop they would be read again for every chunk (the X' stores in between may alias
  // them, as far as the compiler can tell).
  constexpr bool AREG = XI > 1 && D <= 8 && RG == 1;
  float Ar[AREG ? D * D + D : 1];
  if constexpr (AREG) {
#pragma unroll
    for (int i = 0; i < D * D + D; ++i) Ar[i] = As[i];   // B follows A in LDS
  }
  const float* Au = AREG ? Ar : As;
  const float* Bu = AREG ? Ar + D * D : Bs;
#pragma unroll
  for (int j = 0; j < XI; ++j) {
    const int i = t + j * GWF * 64;
    if (i >= nitems) break;
    const int kc = i & 15, gm = i >> 4;
    const int m = gm % M, kb = gm / M;
    uint32_t hi[4], lo[4];
    float scale, bsum;
    const bool in_k = kb * GK + kc * 16 < K;
    const uint4 z4 = make_uint4(0, 0, 0, 0);
    xprime_chunk<D>(in_k ? xv[j][0] : z4, in_k ? xv[j][1] : z4, Au, Bu, hi, lo, scale, bsum);
    const int q = kc >> 2, s = kc & 3;
    *reinterpret_cast<uint4*>(gsm + (((kb * 8 + 2 * s) * 4 + q) * M + m) * 16) =
        make_uint4(hi[0], hi[1], hi[2], hi[3]);
    *reinterpret_cast<uint4*>(gsm + (((kb * 8 + 2 * s + 1) * 4 + q) * M + m) * 16) =
        make_uint4(lo[0], lo[1], lo[2], lo[3]);
    if (kc == 0) ris[kb * 16 + m] = make_float2(scale, bsum);
  }
  __syncthreads();

  // 4. the products. A-operand lane row m = lane % 16. With one row group per workgroup,
  //    each block's 8 fragments and scales are read one block ahead, so that the LDS
  //    reads run under the previous block's MFMAs instead of each step waiting for its
  //    own two; rows m >= M then read row 0's X' (a valid address): they only reach
  //    output rows m >= M, whose block scales are zero and which are never stored. With
  //    two row groups the workgroups must fit two to a CU (128 VGPRs), which leaves no
  //    room for the second set of fragments: those read each step's two fragments as it
  //    comes, rows m >= M as zeros.
  f32x4 acc[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint8_t* ri = gsm + XB + kq * 32;
  struct Frags {
    i32x4 h[4], l[4];
    f32x4 r0, r1;
  };
  auto block_mfma = [&](const Frags& f, int u) {
    i32x4 chi[RG], clo[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g) chi[g] = clo[g] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        const uint32_t w = cw[u][g][s];
        i32x4 bz;
        bz[0] = (int)(w & 0x03030303u);
        bz[1] = (int)((w >> 2) & 0x03030303u);
        bz[2] = (int)((w >> 4) & 0x03030303u);
        bz[3] = (int)((w >> 6) & 0x03030303u);
        chi[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.h[s], bz, chi[g], 0, 0, 0);
        clo[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.l[s], bz, clo[g], 0, 0, 0);
      }
    }
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      f32x4& a = acc[g];
      a[0] = __builtin_fmaf((float)(chi[g][0] * 256 + clo[g][0]), f.r0[0], a[0] + f.r0[1]);
      a[1] = __builtin_fmaf((float)(chi[g][1] * 256 + clo[g][1]), f.r0[2], a[1] + f.r0[3]);
      a[2] = __builtin_fmaf((float)(chi[g][2] * 256 + clo[g][2]), f.r1[0], a[2] + f.r1[1]);
      a[3] = __builtin_fmaf((float)(chi[g][3] * 256 + clo[g][3]), f.r1[2], a[3] + f.r1[3]);
    }
  };
  if constexpr (RG == 1) {
    const uint8_t* xl = gsm + (kq * M + (nl < M ? nl : 0)) * 16;
    auto read_frags = [&](int kb, Frags& f) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        f.h[s] = *reinterpret_cast<const i32x4*>(xl + (kb * 8 + 2 * s) * 4 * M * 16);
        f.l[s] = *reinterpret_cast<const i32x4*>(xl + (kb * 8 + 2 * s + 1) * 4 * M * 16);
      }
      f.r0 = *reinterpret_cast<const f32x4*>(ri + kb * 128);
      f.r1 = *reinterpret_cast<const f32x4*>(ri + kb * 128 + 16);
    };
    Frags fr[2];
    read_frags(min(wave, nkb - 1), fr[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < KSW; ++u) {
      const int kb = wave + GWF * u;
      if (kb >= nkb) break;
      if (u + 1 < KSW) read_frags(min(kb + GWF, nkb - 1), fr[(u + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);           // keep the reads ahead of the MFMAs
      block_mfma(fr[u & 1], u);
    }
  } else {
    const bool has_a = nl < M;
    const uint8_t* xl = gsm + (kq * M + nl) * 16;
#pragma unroll
    for (int u = 0; u < KSW; ++u) {
      const int kb = wave + GWF * u;
      if (kb >= nkb) break;
      Frags f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        f.h[s] = f.l[s] = i32x4{0, 0, 0, 0};
        if (has_a) {
          f.h[s] = *reinterpret_cast<const i32x4*>(xl + (kb * 8 + 2 * s) * 4 * M * 16);
          f.l[s] = *reinterpret_cast<const i32x4*>(xl + (kb * 8 + 2 * s + 1) * 4 * M * 16);
        }
      }
      f.r0 = *reinterpret_cast<const f32x4*>(ri + kb * 128);
      f.r1 = *reinterpret_cast<const f32x4*>(ri + kb * 128 + 16);
      block_mfma(f, u);
    }
  }
  // 5. the GWF partial sums of each row, in wave order
  __syncthreads();                                 // the X' area becomes the reduction area
  f32x4* red = reinterpret_cast<f32x4*>(gsm);
#pragma unroll
  for (int g = 0; g < RG; ++g) red[(wave * RG + g) * 64 + lane] = acc[g];
  __syncthreads();
  if (wave < RG) {
    const int g = wave;
    f32x4 v = red[g * 64 + lane];
#pragma unroll
    for (int w = 1; w < GWF; ++w) {
      const f32x4 o = red[(w * RG + g) * 64 + lane];
      v[0] += o[0]; v[1] += o[1]; v[2] += o[2]; v[3] += o[3];
    }
    const int n = n0 + 16 * g + nl;
    if (n < N) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * kq + r;
        if (m < M) reinterpret_cast<__bf16*>(Y)[(int64_t)m * N + n] = (__bf16)v[r];
      }
    }
  }
}

template <int D, int RG, int KSW, int MT>
static hipError_t launch_fused(dim3 grid, size_t shm, hipStream_t s, const uint16_t* X,
                               const GemvBatch& b, int K, int M) {
  // Dynamic LDS beyond 64 KiB must be requested for the kernel, once per device: a
  // process-wide cache of the devices done (the first 64; beyond that it is requested on
  // every launch). A failed request is returned, and not cached.
  static std::atomic<uint64_t> done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? uint64_t(1) << dev : 0;
  if (!bit || !(done.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv_fused<D, RG, KSW, MT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)GEMV_LDS_MAX);
    if (e != hipSuccess) return e;
    done.fetch_or(bit, std::memory_order_acq_rel);
  }
  LCVQ_LAUNCH(PROF_GEMV, (k_gemv_fused<D, RG, KSW, MT>), grid, dim3(GWF * 64), shm, s, X, b, K,
              M);
  return hipGetLastError();
}

// The instances gemv_fused() can reach: M = 3, 4 with two row groups only for K up to 32
// blocks (KSW <= 4); M = 5..16 with K up to 16 blocks (KSW = 2); four row groups only for
// M = 1, 2 and K up to 16 blocks.
template <int D, int RG, int KSW>
static hipError_t launch_fused_m(int M, dim3 grid, size_t shm, hipStream_t s, const uint16_t* X,
                                 const GemvBatch& b, int K) {
  if (M == 1) return launch_fused<D, RG, KSW, 1>(grid, shm, s, X, b, K, M);
  if (M == 2) return launch_fused<D, RG, KSW, 2>(grid, shm, s, X, b, K, M);
  if constexpr (RG <= 2 && (KSW <= 4 || RG == 1)) {
    if (M == 3) return launch_fused<D, RG, KSW, 3>(grid, shm, s, X, b, K, M);
    if (M == 4) return launch_fused<D, RG, KSW, 4>(grid, shm, s, X, b, K, M);
  }
  if constexpr (RG <= 2 && KSW <= 2) {     // the X' items a thread holds grow with the bound
    if (M <= 8) return launch_fused<D, RG, KSW, 8>(grid, shm, s, X, b, K, M);
    if (M <= 12) return launch_fused<D, RG, KSW, 12>(grid, shm, s, X, b, K, M);
    if (M <= 16) return launch_fused<D, RG, KSW, 16>(grid, shm, s, X, b, K, M);
  }
  return hipErrorInvalidValue;       // not reached: gemv_fused() picks only the cases above
}

template <int D>
static hipError_t launch_fused_d(int M, int K, int rg, size_t shm, hipStream_t s,
                                 const uint16_t* X, const GemvBatch& b, int wgs) {
  const int pw = (gemv_blocks(K) + GWF - 1) / GWF;
  const dim3 grid(wgs);
#define LCVQ_FUSED(RG, KSW) return launch_fused_m<D, RG, KSW>(M, grid, shm, s, X, b, K)
  if (rg == 4) {
    LCVQ_FUSED(4, 2);               // gemv_row_groups() keeps four groups to K <= 4096
  } else if (rg == 2) {
    if (pw <= 2) LCVQ_FUSED(2, 2);
    else if (pw <= 4) LCVQ_FUSED(2, 4);
    else LCVQ_FUSED(2, 8);
  } else {
    if (pw <= 2) LCVQ_FUSED(1, 2);
    else if (pw <= 4) LCVQ_FUSED(1, 4);
    else LCVQ_FUSED(1, 8);
  }
#undef LCVQ_FUSED
}

// One fused launch over the matrices of `b` (count, packed, A16, B16, Y, N filled in).
hipError_t launch_gemv_fused(const uint16_t* X, int M, int K, int d, GemvBatch b,
                             hipStream_t s) {
  int64_t rows = 0;
  for (int i = 0; i < b.count; ++i) rows += b.N[i];
  const int rg = gemv_row_groups(M, K, rows);
  int wgs = 0;
  for (int i = 0; i < b.count; ++i) {
    b.wg0[i] = wgs;
    wgs += (b.N[i] + 16 * rg - 1) / (16 * rg);
  }
  const size_t shm = gemv_fused_lds(M, K, d, rg);
  switch (d) {
    case 4: return launch_fused_d<4>(M, K, rg, shm, s, X, b, wgs);
    case 8: return launch_fused_d<8>(M, K, rg, shm, s, X, b, wgs);
    default: return launch_fused_d<16>(M, K, rg, shm, s, X, b, wgs);
  }
}

hipError_t launch_gemv(const uint16_t* X, int M, int N, int K, const uint16_t* A16,
                       const uint16_t* B16, int d, const uint8_t* packed, int shuffled,
                       uint16_t* Y, int8_t* xq, float* rowinfo, hipStream_t s) {
  const int nkb = gemv_blocks(K);
  // Two row groups per workgroup when N still gives a workgroup per CU.
  const bool two = N >= 2 * 16 * 256;
  if (gemv_fused(M, K, N, d)) {
    GemvBatch b = {};
    b.count = 1;
    b.packed[0] = packed; b.A16[0] = A16; b.B16[0] = B16; b.Y[0] = Y; b.N[0] = N;
    b.shuffled[0] = shuffled;
    return launch_gemv_fused(X, M, K, d, b, s);
  }
  float2* ri = reinterpret_cast<float2*>(rowinfo);
  // Two launches: the timing hook, when armed for the decode product, brackets both with
  // events on the stream (the prologue's time is part of the product's).
  hipEvent_t e0, e1;
  const bool timed = take_profile(PROF_GEMV, &e0, &e1);
  if (timed) (void)hipEventRecord(e0, s);
  const dim3 pgrid(nkb), pblock(256);
  switch (d) {
    case 4: hipLaunchKernelGGL(k_gemv_prologue<4>, pgrid, pblock, 0, s, X, M, K, A16, B16, xq, ri); break;
    case 8: hipLaunchKernelGGL(k_gemv_prologue<8>, pgrid, pblock, 0, s, X, M, K, A16, B16, xq, ri); break;
    default: hipLaunchKernelGGL(k_gemv_prologue<16>, pgrid, pblock, 0, s, X, M, K, A16, B16, xq, ri); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    if (timed) (void)hipEventRecord(e1, s);
    return e;
  }
  const int per_wave = (nkb + GW - 1) / GW;
  const dim3 grid(two ? (N + 31) / 32 : N / 16), block(GW * 64);
#define LCVQ_GEMV(RG, KSW) \
  hipLaunchKernelGGL((k_gemv<RG, KSW>), grid, block, 0, s, xq, ri, packed, shuffled, M, N, K, Y)
  if (two) {
    if (per_wave <= 1) LCVQ_GEMV(2, 1);
    else LCVQ_GEMV(2, 2);
  } else {
    if (per_wave <= 1) LCVQ_GEMV(1, 1);
    else LCVQ_GEMV(1, 2);
  }
#undef LCVQ_GEMV
  e = hipGetLastError();
  if (timed) (void)hipEventRecord(e1, s);
  return e;
}

}  // namespace lcvq
