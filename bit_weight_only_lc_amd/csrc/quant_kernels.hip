// Elementwise and layout kernels of the LC-VQ path (gfx950):
//  * the quantizer z = clamp(round(Wp), 0, 3) with mask, packing and an optional
//    float32 decode (LC-QAT summary, Methodology 1 and 3);
//  * 2-bit pack / unpack;
//  * the transposed code layout the dX product reads;
//  * the forward prologue X' = X (I kron A) and the backward prologue r = dY 1.
// All are HBM-bound: each thread owns 16 consecutive elements so that its codes form
// exactly one 32-bit packed word, and every d-vector (d <= 16) lies inside one thread.
#include "lcvq_device.h"
#include "lcvq_internal.h"

namespace lcvq {

// Index of the R16 word holding codes (row, 16*w .. 16*w+15) in the blocked layout
// the GEMM loaders read: rows in blocks of 256, contraction in steps of 64, and each
// (row block, step) slab of 256 rows x 4 words contiguous (4 KiB). Inside a row the
// word w sits at position (w + row/8) mod 4, which spreads the MFMA fragment reads of
// 32 consecutive rows over all LDS banks.
__device__ __forceinline__ int64_t r16_blocked_index(int64_t row, int64_t w, int64_t ksteps) {
  return ((row >> 8) * ksteps + (w >> 2)) * 1024 + (row & 255) * 4 + (((w & 3) + ((row >> 3) & 3)) & 3);
}

// ------------------------------------------------------------------ quantizer
// Each wave streams a contiguous chunk of 1024 proxies with four fully coalesced
// 16-byte loads per lane (lane l holds elements 256 j + 4 l .. +3 of load j). A group of
// 16 consecutive codes (one packed word, one R16 word, one d-vector for d <= 16) is
// spread over 4 neighbouring lanes and gathered with lane shuffles.
template <int D>   // D = 0: no float32 decode requested; (bx, gx) = block, grid size
__device__ __forceinline__ void quantize_body(
    int bx, int gx, const float* __restrict__ wp, int64_t total /* N*K */, int64_t K,
    uint8_t* __restrict__ z_out, uint8_t* __restrict__ packed_out,
    uint8_t* __restrict__ mask_out, uint32_t* __restrict__ r16_out,
    float* __restrict__ what_out, const float* __restrict__ A,
    const float* __restrict__ B) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  constexpr int DD = D > 0 ? D : 1;
  const int lane = threadIdx.x & 63;
  const int q = lane & 3;
  const int64_t nchunks = (total + 1023) >> 10;
  const int64_t wstride = (int64_t)gx * 4;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int64_t ch = (int64_t)bx * 4 + wv; ch < nchunks; ch += wstride) {
    const int64_t base = ch << 10;
    // Row of the chunk's first element (one scalar division per chunk); a lane's element
    // lies less than 1024 elements further, i.e. in row0 or a few rows later.
    const int64_t row0 = r16_out ? base / K : 0;
    const int off0 = (int)(base - row0 * K);
    // 64-bit chunk bases are uniform (scalar); per-lane offsets stay 32-bit
    const int rem = (int)(total - base < 1024 ? total - base : 1024);
    const float* wpc = wp + base;
    f4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int le = 256 * j + 4 * lane;
      v[j] = le < rem ? __builtin_nontemporal_load(reinterpret_cast<const f4*>(wpc + le))
                      : f4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int le = 256 * j + 4 * lane;
      const int64_t e = base + le;
      uint32_t byte = 0, m4 = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float r = __builtin_rintf(v[j][t]);            // round half to even
        // maxNum/minNum return the number for a NaN operand: NaN -> 0, +inf -> 3,
        // -inf -> 0. The mask is 1 exactly when the clamp left r unchanged (never for
        // NaN or infinities).
        const float cf = fminf(fmaxf(r, 0.f), 3.f);
        byte |= (uint32_t)(int)cf << (2 * t);
        m4 |= (uint32_t)(cf == r) << t;
      }
      const uint32_t mpair = m4 | ((uint32_t)__shfl_xor((int)m4, 1) << 4);
      // R16 word of this lane's 16-code group: lane q of the group holds codes 4q..4q+3;
      // its even codes go to bits 5 + 2p and its odd codes to bits 21 + 2p of an 8-code
      // half (p = position in the half), and the second half is rotated left by 8, so
      // each lane places its two 2-code runs with one rotate and the four lanes OR them.
      uint32_t rw = 0;
      if (r16_out) {
        const uint32_t E = (byte & 3u) | ((byte >> 2) & 0xCu);
        const uint32_t O = ((byte >> 2) & 3u) | ((byte >> 4) & 0xCu);
        const uint64_t v = (uint64_t)((E << 5) | (O << 21)) << (4 * (q & 1) + 8 * (q >> 1));
        rw = (uint32_t)v | (uint32_t)(v >> 32);
        rw |= (uint32_t)__shfl_xor((int)rw, 1);
        rw |= (uint32_t)__shfl_xor((int)rw, 2);
      }
      // the packed word of the group, for the float32 decode only
      uint32_t w = 0;
      if (D > 0 && what_out) {
        const int g0 = lane & ~3;
        w = (uint32_t)__shfl((int)byte, g0) | (uint32_t)__shfl((int)byte, g0 + 1) << 8 |
            (uint32_t)__shfl((int)byte, g0 + 2) << 16 | (uint32_t)__shfl((int)byte, g0 + 3) << 24;
      }
      if (le < rem) {
        if (packed_out) packed_out[(base >> 2) + (le >> 2)] = (uint8_t)byte;
        if (mask_out && !(lane & 1)) mask_out[(base >> 3) + (le >> 3)] = (uint8_t)mpair;
        if (z_out)
          *reinterpret_cast<uint32_t*>(z_out + e) =
              (byte & 3u) | ((byte >> 2) & 3u) << 8 | ((byte >> 4) & 3u) << 16 | (byte >> 6) << 24;
        if (r16_out && q == 0) {
          const int off = off0 + 256 * j + 4 * lane;   // < K + 1024
          int dr, col;
          if (K >= 1024) {
            dr = off >= K;
            col = off - (dr ? (int)K : 0);
          } else {
            dr = (int)((uint32_t)off / (uint32_t)K);
            col = off - dr * (int)K;
          }
          r16_out[r16_blocked_index(row0 + dr, col >> 4, K >> 6)] = rw;
        }
        if (D > 0 && what_out) {
          // What[n, g*d+i] = B[i] + sum_j A[i][j] z[n, g*d+j], in float32.
          float o[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int p = 4 * q + t;             // position in the 16-group
            const int v0 = (p / DD) * DD, i = p % DD;
            float sacc = B[i];
#pragma unroll
            for (int jj = 0; jj < DD; ++jj)
              sacc = __builtin_fmaf(A[i * DD + jj], (float)((w >> (2 * (v0 + jj))) & 3u), sacc);
            o[t] = sacc;
          }
          *reinterpret_cast<float4*>(what_out + e) = make_float4(o[0], o[1], o[2], o[3]);
        }
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void k_quantize(
    const float* __restrict__ wp, int64_t total, int64_t K, uint8_t* __restrict__ z_out,
    uint8_t* __restrict__ packed_out, uint8_t* __restrict__ mask_out,
    uint32_t* __restrict__ r16_out, float* __restrict__ what_out, const float* __restrict__ A,
    const float* __restrict__ B) {
  quantize_body<D>(blockIdx.x, gridDim.x, wp, total, K, z_out, packed_out, mask_out, r16_out,
                   what_out, A, B);
}

// ------------------------------------------------------------------ pack / unpack
// Code k = 4b + t of a row goes to bits [2t, 2t+1] of byte b. A dword of four one-byte
// codes packs into one byte, and a packed byte unpacks into one dword:
__device__ __forceinline__ uint32_t pack_dword(uint32_t w) {
  const uint32_t x = w & 0x03030303u;              // codes in bits 0-1 of each byte
  const uint32_t y = (x | (x >> 6)) & 0x000F000Fu; // bytes 0 and 2: two codes each
  return (y | (y >> 12)) & 0xFFu;
}
__device__ __forceinline__ uint32_t unpack_byte(uint32_t b) {
  const uint32_t y = (b | (b << 12)) & 0x000F000Fu;
  return (y | (y << 6)) & 0x03030303u;
}
__device__ __forceinline__ uint32_t pack_group(const u32x4& q) {   // 16 codes -> 1 word
  return pack_dword(q[0]) | (pack_dword(q[1]) << 8) | (pack_dword(q[2]) << 16) |
         (pack_dword(q[3]) << 24);
}
__device__ __forceinline__ u32x4 unpack_group(uint32_t p) {       // 1 word -> 16 codes
  return u32x4{unpack_byte(p & 0xFFu), unpack_byte((p >> 8) & 0xFFu),
               unpack_byte((p >> 16) & 0xFFu), unpack_byte(p >> 24)};
}

// A group is 16 codes (16 bytes unpacked, one 4-byte word packed). Each wave takes
// chunks of 256 consecutive groups: lane l handles groups 64 j + l, j = 0..3, with the
// four loads issued together, so that every load and store instruction of the wave covers
// one contiguous run (1 KiB of codes or 256 bytes of words) and each lane keeps four
// loads in flight. Groups past the end read the last group and are not stored.
constexpr int PACK_CHUNK = 256;
__global__ __launch_bounds__(256) void k_pack2b(const uint8_t* __restrict__ z, int64_t groups,
                                                uint32_t* __restrict__ packed) {
  const int lane = threadIdx.x & 63;
  const int64_t nchunks = (groups + PACK_CHUNK - 1) / PACK_CHUNK;
  const u32x4* zi = reinterpret_cast<const u32x4*>(z);
  for (int64_t c = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); c < nchunks;
       c += (int64_t)gridDim.x * 4) {
    u32x4 q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t g = c * PACK_CHUNK + 64 * j + lane;
      q[j] = __builtin_nontemporal_load(zi + (g < groups ? g : groups - 1));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t g = c * PACK_CHUNK + 64 * j + lane;
      if (g < groups) packed[g] = pack_group(q[j]);
    }
  }
}

// The inverse, with the same chunks: four 4-byte loads and four 16-byte stores per lane.
__global__ __launch_bounds__(256) void k_unpack2b(const uint32_t* __restrict__ packed,
                                                  int64_t groups, uint8_t* __restrict__ z) {
  const int lane = threadIdx.x & 63;
  const int64_t nchunks = (groups + PACK_CHUNK - 1) / PACK_CHUNK;
  u32x4* zo = reinterpret_cast<u32x4*>(z);
  for (int64_t c = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); c < nchunks;
       c += (int64_t)gridDim.x * 4) {
    uint32_t p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t g = c * PACK_CHUNK + 64 * j + lane;
      p[j] = __builtin_nontemporal_load(packed + (g < groups ? g : groups - 1));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t g = c * PACK_CHUNK + 64 * j + lane;
      if (g < groups) zo[g] = unpack_group(p[j]);
    }
  }
}

// ------------------------------------------------------------------ transposed codes
// Canonical packed [N][K/4] -> R16 words along n, blocked for the dX product whose
// operand rows are k: word (k, n/16) of the blocked layout with contraction length N.
// One block handles 64 rows n x 256 columns k: the 64 x 16 packed words go through LDS
// and each thread then assembles the words of one column k for the 4 groups of 16 n.
__device__ __forceinline__ void r16t_body(int bx, int by, const uint8_t* __restrict__ packed,
                                          int64_t N, int64_t K, uint32_t* __restrict__ r16t) {
  __shared__ uint32_t tile[64][17];
  const int tid = threadIdx.x;
  const int64_t n0 = (int64_t)by * 64, k0 = (int64_t)bx * 256;
  const int kcols = K - k0 < 256 ? (int)(K - k0) : 256;   // a multiple of 64
  {
    const int nr = tid >> 2, kq = tid & 3;
    uint4 w = make_uint4(0, 0, 0, 0);
    if (kq * 64 < kcols)
      w = *reinterpret_cast<const uint4*>(packed + (n0 + nr) * (K >> 2) + (k0 >> 2) + kq * 16);
    tile[nr][kq * 4 + 0] = w.x;
    tile[nr][kq * 4 + 1] = w.y;
    tile[nr][kq * 4 + 2] = w.z;
    tile[nr][kq * 4 + 3] = w.w;
  }
  __syncthreads();
  const int kr = tid;                       // column k0 + kr
  if (kr >= kcols) return;
  const int sh = 2 * (kr & 15), wc = kr >> 4;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    uint32_t c[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) c[t] = (tile[16 * g + t][wc] >> sh) & 3u;
    r16t[r16_blocked_index(k0 + kr, (n0 >> 4) + g, N >> 6)] = r16_encode(c);
  }
}

__global__ __launch_bounds__(256) void k_codes_to_r16t(const uint8_t* __restrict__ packed,
                                                       int64_t N, int64_t K,
                                                       uint32_t* __restrict__ r16t) {
  r16t_body(blockIdx.x, blockIdx.y, packed, N, K, r16t);
}

// ------------------------------------------------------------------ block reduction
__device__ __forceinline__ float block_sum_256(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

template <typename T> __device__ __forceinline__ void load16(const T* p, float out[16]);
template <> __device__ __forceinline__ void load16<uint16_t>(const uint16_t* p, float out[16]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  const uint4 a = q[0], b = q[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) { out[2 * i] = bf16lo_to_f32(w[i]); out[2 * i + 1] = bf16hi_to_f32(w[i]); }
}
template <> __device__ __forceinline__ void load16<float>(const float* p, float out[16]) {
  const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) { float4 f = q[i]; out[4*i] = f.x; out[4*i+1] = f.y; out[4*i+2] = f.z; out[4*i+3] = f.w; }
}

// ------------------------------------------------------------------ forward prologue
// Folds A into the activations (exact algebra, see the GEMM):
//   X'[m, g*d+j] = sum_i X[m, g*d+i] A[i][j]          rounded to bf16 -> X'b
//   xs[m, k]     = 2 * X'b[m, k]                        (bf16, exact)
//   beta[m]      = sum_k X[m, k] B[k % d] - 4 sum_k X'b[m, k]
// so that Y[m, n] = sum_k xs[m, k] v(z[n, k]) + beta[m], with v(c) = 2 + c/2.
// With float32 activations X' is kept to about 16 bits: xs_lo = 2 bf16(X' - X'b) is a
// second operand added by a second pass of the product, and beta uses X'b + X'lo.
// One block per row m; each thread takes 16 consecutive columns per step.
template <typename T, int D>
__device__ __forceinline__ void fwd_prologue_body(int64_t m, const T* __restrict__ X, int64_t K,
                                                      const float* __restrict__ A,
                                                      const float* __restrict__ B,
                                                      uint16_t* __restrict__ xs,
                                                      uint16_t* __restrict__ xs_lo,
                                                      float* __restrict__ beta) {
  __shared__ float red[4];
  __shared__ float Asm[D * D], Bsm[D];
  __shared__ float xsl[D > 8 ? 256 * 17 : 1];     // d = 16: each thread's 16 inputs (padded)
  // A and B are the same for every lane: for d <= 8 they are read with scalar loads into
  // scalar registers (64 + 8 values), which keeps the vector registers for the data;
  // for d = 16 they are staged in LDS.
  const float* As = A;
  const float* Bs = B;
  if (D > 8) {
    if (threadIdx.x < D * D) Asm[threadIdx.x] = A[threadIdx.x];
    if (threadIdx.x < D) Bsm[threadIdx.x] = B[threadIdx.x];
    __syncthreads();
    As = Asm;
    Bs = Bsm;
  }
  const T* xrow = X + m * K;
  uint16_t* orow = xs + m * K;
  float acc = 0.f;
  for (int64_t c = threadIdx.x; c < (K >> 4); c += blockDim.x) {
    float x[16];
    load16<T>(xrow + c * 16, x);
    float xp[16];
    if (D <= 8) {
#pragma unroll
      for (int v0 = 0; v0 < 16; v0 += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
          float sum = 0.f;
#pragma unroll
          for (int i = 0; i < D; ++i) sum = __builtin_fmaf(x[v0 + i], As[i * D + j], sum);
          xp[v0 + j] = sum;
        }
      }
    } else {
      // One row of A at a time from LDS, so that only the 16 outputs stay in registers.
      // The row index runs at run time, so x[i] is read back from the thread's own LDS
      // slot rather than selected among 16 registers.
      float* xt = xsl + threadIdx.x * 17;
#pragma unroll
      for (int j = 0; j < 16; ++j) xt[j] = x[j];
#pragma unroll
      for (int j = 0; j < 16; ++j) xp[j] = 0.f;
#pragma unroll 1
      for (int i = 0; i < D; ++i) {
        const float xi = xt[i];
#pragma unroll
        for (int j = 0; j < 16; ++j) xp[j] = __builtin_fmaf(xi, As[i * D + j], xp[j]);
      }
    }
#pragma unroll
    for (int v0 = 0; v0 < 16; v0 += D) {
#pragma unroll
      for (int i = 0; i < D; ++i) acc = __builtin_fmaf(x[v0 + i], Bs[i], acc);
    }
    uint32_t o[8], ol[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t pb = pack_bf16x2(xp[2 * i], xp[2 * i + 1]);
      const float e0 = bf16lo_to_f32(pb), e1 = bf16hi_to_f32(pb);
      o[i] = pack_bf16x2(2.f * e0, 2.f * e1);
      if (xs_lo) {
        const uint32_t pl = pack_bf16x2(xp[2 * i] - e0, xp[2 * i + 1] - e1);
        const float l0 = bf16lo_to_f32(pl), l1 = bf16hi_to_f32(pl);
        ol[i] = pack_bf16x2(2.f * l0, 2.f * l1);
        acc -= 4.f * ((e0 + l0) + (e1 + l1));
      } else {
        acc -= 4.f * (e0 + e1);
      }
    }
    uint4* dst = reinterpret_cast<uint4*>(orow + c * 16);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    if (xs_lo) {
      uint4* dl = reinterpret_cast<uint4*>(xs_lo + m * K + c * 16);
      dl[0] = make_uint4(ol[0], ol[1], ol[2], ol[3]);
      dl[1] = make_uint4(ol[4], ol[5], ol[6], ol[7]);
    }
  }
  const float sum = block_sum_256(acc, red);
  if (threadIdx.x == 0) beta[m] = sum;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void k_fwd_prologue(const T* __restrict__ X, int64_t K,
                                                      const float* __restrict__ A,
                                                      const float* __restrict__ B,
                                                      uint16_t* __restrict__ xs,
                                                      uint16_t* __restrict__ xs_lo,
                                                      float* __restrict__ beta) {
  fwd_prologue_body<T, D>(blockIdx.x, X, K, A, B, xs, xs_lo, beta);
}

// ------------------------------------------------------------------ backward prologue
// r[m] = sum_n dY[m, n] (float32). With float32 activations, also splits dY and X into
// bf16 pairs hi + lo (hi = bf16(x), lo = bf16(x - hi)) for the matrix-core products,
// which then add the cross terms in extra passes.
__device__ __forceinline__ void split16(const float x[16], uint16_t* hi, uint16_t* lo) {
  uint32_t h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    l[i] = pack_bf16x2(x[2 * i] - bf16lo_to_f32(h[i]), x[2 * i + 1] - bf16hi_to_f32(h[i]));
  }
  uint4* dh = reinterpret_cast<uint4*>(hi);
  uint4* dl = reinterpret_cast<uint4*>(lo);
  dh[0] = make_uint4(h[0], h[1], h[2], h[3]);
  dh[1] = make_uint4(h[4], h[5], h[6], h[7]);
  dl[0] = make_uint4(l[0], l[1], l[2], l[3]);
  dl[1] = make_uint4(l[4], l[5], l[6], l[7]);
}

template <typename T>
__device__ __forceinline__ void bwd_prologue_body(int64_t m, const T* __restrict__ dY,
                                                  const T* __restrict__ X, int64_t N,
                                                  int64_t K, float* __restrict__ r,
                                                  uint16_t* __restrict__ dy_hi,
                                                  uint16_t* __restrict__ dy_lo,
                                                  uint16_t* __restrict__ x_hi,
                                                  uint16_t* __restrict__ x_lo) {
  __shared__ float red[4];
  float acc = 0.f;
  for (int64_t c = threadIdx.x; c < (N >> 4); c += blockDim.x) {
    float y[16];
    load16<T>(dY + m * N + c * 16, y);
    if (dy_hi) split16(y, dy_hi + m * N + c * 16, dy_lo + m * N + c * 16);
#pragma unroll
    for (int i = 0; i < 16; ++i) acc += y[i];
  }
  if (x_hi) {
    for (int64_t c = threadIdx.x; c < (K >> 4); c += blockDim.x) {
      float x[16];
      load16<T>(X + m * K + c * 16, x);
      split16(x, x_hi + m * K + c * 16, x_lo + m * K + c * 16);
    }
  }
  const float s = block_sum_256(acc, red);
  if (threadIdx.x == 0) r[m] = s;
}

// r[m] = sum_n dY[m, n] for bf16 dY: one wave per row. Every lane issues all of its
// 16-byte loads of a sweep before using any (clamped addresses, no branch, so none of
// them is waited for early), then the wave adds its lanes. N is a multiple of 64.
constexpr int ROWSUM_U = 8;                   // loads in flight per lane
__device__ __forceinline__ void rowsum_bf16_wave(int64_t m, const uint16_t* __restrict__ dY,
                                                 int64_t N, float* __restrict__ r, int lane) {
  const uint4* row = reinterpret_cast<const uint4*>(dY + m * N);
  const int64_t chunks = N >> 3;              // 8 bf16 per 16 bytes
  float acc = 0.f;
  for (int64_t c0 = 0; c0 < chunks; c0 += 64 * ROWSUM_U) {
    uint4 v[ROWSUM_U];
#pragma unroll
    for (int u = 0; u < ROWSUM_U; ++u) v[u] = row[min(c0 + u * 64 + lane, chunks - 1)];
#pragma unroll
    for (int u = 0; u < ROWSUM_U; ++u) {
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) t += bf16lo_to_f32(w[i]) + bf16hi_to_f32(w[i]);
      acc += c0 + u * 64 + lane < chunks ? t : 0.f;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) r[m] = acc;
}

// ------------------------------------------------------------------ merged launches
// Work that does not depend on each other shares one launch: block ranges of one grid
// run the two parts, which saves a kernel boundary and lets the VALU-bound quantizer
// overlap the memory-bound prologue.
//   forward:  blocks [0, qblocks) quantize, then one block per activation row m;
//   backward: the blocks of the transposed codes (VALU work, first so that it overlaps
//             the rest), then the row blocks (r = dY 1; bf16: 4 rows per block, one per
//             wave; float32, which also writes the hi/lo splits: one row per block).
template <typename T, int DQ, int D>
__global__ __launch_bounds__(256) void k_fwd_prep(const float* __restrict__ wp, int64_t total,
                                                  int64_t K, uint8_t* __restrict__ packed,
                                                  uint8_t* __restrict__ mask,
                                                  uint32_t* __restrict__ r16,
                                                  float* __restrict__ what, int qblocks,
                                                  const T* __restrict__ X, int64_t KX,
                                                  const float* __restrict__ A,
                                                  const float* __restrict__ B,
                                                  uint16_t* __restrict__ xs,
                                                  uint16_t* __restrict__ xs_lo,
                                                  float* __restrict__ beta) {
  if ((int)blockIdx.x < qblocks)
    quantize_body<DQ>(blockIdx.x, qblocks, wp, total, K, nullptr, packed, mask, r16, what, A, B);
  else
    fwd_prologue_body<T, D>((int64_t)blockIdx.x - qblocks, X, KX, A, B, xs, xs_lo, beta);
}

template <typename T> constexpr int bwd_rows_per_block() { return sizeof(T) == 2 ? 4 : 1; }

template <typename T>
__global__ __launch_bounds__(256) void k_bwd_prep(const T* __restrict__ dY,
                                                  const T* __restrict__ X, int64_t M,
                                                  int64_t N, int64_t K, float* __restrict__ r,
                                                  uint16_t* __restrict__ dy_hi,
                                                  uint16_t* __restrict__ dy_lo,
                                                  uint16_t* __restrict__ x_hi,
                                                  uint16_t* __restrict__ x_lo,
                                                  const uint8_t* __restrict__ packed,
                                                  uint32_t* __restrict__ r16t, int kblocks,
                                                  int tblocks) {
  constexpr int RPB = bwd_rows_per_block<T>();
  if ((int64_t)blockIdx.x < tblocks) {
    const int vb = (int)blockIdx.x;
    r16t_body(vb % kblocks, vb / kblocks, packed, N, K, r16t);
  } else {
    const int64_t rb = (int64_t)blockIdx.x - tblocks;
    if constexpr (RPB == 4) {
      const int64_t m = rb * 4 + (threadIdx.x >> 6);
      if (m < M) rowsum_bf16_wave(m, dY, N, r, threadIdx.x & 63);
    } else {
      bwd_prologue_body<T>(rb, dY, X, N, K, r, dy_hi, dy_lo, x_hi, x_lo);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_bwd_prologue(const T* __restrict__ dY,
                                                      const T* __restrict__ X, int64_t N,
                                                      int64_t K, float* __restrict__ r,
                                                      uint16_t* __restrict__ dy_hi,
                                                      uint16_t* __restrict__ dy_lo,
                                                      uint16_t* __restrict__ x_hi,
                                                      uint16_t* __restrict__ x_lo) {
  bwd_prologue_body<T>(blockIdx.x, dY, X, N, K, r, dy_hi, dy_lo, x_hi, x_lo);
}

// ------------------------------------------------------------------ launchers
static int grid_for(int64_t groups) {
  int64_t g = (groups + 255) / 256;
  if (g > 65536) g = 65536;
  return (int)(g < 1 ? 1 : g);
}

hipError_t launch_quantize(const float* wp, int64_t N, int64_t K, uint8_t* z, uint8_t* packed,
                           uint8_t* mask, uint32_t* r16, float* what, const float* A,
                           const float* B, int d, hipStream_t s) {
  const int64_t total = N * K;
  int64_t blocks = ((total + 1023) / 1024 + 3) / 4;
  if (blocks > 65535) blocks = 65535;
  if (blocks < 1) blocks = 1;
  const dim3 g((unsigned)blocks);
  if (!what) {
    LCVQ_LAUNCH(PROF_QUANTIZE, k_quantize<0>, g, dim3(256), 0, s, wp, total, K, z, packed, mask,
                r16, what, A, B);
  } else if (d == 4) {
    LCVQ_LAUNCH(PROF_QUANTIZE, k_quantize<4>, g, dim3(256), 0, s, wp, total, K, z, packed, mask,
                r16, what, A, B);
  } else if (d == 8) {
    LCVQ_LAUNCH(PROF_QUANTIZE, k_quantize<8>, g, dim3(256), 0, s, wp, total, K, z, packed, mask,
                r16, what, A, B);
  } else {
    LCVQ_LAUNCH(PROF_QUANTIZE, k_quantize<16>, g, dim3(256), 0, s, wp, total, K, z, packed, mask,
                r16, what, A, B);
  }
  return hipGetLastError();
}

// pack / unpack: one workgroup of four waves per 4 chunks of 256 groups
hipError_t launch_pack2b(const uint8_t* z, int64_t N, int64_t K, uint8_t* packed, hipStream_t s) {
  const int64_t groups = N * K / 16;
  LCVQ_LAUNCH(PROF_PACK, k_pack2b, dim3(grid_for((groups + 3) / 4)), dim3(256), 0, s, z, groups,
              reinterpret_cast<uint32_t*>(packed));
  return hipGetLastError();
}

hipError_t launch_unpack2b(const uint8_t* packed, int64_t N, int64_t K, uint8_t* z, hipStream_t s) {
  const int64_t groups = N * K / 16;
  LCVQ_LAUNCH(PROF_UNPACK, k_unpack2b, dim3(grid_for((groups + 3) / 4)), dim3(256), 0, s,
              reinterpret_cast<const uint32_t*>(packed), groups, z);
  return hipGetLastError();
}

hipError_t launch_codes_to_r16t(const uint8_t* packed, int64_t N, int64_t K, uint32_t* r16t,
                                hipStream_t s) {
  hipLaunchKernelGGL(k_codes_to_r16t, dim3((unsigned)((K + 255) / 256), (unsigned)(N / 64)), dim3(256), 0,
                     s, packed, N, K, r16t);
  return hipGetLastError();
}

template <int D>
static void fwd_prologue_d(const void* X, bool x_f32, int64_t M, int64_t K, const float* A,
                           const float* B, uint16_t* xs, uint16_t* xs_lo, float* beta,
                           hipStream_t s) {
  if (x_f32)
    hipLaunchKernelGGL((k_fwd_prologue<float, D>), dim3((unsigned)M), dim3(256), 0, s,
                       static_cast<const float*>(X), K, A, B, xs, xs_lo, beta);
  else
    hipLaunchKernelGGL((k_fwd_prologue<uint16_t, D>), dim3((unsigned)M), dim3(256), 0, s,
                       static_cast<const uint16_t*>(X), K, A, B, xs, (uint16_t*)nullptr, beta);
}

hipError_t launch_fwd_prologue(const void* X, bool x_f32, int64_t M, int64_t K, const float* A,
                               const float* B, int d, uint16_t* xs, uint16_t* xs_lo,
                               float* beta, hipStream_t s) {
  if (d == 4) fwd_prologue_d<4>(X, x_f32, M, K, A, B, xs, xs_lo, beta, s);
  else if (d == 8) fwd_prologue_d<8>(X, x_f32, M, K, A, B, xs, xs_lo, beta, s);
  else fwd_prologue_d<16>(X, x_f32, M, K, A, B, xs, xs_lo, beta, s);
  return hipGetLastError();
}

static int quantize_blocks(int64_t total) {
  int64_t blocks = ((total + 1023) / 1024 + 3) / 4;
  if (blocks > 65535) blocks = 65535;
  return (int)(blocks < 1 ? 1 : blocks);
}

template <typename T, int DQ, int D>
static void fwd_prep_launch(const float* wp, int64_t N, int64_t K, uint8_t* packed, uint8_t* mask,
                            uint32_t* r16, float* what, const T* X, int64_t M, const float* A,
                            const float* B, uint16_t* xs, uint16_t* xs_lo, float* beta,
                            hipStream_t s) {
  const int qb = quantize_blocks(N * K);
  LCVQ_LAUNCH(PROF_QUANTIZE, (k_fwd_prep<T, DQ, D>), dim3((unsigned)(qb + M)), dim3(256), 0, s,
              wp, N * K, K, packed, mask, r16, what, qb, X, K, A, B, xs, xs_lo, beta);
}

template <typename T, int D>
static void fwd_prep_t(const float* wp, int64_t N, int64_t K, uint8_t* packed, uint8_t* mask,
                       uint32_t* r16, float* what, const void* X, int64_t M, const float* A,
                       const float* B, uint16_t* xs, uint16_t* xs_lo, float* beta,
                       hipStream_t s) {
  const T* x = static_cast<const T*>(X);
  if (what)
    fwd_prep_launch<T, D, D>(wp, N, K, packed, mask, r16, what, x, M, A, B, xs, xs_lo, beta, s);
  else
    fwd_prep_launch<T, 0, D>(wp, N, K, packed, mask, r16, what, x, M, A, B, xs, xs_lo, beta, s);
}

template <int D>
static void fwd_prep_d(const float* wp, int64_t N, int64_t K, uint8_t* packed, uint8_t* mask,
                       uint32_t* r16, float* what, const void* X, bool x_f32, int64_t M,
                       const float* A, const float* B, uint16_t* xs, uint16_t* xs_lo,
                       float* beta, hipStream_t s) {
  if (x_f32)
    fwd_prep_t<float, D>(wp, N, K, packed, mask, r16, what, X, M, A, B, xs, xs_lo, beta, s);
  else
    fwd_prep_t<uint16_t, D>(wp, N, K, packed, mask, r16, what, X, M, A, B, xs, nullptr, beta, s);
}

hipError_t launch_fwd_prep(const float* wp, int64_t N, int64_t K, uint8_t* packed, uint8_t* mask,
                           uint32_t* r16, float* what, const void* X, bool x_f32, int64_t M,
                           const float* A, const float* B, int d, uint16_t* xs,
                           uint16_t* xs_lo, float* beta, hipStream_t s) {
  if (d == 4) fwd_prep_d<4>(wp, N, K, packed, mask, r16, what, X, x_f32, M, A, B, xs, xs_lo, beta, s);
  else if (d == 8) fwd_prep_d<8>(wp, N, K, packed, mask, r16, what, X, x_f32, M, A, B, xs, xs_lo, beta, s);
  else fwd_prep_d<16>(wp, N, K, packed, mask, r16, what, X, x_f32, M, A, B, xs, xs_lo, beta, s);
  return hipGetLastError();
}

hipError_t launch_bwd_prep(const void* dY, const void* X, bool f32, int64_t M, int64_t N,
                           int64_t K, float* r, uint16_t* dy_hi, uint16_t* dy_lo,
                           uint16_t* x_hi, uint16_t* x_lo, const uint8_t* packed,
                           uint32_t* r16t, hipStream_t s) {
  const int kblocks = (int)((K + 255) / 256);
  const int64_t rb = r16t ? (int64_t)kblocks * (N / 64) : 0;
  const int rpb = f32 ? bwd_rows_per_block<float>() : bwd_rows_per_block<uint16_t>();
  const dim3 g((unsigned)((M + rpb - 1) / rpb + rb)), b(256);
  if (f32)
    LCVQ_LAUNCH(PROF_BWD_PREP, k_bwd_prep<float>, g, b, 0, s, static_cast<const float*>(dY),
                static_cast<const float*>(X), M, N, K, r, dy_hi, dy_lo, x_hi, x_lo, packed,
                r16t, kblocks, (int)rb);
  else
    LCVQ_LAUNCH(PROF_BWD_PREP, k_bwd_prep<uint16_t>, g, b, 0, s,
                static_cast<const uint16_t*>(dY), static_cast<const uint16_t*>(X), M, N, K, r,
                (uint16_t*)nullptr, (uint16_t*)nullptr, (uint16_t*)nullptr, (uint16_t*)nullptr,
                packed, r16t, kblocks, (int)rb);
  return hipGetLastError();
}

hipError_t launch_bwd_prologue(const void* dY, const void* X, bool f32, int64_t M, int64_t N,
                               int64_t K, float* r, uint16_t* dy_hi, uint16_t* dy_lo,
                               uint16_t* x_hi, uint16_t* x_lo, hipStream_t s) {
  if (f32)
    hipLaunchKernelGGL(k_bwd_prologue<float>, dim3((unsigned)M), dim3(256), 0, s,
                       static_cast<const float*>(dY), static_cast<const float*>(X), N, K, r,
                       dy_hi, dy_lo, x_hi, x_lo);
  else
    hipLaunchKernelGGL(k_bwd_prologue<uint16_t>, dim3((unsigned)M), dim3(256), 0, s,
                       static_cast<const uint16_t*>(dY), static_cast<const uint16_t*>(X), N,
                       K, r, (uint16_t*)nullptr, (uint16_t*)nullptr, (uint16_t*)nullptr,
                       (uint16_t*)nullptr);
  return hipGetLastError();
}

}  // namespace lcvq
