// Matrix-core products of the LC-VQ layer on gfx950 (bf16 MFMA, float32 accumulate).
//
// The decode c = A z + B (LC-QAT summary, Methodology 1) is linear, so A and B are moved
// off the weight operand and the products run directly on the 2-bit codes; the summary's
// training pipeline likewise reorganises the computation around INT2 x FP16 matrix
// products (Methodology 3):
//   forward  Y  = X What^T            = X' Z^T + (X (1 kron B)) 1^T,   X' = X (I kron A)
//   dX          = dY What             = (dY Z)(I kron A^T) + (dY 1)(1 kron B)^T
//   dWp, dA, dB from G = dY^T X       (straight-through epilogue on the accumulators)
// A code c enters a product as v(c) = 2 + c/2, exact in bf16 (see codes_expand); the
// constant part is removed through the row terms prepared by the prologue kernels.
//
// Two kernel templates cover the three products (k_gemm_ring: forward and dX; k_gemm_dw).
// C (P x Q) = sum_r L[p, r] R[q, r] is computed in 256 x 256 tiles (32x32x16 bf16 MFMA,
// contraction staged through LDS in steps of 64):
//   FWD: L = X' (bf16 rows m),        R = codes (rows n)       8 waves, 4-slot LDS ring
//   DX : L = codes transposed (rows k), R = dY (bf16 rows m)   8 waves, 4-slot LDS ring
//   DW : L = X^T (rows k), R = dY^T (rows n); both tiles arrive in their natural layout
//        and are transposed by the LDS reads; 8 waves, double buffer.
// With 8 waves two waves share each SIMD, so one wave's LDS waits and code expansion
// overlap the other wave's MFMAs.
#include "lcvq_device.h"
#include "lcvq_internal.h"

namespace lcvq {

constexpr int BT = 256;        // C tile edge
constexpr int BK = 64;         // contraction per stage
constexpr int ROWB = 128;      // bytes per LDS tile row (64 bf16)
constexpr int TILEB = BT * ROWB;

enum { OP_FWD = 0, OP_DX = 1, OP_DW = 2 };

// Waves per workgroup of the forward and dX products (4 or 8).
#ifndef LCVQ_FWD_WAVES
#define LCVQ_FWD_WAVES 8
#endif
#ifndef LCVQ_DX_WAVES
#define LCVQ_DX_WAVES 8
#endif
// Wave rows of the 8-wave forward product (2: waves own 128 x 64, 4: 64 x 128).
#ifndef LCVQ_FWD_WGP
#define LCVQ_FWD_WGP 2
#endif

// Wave layout of the 8-wave products: WGP wave rows x WGQ wave columns; a wave owns
// 32*WI rows and 32*WJ columns of the C tile. The operand made of codes is spread over
// the wave dimension with fewer waves, so that each wave expands as few code fragments
// as possible (forward: codes are columns; dX: codes are rows).
// With 4 waves (one per SIMD) each wave owns a 128 x 128 quarter of the tile: 16
// accumulator blocks of 32 x 32 (256 values, held in the accumulation registers) and 4
// + 4 operand fragments per contraction sub-step, i.e. fewer LDS bytes per MFMA.
template <int OP, int NWV = 8> struct Tiling {
  static constexpr int NW = NWV;
  static constexpr int WGP = NW == 4 ? 2 : (OP == OP_DX ? 4 : LCVQ_FWD_WGP);
  static constexpr int WGQ = NW / WGP;
  static constexpr int WI = 8 / WGP;
  static constexpr int WJ = 8 / WGQ;
};

struct GemmArgs {
  int P, Q, R;                 // C is P x Q; contraction length R
  int tilesP, tilesQ, ntiles;
  // Operand matrices per pass. bf16 activations need one pass; float32 activations are
  // split into bf16 hi + lo and the products add hi*hi + lo*hi (+ hi*lo) over 2-3 passes.
  const uint16_t* Lmat[3];     // FWD: X' [M][K]; DW: X [M][K]
  const uint16_t* Rmat[3];     // DX, DW: dY [M][N]
  int npass;
  const uint32_t* codes;       // FWD: R16 of Z along k; DX: R16 of Z^T along n (blocked)
  int M, N, K;
  const float* rowvec;         // FWD: beta [M]; DX: r [M]
  const float* A;              // [d][d]
  const float* B;              // [d]
  void* out;                   // FWD: Y [M][N]; DX: dX [M][K]
  int out_f32;
  float* dwp;                  // DW: [N][K]
  const uint8_t* packed;       // DW: canonical codes [N][K/4]
  const uint8_t* mask;         // DW: mask bits [N][K/8]
  float* partials;             // DW: [ntiles][d*d + d]
  const float* dge_wp;         // DW with the DGE estimator: proxies [N][K], else NULL
  // DX launched after DW: the DW tiles' dA/dB partials [red_tiles][d*d + d] to reduce
  // into red_dA, red_dB (NULL: nothing to reduce)
  const float* red_partials;
  int red_tiles;
  float* red_dA;
  float* red_dB;
  float dge_alpha, dge_c;      // sharpness and alpha / (2 tanh(alpha / 2))
};

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * ROWB + ((chunk ^ swz(row)) << 4); }

// Tiles are spread so that consecutive workgroup ids land on different XCDs (the
// dispatcher deals workgroups round-robin over the 8 XCDs) while each XCD works on a
// compact group of GR tile-rows, which keeps its operand panels in its own L2.
template <int GR>
__device__ __forceinline__ bool map_tile(int b, int tilesP, int tilesQ, int ntiles, int& tp, int& tq, int& t) {
  const int per = (ntiles + 7) >> 3;
  t = (b & 7) * per + (b >> 3);
  if (t >= ntiles) return false;
  const int group = t / (GR * tilesQ);
  const int within = t - group * GR * tilesQ;
  int rows = tilesP - group * GR;
  if (rows > GR) rows = GR;
  tp = group * GR + within % rows;
  tq = within / rows;
  return true;
}

__device__ __forceinline__ void store_out4(void* out, int f32, int64_t idx, float a, float b, float c, float d) {
  if (f32) {
    __builtin_nontemporal_store(f32x4{a, b, c, d},
                                reinterpret_cast<f32x4*>(static_cast<float*>(out) + idx));
  } else {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + idx) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
  }
}

// ---- epilogues -----------------------------------------------------------------------
// Outputs (Y, dX, dWp) are written once and not read again by the kernel: they go out as
// non-temporal stores, which measured 1-3 us faster per product than ordinary ones.
// Accumulator layout (32x32 block): lane l holds column l%32 and, in register r, row
// 8*(r/4) + 4*(l/32) + r%4. For DX and DW the rows run along the d-vectors: a swap of
// register halves between lanes l and l^32 (gather_dvectors) gives every lane whole
// d-vectors, the d x d mix runs in registers, and the results go through a per-wave
// LDS area (rows of 33 floats) only to be written back transposed, each group of 8
// lanes covering consecutive elements of one output row. The forward epilogue stages
// row-major strips the same way for 16-byte stores.

constexpr int SROW = 33;                  // padded row of the staging area (floats)

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding; the other counters are not waited on.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Writes a staged 32 x 32 block (rows = contraction-side index k, columns = output row)
// transposed to out[row][k] (row stride ld elements), float32 or bf16.
__device__ __forceinline__ void store_block_rows(const float* S, void* out, int f32, int64_t ld,
                                                 int row0, int rows, int k0, int K, int lane) {
  const int kq = (lane & 7) * 4;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int rr = it * 8 + (lane >> 3);
    const int row = row0 + rr;
    if (row < rows && k0 + kq < K) {
      const float v0 = S[(kq + 0) * SROW + rr], v1 = S[(kq + 1) * SROW + rr];
      const float v2 = S[(kq + 2) * SROW + rr], v3 = S[(kq + 3) * SROW + rr];
      store_out4(out, f32, (int64_t)row * ld + k0 + kq, v0, v1, v2, v3);
    }
  }
}

// Slope of the DGE curve s(w) = floor(w) + 1/2 + tanh(alpha (f - 1/2)) / (2 tanh(alpha/2)),
// f = w - floor(w): c (1 - tanh^2(alpha (f - 1/2))) with c = alpha / (2 tanh(alpha / 2)).
// Zero for non-finite proxies (the clamp masks them).
__device__ __forceinline__ float dge_slope(float w, float alpha, float c) {
  if (!__builtin_isfinite(w)) return 0.f;
  const float t = tanhf(alpha * ((w - floorf(w)) - 0.5f));
  return c * (1.f - t * t);
}

// store_block_rows for dWp under the DGE estimator: each value is multiplied by the
// slope at its proxy, read as the same 4 consecutive floats of Wp [N][K]. All four
// proxy loads are issued before the first store: the compiler cannot move a load of Wp
// above a store to dWp (they might alias), and one HBM round trip per store would
// serialize the epilogue. (Loading a block ahead of its store spills the epilogue.)
__device__ __forceinline__ void store_block_rows_dge(const float* S, float* out, const float* wp,
                                                     float alpha, float c, int64_t ld, int row0,
                                                     int rows, int k0, int K, int lane) {
  const int kq = (lane & 7) * 4;
  float4 w[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = row0 + it * 8 + (lane >> 3);
    const bool in = row < rows && k0 + kq < K;
    // a valid address either way; values of rows or columns past the end are not used
    const int64_t idx = in ? (int64_t)row * ld + k0 + kq : 0;
    w[it] = *reinterpret_cast<const float4*>(wp + idx);
  }
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int rr = it * 8 + (lane >> 3);
    const int row = row0 + rr;
    if (row < rows && k0 + kq < K) {
      const int64_t idx = (int64_t)row * ld + k0 + kq;
      __builtin_nontemporal_store(f32x4{S[(kq + 0) * SROW + rr] * dge_slope(w[it].x, alpha, c),
                                        S[(kq + 1) * SROW + rr] * dge_slope(w[it].y, alpha, c),
                                        S[(kq + 2) * SROW + rr] * dge_slope(w[it].z, alpha, c),
                                        S[(kq + 3) * SROW + rr] * dge_slope(w[it].w, alpha, c)},
                                  reinterpret_cast<f32x4*>(out + idx));
    }
  }
}

// Forward epilogue: Y[p, q] = C[p, q] + beta[p]. Each 32-row strip of the wave's
// 32 x 32*WJ sub-tile is staged row-major through the wave's LDS area (the ring is
// free by now), then written with 16-byte stores, so that every store instruction
// covers whole 32*WJ-element runs of 16 / WJ output rows.
template <int NW, int WI, int WJ>
__device__ void epilogue_fwd(const GemmArgs& a, f32x16 acc[WI][WJ], int p0, int q0, int wp,
                             int wq, int lane, int wave, uint8_t* smem) {
  constexpr int CW = 32 * WJ, SR = CW + 4;             // strip width, padded LDS row
  constexpr int LPR = CW / 8, RPI = 64 / LPR;          // lanes per row, rows per store
  static_assert(NW * 32 * SR * 4 <= 144 * 1024, "forward staging area");
  float* S = reinterpret_cast<float*>(smem) + wave * 32 * SR;
  const int col = lane & 31, h = lane >> 5;
  const int qb = q0 + wq * CW, c8 = (lane % LPR) * 8, q = qb + c8;
  // All of this lane's beta values are loaded before the first store: vector loads and
  // stores share one counter (vmcnt), so a load issued after a store can only be waited
  // for together with that store.
  constexpr int NIT = 32 / RPI;
  float bv[WI][NIT];
#pragma unroll
  for (int i = 0; i < WI; ++i)
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int p = p0 + wp * 32 * WI + i * 32 + it * RPI + lane / LPR;
      bv[i][it] = a.rowvec[p < a.M ? p : a.M - 1];
    }
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int pb = p0 + wp * 32 * WI + i * 32;
    wave_sync();
#pragma unroll
    for (int j = 0; j < WJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        S[(8 * (r >> 2) + 4 * h + (r & 3)) * SR + j * 32 + col] = acc[i][j][r];
    wave_sync();
    // Settle every beta load here, before the first store: a wait for one of them
    // placed after stores would also wait for those stores to complete.
    if (i == 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int rr = it * RPI + lane / LPR, p = pb + rr;
      if (p < a.M && q < a.N) {
        const float b = bv[i][it];
        const f32x4 x = *reinterpret_cast<const f32x4*>(S + rr * SR + c8);
        const f32x4 y = *reinterpret_cast<const f32x4*>(S + rr * SR + c8 + 4);
        const int64_t idx = (int64_t)p * a.N + q;
        if (a.out_f32) {
          float* o = static_cast<float*>(a.out) + idx;
          __builtin_nontemporal_store(x + b, reinterpret_cast<f32x4*>(o));
          __builtin_nontemporal_store(y + b, reinterpret_cast<f32x4*>(o + 4));
        } else {
          __builtin_nontemporal_store(
              u32x4{pack_bf16x2(x[0] + b, x[1] + b), pack_bf16x2(x[2] + b, x[3] + b),
                    pack_bf16x2(y[0] + b, y[1] + b), pack_bf16x2(y[2] + b, y[3] + b)},
              reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.out) + idx));
        }
      }
    }
  }
}

// Writes a staged 64 x 32 area (rows = contraction-side index k, columns = output row)
// transposed to out[row][k0 .. k0+63] (row stride ld elements), float32 or bf16: each
// group of 8 lanes covers the 64 consecutive k of one output row, 8 per lane.
__device__ __forceinline__ void store_block_rows64(const float* S, void* out, int f32,
                                                   int64_t ld, int row0, int rows, int k0,
                                                   int K, int lane) {
  const int kq = (lane & 7) * 8;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int rr = it * 8 + (lane >> 3);
    const int row = row0 + rr;
    if (row < rows && k0 + kq < K) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = S[(kq + e) * SROW + rr];
      const int64_t idx = (int64_t)row * ld + k0 + kq;
      if (f32) {
        float* o = static_cast<float*>(out) + idx;
        __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(o));
        __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]},
                                    reinterpret_cast<f32x4*>(o + 4));
      } else {
        __builtin_nontemporal_store(
            u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                  pack_bf16x2(v[6], v[7])},
            reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + idx));
      }
    }
  }
}

// Whole d-vectors per lane. In a 32x32 accumulator block, lane (column l%32, half
// h = l/32) holds rows 8*(r/4) + 4h + r%4 in register r: for d = 4 these are complete
// d-vectors already, for d = 8 and 16 each vector is split between lanes l and l^32.
// Swapping registers 0..7 of the upper half with registers 8..15 of the lower half
// (v_permlane32_swap: the first operand's lanes 32..63 trade places with the second
// operand's lanes 0..31) leaves every lane with whole vectors: d = 8, vectors 2h and
// 2h+1; d = 16, vector h. Element e of local vector v then sits in register
// 4*bsel + e%4 with bsel as in dvec_reg.
template <int D>
__device__ __forceinline__ void gather_dvectors(f32x16& c) {
  if (D == 4) return;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(c[r]),
                                                    __float_as_uint(c[r + 8]), false, false);
    c[r] = __uint_as_float(s[0]);
    c[r + 8] = __uint_as_float(s[1]);
  }
}
template <int D>
__host__ __device__ constexpr int dvec_reg(int v, int e) {
  const int j = e >> 2;
  const int bsel = D == 4 ? v : D == 8 ? (j << 1) | v : ((j & 1) << 1) | (j >> 1);
  return 4 * bsel + (e & 3);
}
// Row (index k within the block) of element e of local vector v in lane half h.
template <int D>
__device__ __forceinline__ int dvec_row(int v, int e, int h) {
  const int g = D == 4 ? 2 * v + h : D == 8 ? 2 * h + v : h;
  return g * D + e;
}

// dX[m, g*d+i] = 2 sum_j A[i][j] C[g*d+j, m] + (B[i] - 4 sum_j A[i][j]) r[m]
// where C = sum_n v(z[n, k]) dY[m, n] is the accumulator (rows k, columns m).
// The d x d product runs on whole vectors in registers (gather_dvectors); the results
// go through the wave's LDS area only for the transposed store. Blocks are taken in
// pairs along k, so that each output row receives 128 contiguous bytes (bf16) per
// store instruction.
constexpr int DX_WAVE_LDS = 64 * SROW * 4;   // per-wave staging area: 64 x 33 floats

template <int D, int WI, int WJ>
__device__ void epilogue_dx(const GemmArgs& a, f32x16 acc[WI][WJ], int p0, int q0, int wp, int wq,
                            int lane, float* S, const float* Alds) {
  static_assert(WI % 2 == 0, "k blocks are staged in pairs");
  constexpr int NV = 16 / D;                  // whole vectors per lane and block
  constexpr int IIU = D == 16 ? 4 : D;        // output rows unrolled together
  // row terms B[i] - 4 sum_j A[i][j] (d <= 8; d = 16 keeps them in LDS), read as scalar
  // loads through constant-address-space pointers
  float bp[D];
  if constexpr (D != 16) {
    const LCVQ_CONST float* Ac = (const LCVQ_CONST float*)a.A;
    const LCVQ_CONST float* Bc = (const LCVQ_CONST float*)a.B;
#pragma unroll
    for (int i = 0; i < D; ++i) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < D; ++j) s += Ac[i * D + j];
      bp[i] = Bc[i] - 4.f * s;
    }
  }
  const int q = lane & 31, h = lane >> 5;
  // r of this lane's rows, loaded before the first store (vector loads and stores share
  // one counter, so a load issued after a store is waited for together with it)
  float rmv[WJ];
#pragma unroll
  for (int j = 0; j < WJ; ++j) {
    const int m = q0 + wq * 32 * WJ + j * 32 + q;
    const float r = a.rowvec[m < a.M ? m : a.M - 1];
    rmv[j] = m < a.M ? r : 0.f;
  }
#pragma unroll
  for (int j = 0; j < WJ; ++j)
#pragma unroll
    for (int i2 = 0; i2 < WI / 2; ++i2) {
      const int kb = p0 + wp * 32 * WI + i2 * 64;
      const int mb = q0 + wq * 32 * WJ + j * 32;
      const float rm = rmv[j];
      // Re-read A for every block pair instead of keeping d*d values live across the
      // unrolled sequence: d <= 8 through a constant-address-space pointer, so that the
      // reads are scalar loads from the scalar cache (through a generic pointer they would
      // be vector loads, each waited for); d = 16 from the copy in LDS.
      const LCVQ_CONST float* Ac = (const LCVQ_CONST float*)a.A;
      const LCVQ_LDS float* Al = (const LCVQ_LDS float*)Alds;
      if constexpr (D == 16) asm volatile("" : "+v"(Al));
      else asm volatile("" : "+s"(Ac));
      auto Aat = [&](int idx) -> float {
        if constexpr (D == 16) return Al[idx];
        else return Ac[idx];
      };
      wave_sync();
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        f32x16& c = acc[2 * i2 + half][j];
        gather_dvectors<D>(c);
        float* Sh = S + half * 32 * SROW;
        // d = 16: the output rows go four at a time, with their A rows and row terms read
        // from LDS, instead of all 256 coefficients at once (which spills).
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll IIU
          for (int ii = 0; ii < D; ++ii) {
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < D; ++e) s = __builtin_fmaf(Aat(ii * D + e), c[dvec_reg<D>(v, e)], s);
            const float bpi = D == 16 ? Al[D * D + ii] : bp[ii];
            Sh[dvec_row<D>(v, ii, h) * SROW + q] = __builtin_fmaf(2.f, s, bpi * rm);
          }
      }
      wave_sync();
      // Settle the loads issued before the epilogue (r, and dW's partials when this tile
      // reduces them) before the first store: a wait for them placed after stores would
      // also wait for those stores to complete.
      if (j == 0 && i2 == 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      store_block_rows64(S, a.out, a.out_f32, a.K, mb, a.M, kb, a.K, lane);
    }
}

// Straight-through epilogue on G (rows k, columns n):
//   dWp[n, g*d+j] = mask * sum_i A[i][j] G[g*d+i, n]
//   dA[i][j] += G[g*d+i, n] z[n, g*d+j],   dB[i] += G[g*d+i, n]
// Per-lane partial sums are reduced over the wave through LDS, then over the waves,
// in a fixed order, into this tile's slot of `partials`.
// dW LDS map: the double buffer (2 x 64 KiB) during the main loop, then per-wave
// epilogue areas below 128 KiB; the tile's codes (256 columns n x 64 bytes) and mask bits
// (256 x 32 bytes) live above it from kernel start, for the straight-through epilogue.
constexpr int DW_CODES_OFF = 128 * 1024;
constexpr int DW_MASK_OFF = DW_CODES_OFF + 256 * 64;    // 144 KiB
constexpr int DW_SMEM = DW_MASK_OFF + 256 * 32;         // 152 KiB

template <int D, int NW, int WJ>
__device__ void epilogue_dw(const GemmArgs& a, f32x16 acc[4][WJ], int p0, int q0, int wp, int wq,
                            int lane, int wave, int tile, uint8_t* smem, const float* Alds) {
  constexpr int NP = D == 16 ? 8 : 1;          // passes over the columns j of dA (d = 16: two
                                               // columns a pass, so no partial sums spill)
  constexpr int JW = D / NP;
  constexpr int NA = D * JW;                   // dA partials per lane and pass
  constexpr int NR = NA + D;                   // + dB partials (first pass)
  constexpr int RROW = NR + 1;
  constexpr int WREG = 12 * 1024;              // per-wave LDS area: staging, then reduction
  static_assert(32 * RROW * 4 <= WREG && 32 * SROW * 4 <= WREG, "per-wave LDS area");
  float* S = reinterpret_cast<float*>(smem + wave * WREG);
  float* red = S;                              // reused after the blocks of a pass
  float* wsum = reinterpret_cast<float*>(smem + NW * WREG);      // [NP][NW][NR]
  const int q = lane & 31, h = lane >> 5;
  float dB[D];
#pragma unroll
  for (int e = 0; e < D; ++e) dB[e] = 0.f;
#pragma unroll
  for (int pass = 0; pass < NP; ++pass) {
    float dA[NA];
#pragma unroll
    for (int x = 0; x < NA; ++x) dA[x] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < WJ; ++j) {
        const int kb = p0 + wp * 128 + i * 32;
        const int nb = q0 + wq * 32 * WJ + j * 32;
        const int n = nb + q;
        // A: scalar loads through a constant-address-space pointer (d = 16: LDS copy).
        const LCVQ_CONST float* Ac = (const LCVQ_CONST float*)a.A;
        const LCVQ_LDS float* Al = (const LCVQ_LDS float*)Alds;
        if constexpr (D == 16) asm volatile("" : "+v"(Al));
        else asm volatile("" : "+s"(Ac));
        auto Aat = [&](int idx) -> float {
          if constexpr (D == 16) return Al[idx];
          else return Ac[idx];
        };
        f32x16& c = acc[i][j];
        __builtin_amdgcn_sched_barrier(0);   // keep each block's work within its block
        if (pass == 0) {
          gather_dvectors<D>(c);        // whole d-vectors per lane from here on
          wave_sync();                  // the previous block's store has read S
        }
#pragma unroll
        for (int v = 0; v < 16 / D; ++v) {
          const int kr = dvec_row<D>(v, 0, h);       // first row of this vector in the block
          const int kv = kb + kr;
          float T[D];
#pragma unroll
          for (int e = 0; e < D; ++e) T[e] = c[dvec_reg<D>(v, e)];
          // The tile's codes and mask bits were brought into LDS at kernel start; the
          // offsets stay inside the tile's area (n - q0 < 256, kv - p0 < 256) whether or
          // not the vector is inside G, so the reads need no branch. Rows and columns
          // past the end of G hold clamped-operand values, not zeros: they must not
          // reach dA or dB.
          const bool valid = n < a.N && kv < a.K;
          const uint8_t* zp = smem + DW_CODES_OFF + (n - q0) * 64 + ((kv - p0) >> 2);
          const uint8_t* mp = smem + DW_MASK_OFF + (n - q0) * 32 + ((kv - p0) >> 3);
          uint32_t zw, mw;
          if (D == 4) { zw = zp[0]; mw = (mp[0] >> (kv & 4)) & 0xFu; }
          if (D == 8) { zw = *reinterpret_cast<const uint16_t*>(zp); mw = mp[0]; }
          if (D == 16) { zw = *reinterpret_cast<const uint32_t*>(zp); mw = *reinterpret_cast<const uint16_t*>(mp); }
          zw = valid ? zw : 0u;
          mw = valid ? mw : 0u;
          if (pass == 0) {
#pragma unroll
            for (int jj = 0; jj < D; ++jj) {
              float sum = 0.f;
#pragma unroll
              for (int e = 0; e < D; ++e) sum = __builtin_fmaf(Aat(e * D + jj), T[e], sum);
              S[(kr + jj) * SROW + q] = ((mw >> jj) & 1u) ? sum : 0.f;
            }
#pragma unroll
            for (int e = 0; e < D; ++e) dB[e] += valid ? T[e] : 0.f;
          }
#pragma unroll
          for (int jj = 0; jj < JW; ++jj) {
            const float zj = (float)((zw >> (2 * (pass * JW + jj))) & 3u);
#pragma unroll
            for (int e = 0; e < D; ++e) dA[e * JW + jj] = __builtin_fmaf(T[e], zj, dA[e * JW + jj]);
          }
        }
        if (pass == 0) {
          wave_sync();
          if (a.dge_wp)
            store_block_rows_dge(S, a.dwp, a.dge_wp, a.dge_alpha, a.dge_c, a.K, nb, a.N, kb,
                                 a.K, lane);
          else
            store_block_rows(S, a.dwp, 1, a.K, nb, a.N, kb, a.K, lane);
        }
      }
    // Wave reduction: lanes l and l+32 hold the same entries for different vectors; add
    // them with one exchange, then lane l < 32 writes its row and lanes sum columns.
#pragma unroll
    for (int x = 0; x < NA; ++x) dA[x] += __shfl_xor(dA[x], 32);
    float dBp[D];
#pragma unroll
    for (int x = 0; x < D; ++x) dBp[x] = pass == 0 ? dB[x] + __shfl_xor(dB[x], 32) : 0.f;
    wave_sync();
    if (lane < 32) {
#pragma unroll
      for (int x = 0; x < NA; ++x) red[lane * RROW + x] = dA[x];
#pragma unroll
      for (int x = 0; x < D; ++x) red[lane * RROW + NA + x] = dBp[x];
    }
    wave_sync();
    for (int x = lane; x < NR; x += 64) {
      float sum = 0.f;
      for (int l = 0; l < 32; ++l) sum += red[l * RROW + x];
      wsum[(pass * NW + wave) * NR + x] = sum;
    }
  }
  __syncthreads();
  for (int o = threadIdx.x; o < D * D + D; o += blockDim.x) {
    float sum = 0.f;
    if (o < D * D) {
      const int e = o / D, jj = o % D;
      const int pass = jj / JW, x = e * JW + (jj % JW);
      for (int w = 0; w < NW; ++w) sum += wsum[(pass * NW + w) * NR + x];
    } else {
      const int x = NA + (o - D * D);
      for (int w = 0; w < NW; ++w) sum += wsum[w * NR + x];
    }
    a.partials[(int64_t)tile * (D * D + D) + o] = sum;
  }
}

// ---- ring pipeline for the products with one 2-bit operand (FWD, DX) -----------------
// Each stage of 64 contraction steps occupies one LDS slot: the bf16 operand tile
// (256 rows x 128 bytes, swizzled) and the raw R16 code words of the other operand
// (256 rows x 16 bytes). Both arrive by direct global->LDS loads, four slots deep, so
// three stages are in flight while one is consumed. Codes are expanded to bf16 only
// when a wave reads its MFMA fragment, which halves the LDS traffic per stage.
// Within a row, word w of the R16 slab sits at position (w + row/8) mod 4 (the global
// blocked layout is written that way), which keeps the fragment reads conflict-free.
constexpr int RING = 4;
constexpr int CODEB = 256 * 16;
constexpr int SLOTB = TILEB + CODEB;
// Loads per lane and stage: RPW/8 bf16-tile loads (8 rows each) + RPW/16 code loads
// (16 rows of 16 bytes each), RPW = 256 / NW rows per wave.
template <int NW> constexpr int ring_loads() { return (256 / NW) / 8 + (256 / NW) / 16; }

// Wave w fills tile rows [RPW w, RPW (w+1)) and the code words of the same rows.
template <int NW>
__device__ __forceinline__ void issue_ring_stage(uint8_t* slot, const uint16_t* mat, int64_t ld,
                                                 int row0, int rows_total, int k0,
                                                 const uint32_t* codes, int rowblock, int nk,
                                                 int kt, int wave, int lane) {
  constexpr int RPW = 256 / NW;
#pragma unroll
  for (int i = 0; i < RPW / 8; ++i) {
    const int r = wave * RPW + i * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    int g = row0 + r;
    g = g < rows_total ? g : rows_total - 1;
    const uint16_t* src = mat + (int64_t)g * ld + k0 + c * 8;
    __builtin_amdgcn_global_load_lds(src, (LCVQ_LDS void*)(slot + (wave * RPW + i * 8) * ROWB), 16, 0, 0);
  }
  const uint32_t* slab = codes + ((int64_t)rowblock * nk + kt) * 1024;
#pragma unroll
  for (int h = 0; h < RPW / 16; ++h) {
    const int w0 = (wave * RPW + h * 16) * 4;           // first word of these 16 rows
    __builtin_amdgcn_global_load_lds(slab + w0 + lane, (LCVQ_LDS void*)(slot + TILEB + w0 * 4), 4, 0, 0);
  }
}

// The R16 word of tile row `row` for sub-step s, and its expansion into the MFMA
// fragment (8 consecutive codes as v(c) bf16) for half h of the 16-code word.
__device__ __forceinline__ uint32_t codes_word(const uint8_t* ctile, int row, int s) {
  return *reinterpret_cast<const uint32_t*>(ctile + row * 16 + (((s + (row >> 3)) & 3) << 2));
}
// Expansion constants held in registers: gfx950's three-operand encodings take no 32-bit
// literal and at most one scalar operand, so with the mask in a scalar register and the
// exponent bits in a vector register each dword is one shift and one v_and_or_b32.
struct ExpandK {
  uint32_t mask;   // 0x00600060, scalar
  uint32_t one;    // 0x40004000, vector
  uint32_t rot;    // 8 for lanes 32..63 (second half of the word), else 0
};
__device__ __forceinline__ ExpandK expand_consts(int lane) {
  ExpandK k;
  asm volatile("s_mov_b32 %0, 0x600060" : "=s"(k.mask));
  asm volatile("v_mov_b32 %0, 0x40004000" : "=v"(k.one));
  k.rot = (uint32_t)(lane >> 5) << 3;
  return k;
}
__device__ __forceinline__ bf16x8 codes_expand(uint32_t w, const ExpandK& k) {
  const uint32_t src = __builtin_amdgcn_alignbit(w, w, k.rot);
  u32x4 o;
#pragma unroll
  for (int p = 0; p < 4; ++p) o[p] = ((src >> (2 * p)) & k.mask) | k.one;
  return __builtin_bit_cast(bf16x8, o);
}

// Sub-step fragments: NB bf16 fragments read from the swizzled tile and NC code words.
template <bool CODES_ARE_L, int WI, int WJ>
struct RingFrags {
  static constexpr int NB = CODES_ARE_L ? WJ : WI;   // bf16-tile fragments
  static constexpr int NC = CODES_ARE_L ? WI : WJ;   // code fragments
  bf16x8 b[NB];
  uint32_t w[NC];
  bf16x8 c[NC];
};

template <bool CODES_ARE_L, int WI, int WJ>
__device__ __forceinline__ void ring_read(const uint8_t* slot, int s, int wp, int wq, int lane,
                                          RingFrags<CODES_ARE_L, WI, WJ>& f) {
  using F = RingFrags<CODES_ARE_L, WI, WJ>;
  const int chunk = 2 * s + (lane >> 5);
  const int tb = CODES_ARE_L ? wq * 32 * WJ : wp * 32 * WI;  // bf16-tile rows
  const int cb = CODES_ARE_L ? wp * 32 * WI : wq * 32 * WJ;  // code rows
  // code words first: their expansion is the first consumer
#pragma unroll
  for (int i = 0; i < F::NC; ++i) f.w[i] = codes_word(slot + TILEB, cb + i * 32 + (lane & 31), s);
#pragma unroll
  for (int i = 0; i < F::NB; ++i) {
    const int row = tb + i * 32 + (lane & 31);
    f.b[i] = *reinterpret_cast<const bf16x8*>(slot + lds_off(row, chunk));
  }
}

template <bool CODES_ARE_L, int WI, int WJ>
__device__ __forceinline__ void ring_expand(RingFrags<CODES_ARE_L, WI, WJ>& f, const ExpandK& k) {
#pragma unroll
  for (int i = 0; i < RingFrags<CODES_ARE_L, WI, WJ>::NC; ++i) f.c[i] = codes_expand(f.w[i], k);
}

// The MFMAs of one sub-step on fragments fc, with the expansion of the next fragments fn
// (whose LDS reads were issued just before) interleaved between them.
template <bool CODES_ARE_L, int WI, int WJ>
__device__ __forceinline__ void ring_mfma(const RingFrags<CODES_ARE_L, WI, WJ>& fc,
                                          RingFrags<CODES_ARE_L, WI, WJ>& fn,
                                          f32x16 acc[WI][WJ], const ExpandK& ek) {
  using F = RingFrags<CODES_ARE_L, WI, WJ>;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < WI; ++i)
#pragma unroll
    for (int j = 0; j < WJ; ++j) {
      const bf16x8 av = CODES_ARE_L ? fc.c[i] : fc.b[i];
      const bf16x8 bv = CODES_ARE_L ? fc.b[j] : fc.c[j];
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[i][j], 0, 0, 0);
    }
  ring_expand<CODES_ARE_L, WI, WJ>(fn, ek);
  constexpr int NV = (F::NC * 10 + WI * WJ - 1) / (WI * WJ);  // VALU per MFMA slot
#pragma unroll
  for (int g = 0; g < WI * WJ; ++g) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// dA and dB from the dW product's per-tile partials, summed in a fixed order: output o by
// tile o mod ntiles; thread t adds partials t, t + NT, ... of it, each wave adds its 64
// thread sums by a butterfly of lane exchanges, and thread 0 adds the NT / 64 wave sums
// in wave order. `first` is thread tid's sum for output `tile` when the caller loaded it
// ahead (`have_first`). Barriers are plain s_barrier: __syncthreads() would also wait for
// the epilogue's outstanding stores.
template <int D, int NT>
__device__ void reduce_dw_partials(const GemmArgs& a, int tile, int ntiles, int tid, float* red,
                                   float first, bool have_first) {
  constexpr int NOUT = D * D + D;
  for (int o = tile; o < NOUT; o += ntiles) {
    float s = 0.f;
    if (o == tile && have_first) {
      s = first;
    } else {
      for (int i = tid; i < a.red_tiles; i += NT) s += a.red_partials[(int64_t)i * NOUT + o];
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
    if ((tid & 63) == 0) red[tid >> 6] = s;
    __builtin_amdgcn_s_waitcnt(0xC07F);                   // lgkmcnt(0): the LDS write
    asm volatile("s_barrier" ::: "memory");
    if (tid == 0) {
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < NT / 64; ++w) t += red[w];
      if (o < D * D) a.red_dA[o] = t;
      else a.red_dB[o - D * D] = t;
    }
    asm volatile("s_barrier" ::: "memory");               // red is reused next round
  }
}

template <int NW>
__device__ __forceinline__ void wait_vm_stages(int stages_after) {
  constexpr int L = ring_loads<NW>();
  static_assert(2 * L < 64, "vmcnt range");
  if (stages_after >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * L));
  else if (stages_after == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(L));
  else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// ---- the kernel ----------------------------------------------------------------------
// FWD and dX: NW waves (4 or 8), 4-slot ring of direct global->LDS loads.
template <int OP, int D, int NW>
__global__ __launch_bounds__(NW * 64, 1) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void k_gemm_ring(GemmArgs a) {
  using T = Tiling<OP, NW>;
  constexpr int WI = T::WI, WJ = T::WJ;
  constexpr bool CL = OP == OP_DX;               // codes are the L operand for dX
  __shared__ __attribute__((aligned(1024))) uint8_t smem[RING * SLOTB];   // 144 KiB
  int tp, tq, tile;
  // The bf16 operand's panels (2 MiB each at K or N = 4096) outweigh the code panels
  // (256 KiB), so each XCD takes few tiles along the bf16 operand: forward tile-rows
  // are rows of X', dX tile-columns are rows of dY.
  constexpr int GR = OP == OP_FWD ? 2 : 16;
  if (!map_tile<GR>(blockIdx.x, a.tilesP, a.tilesQ, a.ntiles, tp, tq, tile)) return;
  const int p0 = tp * BT, q0 = tq * BT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wp = wave / T::WGQ, wq = wave % T::WGQ;
  const int nk = (a.R + BK - 1) / BK;

  f32x16 acc[WI][WJ];
#pragma unroll
  for (int i = 0; i < WI; ++i)
#pragma unroll
    for (int j = 0; j < WJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // One pipelined pass over the contraction per bf16 operand (bf16 activations: one
  // pass; float32 activations: hi and lo halves in two passes).
  for (int pass = 0; pass < a.npass; ++pass) {
    const uint16_t* mat = CL ? (pass == 0 ? a.Rmat[0] : a.Rmat[1])
                             : (pass == 0 ? a.Lmat[0] : a.Lmat[1]);
    const int64_t ld = CL ? a.N : a.K;
    const int row0 = CL ? q0 : p0;
    const int rowblock = CL ? tp : tq;
#pragma unroll
    for (int st = 0; st < RING - 1; ++st)
      if (st < nk)
        issue_ring_stage<NW>(smem + st * SLOTB, mat, ld, row0, a.M, st * BK, a.codes, rowblock,
                             nk, st, wave, lane);
    // The barrier of each stage sits before its last sub-step, so that the first
    // fragments of the next stage are read and expanded under that sub-step's MFMAs
    // instead of after a barrier at the stage boundary. Plain s_barrier: __syncthreads()
    // would also wait for every outstanding load (a workgroup release fence), which would
    // drain the ring; the memory clobber keeps LDS reads from moving across it.
    using F = RingFrags<CL, WI, WJ>;
    F f[2];
    const ExpandK ek = expand_consts(lane);
    wait_vm_stages<NW>(nk - 1 < 2 ? nk - 1 : 2);
    asm volatile("s_barrier" ::: "memory");
    ring_read<CL, WI, WJ>(smem, 0, wp, wq, lane, f[0]);
    ring_expand<CL, WI, WJ>(f[0], ek);
    for (int kt = 0; kt < nk; ++kt) {
      const uint8_t* slot = smem + (kt % RING) * SLOTB;
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        ring_read<CL, WI, WJ>(slot, s + 1, wp, wq, lane, f[(s & 1) ^ 1]);
        ring_mfma<CL, WI, WJ>(f[s & 1], f[(s & 1) ^ 1], acc, ek);
      }
      // Stage kt + 1 must have landed (stage kt + 2 may still be in flight); after the
      // barrier every wave is past sub-step 2 of stage kt, so stage kt - 1's slot is free
      // for stage kt + 3.
      wait_vm_stages<NW>(kt + 2 < nk ? 1 : 0);
      asm volatile("s_barrier" ::: "memory");
      if (kt + RING - 1 < nk)
        issue_ring_stage<NW>(smem + ((kt + RING - 1) % RING) * SLOTB, mat, ld, row0, a.M,
                             (kt + RING - 1) * BK, a.codes, rowblock, nk, kt + RING - 1, wave,
                             lane);
      // Sub-step 3, with stage kt + 1's first fragments read and expanded under it (on
      // the last stage this reads a free slot; the values are not used).
      ring_read<CL, WI, WJ>(smem + ((kt + 1) % RING) * SLOTB, 0, wp, wq, lane, f[0]);
      ring_mfma<CL, WI, WJ>(f[1], f[0], acc, ek);
    }
    __syncthreads();
  }

  if (OP == OP_FWD) {
    epilogue_fwd<NW, WI, WJ>(a, acc, p0, q0, wp, wq, lane, wave, smem);
  } else {
    // The ring is free after the last barrier: per-wave staging areas of 8.25 KiB, and
    // for d = 16 a copy of A at 120 KiB followed by the row terms B[i] - 4 sum_j A[i][j].
    float* Alds = reinterpret_cast<float*>(smem + 120 * 1024);
    if (D == 16) {
      if (tid < D * D) Alds[tid] = a.A[tid];
      if (tid < D) {
        float sa = 0.f;
        for (int j = 0; j < D; ++j) sa += a.A[tid * D + j];
        Alds[D * D + tid] = a.B[tid] - 4.f * sa;
      }
      __syncthreads();
    }
    static_assert(NW * DX_WAVE_LDS <= 120 * 1024, "dX staging below the copy of A");
    // This tile's first dA/dB output (o = tile) from dW's partials: loaded here, before
    // the epilogue's stores, when one load per thread covers the partials.
    // The load is unconditional, from a valid address (A when there is nothing to
    // reduce): a load inside a branch would be waited for at once where the branch joins.
    constexpr int NOUT = D * D + D;
    const bool have_first = a.red_partials && tile < NOUT && a.red_tiles <= NW * 64;
    const float* fsrc = a.red_partials
                            ? a.red_partials + (int64_t)(tid < a.red_tiles ? tid : 0) * NOUT +
                                  (tile < NOUT ? tile : 0)
                            : a.A;
    const float fv = *fsrc;
    epilogue_dx<D, WI, WJ>(a, acc, p0, q0, wp, wq, lane,
                           reinterpret_cast<float*>(smem + wave * DX_WAVE_LDS), Alds);
    // wave sums at 128 KiB: above the staging areas and the copy of A
    if (a.red_partials)
      reduce_dw_partials<D, NW * 64>(a, tile, a.ntiles, tid,
                                     reinterpret_cast<float*>(smem + 128 * 1024),
                                     tid < a.red_tiles ? fv : 0.f, have_first);
  }
}

// ---- dW product: both operands arrive in their natural [m][column] layout ------------
// G^T[k, n] = sum_m X[m, k] dY[m, n] contracts over the rows of both matrices. Their
// tiles (64 rows m x 256 columns, 512 bytes per row) go straight from HBM into LDS, and
// the MFMA fragments (8 consecutive m for one column) are read with gfx950's
// transposing LDS read ds_read_b64_tr_b16: within each group of 16 lanes, lane t
// receives element t%4 of the 64-bit pieces supplied by lanes 4e + t/4, e = 0..3.
// Source lane t of a group therefore points at row m0 + t/4, columns c0 + 4(t%4); the
// group gets columns c0 .. c0+15 with 4 consecutive m each. Two reads (m, m+4) fill an
// 8-element operand. 16-byte chunks are XOR-swizzled by 4*(m mod 4), which spreads the
// 8 rows x 4 chunks of one read evenly over the banks.
typedef short v4i16 __attribute__((ext_vector_type(4)));
constexpr int TROWB = 512;                     // bytes per LDS row of a transposed tile
constexpr int TTILEB = 64 * TROWB;             // 32 KiB
__device__ __forceinline__ int tswz(int m) { return (m & 3) << 2; }

__device__ __forceinline__ bf16x8 trans_frag(const uint8_t* tile, int colbase, int s, int lane) {
  const int g = lane >> 4, t = lane & 15;
  const int col = colbase + 16 * (g & 1) + 4 * (t & 3);
  const int m = 16 * s + 8 * (g >> 1) + (t >> 2);
  const int m2 = m + 4;
  const LCVQ_LDS uint8_t* base = (const LCVQ_LDS uint8_t*)tile;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (LCVQ_LDS v4i16*)(base + m * TROWB + (((col >> 3) ^ tswz(m)) << 4) + ((col & 4) << 1)));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (LCVQ_LDS v4i16*)(base + m2 * TROWB + (((col >> 3) ^ tswz(m2)) << 4) + ((col & 4) << 1)));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// One stage: 64 rows m of X (columns p0..p0+255) and of dY (columns q0..q0+255). Wave w
// fills rows [8w, 8w+8) of each tile, 2 rows per instruction (lane l: row l/32, physical
// chunk l%32). Rows past M are written as zeros (they are contraction terms); columns
// past the end are clamped (they only feed C entries that are never stored).
__device__ __forceinline__ void issue_dw_stage(uint8_t* slot, const uint16_t* X, const uint16_t* dY,
                                               int M, int N, int K, int m0, int p0, int q0,
                                               int wave, int lane) {
#pragma unroll
  for (int op = 0; op < 2; ++op) {
    const uint16_t* mat = op == 0 ? X : dY;
    const int ld = op == 0 ? K : N;
    const int c0 = op == 0 ? p0 : q0;
    uint8_t* tile = slot + op * TTILEB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wave * 8 + i * 2 + (lane >> 5);
      const int phys = lane & 31;
      const int c = phys ^ tswz(r);
      int col = c0 + c * 8;
      col = col < ld ? col : ld - 8;
      const int m = m0 + r;
      if (m < M) {
        const uint16_t* src = mat + (int64_t)m * ld + col;
        __builtin_amdgcn_global_load_lds(src, (LCVQ_LDS void*)(tile + (wave * 8 + i * 2) * TROWB), 16, 0, 0);
      } else {
        *reinterpret_cast<uint4*>(tile + r * TROWB + phys * 16) = make_uint4(0, 0, 0, 0);
      }
    }
  }
}

// Stages after the first: the two rows of each load instruction are uniform, so a load
// is a scalar row base plus one of two per-lane byte offsets (the swizzle of rows 2i and
// 2i + 1 alternates with i), which keeps few address registers live in the main loop.
// In a stage that runs past M, a load whose pair of rows reaches M reads row
// min(row, M - 1) into both halves (a valid row: such a stage is never the first, so
// M > 64), and zero_dw_rows then clears the rows at or past M, which are contraction
// terms.
struct DwLaneOffsets {
  uint32_t v[2][2];            // [operand][i & 1]
};
__device__ __forceinline__ DwLaneOffsets dw_lane_offsets(int N, int K, int p0, int q0, int lane) {
  DwLaneOffsets o;
#pragma unroll
  for (int op = 0; op < 2; ++op) {
    const int ld = op == 0 ? K : N;
    const int c0 = op == 0 ? p0 : q0;
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int r = par * 2 + (lane >> 5);             // row mod 4 of this lane's load
      const int c = (lane & 31) ^ tswz(r);
      int col = c0 + c * 8;
      col = col < ld ? col : ld - 8;
      o.v[op][par] = (uint32_t)(((lane >> 5) * ld + col) * 2);
    }
  }
  return o;
}
__device__ __forceinline__ void issue_dw_stage_rows(uint8_t* slot, const uint16_t* X,
                                                    const uint16_t* dY, int M, int N, int K,
                                                    int m0, const DwLaneOffsets& o, int wave,
                                                    int lane) {
#pragma unroll
  for (int op = 0; op < 2; ++op) {
    const uint16_t* mat = op == 0 ? X : dY;
    const int ld = op == 0 ? K : N;
    uint8_t* tile = slot + op * TTILEB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int row = m0 + wave * 8 + i * 2;                   // uniform
      uint32_t off = o.v[op][i & 1];
      if (row + 1 >= M) {
        // the second row of the pair (or both) lies past M: both halves read row
        // min(row, M - 1), whose copy in a row past M is cleared afterwards
        row = row < M ? row : M - 1;
        off -= (uint32_t)((lane >> 5) * ld * 2);
      }
      const uint8_t* base = reinterpret_cast<const uint8_t*>(mat + (int64_t)row * ld);
      __builtin_amdgcn_global_load_lds(base + off,
                                       (LCVQ_LDS void*)(tile + (wave * 8 + i * 2) * TROWB), 16, 0, 0);
    }
  }
}
// Wave w clears its own rows [8w, 8w + 8) of both tiles where m0 + row >= M; called after
// its loads have landed and before the stage's barrier.
__device__ __forceinline__ void zero_dw_rows(uint8_t* slot, int m0, int M, int wave, int lane) {
#pragma unroll
  for (int op = 0; op < 2; ++op)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wave * 8 + i * 2 + (lane >> 5);
      if (m0 + r >= M)
        *reinterpret_cast<uint4*>(slot + op * TTILEB + r * TROWB + (lane & 31) * 16) =
            make_uint4(0, 0, 0, 0);
    }
}

template <int WJ>
struct DwFrags {
  bf16x8 a[4], b[WJ];
};

template <int WJ>
__device__ __forceinline__ void dw_read(const uint8_t* slot, int s, int wp, int wq, int lane,
                                        DwFrags<WJ>& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f.a[i] = trans_frag(slot, wp * 128 + i * 32, s, lane);
#pragma unroll
  for (int j = 0; j < WJ; ++j) f.b[j] = trans_frag(slot + TTILEB, wq * 32 * WJ + j * 32, s, lane);
}

template <int WJ>
__device__ __forceinline__ void dw_mfma(const DwFrags<WJ>& f, f32x16 acc[4][WJ]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < WJ; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// Codes: 16-byte direct loads, 2 per lane; mask: 4-byte direct loads (mask rows are only
// 8-byte aligned), 4 per lane. Columns past N and k past K read a valid address; those
// entries are never used.
__device__ __forceinline__ void issue_dw_codes(uint8_t* smem, const uint8_t* packed,
                                               const uint8_t* mask, int N, int K, int p0,
                                               int q0, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = (wave * 2 + i) * 64 + lane;            // 16-byte chunk of the code tile
    int n = q0 + (c >> 2);
    n = n < N ? n : N - 1;
    int kb = p0 + (c & 3) * 64;
    kb = kb < K ? kb : 0;
    const uint8_t* src = packed + (int64_t)n * (K >> 2) + (kb >> 2);
    __builtin_amdgcn_global_load_lds(src, (LCVQ_LDS void*)(smem + DW_CODES_OFF + (wave * 2 + i) * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = (wave * 4 + i) * 64 + lane;            // 4-byte word of the mask tile
    int n = q0 + (c >> 3);
    n = n < N ? n : N - 1;
    int kb = p0 + (c & 7) * 32;
    kb = kb < K ? kb : 0;
    const uint8_t* src = mask + (int64_t)n * (K >> 3) + (kb >> 3);
    __builtin_amdgcn_global_load_lds(src, (LCVQ_LDS void*)(smem + DW_MASK_OFF + (wave * 4 + i) * 256), 4, 0, 0);
  }
}

// dW: 8 waves (512 threads), double-buffered direct loads into LDS (2 x 64 KiB).
template <int D>
__global__ __launch_bounds__(512, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_gemm_dw(GemmArgs a) {
  constexpr int NW = 8, WGQ = 4, WJ = 2;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[DW_SMEM];   // 152 KiB
  int tp, tq, tile;
  // X and dY panels weigh the same: 4 x 8 tiles per XCD reads the fewest panels.
  if (!map_tile<4>(blockIdx.x, a.tilesP, a.tilesQ, a.ntiles, tp, tq, tile)) return;
  const int p0 = tp * BT, q0 = tq * BT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wp = wave / WGQ, wq = wave % WGQ;
  const int nk = (a.R + BK - 1) / BK;
  const DwLaneOffsets lo = dw_lane_offsets(a.N, a.K, p0, q0, lane);
  issue_dw_codes(smem, a.packed, a.mask, a.N, a.K, p0, q0, wave, lane);

  f32x16 acc[4][WJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < WJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  for (int pass = 0; pass < a.npass; ++pass) {
    const uint16_t* Lp = pass == 0 ? a.Lmat[0] : (pass == 1 ? a.Lmat[1] : a.Lmat[2]);
    const uint16_t* Rp = pass == 0 ? a.Rmat[0] : (pass == 1 ? a.Rmat[1] : a.Rmat[2]);
    issue_dw_stage(smem, Lp, Rp, a.M, a.N, a.K, 0, p0, q0, wave, lane);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // Every transposing LDS read of a stage is issued before the next stage's direct
    // loads: the compiler makes an LDS read that follows a direct global->LDS load in
    // program order wait for that load, which would serialize the two. Sub-steps 0-2 are
    // read first, sub-step 3 into sub-step 0's registers once its MFMAs have issued, and
    // the next stage's loads then run under the MFMAs of sub-steps 1-3.
    for (int kt = 0; kt < nk; ++kt) {
      const uint8_t* slot = smem + (kt & 1) * 2 * TTILEB;
      DwFrags<WJ> f0, f1, f2;
      dw_read<WJ>(slot, 0, wp, wq, lane, f0);
      dw_read<WJ>(slot, 1, wp, wq, lane, f1);
      dw_read<WJ>(slot, 2, wp, wq, lane, f2);
      __builtin_amdgcn_sched_barrier(0);
      dw_mfma<WJ>(f0, acc);
      __builtin_amdgcn_sched_barrier(0);
      dw_read<WJ>(slot, 3, wp, wq, lane, f0);
      __builtin_amdgcn_sched_barrier(0);
      uint8_t* next = smem + ((kt & 1) ^ 1) * 2 * TTILEB;
      if (kt + 1 < nk)
        issue_dw_stage_rows(next, Lp, Rp, a.M, a.N, a.K, (kt + 1) * BK, lo, wave, lane);
      __builtin_amdgcn_sched_barrier(0);
      dw_mfma<WJ>(f1, acc);
      dw_mfma<WJ>(f2, acc);
      dw_mfma<WJ>(f0, acc);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0);
      if (kt + 1 < nk && (kt + 1) * BK + wave * 8 + 8 > a.M)
        zero_dw_rows(next, (kt + 1) * BK, a.M, wave, lane);
      __syncthreads();
    }
  }
  // The buffers are free after the last barrier: per-wave areas of 12 KiB from 0, the
  // per-wave sums after them, and for d = 16 a copy of A at 120 KiB.
  float* Alds = reinterpret_cast<float*>(smem + 120 * 1024);
  if (D == 16) {
    if (tid < D * D) Alds[tid] = a.A[tid];
    __syncthreads();
  }
  epilogue_dw<D, NW, WJ>(a, acc, p0, q0, wp, wq, lane, wave, tile, smem, Alds);
}

// One block per output: thread t adds tiles t, t+256, ... in order, then a fixed
// binary tree in LDS combines the 256 thread sums.
__global__ __launch_bounds__(256) void k_reduce_partials(const float* __restrict__ partials,
                                                         int ntiles, int nout,
                                                         float* __restrict__ dA,
                                                         float* __restrict__ dB, int d) {
  __shared__ float red[256];
  const int o = blockIdx.x, t = threadIdx.x;
  float s = 0.f;
  for (int i = t; i < ntiles; i += 256) s += partials[(int64_t)i * nout + o];
  red[t] = s;
  __syncthreads();
#pragma unroll
  for (int w = 128; w >= 1; w >>= 1) {
    if (t < w) red[t] += red[t + w];
    __syncthreads();
  }
  if (t == 0) {
    if (o < d * d) dA[o] = red[0];
    else dB[o - d * d] = red[0];
  }
}

// ---- launchers -----------------------------------------------------------------------
template <int OP>
static hipError_t launch_op(GemmArgs& a, int d, hipStream_t s) {
  a.tilesP = (a.P + BT - 1) / BT;
  a.tilesQ = (a.Q + BT - 1) / BT;
  a.ntiles = a.tilesP * a.tilesQ;
  const int grid = ((a.ntiles + 7) / 8) * 8;
  if constexpr (OP == OP_DW) {
    switch (d) {
      case 4: LCVQ_LAUNCH(PROF_DW, k_gemm_dw<4>, dim3(grid), dim3(512), 0, s, a); break;
      case 8: LCVQ_LAUNCH(PROF_DW, k_gemm_dw<8>, dim3(grid), dim3(512), 0, s, a); break;
      default: LCVQ_LAUNCH(PROF_DW, k_gemm_dw<16>, dim3(grid), dim3(512), 0, s, a); break;
    }
  } else {
    constexpr int id = OP == OP_FWD ? PROF_FWD : PROF_DX;
    constexpr int NW = OP == OP_FWD ? LCVQ_FWD_WAVES : LCVQ_DX_WAVES;
    switch (d) {
      case 4: LCVQ_LAUNCH(id, (k_gemm_ring<OP, 4, NW>), dim3(grid), dim3(NW * 64), 0, s, a); break;
      case 8: LCVQ_LAUNCH(id, (k_gemm_ring<OP, 8, NW>), dim3(grid), dim3(NW * 64), 0, s, a); break;
      default: LCVQ_LAUNCH(id, (k_gemm_ring<OP, 16, NW>), dim3(grid), dim3(NW * 64), 0, s, a); break;
    }
  }
  return hipGetLastError();
}

int gemm_tiles(int64_t P, int64_t Q) { return (int)(((P + BT - 1) / BT) * ((Q + BT - 1) / BT)); }

hipError_t launch_gemm_fwd(const uint16_t* xs, const uint16_t* xs_lo, const uint32_t* r16,
                           const float* beta, int M, int N, int K, int d, void* Y, bool y_f32,
                           hipStream_t s) {
  GemmArgs a = {};
  a.P = M; a.Q = N; a.R = K;
  a.Lmat[0] = xs; a.Lmat[1] = xs_lo;
  a.npass = xs_lo ? 2 : 1;
  a.codes = r16; a.rowvec = beta;
  a.M = M; a.N = N; a.K = K;
  a.out = Y; a.out_f32 = y_f32;
  return launch_op<OP_FWD>(a, d, s);
}

hipError_t launch_gemm_dx(const uint32_t* r16t, const uint16_t* dy, const uint16_t* dy_lo,
                          const float* r, const float* A, const float* B, int M, int N, int K,
                          int d, void* dX, bool f32, const float* dw_partials, float* dA,
                          float* dB, hipStream_t s) {
  GemmArgs a = {};
  if (dw_partials) {                         // the dW product's tiles: ceil(K/BT) x ceil(N/BT)
    a.red_partials = dw_partials;
    a.red_tiles = ((K + BT - 1) / BT) * ((N + BT - 1) / BT);
    a.red_dA = dA;
    a.red_dB = dB;
  }
  a.P = K; a.Q = M; a.R = N;
  a.codes = r16t;
  a.Rmat[0] = dy; a.Rmat[1] = dy_lo;
  a.npass = dy_lo ? 2 : 1;
  a.rowvec = r; a.A = A; a.B = B;
  a.M = M; a.N = N; a.K = K;
  a.out = dX; a.out_f32 = f32;
  return launch_op<OP_DX>(a, d, s);
}

hipError_t launch_gemm_dw(const uint16_t* x, const uint16_t* x_lo, const uint16_t* dy,
                          const uint16_t* dy_lo, const uint8_t* packed, const uint8_t* mask,
                          const float* A, int M, int N, int K, int d, float* dWp,
                          float* partials, float* dA, float* dB, const float* dge_wp,
                          float dge_alpha, bool reduce, hipStream_t s) {
  GemmArgs a = {};
  a.P = K; a.Q = N; a.R = M;
  a.Lmat[0] = x; a.Rmat[0] = dy;
  a.npass = 1;
  if (x_lo && dy_lo) {        // hi*hi + lo*hi + hi*lo
    a.Lmat[1] = x_lo; a.Rmat[1] = dy;
    a.Lmat[2] = x; a.Rmat[2] = dy_lo;
    a.npass = 3;
  }
  a.A = A;
  a.M = M; a.N = N; a.K = K;
  a.dwp = dWp; a.packed = packed; a.mask = mask; a.partials = partials;
  a.dge_wp = dge_wp;
  a.dge_alpha = dge_alpha;
  a.dge_c = dge_wp ? (float)((double)dge_alpha / (2.0 * tanh((double)dge_alpha / 2.0))) : 0.f;
  hipError_t e = launch_op<OP_DW>(a, d, s);
  if (e != hipSuccess || !reduce) return e;
  hipLaunchKernelGGL(k_reduce_partials, dim3(d * d + d), dim3(256), 0, s, partials, a.ntiles,
                     d * d + d, dA, dB, d);
  return hipGetLastError();
}

}  // namespace lcvq
