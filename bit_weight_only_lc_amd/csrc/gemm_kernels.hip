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
// contraction staged through LDS in steps of 64; the forward also in 128 x 256 tiles when
// the larger ones would leave most CUs idle):
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
// The forward can also run 128 x 256 tiles (BPT = 128 rows of X'), for launches whose
// 256 x 256 tiles would leave most of the chip idle: 8 waves of 64 x 64 (2 x 2 blocks).
template <int OP, int NWV = 8, int BPT = 256> struct Tiling {
  static constexpr int NW = NWV;
  static constexpr int WGP = BPT == 128 ? 2 : (NW == 4 ? 2 : (OP == OP_DX ? 4 : LCVQ_FWD_WGP));
  static constexpr int WGQ = NW / WGP;
  static constexpr int WI = BPT / 32 / WGP;
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
  const uint32_t* codes;       // FWD: R16 of Z along k; DX, DW: R16 of Z^T along n (blocked)
  int M, N, K;
  const float* rowvec;         // FWD: beta [M]; DX: r [M]
  const float* A;              // [d][d]
  const float* B;              // [d]
  void* out;                   // FWD: Y [M][N]; DX: dX [M][K]
  int out_f32;
  float* dwp;                  // DW: [N][K]
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
  // Split contraction (launches with few tiles), in two launches of the same kernel:
  // phase 1 runs `splits` workgroups per tile, each over its share of the contraction,
  // and writes its float32 partial tile to split_ws [ntiles][splits][256 * 256]; phase 2
  // runs one workgroup per tile, which adds the partials in split order and runs the
  // epilogue. splits = 1: one launch, one workgroup per tile.
  int splits;
  float* split_ws;
  // Tail split (forward and dW, hyb_L > 0): tile t = x * hyb_per + i of XCD x (map_tile's
  // order); the first hyb_F of each XCD's tiles run unsplit in one launch, the last hyb_L
  // split their contraction in two (splits = 2) over a phase 1 and a phase 2 launch; their
  // partial tiles are indexed x * hyb_L + (i - hyb_F).
  int hyb_per, hyb_F, hyb_L;
  int bpt;                     // forward: tile rows along P, 256 or 128 (host side)
};

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * ROWB + ((chunk ^ swz(row)) << 4); }

// Tiles are spread so that consecutive workgroup ids land on different XCDs (the
// dispatcher deals workgroups round-robin over the 8 XCDs) while each XCD works on a
// compact group of GR tile-rows, which keeps its operand panels in its own L2.
template <int GR>
__device__ __forceinline__ void tile_coords(int t, int tilesP, int tilesQ, int& tp, int& tq) {
  const int group = t / (GR * tilesQ);
  const int within = t - group * GR * tilesQ;
  int rows = tilesP - group * GR;
  if (rows > GR) rows = GR;
  tp = group * GR + within % rows;
  tq = within / rows;
}
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

// Split launches: job b -> (tile b mod ntiles, split b / ntiles). The dispatcher deals
// workgroups round-robin over the 8 XCDs, so the jobs of one tile share an XCD whenever
// ntiles is a multiple of 8 and exchange their partials through its L2.
__device__ __forceinline__ bool map_split(int b, int tilesQ, int ntiles, int splits, int& tp,
                                          int& tq, int& tile, int& split) {
  if (b >= ntiles * splits) return false;
  tile = b % ntiles;
  split = b / ntiles;
  tp = tile / tilesQ;
  tq = tile % tilesQ;
  return true;
}

// Tail split: workgroup b of a launch with `per_tile` workgroups per leftover tile -> its
// XCD's leftover tile (numbered as map_tile<GR> numbers the tiles, so that the tile's
// workgroups of both phases share the XCD that the unsplit tiles of that range use), the
// index of its partial tiles, and j = its slot among the tile's workgroups (split or
// epilogue group).
template <int GR>
__device__ __forceinline__ bool map_hybrid(const GemmArgs& a, int b, int per_tile, int& tp,
                                           int& tq, int& tile, int& pidx, int& j) {
  const int x = b & 7, w = b >> 3;
  const int li = w % a.hyb_L;
  j = w / a.hyb_L;
  if (j >= per_tile) return false;
  tile = x * a.hyb_per + a.hyb_F + li;
  pidx = x * a.hyb_L + li;
  tile_coords<GR>(tile, a.tilesP, a.tilesQ, tp, tq);
  return true;
}

// Stages [kt0, kt1) of nk that job `split` of `splits` contracts over.
__device__ __forceinline__ void split_range(int nk, int split, int splits, int& kt0, int& kt1) {
  kt0 = (int)((int64_t)nk * split / splits);
  kt1 = (int)((int64_t)nk * (split + 1) / splits);
}

// Partial tiles of a split launch: float4 [tile][split][block][register quad][thread], so
// that each store or load instruction of a workgroup covers 1 KiB.
template <int WI, int WJ>
__device__ __forceinline__ void split_store(const GemmArgs& a, const f32x16 (&acc)[WI][WJ],
                                            int tile, int split, int tid) {
  const int nt = blockDim.x;
  constexpr int NQ = WI * WJ * 4;                    // float4 per thread
  f32x4* mine = reinterpret_cast<f32x4*>(a.split_ws) + ((int64_t)tile * a.splits + split) * NQ * nt;
#pragma unroll
  for (int i = 0; i < WI; ++i)
#pragma unroll
    for (int j = 0; j < WJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        mine[((i * WJ + j) * 4 + q) * nt + tid] =
            f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
}

// Phase 2: the tile's accumulators as the sum of its partials, added in split order.
// Addresses are one uniform base plus this thread's byte offset, so the loads need no
// per-load address registers; split 0 is loaded straight into the accumulators (all its
// loads in flight at once), each later split in two batches of WI*WJ*2 loads.
// nt: the phase-1 workgroup size; tid: the phase-1 thread whose accumulators are loaded.
template <int WI, int WJ>
__device__ __forceinline__ void split_load(const GemmArgs& a, f32x16 (&acc)[WI][WJ], int tile,
                                           int tid, int nt) {
  constexpr int NQ = WI * WJ * 4;                    // float4 per thread
  constexpr int HQ = NQ / 2;
  const int64_t step = (int64_t)nt * 16;             // bytes between a thread's float4s
  const uint32_t lo = (uint32_t)tid * 16u;
  const char* base = reinterpret_cast<const char*>(a.split_ws) + (int64_t)tile * a.splits * NQ * step;
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(base + k * step + lo);
    f32x16& c = acc[k / (WJ * 4)][(k / 4) % WJ];
#pragma unroll
    for (int e = 0; e < 4; ++e) c[4 * (k % 4) + e] = v[e];
  }
  for (int sp = 1; sp < a.splits; ++sp) {
    const char* src = base + (int64_t)sp * NQ * step;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 t[HQ];
#pragma unroll
      for (int k = 0; k < HQ; ++k)
        t[k] = *reinterpret_cast<const f32x4*>(src + (h * HQ + k) * step + lo);
#pragma unroll
      for (int k = 0; k < HQ; ++k) {
        const int kk = h * HQ + k;
        f32x16& c = acc[kk / (WJ * 4)][(kk / 4) % WJ];
#pragma unroll
        for (int e = 0; e < 4; ++e) c[4 * (kk % 4) + e] += t[k][e];
      }
    }
  }
}

// ---- epilogues -----------------------------------------------------------------------
// Outputs (Y, dX, dWp) are written once and not read again by the kernel: they go out as
// non-temporal stores, which measured 1-3 us faster per product than ordinary ones.
// Accumulator layout (32x32 block): lane l holds column l%32 and, in register r, row
// 8*(r/4) + 4*(l/32) + r%4. For DX and DW the rows run along the d-vectors, and the d x d
// mix of every 32-row block is one block-diagonal 32 x 32 matrix: it runs on the matrix
// cores with the accumulator block as the B operand, and the results go through a
// per-wave LDS area only to be written back transposed, each group of 8 lanes covering
// consecutive elements of one output row. The forward epilogue stages row-major strips
// the same way for 16-byte stores.

constexpr int SROW = 33;                  // padded row of the staging area (floats)

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding; the other counters are not waited on.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// dW's staging area holds a 32 x 32 block as [n][k] (row stride SROWT floats, 16-byte
// aligned), so that a lane's d-vector (consecutive k of one n) goes in with 16-byte writes
// and each store's four consecutive k come out with one 16-byte read. The block's rows n
// go to out[row0 + n][k0 .. k0 + 31]; each group of 8 lanes covers one row.
constexpr int SROWT = 36;
__device__ __forceinline__ void store_block_rows_t(const float* S, float* out, int64_t ld,
                                                   int row0, int rows, int k0, int K,
                                                   int lane) {
  const int kq = (lane & 7) * 4;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int rr = it * 8 + (lane >> 3);
    const int row = row0 + rr;
    if (row < rows && k0 + kq < K) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(S + rr * SROWT + kq);
      __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(out + (int64_t)row * ld + k0 + kq));
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

// store_block_rows_t for dWp under the DGE estimator: each value is multiplied by the
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
      const f32x4 v = *reinterpret_cast<const f32x4*>(S + rr * SROWT + kq);
      __builtin_nontemporal_store(f32x4{v[0] * dge_slope(w[it].x, alpha, c),
                                        v[1] * dge_slope(w[it].y, alpha, c),
                                        v[2] * dge_slope(w[it].z, alpha, c),
                                        v[3] * dge_slope(w[it].w, alpha, c)},
                                  reinterpret_cast<f32x4*>(out + idx));
    }
  }
}

// Forward epilogue: Y[p, q] = C[p, q] + beta[p]. Each 32-row strip of the wave's
// 32 x 32*WJ sub-tile is staged row-major through the wave's LDS area (the ring is
// free by now), then written with 16-byte stores, so that every store instruction
// covers whole 32*WJ-element runs of 16 / WJ output rows.
template <int NW, int WI, int WJ>
__device__ __forceinline__ void epilogue_fwd(const GemmArgs& a, f32x16 acc[WI][WJ], int p0, int q0, int wp,
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

// dX[m, g*d+i] = 2 sum_j A[i][j] C[g*d+j, m] + (B[i] - 4 sum_j A[i][j]) r[m]
// where C = sum_n v(z[n, k]) dY[m, n] is the accumulator (rows k, columns m). The d x d
// mix 2 (I kron A) runs on the matrix cores with C in the accumulator layout as its B
// operand (bf16 hi + lo halves of C and of the mix: hi*hi + lo*hi + hi*lo, about 16 bits
// of C kept); the results go through the wave's LDS area only for the transposed store.
// Blocks are taken in pairs along k, so that each output row receives 128 contiguous
// bytes (bf16) per store instruction.
constexpr int DX_WAVE_LDS = 64 * SROW * 4;   // per-wave staging area: 64 x 33 floats

template <int D, int WI, int WJ>
__device__ __forceinline__ void epilogue_dx(const GemmArgs& a, f32x16 acc[WI][WJ], int p0, int q0, int wp, int wq,
                            int lane, float* S, const float* Alds) {
  static_assert(WI % 2 == 0, "k blocks are staged in pairs");
  const int q = lane & 31, h = lane >> 5;
  // Mix operands: lane (row q, half h) holds, for the MFMA over accumulator registers
  // 8t .. 8t+7 (slot e: row k = 16t + 8(e/4) + 4h + e%4 of C), the entry 2 A[q % d][k % d]
  // of 2 (I kron A) inside q's d-vector, else 0, as bf16 hi + lo halves. (d = 16: A from its
  // LDS copy.)
  bf16x8 AMh[2], AMl[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = 16 * t + 8 * (e >> 2) + 4 * h + (e & 3);
      const int idx = (q % D) * D + k % D;
      const float av = D == 16 ? Alds[idx] : a.A[idx];
      const float m = k / D == q / D ? 2.f * av : 0.f;
      const __bf16 mh = (__bf16)m;
      AMh[t][e] = mh;
      AMl[t][e] = (__bf16)(m - (float)mh);
    }
  // Row terms B[i] - 4 sum_j A[i][j] of this lane's output rows: register r holds row
  // 8(r/4) + 4h + r%4, i.e. i = that row mod d, slot rslot(r).
  constexpr int NBP = D == 16 ? 8 : 4;
  auto rslot = [](int r) { return D == 16 ? ((r >> 2) & 1) * 4 + (r & 3) : (r & 3); };
  float bpl[NBP];
#pragma unroll
  for (int x = 0; x < NBP; ++x) {
    const int i = D == 16 ? 8 * (x >> 2) + 4 * h + (x & 3) : (D == 8 ? 4 * h + x : x);
    if constexpr (D == 16) {
      bpl[x] = Alds[D * D + i];
    } else {
      float sa = 0.f;
#pragma unroll
      for (int j = 0; j < D; ++j) sa += a.A[i * D + j];
      bpl[x] = a.B[i] - 4.f * sa;
    }
  }
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
      wave_sync();
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const f32x16 c = acc[2 * i2 + half][j];
        uint32_t ch[8], cl[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          ch[p] = pack_bf16x2(c[2 * p], c[2 * p + 1]);
          cl[p] = pack_bf16x2(c[2 * p] - bf16lo_to_f32(ch[p]), c[2 * p + 1] - bf16hi_to_f32(ch[p]));
        }
        const bf16x8 Ch0 = __builtin_bit_cast(bf16x8, u32x4{ch[0], ch[1], ch[2], ch[3]});
        const bf16x8 Ch1 = __builtin_bit_cast(bf16x8, u32x4{ch[4], ch[5], ch[6], ch[7]});
        const bf16x8 Cl0 = __builtin_bit_cast(bf16x8, u32x4{cl[0], cl[1], cl[2], cl[3]});
        const bf16x8 Cl1 = __builtin_bit_cast(bf16x8, u32x4{cl[4], cl[5], cl[6], cl[7]});
        f32x16 o;
#pragma unroll
        for (int r = 0; r < 16; ++r) o[r] = 0.f;
        o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(AMh[0], Ch0, o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(AMh[1], Ch1, o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(AMl[0], Ch0, o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(AMl[1], Ch1, o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(AMh[0], Cl0, o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(AMh[1], Cl1, o, 0, 0, 0);
        float* Sh = S + half * 32 * SROW;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          Sh[(8 * (r >> 2) + 4 * h + (r & 3)) * SROW + q] = __builtin_fmaf(bpl[rslot(r)], rm, o[r]);
      }
      wave_sync();
      // Settle the loads issued before the epilogue (r, and dW's partials when this tile
      // reduces them) before the first store: a wait for them placed after stores would
      // also wait for those stores to complete.
      if (j == 0 && i2 == 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      store_block_rows64(S, a.out, a.out_f32, a.K, mb, a.M, kb, a.K, lane);
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
// Loads per lane and stage: RB/NW/8 bf16-tile loads (8 rows each) + 256/NW/16 code loads
// (16 rows of 16 bytes each); the bf16 tile has RB rows (256, or 128 for the forward's
// 128 x 256 tiles), the code tile always 256.
template <int NW, int RB = 256> constexpr int ring_loads() { return (RB / NW) / 8 + (256 / NW) / 16; }

// Wave w fills bf16-tile rows [RB/NW w, RB/NW (w+1)) and code rows [256/NW w, 256/NW (w+1)).
template <int NW, int RB = 256>
__device__ __forceinline__ void issue_ring_stage(uint8_t* slot, const uint16_t* mat, int64_t ld,
                                                 int row0, int rows_total, int k0,
                                                 const uint32_t* codes, int rowblock, int nk,
                                                 int kt, int wave, int lane) {
  constexpr int RPW = RB / NW, CPW = 256 / NW;
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
  for (int h = 0; h < CPW / 16; ++h) {
    const int w0 = (wave * CPW + h * 16) * 4;           // first word of these 16 rows
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
__device__ __forceinline__ void reduce_dw_partials(const GemmArgs& a, int tile, int ntiles, int tid, float* red,
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

template <int NW, int RB = 256>
__device__ __forceinline__ void wait_vm_stages(int stages_after) {
  constexpr int L = ring_loads<NW, RB>();
  static_assert(2 * L < 64, "vmcnt range");
  if (stages_after >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * L));
  else if (stages_after == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(L));
  else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// ---- the kernel ----------------------------------------------------------------------
// FWD and dX: NW waves (4 or 8), 4-slot ring of direct global->LDS loads.
// SPL: 0 one workgroup per tile; 1 phase 1 of a split launch (forward only; phase 2 is
// k_gemm_fwd_epi). BPT: tile rows along P (128 only for the forward without a split).
template <int OP, int D, int NW, int SPL = 0, int BPT = 256>
__global__ __launch_bounds__(NW * 64, 1) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void k_gemm_ring(GemmArgs a) {
  static_assert(SPL == 0 || (SPL == 1 && OP == OP_FWD), "phase 2 of a split forward is k_gemm_fwd_epi");
  static_assert(BPT == 256 || (BPT == 128 && OP == OP_FWD && SPL == 0 && NW == 8), "128-row tiles: forward only");
  using T = Tiling<OP, NW, BPT>;
  constexpr int WI = T::WI, WJ = T::WJ;
  constexpr bool CL = OP == OP_DX;               // codes are the L operand for dX
  constexpr int RB = CL ? 256 : BPT;             // rows of the bf16 operand's tile
  __shared__ __attribute__((aligned(1024))) uint8_t smem[RING * SLOTB];   // 144 KiB
  int tp, tq, tile;
  // The bf16 operand's panels (2 MiB each at K or N = 4096) outweigh the code panels
  // (256 KiB), so each XCD takes few tiles along the bf16 operand: forward tile-rows
  // are rows of X', dX tile-columns are rows of dY.
  constexpr int GR = OP == OP_FWD ? 2 : 16;
  int split = 0, pidx = 0;
  if constexpr (SPL == 1) {
    if (a.hyb_L) {
      if (!map_hybrid<GR>(a, blockIdx.x, 2, tp, tq, tile, pidx, split)) return;
    } else {
      if (!map_split(blockIdx.x, a.tilesQ, a.ntiles, a.splits, tp, tq, tile, split)) return;
      pidx = tile;
    }
  } else if (!map_tile<GR>(blockIdx.x, a.tilesP, a.tilesQ, a.ntiles, tp, tq, tile)) {
    return;
  }
  const int p0 = tp * BPT, q0 = tq * BT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wp = wave / T::WGQ, wq = wave % T::WGQ;
  const int nkt = (a.R + BK - 1) / BK;               // stages of the whole contraction
  int kt0 = 0, kt1 = nkt;
  if constexpr (SPL == 1) split_range(nkt, split, a.splits, kt0, kt1);
  const int nk = kt1 - kt0;                          // stages of this job

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
        issue_ring_stage<NW, RB>(smem + st * SLOTB, mat, ld, row0, a.M, (kt0 + st) * BK, a.codes,
                                 rowblock, nkt, kt0 + st, wave, lane);
    // The barrier of each stage sits before its last sub-step, so that the first
    // fragments of the next stage are read and expanded under that sub-step's MFMAs
    // instead of after a barrier at the stage boundary. Plain s_barrier: __syncthreads()
    // would also wait for every outstanding load (a workgroup release fence), which would
    // drain the ring; the memory clobber keeps LDS reads from moving across it.
    using F = RingFrags<CL, WI, WJ>;
    F f[2];
    const ExpandK ek = expand_consts(lane);
    wait_vm_stages<NW, RB>(nk - 1 < 2 ? nk - 1 : 2);
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
      wait_vm_stages<NW, RB>(kt + 2 < nk ? 1 : 0);
      asm volatile("s_barrier" ::: "memory");
      if (kt + RING - 1 < nk)
        issue_ring_stage<NW, RB>(smem + ((kt + RING - 1) % RING) * SLOTB, mat, ld, row0, a.M,
                                 (kt0 + kt + RING - 1) * BK, a.codes, rowblock, nkt,
                                 kt0 + kt + RING - 1, wave, lane);
      // Sub-step 3, with stage kt + 1's first fragments read and expanded under it (on
      // the last stage this reads a free slot; the values are not used).
      ring_read<CL, WI, WJ>(smem + ((kt + 1) % RING) * SLOTB, 0, wp, wq, lane, f[0]);
      ring_mfma<CL, WI, WJ>(f[1], f[0], acc, ek);
    }
    __syncthreads();
  }
  if constexpr (SPL == 1) {
    split_store<WI, WJ>(a, acc, pidx, split, tid);
    return;
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

// Phase 2 of a split forward launch, spread over FWD_EPI_G workgroups per tile: workgroup
// b takes tile b mod ntiles (as the phase-1 jobs, so that both phases of a tile share an
// XCD, whose L2 holds the partials) and group g = b / ntiles, i.e. the tile's waves
// v = FWD_EPI_NW g .. + FWD_EPI_NW - 1 of the 8-wave forward layout. It adds their partial
// accumulators in split order and runs their part of the forward epilogue (per wave).
constexpr int FWD_EPI_NW = 2;
constexpr int FWD_EPI_G = 8 / FWD_EPI_NW;
__global__ __launch_bounds__(FWD_EPI_NW * 64) void k_gemm_fwd_epi(GemmArgs a) {
  using T = Tiling<OP_FWD, 8>;
  constexpr int WI = T::WI, WJ = T::WJ;
  __shared__ __attribute__((aligned(16))) uint8_t smem[FWD_EPI_NW * 32 * (32 * WJ + 4) * 4];
  int tile, g, tp, tq, pidx;
  if (a.hyb_L) {
    if (!map_hybrid<2>(a, blockIdx.x, FWD_EPI_G, tp, tq, tile, pidx, g)) return;
  } else {
    tile = (int)blockIdx.x % a.ntiles;
    g = (int)blockIdx.x / a.ntiles;
    if (g >= FWD_EPI_G) return;
    tp = tile / a.tilesQ;                                // as map_split
    tq = tile % a.tilesQ;
    pidx = tile;
  }
  const int p0 = tp * BT, q0 = tq * BT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int lw = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int v = FWD_EPI_NW * g + lw;
  const int wp = v / T::WGQ, wq = v % T::WGQ;
  f32x16 acc[WI][WJ];
  split_load<WI, WJ>(a, acc, pidx, v * 64 + lane, 512);
  epilogue_fwd<FWD_EPI_NW, WI, WJ>(a, acc, p0, q0, wp, wq, lane, lw, smem);
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

// `buf` is the LDS array itself and `tile` the tile's byte offset in it: each read's
// address is one offset from the array, so that the compiler can attribute the read to
// that array (its alias scope is carried only along short chains of address arithmetic).
__device__ __forceinline__ bf16x8 trans_frag(const uint8_t* buf, int tile, int colbase, int s,
                                             int lane) {
  const int g = lane >> 4, t = lane & 15;
  const int col = colbase + 16 * (g & 1) + 4 * (t & 3);
  const int m = 16 * s + 8 * (g >> 1) + (t >> 2);
  const int m2 = m + 4;
  const LCVQ_LDS uint8_t* base = (const LCVQ_LDS uint8_t*)buf;
  const int off_lo = tile + m * TROWB + (((col >> 3) ^ tswz(m)) << 4) + ((col & 4) << 1);
  const int off_hi = tile + m2 * TROWB + (((col >> 3) ^ tswz(m2)) << 4) + ((col & 4) << 1);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LCVQ_LDS v4i16*)(base + off_lo));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LCVQ_LDS v4i16*)(base + off_hi));
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
// Operand OPN (0: X, 1: dY) of one stage, so that a stage's loads can be issued in two
// halves.
template <int OPN>
__device__ __forceinline__ void issue_dw_stage_rows_op(uint8_t* slot, const uint16_t* X,
                                                       const uint16_t* dY, int M, int N, int K,
                                                       int m0, const DwLaneOffsets& o, int wave,
                                                       int lane) {
  const uint16_t* mat = OPN == 0 ? X : dY;
  const int ld = OPN == 0 ? K : N;
  uint8_t* tile = slot + OPN * TTILEB;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int row = m0 + wave * 8 + i * 2;                   // uniform
    uint32_t off = o.v[OPN][i & 1];
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
__device__ __forceinline__ void issue_dw_stage_rows(uint8_t* slot, const uint16_t* X,
                                                    const uint16_t* dY, int M, int N, int K,
                                                    int m0, const DwLaneOffsets& o, int wave,
                                                    int lane) {
  issue_dw_stage_rows_op<0>(slot, X, dY, M, N, K, m0, o, wave, lane);
  issue_dw_stage_rows_op<1>(slot, X, dY, M, N, K, m0, o, wave, lane);
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
  for (int i = 0; i < 4; ++i) f.a[i] = trans_frag(slot, 0, wp * 128 + i * 32, s, lane);
#pragma unroll
  for (int j = 0; j < WJ; ++j) f.b[j] = trans_frag(slot, TTILEB, wq * 32 * WJ + j * 32, s, lane);
}

// The same fragments from per-lane byte offsets computed once (dw_frag_offsets): the
// fragment of sub-step s starts 16 s rows = 8192 bytes further, and its second half
// (rows m + 4, same swizzle) 2048 bytes further. Each read address is then the LDS array
// plus one opaque offset plus a constant, a chain short enough that the compiler keeps
// the read attributed to its array.
struct DwOffsets {
  int a[4], b[2];
};
__device__ __forceinline__ int dw_frag_off(int k, int lane) {   // column block 32 k, s = 0
  const int g = lane >> 4, t = lane & 15;
  const int col = 32 * k + 16 * (g & 1) + 4 * (t & 3);
  const int m = 8 * (g >> 1) + (t >> 2);
  return m * TROWB + (((col >> 3) ^ tswz(m)) << 4) + ((col & 4) << 1);
}
__device__ __forceinline__ DwOffsets dw_frag_offsets(int wp, int wq, int lane) {
  DwOffsets o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o.a[i] = dw_frag_off(4 * wp + i, lane);
    asm volatile("" : "+v"(o.a[i]));
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    o.b[j] = TTILEB + dw_frag_off(2 * wq + j, lane);
    asm volatile("" : "+v"(o.b[j]));
  }
  return o;
}
__device__ __forceinline__ bf16x8 trans_frag_at(const uint8_t* buf, int off) {
  const LCVQ_LDS uint8_t* base = (const LCVQ_LDS uint8_t*)buf;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LCVQ_LDS v4i16*)(base + off));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LCVQ_LDS v4i16*)(base + off + 4 * TROWB));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ void dw_read_at(const uint8_t* buf, int s, const DwOffsets& o,
                                           DwFrags<2>& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f.a[i] = trans_frag_at(buf, o.a[i] + s * 16 * TROWB);
#pragma unroll
  for (int j = 0; j < 2; ++j) f.b[j] = trans_frag_at(buf, o.b[j] + s * 16 * TROWB);
}

template <int WJ>
__device__ __forceinline__ void dw_mfma(const DwFrags<WJ>& f, f32x16 acc[4][WJ]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < WJ; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// Straight-through epilogue on G (rows k, columns n), its d x d contractions on the
// matrix cores (idle by then):
//   dWp[n, k] = mask * sum_k' Mix[k][k'] G[k', n],   Mix = I kron A^T (block diagonal)
//   dA[i][j]  = sum G[g*d+i, n] z[n, g*d+j] = 2 sum G[g*d+i, n] v(z[n, g*d+j]) - 4 dB[i]
//   dB[i]     = sum G[g*d+i, n]
// with v(z) = 2 + z/2, the code operand of the other products. G enters the MFMAs as bf16
// hi + lo halves, and Mix likewise (hi*hi + lo*hi + hi*lo), so both products keep about
// 16 bits of G. The mix takes G in the accumulator layout as its B operand (contraction
// over k). dA contracts over n, the lane index of G: each block's G halves go through the
// wave's LDS area as [n][k] and come back with transposing reads as the A operand, against
// v(z) fragments expanded from the tile's transposed code words (the dX product's code
// layout). Each wave's sums run over all its blocks; the waves' sums are then added in a
// fixed order into the tile's partial row `prow`.
// dW LDS map: two arrays. The main loop's double buffer is stage buffer 0 at the start of
// the first array and stage buffer 1, the second array (64 KiB each); the tile's
// transposed code words (4 slabs of 256 rows k x 16 bytes) and mask bits (256 columns n x
// 32 bytes) follow buffer 0 in the first array from kernel start. The two buffers are
// separate arrays so that the compiler can tell a direct load into one from a read of
// the other: with one array it makes every LDS read wait for the direct loads issued
// before it. The epilogue's per-wave areas then take waves 0-4 in buffer 0 and waves 5-7,
// the waves' sums and A's copy in buffer 1.
constexpr int DW_CODES_OFF = 64 * 1024;
constexpr int DW_MASK_OFF = DW_CODES_OFF + 4 * 4096;    // 80 KiB
constexpr int DW_SMEM0 = DW_MASK_OFF + 256 * 32;        // 88 KiB
constexpr int DW_SMEM1 = 64 * 1024;
constexpr int DW_WREG = 12 * 1024;                      // per-wave epilogue area
constexpr int DW_WAVES_IN_B0 = 5;
constexpr int DW_WSUM_OFF = (8 - DW_WAVES_IN_B0) * DW_WREG;   // in buffer 1
constexpr int DW_A_OFF = 56 * 1024;                           // in buffer 1
constexpr int GTROWB = 72;                 // bytes per row n of a staged bf16 half of G

// ALDS: A is read from its copy in LDS (d = 16, and the second phase of a split launch).
// area: this wave's DW_WREG bytes of LDS (staging, then its reduction); wsum: the waves'
// sums [NW][d*d + d]; codes_lds, mask_lds: the tile's code words and mask bits in LDS.
template <int D, int NW, int WJ, bool ALDS>
__device__ __forceinline__ void epilogue_dw(const GemmArgs& a, f32x16 acc[4][WJ], int p0, int q0, int wp, int wq,
                            int lane, int wave, int prow, uint8_t* area, float* wsum,
                            const uint8_t* codes_lds, const uint8_t* mask_lds, const float* Alds) {
  constexpr int SBYTES = 32 * SROWT * 4;
  constexpr int GTB = 32 * GTROWB;
  constexpr int NO = D * D + D;
  constexpr int DBS = D == 16 ? 8 : 4;         // dB partial sums per lane
  constexpr int RRED = 17;                     // row of the wave reduction (16 + pad)
  static_assert(SBYTES + 2 * GTB <= DW_WREG && (64 * RRED + 16) * 4 <= DW_WREG,
                "per-wave LDS area");
  float* S = reinterpret_cast<float*>(area);
  uint8_t* GTh = area + SBYTES;
  uint8_t* GTl = GTh + GTB;
  const int q = lane & 31, h = lane >> 5;

  // Mix operands. In the MFMA over accumulator registers 8t .. 8t+7, slot e of lane half h
  // holds row k = 16t + 8(e/4) + 4h + e%4 of the block; lane (row q, half h) holds
  // Mix[q][k] for those k: A[k % d][q % d] inside q's d-vector, else 0.
  bf16x8 AMh[2], AMl[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = 16 * t + 8 * (e >> 2) + 4 * h + (e & 3);
      const int idx = (k % D) * D + q % D;
      const float av = ALDS ? Alds[idx] : a.A[idx];
      const float m = k / D == q / D ? av : 0.f;
      const __bf16 mh = (__bf16)m;
      AMh[t][e] = mh;
      AMl[t][e] = (__bf16)(m - (float)mh);
    }
  const ExpandK ek = expand_consts(lane);
  const bool full = p0 + BT <= a.K && q0 + BT <= a.N;
  f32x16 P;
  float dBp[DBS];
#pragma unroll
  for (int r = 0; r < 16; ++r) P[r] = 0.f;
#pragma unroll
  for (int x = 0; x < DBS; ++x) dBp[x] = 0.f;

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < WJ; ++j) {
      const int kb = p0 + wp * 128 + i * 32;
      const int nb = q0 + wq * 32 * WJ + j * 32;
      const int n = nb + q;
      __builtin_amdgcn_sched_barrier(0);   // keep each block's work within its block
      f32x16 g = acc[i][j];
      // Rows and columns past the end of G hold clamped-operand values: they must not
      // reach dA or dB (their dWp entries are not stored).
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int k = kb + 8 * (r >> 2) + 4 * h + (r & 3);
          g[r] = n < a.N && k < a.K ? g[r] : 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int slot = D == 16 ? ((r >> 2) & 1) * 4 + (r & 3) : (r & 3);
        dBp[slot] += g[r];
      }
      uint32_t gh[8], gl[8];
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        gh[p] = pack_bf16x2(g[2 * p], g[2 * p + 1]);
        gl[p] = pack_bf16x2(g[2 * p] - bf16lo_to_f32(gh[p]), g[2 * p + 1] - bf16hi_to_f32(gh[p]));
      }
      const bf16x8 Gh0 = __builtin_bit_cast(bf16x8, u32x4{gh[0], gh[1], gh[2], gh[3]});
      const bf16x8 Gh1 = __builtin_bit_cast(bf16x8, u32x4{gh[4], gh[5], gh[6], gh[7]});
      const bf16x8 Gl0 = __builtin_bit_cast(bf16x8, u32x4{gl[0], gl[1], gl[2], gl[3]});
      const bf16x8 Gl1 = __builtin_bit_cast(bf16x8, u32x4{gl[4], gl[5], gl[6], gl[7]});
      f32x16 o;
#pragma unroll
      for (int r = 0; r < 16; ++r) o[r] = 0.f;
      o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(AMh[0], Gh0, o, 0, 0, 0);
      o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(AMh[1], Gh1, o, 0, 0, 0);
      o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(AMl[0], Gh0, o, 0, 0, 0);
      o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(AMl[1], Gh1, o, 0, 0, 0);
      o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(AMh[0], Gl0, o, 0, 0, 0);
      o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(AMh[1], Gl1, o, 0, 0, 0);
      // mask bits of (n, kb .. kb+31): register r of o is row 8(r/4) + 4h + r%4
      const uint32_t mw =
          *reinterpret_cast<const uint32_t*>(mask_lds + (n - q0) * 32 + ((kb - p0) >> 3)) >> (4 * h);
      wave_sync();                    // the previous block's store and reads are done
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = ((mw >> (8 * qq + e)) & 1u) ? o[4 * qq + e] : 0.f;
        *reinterpret_cast<f32x4*>(S + q * SROWT + 8 * qq + 4 * h) = v;
        *reinterpret_cast<uint2*>(GTh + q * GTROWB + (8 * qq + 4 * h) * 2) =
            make_uint2(gh[2 * qq], gh[2 * qq + 1]);
        *reinterpret_cast<uint2*>(GTl + q * GTROWB + (8 * qq + 4 * h) * 2) =
            make_uint2(gl[2 * qq], gl[2 * qq + 1]);
      }
      wave_sync();
      // dA over the block's 32 n in two contraction steps of 16: the A operand (rows k,
      // contraction n) by transposing reads of the staged halves, the B operand (rows n,
      // columns k) from the code words of rows k = kb .. kb+31.
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int g4 = lane >> 4, t = lane & 15;
        const int col = 16 * (g4 & 1) + 4 * (t & 3);
        const int row = 16 * u + 8 * (g4 >> 1) + (t >> 2);
        typedef short v8i16 __attribute__((ext_vector_type(8)));
        const LCVQ_LDS uint8_t* bh = (const LCVQ_LDS uint8_t*)GTh;
        const LCVQ_LDS uint8_t* bl = (const LCVQ_LDS uint8_t*)GTl;
        const v4i16 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LCVQ_LDS v4i16*)(bh + row * GTROWB + col * 2));
        const v4i16 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LCVQ_LDS v4i16*)(bh + (row + 4) * GTROWB + col * 2));
        const v4i16 l0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LCVQ_LDS v4i16*)(bl + row * GTROWB + col * 2));
        const v4i16 l1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LCVQ_LDS v4i16*)(bl + (row + 4) * GTROWB + col * 2));
        const bf16x8 Ah = __builtin_bit_cast(bf16x8, v8i16{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]});
        const bf16x8 Al = __builtin_bit_cast(bf16x8, v8i16{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]});
        const int nl = nb - q0 + 16 * u;
        const uint32_t w = codes_word(codes_lds + (nl >> 6) * 4096, kb - p0 + q, (nl >> 4) & 3);
        const bf16x8 bv = codes_expand(w, ek);
        P = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ah, bv, P, 0, 0, 0);
        P = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Al, bv, P, 0, 0, 0);
      }
      if (a.dge_wp)
        store_block_rows_dge(S, a.dwp, a.dge_wp, a.dge_alpha, a.dge_c, a.K, nb, a.N, kb, a.K,
                             lane);
      else
        store_block_rows_t(S, a.dwp, a.K, nb, a.N, kb, a.K, lane);
    }

  // The wave's sums. dB: the lanes of a half hold the same slots (both halves, d = 4).
#pragma unroll
  for (int x = 0; x < DBS; ++x) {
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) dBp[x] += __shfl_xor(dBp[x], off);
    if (D == 4) dBp[x] += __shfl_xor(dBp[x], 32);
  }
  float* red = S;                              // [64][RRED] P, then dB of the two halves
  wave_sync();
#pragma unroll
  for (int r = 0; r < 16; ++r) red[lane * RRED + r] = P[r];
  if (q == 0) {
#pragma unroll
    for (int x = 0; x < DBS; ++x) red[64 * RRED + h * 8 + x] = dBp[x];
  }
  wave_sync();
  // P entry (row k, column k') sits in lane 32 h + k' % 32, register r with
  // k = 8(r/4) + 4h + r%4; dA[i][j] adds the entries with k = g d + i, k' = g d + j.
  auto dB_of = [&](int i) -> float {
    if (D == 8) return red[64 * RRED + (i >> 2) * 8 + (i & 3)];
    if (D == 4) return red[64 * RRED + i];
    return red[64 * RRED + ((i >> 2) & 1) * 8 + 4 * (i >> 3) + (i & 3)];
  };
  for (int o = lane; o < NO; o += 64) {
    float v;
    if (o < D * D) {
      const int i = o / D, j = o % D;
      float sum = 0.f;
      if (D == 8) {
        for (int g2 = 0; g2 < 4; ++g2) sum += red[(32 * (i >> 2) + 8 * g2 + j) * RRED + 4 * g2 + (i & 3)];
      } else if (D == 4) {
        for (int g2 = 0; g2 < 8; ++g2) sum += red[(32 * (g2 & 1) + 4 * g2 + j) * RRED + 4 * (g2 >> 1) + i];
      } else {
        for (int g2 = 0; g2 < 2; ++g2)
          sum += red[(32 * ((i >> 2) & 1) + 16 * g2 + j) * RRED + 4 * (2 * g2 + (i >> 3)) + (i & 3)];
      }
      v = 2.f * sum - 4.f * dB_of(i);
    } else {
      v = dB_of(o - D * D);
    }
    wsum[wave * NO + o] = v;
  }
  __syncthreads();
  for (int o = threadIdx.x; o < NO; o += blockDim.x) {
    float sum = 0.f;
    for (int w = 0; w < NW; ++w) sum += wsum[w * NO + o];
    a.partials[(int64_t)prow * NO + o] = sum;
  }
}

// The tile's transposed code words (the dX product's layout: per 256-row block of k and
// 64-column stage of n, a 4 KiB slab of 256 rows x 4 R16 words): the four slabs of stages
// q0/64 .. q0/64 + 3, 16-byte direct loads, 2 per lane. Stages past N read the last one
// (their G columns are zero). Mask bits: 4-byte direct loads (mask rows are only 8-byte
// aligned), 4 per lane; columns past N and k past K read a valid address, never used.
__device__ __forceinline__ void issue_dw_codes(uint8_t* codes_lds, uint8_t* mask_lds,
                                               const uint32_t* r16t, const uint8_t* mask,
                                               int N, int K, int p0, int q0, int wave,
                                               int lane) {
  const int nks = N >> 6;                                // stages along n
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = (wave * 2 + i) * 64 + lane;            // 16-byte chunk of the 16 KiB
    int kt = (q0 >> 6) + (c >> 8);
    kt = kt < nks ? kt : nks - 1;
    const uint32_t* src = r16t + ((int64_t)(p0 >> 8) * nks + kt) * 1024 + (c & 255) * 4;
    __builtin_amdgcn_global_load_lds(src, (LCVQ_LDS void*)(codes_lds + (wave * 2 + i) * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = (wave * 4 + i) * 64 + lane;            // 4-byte word of the mask tile
    int n = q0 + (c >> 3);
    n = n < N ? n : N - 1;
    int kb = p0 + (c & 7) * 32;
    kb = kb < K ? kb : 0;
    const uint8_t* src = mask + (int64_t)n * (K >> 3) + (kb >> 3);
    __builtin_amdgcn_global_load_lds(src, (LCVQ_LDS void*)(mask_lds + (wave * 4 + i) * 256), 4, 0, 0);
  }
}

// dW: 8 waves (512 threads), double-buffered direct loads into LDS (2 x 64 KiB).
// SPL = 0: one workgroup per tile, with the epilogue; SPL = 1: phase 1 of a split launch
// (partial tiles out; phase 2 is k_gemm_dw_epi).
template <int D, int SPL = 0>
__global__ __launch_bounds__(512, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_gemm_dw(GemmArgs a) {
  static_assert(SPL == 0 || SPL == 1, "phase 2 of a split dW is k_gemm_dw_epi");
  constexpr int NW = 8, WGQ = 4, WJ = 2;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[DW_SMEM0];   // buffer 0, codes, mask
  __shared__ __attribute__((aligned(1024))) uint8_t smem1[DW_SMEM1];  // buffer 1
  int tp, tq, tile;
  // X and dY panels weigh the same: 4 x 8 tiles per XCD reads the fewest panels.
  int split = 0, pidx = 0;
  if constexpr (SPL == 1) {
    if (a.hyb_L) {
      if (!map_hybrid<4>(a, blockIdx.x, 2, tp, tq, tile, pidx, split)) return;
    } else {
      if (!map_split(blockIdx.x, a.tilesQ, a.ntiles, a.splits, tp, tq, tile, split)) return;
      pidx = tile;
    }
  } else if (!map_tile<4>(blockIdx.x, a.tilesP, a.tilesQ, a.ntiles, tp, tq, tile)) {
    return;
  }
  const int p0 = tp * BT, q0 = tq * BT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wp = wave / WGQ, wq = wave % WGQ;
  int kt0 = 0, kt1 = (a.R + BK - 1) / BK;
  if constexpr (SPL == 1) split_range(kt1, split, a.splits, kt0, kt1);
  const DwLaneOffsets lo = dw_lane_offsets(a.N, a.K, p0, q0, lane);
  static_assert(WJ == 2, "dw_frag_offsets holds two column fragments");
  const DwOffsets fo = dw_frag_offsets(wp, wq, lane);
  if constexpr (SPL == 0)                            // for the epilogue
    issue_dw_codes(smem + DW_CODES_OFF, smem + DW_MASK_OFF, a.codes, a.mask, a.N, a.K, p0, q0,
                   wave, lane);

  f32x16 acc[4][WJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < WJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  for (int pass = 0; pass < (kt1 > kt0 ? a.npass : 0); ++pass) {
    const uint16_t* Lp = pass == 0 ? a.Lmat[0] : (pass == 1 ? a.Lmat[1] : a.Lmat[2]);
    const uint16_t* Rp = pass == 0 ? a.Rmat[0] : (pass == 1 ? a.Rmat[1] : a.Rmat[2]);
    issue_dw_stage(smem, Lp, Rp, a.M, a.N, a.K, kt0 * BK, p0, q0, wave, lane);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // One stage: the current buffer's fragments are read up to two sub-steps ahead of
    // their MFMAs, and the next stage's direct loads go into the other buffer (free since
    // the last barrier) in two halves, X's rows under sub-step 0's MFMAs and dY's under
    // sub-step 1's, so that they land under the rest of the stage without crowding its
    // first reads. The buffers are fixed per call (the loop is unrolled by two), so the
    // compiler sees that the reads of one buffer do not depend on the loads into the
    // other. (Measured against the earlier order, all fragment reads of sub-steps 0-2
    // before one batch of loads: c1 dW 115.5 -> 112.9 us, 896-tile 14336 x 4096 dW at 8192
    // tokens 888 -> 832 us; issuing all loads at the start of the stage was slower.)
    auto stage = [&](const uint8_t* cur, uint8_t* nxt, int kt) __attribute__((always_inline)) {
      DwFrags<WJ> f0, f1;
      dw_read_at(cur, 0, fo, f0);
      dw_read_at(cur, 1, fo, f1);
      __builtin_amdgcn_sched_barrier(0);
      dw_mfma<WJ>(f0, acc);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 1 < kt1)
        issue_dw_stage_rows_op<0>(nxt, Lp, Rp, a.M, a.N, a.K, (kt + 1) * BK, lo, wave, lane);
      __builtin_amdgcn_sched_barrier(0);
      dw_read_at(cur, 2, fo, f0);
      __builtin_amdgcn_sched_barrier(0);
      dw_mfma<WJ>(f1, acc);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 1 < kt1)
        issue_dw_stage_rows_op<1>(nxt, Lp, Rp, a.M, a.N, a.K, (kt + 1) * BK, lo, wave, lane);
      __builtin_amdgcn_sched_barrier(0);
      dw_read_at(cur, 3, fo, f1);
      __builtin_amdgcn_sched_barrier(0);
      dw_mfma<WJ>(f0, acc);
      dw_mfma<WJ>(f1, acc);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0);
      if (kt + 1 < kt1 && (kt + 1) * BK + wave * 8 + 8 > a.M)
        zero_dw_rows(nxt, (kt + 1) * BK, a.M, wave, lane);
      __syncthreads();
    };
    for (int kt = kt0; kt < kt1; kt += 2) {
      stage(smem, smem1, kt);
      if (kt + 1 < kt1) stage(smem1, smem, kt + 1);
    }
  }
  if constexpr (SPL == 1) {
    split_store<4, WJ>(a, acc, pidx, split, tid);
    return;
  }
  // The buffers are free after the last barrier: per-wave areas of 12 KiB (waves 0-4 in
  // buffer 0, 5-7 in buffer 1), the waves' sums and for d = 16 a copy of A in buffer 1.
  static_assert(DW_WAVES_IN_B0 * DW_WREG <= DW_CODES_OFF, "waves 0-4 below the code words");
  static_assert(DW_WSUM_OFF + NW * (D * D + D) * 4 <= DW_A_OFF &&
                DW_A_OFF + D * D * 4 <= DW_SMEM1, "sums and A in buffer 1");
  float* Alds = reinterpret_cast<float*>(smem1 + DW_A_OFF);
  constexpr bool ALDS = D == 16;
  if (ALDS) {
    if (tid < D * D) Alds[tid] = a.A[tid];
    __syncthreads();
  }
  uint8_t* area = wave < DW_WAVES_IN_B0 ? smem + wave * DW_WREG
                                        : smem1 + (wave - DW_WAVES_IN_B0) * DW_WREG;
  epilogue_dw<D, NW, WJ, ALDS>(a, acc, p0, q0, wp, wq, lane, wave, tile, area,
                               reinterpret_cast<float*>(smem1 + DW_WSUM_OFF),
                               smem + DW_CODES_OFF, smem + DW_MASK_OFF, Alds);
}

// Phase 2 of a split dW launch, spread over DW_EPI_G workgroups per tile so that few-tile
// launches still fill the chip with the epilogue's VALU work: workgroup b takes tile
// b mod ntiles (as the phase-1 jobs, so that a tile's workgroups of both phases share an
// XCD, whose L2 holds the partials) and group g = b / ntiles, i.e. the tile's waves
// v = DW_EPI_NW g .. + DW_EPI_NW - 1 of the 8-wave layout of phase 1. It adds their partial
// accumulators in split order and runs their part of the straight-through epilogue; its
// dA/dB sums go to partial row DW_EPI_G * tile + g (tail split: see map_hybrid and prow
// below). LDS: the waves' 12 KiB areas, their
// sums, A, then the whole tile's codes and mask bits.
constexpr int DW_EPI_NW = 2;
constexpr int DW_EPI_G = 8 / DW_EPI_NW;
constexpr int EPI_A_OFF = 28 * 1024;
constexpr int EPI_CODES_OFF = 32 * 1024;
constexpr int EPI_MASK_OFF = EPI_CODES_OFF + 4 * 4096;
constexpr int EPI_SMEM = EPI_MASK_OFF + 256 * 32;       // 56 KiB
template <int D>
__global__ __launch_bounds__(DW_EPI_NW * 64) void k_gemm_dw_epi(GemmArgs a) {
  constexpr int WGQ = 4, WJ = 2;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[EPI_SMEM];
  int tile, g, tp, tq, pidx, prow;
  if (a.hyb_L) {
    if (!map_hybrid<4>(a, blockIdx.x, DW_EPI_G, tp, tq, tile, pidx, g)) return;
    // group 0 writes the tile's own partial row, groups 1-3 rows after the unsplit tiles'
    prow = g == 0 ? tile : a.ntiles + (DW_EPI_G - 1) * pidx + g - 1;
  } else {
    tile = (int)blockIdx.x % a.ntiles;
    g = (int)blockIdx.x / a.ntiles;
    if (g >= DW_EPI_G) return;
    tp = tile / a.tilesQ;                                // as map_split
    tq = tile % a.tilesQ;
    pidx = tile;
    prow = DW_EPI_G * tile + g;
  }
  const int p0 = tp * BT, q0 = tq * BT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int lw = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int v = DW_EPI_NW * g + lw;                       // wave of the 8-wave layout
  const int wp = v / WGQ, wq = v % WGQ;
  for (int vw = lw; vw < 8; vw += DW_EPI_NW)              // the whole tile's codes and mask
    issue_dw_codes(smem + EPI_CODES_OFF, smem + EPI_MASK_OFF, a.codes, a.mask, a.N, a.K, p0,
                   q0, vw, lane);
  float* Alds = reinterpret_cast<float*>(smem + EPI_A_OFF);
  for (int i = tid; i < D * D; i += DW_EPI_NW * 64) Alds[i] = a.A[i];
  f32x16 acc[4][WJ];
  split_load<4, WJ>(a, acc, pidx, v * 64 + lane, 512);
  __builtin_amdgcn_s_waitcnt(0);                          // the codes and mask in LDS
  __syncthreads();
  static_assert(DW_EPI_NW * DW_WREG + DW_EPI_NW * (D * D + D) * 4 <= EPI_A_OFF,
                "per-wave areas and sums below A's copy");
  epilogue_dw<D, DW_EPI_NW, WJ, true>(a, acc, p0, q0, wp, wq, lane, lw, prow,
                                      smem + lw * DW_WREG,
                                      reinterpret_cast<float*>(smem + DW_EPI_NW * DW_WREG),
                                      smem + EPI_CODES_OFF, smem + EPI_MASK_OFF, Alds);
}

// dW tail split: where the 256 x 256 tiles fill whole rounds of the 256 CUs plus a last
// round at most half full (and the count is a multiple of the 8 XCDs), the tiles of the
// full rounds run unsplit and each leftover tile splits its contraction in two, so that
// the leftover work takes half a round instead of a whole one. Per XCD: hyb_per tiles,
// the first hyb_F unsplit, the last hyb_L split. Needs at least 16 contraction stages.
// (The forward takes the same rule for its 256 x 256 tiles.)
static bool tail_split(int64_t nt, int64_t R, int& per, int& F, int& L) {
  const int64_t r = nt % 256;
  if (nt <= 256 || (nt % 8) || r == 0 || r > 128 || (R + BK - 1) / BK < 16) return false;
  per = (int)(nt / 8);
  L = (int)(r / 8);
  F = per - L;
  return true;
}
static bool dw_hybrid(int64_t M, int64_t N, int64_t K, int& per, int& F, int& L) {
  return tail_split(gemm_tiles(K, N), M, per, F, L);
}

// dA/dB partial rows the dW product of this shape writes (the reduction's input).
int dw_partial_rows(int64_t M, int64_t N, int64_t K) {
  const int nt = gemm_tiles(K, N);
  int per, F, L;
  if (gemm_splits(K, N, M) > 1) return nt * DW_EPI_G;
  if (dw_hybrid(M, N, K, per, F, L)) return nt + (DW_EPI_G - 1) * 8 * L;
  return nt;
}

// Bytes of float32 partial tiles the dW product needs (0: none).
size_t dw_split_bytes(int64_t M, int64_t N, int64_t K) {
  int per, F, L;
  if (gemm_splits(K, N, M) > 1) return gemm_split_bytes(K, N, M);
  if (dw_hybrid(M, N, K, per, F, L)) return (size_t)8 * L * 2 * BT * BT * 4;
  return 0;
}

// ---- Gram matrix H = X^T X of calibration activations --------------------------------
// The dW product's main loop with X as both operands: C[p, q] = sum_m X[m, p] X[m, q] on
// 256 x 256 tiles, computed only for tile-row <= tile-column. Every element with p <= q
// is written to H[p][q] and H[q][p] (elements p > q of a diagonal tile are skipped), so H
// is exactly symmetric. Rows m past M are contraction terms and are cleared; columns past
// K are clamped reads whose results are not stored.
__global__ __launch_bounds__(512, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_gram(const uint16_t* __restrict__ X, int M, int K, float* __restrict__ H) {
  constexpr int WGQ = 4, WJ = 2;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TTILEB];   // 128 KiB
  const int T = (K + BT - 1) / BT;
  int t = blockIdx.x, tp = 0;                     // upper tile t -> (tp, tq), row by row
  while (t >= T - tp) {
    t -= T - tp;
    ++tp;
  }
  const int tq = tp + t;
  const int p0 = tp * BT, q0 = tq * BT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wp = wave / WGQ, wq = wave % WGQ;
  const int nk = (M + BK - 1) / BK;
  const DwLaneOffsets lo = dw_lane_offsets(K, K, p0, q0, lane);
  f32x16 acc[4][WJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < WJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  issue_dw_stage(smem, X, X, M, K, K, 0, p0, q0, wave, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {                // the dW product's stage order
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
    if (kt + 1 < nk) issue_dw_stage_rows(next, X, X, M, K, K, (kt + 1) * BK, lo, wave, lane);
    __builtin_amdgcn_sched_barrier(0);
    dw_mfma<WJ>(f1, acc);
    dw_mfma<WJ>(f2, acc);
    dw_mfma<WJ>(f0, acc);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);
    if (kt + 1 < nk && (kt + 1) * BK + wave * 8 + 8 > M) zero_dw_rows(next, (kt + 1) * BK, M, wave, lane);
    __syncthreads();
  }
  // accumulator block (i, j): lane column q = l % 32; register r holds row
  // 8 (r / 4) + 4 (l / 32) + r % 4, so registers 4g .. 4g + 3 are four consecutive rows:
  // H[q][p .. p + 3] is one 16-byte store when all four rows are at or above the diagonal.
  const int col = lane & 31, h = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < WJ; ++j) {
      const int q = q0 + wq * 32 * WJ + j * 32 + col;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int p = p0 + wp * 128 + i * 32 + 8 * g + 4 * h;
        const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                         acc[i][j][4 * g + 3]};
        if (q >= K) continue;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (p + u < K && p + u <= q) H[(int64_t)(p + u) * K + q] = v[u];
        if (p + 3 < q && p + 3 < K) {
          *reinterpret_cast<f32x4*>(H + (int64_t)q * K + p) = v;
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (p + u < K && p + u < q) H[(int64_t)q * K + p + u] = v[u];
        }
      }
    }
}

hipError_t launch_gram(const uint16_t* X, int M, int K, float* H, hipStream_t s) {
  const int T = (K + BT - 1) / BT;
  LCVQ_LAUNCH(PROF_GRAM, k_gram, dim3(T * (T + 1) / 2), dim3(512), 0, s, X, M, K, H);
  return hipGetLastError();
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
int gemm_splits(int64_t P, int64_t Q, int64_t R) {
  const int64_t nt = ((P + BT - 1) / BT) * ((Q + BT - 1) / BT);
  const int64_t nk = (R + BK - 1) / BK;
  // Measured on k/v-shaped layers (8192 tokens): with 64 tiles the split pays (dW 176 ->
  // 121 us), and with 128 tiles (the forward, half the chip) too since the second phase
  // loads its partials in one batch (95 -> 80 us).
  if (nt > 128) return 1;
  int64_t sp = 256 / nt;
  if (sp > 4) sp = 4;
  if (sp > nk / 8) sp = nk / 8;                      // at least 8 stages per job
  return sp < 1 ? 1 : (int)sp;
}

size_t gemm_split_bytes(int64_t P, int64_t Q, int64_t R) {
  const int sp = gemm_splits(P, Q, R);
  if (sp == 1) return 0;
  const size_t nt = (size_t)(((P + BT - 1) / BT) * ((Q + BT - 1) / BT));
  return nt * sp * BT * BT * 4;
}

// The forward runs 128 x 256 tiles, without a split, when its 256 x 256 tiles would
// occupy at most half of the 256 CUs and the 128-row tiles occupy more than half: at
// 8192 tokens and N = 1024 that is 256 tiles in one round, where the split's float32
// partial tiles cost a write and a read of 64 MiB.
bool gemm_fwd_half_tiles(int64_t M, int64_t N) {
  const int64_t tq = (N + BT - 1) / BT;
  return ((M + BT - 1) / BT) * tq <= 128 && ((M + 127) / 128) * tq > 128;
}

// The forward's 256 x 256 tiles: the few-tile split, or the tail split of a last round
// at most half full.
static bool fwd_hybrid(int64_t M, int64_t N, int64_t K, int& per, int& F, int& L) {
  return gemm_splits(M, N, K) == 1 && tail_split(gemm_tiles(M, N), K, per, F, L);
}

size_t gemm_fwd_split_bytes(int64_t M, int64_t N, int64_t K) {
  if (gemm_fwd_half_tiles(M, N)) return 0;
  int per, F, L;
  if (fwd_hybrid(M, N, K, per, F, L)) return (size_t)8 * L * 2 * BT * BT * 4;
  return gemm_split_bytes(M, N, K);
}

template <int OP, int SPL>
static hipError_t launch_op1(GemmArgs& a, int d, int grid, hipStream_t s);

template <int OP>
static hipError_t launch_op(GemmArgs& a, int d, hipStream_t s) {
  a.tilesP = (a.P + BT - 1) / BT;
  a.tilesQ = (a.Q + BT - 1) / BT;
  a.ntiles = a.tilesP * a.tilesQ;
  if constexpr (OP == OP_FWD) {
    if (a.bpt == 128) {
      static_assert(LCVQ_FWD_WAVES == 8, "the forward's 128-row tiles use the 8-wave layout");
      a.tilesP = (a.P + 127) / 128;
      a.ntiles = a.tilesP * a.tilesQ;
      const dim3 g(((a.ntiles + 7) / 8) * 8), b(8 * 64);
      switch (d) {
        case 4: LCVQ_LAUNCH(PROF_FWD, (k_gemm_ring<OP_FWD, 4, 8, 0, 128>), g, b, 0, s, a); break;
        case 8: LCVQ_LAUNCH(PROF_FWD, (k_gemm_ring<OP_FWD, 8, 8, 0, 128>), g, b, 0, s, a); break;
        default: LCVQ_LAUNCH(PROF_FWD, (k_gemm_ring<OP_FWD, 16, 8, 0, 128>), g, b, 0, s, a); break;
      }
      return hipGetLastError();
    }
  }
  if constexpr (OP == OP_DX) {
    return launch_op1<OP, 0>(a, d, ((a.ntiles + 7) / 8) * 8, s);
  } else {
    if (a.hyb_L) {
      // tail split: the full rounds unsplit, then the leftover tiles' two halves and
      // their phase 2; the timing hook, when armed, brackets the three launches
      constexpr int id = OP == OP_FWD ? PROF_FWD : PROF_DW;
      hipEvent_t e0, e1;
      const bool timed = take_profile(id, &e0, &e1);
      if (timed) (void)hipEventRecord(e0, s);
      hipError_t e = launch_op1<OP, 0>(a, d, 8 * a.hyb_F, s);
      if (e == hipSuccess) e = launch_op1<OP, 1>(a, d, 8 * a.hyb_L * 2, s);
      if (e == hipSuccess)
        e = launch_op1<OP, 2>(a, d, 8 * a.hyb_L * (OP == OP_DW ? DW_EPI_G : FWD_EPI_G), s);
      if (timed) (void)hipEventRecord(e1, s);
      return e;
    }
    if (a.splits <= 1) return launch_op1<OP, 0>(a, d, ((a.ntiles + 7) / 8) * 8, s);
    // Split launch: the timing hook, when armed for this product, brackets both phases
    // with events on the stream.
    constexpr int id = OP == OP_FWD ? PROF_FWD : PROF_DW;
    hipEvent_t e0, e1;
    const bool timed = take_profile(id, &e0, &e1);
    if (timed) (void)hipEventRecord(e0, s);
    hipError_t e = launch_op1<OP, 1>(a, d, a.ntiles * a.splits, s);
    if (e != hipSuccess) return e;
    e = launch_op1<OP, 2>(a, d, a.ntiles * (OP == OP_DW ? DW_EPI_G : FWD_EPI_G), s);
    if (timed) (void)hipEventRecord(e1, s);
    return e;
  }
}

template <int OP, int SPL>
static hipError_t launch_op1(GemmArgs& a, int d, int grid, hipStream_t s) {
  if constexpr (OP == OP_DW && SPL == 2) {
    const dim3 b(DW_EPI_NW * 64);
    switch (d) {
      case 4: LCVQ_LAUNCH(PROF_DW, k_gemm_dw_epi<4>, dim3(grid), b, 0, s, a); break;
      case 8: LCVQ_LAUNCH(PROF_DW, k_gemm_dw_epi<8>, dim3(grid), b, 0, s, a); break;
      default: LCVQ_LAUNCH(PROF_DW, k_gemm_dw_epi<16>, dim3(grid), b, 0, s, a); break;
    }
  } else if constexpr (OP == OP_DW) {
    switch (d) {
      case 4: LCVQ_LAUNCH(PROF_DW, (k_gemm_dw<4, SPL>), dim3(grid), dim3(512), 0, s, a); break;
      case 8: LCVQ_LAUNCH(PROF_DW, (k_gemm_dw<8, SPL>), dim3(grid), dim3(512), 0, s, a); break;
      default: LCVQ_LAUNCH(PROF_DW, (k_gemm_dw<16, SPL>), dim3(grid), dim3(512), 0, s, a); break;
    }
  } else if constexpr (OP == OP_FWD && SPL == 2) {
    static_assert(LCVQ_FWD_WAVES == 8, "the forward's spread phase 2 follows the 8-wave layout");
    LCVQ_LAUNCH(PROF_FWD, k_gemm_fwd_epi, dim3(grid), dim3(FWD_EPI_NW * 64), 0, s, a);
  } else {
    constexpr int id = OP == OP_FWD ? PROF_FWD : PROF_DX;
    constexpr int NW = OP == OP_FWD ? LCVQ_FWD_WAVES : LCVQ_DX_WAVES;
    switch (d) {
      case 4: LCVQ_LAUNCH(id, (k_gemm_ring<OP, 4, NW, SPL>), dim3(grid), dim3(NW * 64), 0, s, a); break;
      case 8: LCVQ_LAUNCH(id, (k_gemm_ring<OP, 8, NW, SPL>), dim3(grid), dim3(NW * 64), 0, s, a); break;
      default: LCVQ_LAUNCH(id, (k_gemm_ring<OP, 16, NW, SPL>), dim3(grid), dim3(NW * 64), 0, s, a); break;
    }
  }
  return hipGetLastError();
}

// Measurement helper, no step of the method: the matrix-core issue ceiling the products
// are compared to. One workgroup of 8 waves per CU (2 per SIMD, as in the products); each
// wave runs `iters` rounds of the products' 8 independent 32x32x16 bf16 MFMAs (4 x 2
// accumulator blocks). Operands are pseudo-random bf16 values of magnitude in [0.5, 1)
// with random signs and mantissas, in two sets used on alternate rounds so that the
// operand bits toggle as when data streams through (the matrix cores' power, and so their
// clock, depend on data activity). One word per workgroup goes to sink so that nothing is
// dropped. Flops: iters * 8 * 2 * 32 * 32 * 16 per wave.
__global__ __launch_bounds__(512, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_mfma_probe(int iters, uint32_t* __restrict__ sink) {
  const int tid = threadIdx.x;
  uint32_t h = ((uint32_t)blockIdx.x * 512u + (uint32_t)tid) * 0x9E3779B9u + 0x7F4A7C15u;
  auto next = [&h]() {
    h ^= h << 13; h ^= h >> 17; h ^= h << 5;
    return (h & 0x807F807Fu) | 0x3F003F00u;     // two bf16: sign, exponent -1, mantissa
  };
  bf16x8 a[2][4], b[2][2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a[s2][i] = __builtin_bit_cast(bf16x8, u32x4{next(), next(), next(), next()});
#pragma unroll
    for (int j = 0; j < 2; ++j) b[s2][j] = __builtin_bit_cast(bf16x8, u32x4{next(), next(), next(), next()});
  }
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  for (int it = 0; it < iters; it += 2) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s2][i], b[s2][j], acc[i][j], 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) t += acc[i][j][r];
  __shared__ float w[8];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o);
  if ((tid & 63) == 0) w[tid >> 6] = t;
  __syncthreads();
  if (tid == 0) {
    float u = 0.f;
    for (int k = 0; k < 8; ++k) u += w[k];
    sink[blockIdx.x & 1023] = __builtin_bit_cast(uint32_t, u);
  }
}

// iters (even) rounds on 256 workgroups: iters * 2^29 flops.
hipError_t launch_mfma_probe(int iters, uint32_t* sink, hipStream_t s) {
  LCVQ_LAUNCH(PROF_MFMA_PROBE, k_mfma_probe, dim3(256), dim3(512), 0, s, iters, sink);
  return hipGetLastError();
}

int gemm_tiles(int64_t P, int64_t Q) { return (int)(((P + BT - 1) / BT) * ((Q + BT - 1) / BT)); }

// Split contraction for launches of few tiles; split_ws holds gemm_split_bytes(P, Q, R)
// of partial tiles.
static void set_splits(GemmArgs& a, int64_t P, int64_t Q, int64_t R, void* split_ws) {
  a.splits = split_ws ? gemm_splits(P, Q, R) : 1;
  if (a.splits > 1) a.split_ws = static_cast<float*>(split_ws);
}

hipError_t launch_gemm_fwd(const uint16_t* xs, const uint16_t* xs_lo, const uint32_t* r16,
                           const float* beta, int M, int N, int K, int d, void* Y, bool y_f32,
                           void* split_ws, hipStream_t s) {
  GemmArgs a = {};
  a.bpt = gemm_fwd_half_tiles(M, N) ? 128 : 256;
  if (a.bpt == 256) set_splits(a, M, N, K, split_ws);
  else a.splits = 1;
  if (a.bpt == 256 && a.splits == 1 && split_ws && fwd_hybrid(M, N, K, a.hyb_per, a.hyb_F, a.hyb_L)) {
    a.splits = 2;
    a.split_ws = static_cast<float*>(split_ws);
  }
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
    a.red_tiles = dw_partial_rows(M, N, K);
    a.red_dA = dA;
    a.red_dB = dB;
  }
  a.splits = 1;
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
                          const uint16_t* dy_lo, const uint32_t* r16t, const uint8_t* mask,
                          const float* A, int M, int N, int K, int d, float* dWp,
                          float* partials, float* dA, float* dB, const float* dge_wp,
                          float dge_alpha, bool reduce, void* split_ws, hipStream_t s) {
  GemmArgs a = {};
  set_splits(a, K, N, M, split_ws);
  if (a.splits == 1 && split_ws && dw_hybrid(M, N, K, a.hyb_per, a.hyb_F, a.hyb_L)) {
    a.splits = 2;
    a.split_ws = static_cast<float*>(split_ws);
  }
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
  a.dwp = dWp; a.codes = r16t; a.mask = mask; a.partials = partials;
  a.dge_wp = dge_wp;
  a.dge_alpha = dge_alpha;
  a.dge_c = dge_wp ? (float)((double)dge_alpha / (2.0 * tanh((double)dge_alpha / 2.0))) : 0.f;
  hipError_t e = launch_op<OP_DW>(a, d, s);
  if (e != hipSuccess || !reduce) return e;
  hipLaunchKernelGGL(k_reduce_partials, dim3(d * d + d), dim3(256), 0, s, partials,
                     dw_partial_rows(M, N, K),
                     d * d + d, dA, dB, d);
  return hipGetLastError();
}

}  // namespace lcvq
