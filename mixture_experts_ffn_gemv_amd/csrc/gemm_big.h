// bf16 MFMA grouped GEMM with large tiles for the prefill gate/up and down
// projections.
//
// Workgroup tile: 256 weight rows x BT routes (BT = 256, or 128 when the
// experts average fewer routes), K in steps of 32; 4 waves in a 2 x 2 grid,
// each owning 128 weight rows x BT/2 routes of f32 accumulators built from
// v_mfma_f32_32x32x16_bf16 (4 x BT/64 tiles of 32x32 per wave).  Large tiles
// are what keeps the L2-miss traffic down: every weight byte staged in LDS
// feeds BT routes and every route byte feeds 256 weight rows.
//
// Pipeline: a 3-stage LDS ring and two register staging sets.  In iteration
// kt the workgroup issues the global loads of K-tile kt+3, computes tile kt
// from LDS, and stores tile kt+2 (loaded one iteration earlier) into the ring
// slot freed by tile kt-1, so a load has two iterations of MFMA work to land.
// Rows are 64 bytes (4 chunks of 16 B); chunk c of row r sits at slot
// c ^ ((r >> 2) & 3), which keeps the 16 lanes a ds_read_b128 serves per
// cycle on 16 distinct bank groups.
#pragma once

#include "common.h"
#include "gemm.h"

namespace moe {

constexpr int kBW = 256;     // weight rows per tile
constexpr int kBK = 32;      // K per stage
constexpr int kStages = 3;   // LDS ring depth

__device__ __forceinline__ int swz64(int row, int chunk) {
  return row * kBK + ((chunk ^ ((row >> 2) & 3)) << 3);
}

template <int MODE, int ACT, int BT>
__global__ __launch_bounds__(256, BT == 128 ? 2 : 1) void k_gemm_big(GemmParams p) {
  constexpr int WT = BT / 2;          // routes per wave
  constexpr int NJ = WT / 32;         // 32-wide route blocks per wave
  constexpr int A_ELEMS = kBW * kBK;  // per stage
  constexpr int B_ELEMS = BT * kBK;
  constexpr int NA = kBW * 4 / 256;   // 16-byte A chunks per thread per stage (4)
  constexpr int NB = BT * 4 / 256;    // B chunks per thread per stage (4 or 2)
  __shared__ __attribute__((aligned(16))) uint16_t sA[kStages][A_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t sB[kStages][B_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int nnt = gridDim.y;
  const int ntiles = *p.n_tiles;
  const int L = xcd_valid_remap(blockIdx.y * gridDim.x + blockIdx.x, ntiles * nnt);
  if (L < 0) return;
  int ti, nt;
  grouped_tile(L, ntiles, nnt, ti, nt);
  const int g = p.tile_group[ti];
  const int m0 = p.tile_m0[ti];
  const bool shared = (g == p.E);
  const int count = shared ? p.T : p.counts[g];
  const int base = shared ? 0 : p.offsets[g];
  int K, Nw;
  if constexpr (MODE == GM_GATEUP) { K = p.H; Nw = shared ? p.Is : p.I; }
  else { K = shared ? p.Is : p.I; Nw = p.H; }
  const int nstep = (MODE == GM_GATEUP) ? kBW / 2 : kBW;
  const int n0 = nt * nstep;
  if (n0 >= Nw) return;

  // ---- global -> register staging assignments -------------------------------
  // A: 256 rows x 4 chunks; thread covers chunks q = tid + 256 i (row q/4).
  // GATEUP rows 0..127 are gate features n0.., rows 128..255 the up rows.
  const uint16_t* a_src[NA];
  int a_lds[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int q = tid + 256 * i;
    const int row = q >> 2, c = q & 3;
    a_lds[i] = swz64(row, c);
    const uint16_t* wp;
    if constexpr (MODE == GM_GATEUP) {
      const int f = min(n0 + (row & 127), Nw - 1);   // clamped rows are never stored
      const uint16_t* m = (row < 128) ? (shared ? p.sw0 : p.w0) : (shared ? p.sw1 : p.w1);
      wp = m + ((shared ? 0 : (size_t)g * Nw) + f) * (size_t)K;
    } else {
      const int n = min(n0 + row, Nw - 1);
      wp = (shared ? p.sw0 : p.w0) + ((shared ? 0 : (size_t)g * Nw) + n) * (size_t)K;
    }
    a_src[i] = wp + c * 8;
  }
  const uint16_t* b_src[NB];
  int b_lds[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int q = tid + 256 * i;
    const int row = q >> 2, c = q & 3;
    b_lds[i] = swz64(row, c);
    const int m = min(m0 + row, count - 1);           // clamped routes are never stored
    const uint16_t* ap;
    if constexpr (MODE == GM_DOWN) {
      ap = shared ? p.sact + (size_t)m * K : p.act + (size_t)(base + m) * K;
    } else {
      const int t = shared ? m : p.row_token[base + m];
      ap = p.act + (size_t)t * K;
    }
    b_src[i] = ap + c * 8;
  }

  // ---- wave sub-tile ----------------------------------------------------------
  const int ww = wave & 1, wt = wave >> 1;
  int arow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (MODE == GM_GATEUP)  // blocks 0,1 gate, 2,3 up of the same features
      arow[i] = (i >> 1) * 128 + 64 * ww + 32 * (i & 1);
    else
      arow[i] = 128 * ww + 32 * i;
  }
  const int brow0 = WT * wt;
  f32x16 acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int fr = lane & 31, fk = lane >> 5;
  const int nk = K / kBK;

  u32x4 ra0[NA], rb0[NB], ra1[NA], rb1[NB];
  auto gload = [&](int kt, u32x4 (&ra)[NA], u32x4 (&rb)[NB]) {
    const int ko = kt * kBK;
#pragma unroll
    for (int i = 0; i < NA; ++i) ra[i] = ld16(a_src[i] + ko);
#pragma unroll
    for (int i = 0; i < NB; ++i) rb[i] = ld16(b_src[i] + ko);
  };
  auto lstore = [&](int slot, const u32x4 (&ra)[NA], const u32x4 (&rb)[NB]) {
#pragma unroll
    for (int i = 0; i < NA; ++i) *reinterpret_cast<u32x4*>(&sA[slot][a_lds[i]]) = ra[i];
#pragma unroll
    for (int i = 0; i < NB; ++i) *reinterpret_cast<u32x4*>(&sB[slot][b_lds[i]]) = rb[i];
  };
  auto compute = [&](int slot) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {  // two k-steps of 16
      bf16x8 af[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(&sA[slot][swz64(arow[i] + fr, 2 * s + fk)]);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const bf16x8 bf = *reinterpret_cast<const bf16x8*>(&sB[slot][swz64(brow0 + 32 * j + fr, 2 * s + fk)]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf, acc[i][j], 0, 0, 0);
      }
    }
  };

  // K is a multiple of 64, so nk is even and the loop below runs whole
  // (even, odd) pairs.  Loads and stores are unconditional (the prefetch
  // index is clamped to the last tile): a conditional load would force the
  // wait-count pass to assume the no-load path and wait for every load.
  // prologue: tiles 0 and 1 into the ring, tile 2 in flight in set 0
  gload(0, ra0, rb0);
  lstore(0, ra0, rb0);
  gload(1, ra1, rb1);
  lstore(1, ra1, rb1);
  gload(min(2, nk - 1), ra0, rb0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    // even: tile kt+2 is in set 0, tile kt+3 goes to set 1
    gload(min(kt + 3, nk - 1), ra1, rb1);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the MFMAs
    compute(kt % kStages);
    lstore((kt + 2) % kStages, ra0, rb0);
    __syncthreads();
    // odd: tile kt+3 is in set 1, tile kt+4 goes to set 0
    gload(min(kt + 4, nk - 1), ra0, rb0);
    __builtin_amdgcn_sched_barrier(0);
    compute((kt + 1) % kStages);
    lstore((kt + 3) % kStages, ra1, rb1);
    __syncthreads();
  }

  // ---- epilogue: acc[i][j][4q + v] = weight row arow[i] + 8q + 4*(lane>>5) + v,
  //      route brow0 + 32 j + (lane & 31) -----------------------------------------
  const int rsub = 4 * (lane >> 5);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int m = m0 + brow0 + 32 * j + (lane & 31);
    if (m >= count) continue;
    uint16_t* outp = shared ? reinterpret_cast<uint16_t*>(p.sout) + (size_t)m * Nw
                            : reinterpret_cast<uint16_t*>(p.out) + (size_t)(base + m) * Nw;
    if constexpr (MODE == GM_GATEUP) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int f = n0 + arow[i] + 8 * q + rsub;  // gate rows: tile rows < 128
          if (f < Nw) {
            float hv[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {  // the shared expert is always SwiGLU
              const float gv = acc[i][j][4 * q + v], uv = acc[i + 2][j][4 * q + v];
              hv[v] = (shared ? silu_f(gv) : act_f<ACT>(gv)) * uv;
            }
            u32x2 pk;
            pk[0] = pack_bf16x2(hv[0], hv[1]);
            pk[1] = pack_bf16x2(hv[2], hv[3]);
            *reinterpret_cast<u32x2*>(outp + f) = pk;
          }
        }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + arow[i] + 8 * q + rsub;
          if (n < Nw) {
            u32x2 pk;
            pk[0] = pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
            pk[1] = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
            *reinterpret_cast<u32x2*>(outp + n) = pk;
          }
        }
    }
  }
}

}  // namespace moe
