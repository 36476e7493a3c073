// bf16 MFMA grouped GEMM for many tokens per expert (prefill).
//
// Each workgroup computes a 128 (weight rows) x 128 (routes) tile of
// C^T = W . X^T over K in steps of 64, with v_mfma_f32_32x32x16_bf16 and
// f32 accumulation (on gfx950 the 32x32x16 form sustains about 90% of the
// bf16 peak with one wave per SIMD, the 16x16x32 form about half of it).
// Each wave owns a 64 x 64 sub-tile: 2 x 2 blocks of 32x32.  Weights are
// the MFMA "A" operand, the gathered route activations the "B" operand, so
// each lane ends up holding runs of four consecutive output features of one
// route: epilogue stores are 8-byte contiguous pieces of a route's row.
//
// The route tiles come from a flat list (group, first row) built after the
// expert grouping, so a skewed load only changes the number of tiles, not
// their shape.  A and B tiles are staged through LDS (double-buffered, the
// 16-byte chunks of each 128-byte row XOR-swizzled so the ds_read_b128
// fragment loads are bank-conflict free, see swz).
//
// Modes:
//   GATEUP : rows 0..63 of the weight tile are gate rows n0..n0+63, rows
//            64..127 the up rows of the same features; the epilogue writes
//            h = act(gate) * up as bf16.
//   DOWN   : y = Wd h, bf16.
//   ROUTER : logits = Wr x (+ bias) as f32; row E is the shared gate vector.
#pragma once

#include "common.h"

namespace moe {

constexpr int kTileW = 128;   // weight rows per tile
constexpr int kTileT = 128;   // routes per tile
constexpr int kTileK = 64;    // K per stage

enum GemmMode : int { GM_GATEUP = 0, GM_DOWN = 1, GM_ROUTER = 2 };

struct GemmParams {
  // weights (bf16 bits)
  const uint16_t* w0;    // GATEUP: gate [E,I,H]; DOWN: down [E,H,I]; ROUTER: router [E,H]
  const uint16_t* w1;    // GATEUP: up [E,I,H]
  const uint16_t* sw0;   // shared gate [Is,H] / shared down [H,Is] / shared_gate_inp [H]
  const uint16_t* sw1;   // shared up [Is,H]
  const float* bias;     // ROUTER: [E] or null
  // activations (bf16 bits)
  const uint16_t* act;   // GATEUP/ROUTER: x [T,H]; DOWN: h [R,I]
  const uint16_t* sact;  // DOWN: hs [T,Is]
  // outputs
  void* out;             // GATEUP: h [R,I] bf16; DOWN: y [R,H] bf16; ROUTER: logits [T,ncols] f32
  void* sout;            // GATEUP: hs [T,Is]; DOWN: ys [T,H]
  // grouping
  const int32_t* counts;     // [G]
  const int32_t* offsets;    // [E+1]
  const int32_t* row_token;  // [R]
  const int32_t* tile_group; // [max_tiles]
  const int32_t* tile_m0;
  const int32_t* n_tiles;
  int E, T, H, I, Is, ncols;
  // GATEUP/DOWN on the direct-to-LDS kernel: weights packed into K-step
  // blocks (moe_pack_weights layout) for the routed experts and the shared
  // one; null: the row-major w0/w1/sw0/sw1 are read
  const uint8_t* pk;
  const uint8_t* spk;
};

// LDS tiles are rows of 64 bf16 (128 bytes = 8 chunks of 16 bytes).  A
// ds_read_b128 is served 16 lanes at a time over a 256-byte bank window, and a
// fragment read touches one chunk of 16 consecutive rows: XOR-ing the chunk
// index with (row >> 1) & 7 puts the 8 even rows (and the 8 odd rows) on 8
// different chunks, so the 16 lanes hit 16 distinct bank groups.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 64 + ((chunk ^ ((row >> 1) & 7)) << 3);
}

// Hardware deals workgroups round-robin over the 8 XCDs (block b -> XCD b%8),
// and each XCD has its own L2.
// The grid of the grouped GEMMs is sized for the largest possible number of
// route tiles; only the first n_tiles exist.  xcd_valid_remap deals the
// existing (route tile, weight tile) pairs, nvalid of them, evenly over the
// XCDs (XCD x takes logical tiles [x*q, x*q + q)) and returns -1 for the
// surplus workgroups, which exit.  Sizing the split by the grid instead would
// leave whole XCDs with nothing but empty tiles.
__device__ __forceinline__ int xcd_valid_remap(int b, int nvalid) {
  const int x = b & 7, i = b >> 3;
  const int q = (nvalid + 7) >> 3;
  const int L = x * q + i;
  return (i < q && L < nvalid) ? L : -1;
}

// Grouped order over (route tile, weight tile): groups of kGroupT route tiles
// x all weight tiles, route tiles fastest.  With the XCD remap, the ~64
// workgroups resident on one XCD cover about kGroupT route tiles x 8 weight
// tiles, so each weight slice is fetched into that XCD's L2 once for up to
// kGroupT route tiles of the same expert, and each gathered route tile once
// for 8 weight slices.
constexpr int kGroupT = 8;
__device__ __forceinline__ void grouped_tile(int L, int ntt, int nnt, int& tt, int& nt) {
  const int gsz = kGroupT * nnt;
  const int grp = L / gsz, r = L - grp * gsz;
  const int t0 = grp * kGroupT;
  const int gt = min(kGroupT, ntt - t0);  // last group may be narrower
  tt = t0 + r % gt;
  nt = r / gt;
}

template <int MODE, int ACT>
__global__ __launch_bounds__(256) void k_gemm(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kTileW * kTileK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kTileT * kTileK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  // ---- tile -> (group, rows, weights) --------------------------------------
  int g, m0, count, base;
  int nt_override = blockIdx.y;
  bool shared;
  if constexpr (MODE == GM_ROUTER) {
    g = 0; shared = false; m0 = blockIdx.x * kTileT; count = p.T; base = 0;
    if (m0 >= count) return;
  } else {
    // grid is (max route tiles, weight tiles); see xcd_valid_remap
    const int nnt = gridDim.y;
    const int ntiles = *p.n_tiles;
    const int L = xcd_valid_remap(blockIdx.y * gridDim.x + blockIdx.x, ntiles * nnt);
    if (L < 0) return;
    int ti, ntile;
    grouped_tile(L, ntiles, nnt, ti, ntile);
    nt_override = ntile;
    g = p.tile_group[ti];
    m0 = p.tile_m0[ti];
    shared = (g == p.E);
    count = shared ? p.T : p.counts[g];
    base = shared ? 0 : p.offsets[g];
  }
  int K, Nw;  // reduction length, number of weight rows of this group
  if constexpr (MODE == GM_GATEUP) { K = p.H; Nw = shared ? p.Is : p.I; }
  else if constexpr (MODE == GM_DOWN) { K = shared ? p.Is : p.I; Nw = p.H; }
  else { K = p.H; Nw = p.ncols; }
  const int nstep = (MODE == GM_GATEUP) ? kTileW / 2 : kTileW;
  const int n0 = nt_override * nstep;
  if (n0 >= Nw) return;

  // ---- per-thread global load assignments (4 chunks of A, 4 of B) ----------
  const uint16_t* a_src[4];
  const uint16_t* b_src[4];
  int a_lds[4], b_lds[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + 256 * i;
    const int row = q >> 3, ck = q & 7;
    a_lds[i] = swz(row, ck);
    b_lds[i] = swz(row, ck);
    // weight row; rows past the end are clamped to the last valid row (their
    // results are never stored), so the loads need no branch
    const uint16_t* wp;
    if constexpr (MODE == GM_GATEUP) {
      const int f = min(n0 + (row & 63), Nw - 1);
      const uint16_t* m = (row < 64) ? (shared ? p.sw0 : p.w0) : (shared ? p.sw1 : p.w1);
      wp = m + ((shared ? 0 : (size_t)g * Nw) + f) * (size_t)K;
    } else if constexpr (MODE == GM_DOWN) {
      const int n = min(n0 + row, Nw - 1);
      wp = (shared ? p.sw0 : p.w0) + ((shared ? 0 : (size_t)g * Nw) + n) * (size_t)K;
    } else {
      const int e = min(n0 + row, p.ncols - 1);
      wp = (e < p.E) ? p.w0 + (size_t)e * K : p.sw0;
    }
    a_src[i] = wp + ck * 8;
    // route row, clamped the same way
    const int m = min(m0 + row, count - 1);
    const uint16_t* ap;
    if constexpr (MODE == GM_DOWN) {
      ap = shared ? p.sact + (size_t)m * K : p.act + (size_t)(base + m) * K;
    } else if constexpr (MODE == GM_GATEUP) {
      const int t = shared ? m : p.row_token[base + m];
      ap = p.act + (size_t)t * K;
    } else {
      ap = p.act + (size_t)m * K;
    }
    b_src[i] = ap + ck * 8;
  }

  u32x4 ra[4], rb[4];
  auto gload = [&](int kt) {
    const int ko = kt * kTileK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = ld16(a_src[i] + ko);
      rb[i] = ld16(b_src[i] + ko);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(&sA[buf][a_lds[i]]) = ra[i];
      *reinterpret_cast<u32x4*>(&sB[buf][b_lds[i]]) = rb[i];
    }
  };

  // ---- wave sub-tile: 2 weight blocks x 2 route blocks of 32x32 ------------
  // GATEUP: weight block 0 = gate rows [32ww, +32), block 1 = the up rows of
  // the same features (tile rows 64 + 32ww ...).  Otherwise rows [64ww, +64).
  const int ww = wave & 1, wt = wave >> 1;
  int arow[2], brow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if constexpr (MODE == GM_GATEUP) arow[i] = 64 * i + 32 * ww;
    else arow[i] = 64 * ww + 32 * i;
    brow[i] = 64 * wt + 32 * i;
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = K / kTileK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int fr = lane & 31, fk = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int s = 0; s < 4; ++s) {  // 4 k-steps of 16
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = *reinterpret_cast<const bf16x8*>(&sA[buf][swz(arow[i] + fr, 2 * s + fk)]);
        bfr[i] = *reinterpret_cast<const bf16x8*>(&sB[buf][swz(brow[i] + fr, 2 * s + fk)]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue -------------------------------------------------------------
  // acc[i][j][4q + v]: weight row arow[i] + 8q + 4*(lane>>5) + v,
  //                    route brow[j] + (lane & 31)
  const int rsub = 4 * (lane >> 5);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = m0 + brow[j] + (lane & 31);
    if (m >= count) continue;
    if constexpr (MODE == GM_GATEUP) {
      uint16_t* outp = shared ? reinterpret_cast<uint16_t*>(p.sout) + (size_t)m * Nw
                              : reinterpret_cast<uint16_t*>(p.out) + (size_t)(base + m) * Nw;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f = n0 + arow[0] + 8 * q + rsub;   // gate rows: tile rows < 64
        if (f < Nw) {
          float hv[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {  // the shared expert is always SwiGLU
            const float gv = acc[0][j][4 * q + v], uv = acc[1][j][4 * q + v];
            hv[v] = (shared ? silu_f(gv) : act_f<ACT>(gv)) * uv;
          }
          u32x2 pk;
          pk[0] = pack_bf16x2(hv[0], hv[1]);
          pk[1] = pack_bf16x2(hv[2], hv[3]);
          *reinterpret_cast<u32x2*>(outp + f) = pk;
        }
      }
    } else if constexpr (MODE == GM_DOWN) {
      uint16_t* outp = shared ? reinterpret_cast<uint16_t*>(p.sout) + (size_t)m * Nw
                              : reinterpret_cast<uint16_t*>(p.out) + (size_t)(base + m) * Nw;
#pragma unroll
      for (int i = 0; i < 2; ++i)
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
    } else {
      float* outp = reinterpret_cast<float*>(p.out) + (size_t)m * p.ncols;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int e = n0 + arow[i] + 8 * q + rsub + v;
            if (e < p.ncols) outp[e] = acc[i][j][4 * q + v] + ((e < p.E && p.bias) ? p.bias[e] : 0.f);
          }
    }
  }
}

}  // namespace moe
