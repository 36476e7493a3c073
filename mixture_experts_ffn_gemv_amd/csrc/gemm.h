// bf16 MFMA grouped GEMM for many tokens per expert (prefill).
//
// Each workgroup computes a 128 (weight rows) x 128 (routes) tile of
// C^T = W . X^T over K in steps of 64, with v_mfma_f32_16x16x32_bf16 and
// f32 accumulation.  Weights are the MFMA "A" operand, the gathered route
// activations the "B" operand, so each lane ends up holding four
// consecutive output features of one route: epilogue stores are 8-byte
// contiguous runs of a route's row.
//
// The route tiles come from a flat list (group, first row) built after the
// expert grouping, so a skewed load only changes the number of tiles, not
// their shape.  A and B tiles are staged through LDS (double-buffered, the
// 16-byte chunks of each 128-byte row XOR-swizzled by row & 7 so the
// ds_read_b128 fragment loads are bank-conflict free).
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
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * 64 + ((chunk ^ (row & 7)) << 3); }

template <int MODE, int ACT>
__global__ __launch_bounds__(256) void k_gemm(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kTileW * kTileK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kTileT * kTileK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  // ---- tile -> (group, rows, weights) --------------------------------------
  int g, m0, count, base;
  bool shared;
  if constexpr (MODE == GM_ROUTER) {
    g = 0; shared = false; m0 = blockIdx.x * kTileT; count = p.T; base = 0;
    if (m0 >= count) return;
  } else {
    const int ti = blockIdx.x;
    if (ti >= *p.n_tiles) return;
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
  const int n0 = blockIdx.y * nstep;
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
    // weight row
    const uint16_t* wp = nullptr;
    if constexpr (MODE == GM_GATEUP) {
      const int f = n0 + (row & 63);
      if (f < Nw) {
        const uint16_t* m = (row < 64) ? (shared ? p.sw0 : p.w0) : (shared ? p.sw1 : p.w1);
        wp = m + ((shared ? 0 : (size_t)g * Nw) + f) * (size_t)K;
      }
    } else if constexpr (MODE == GM_DOWN) {
      const int n = n0 + row;
      if (n < Nw) wp = (shared ? p.sw0 : p.w0) + ((shared ? 0 : (size_t)g * Nw) + n) * (size_t)K;
    } else {
      const int e = n0 + row;
      if (e < p.E) wp = p.w0 + (size_t)e * K;
      else if (e < p.ncols) wp = p.sw0;
    }
    a_src[i] = wp ? wp + ck * 8 : nullptr;
    // route row
    const int m = m0 + row;
    const uint16_t* ap = nullptr;
    if (m < count) {
      if constexpr (MODE == GM_DOWN) {
        ap = shared ? p.sact + (size_t)m * K : p.act + (size_t)(base + m) * K;
      } else if constexpr (MODE == GM_GATEUP) {
        const int t = shared ? m : p.row_token[base + m];
        ap = p.act + (size_t)t * K;
      } else {
        ap = p.act + (size_t)m * K;
      }
    }
    b_src[i] = ap ? ap + ck * 8 : nullptr;
  }

  u32x4 ra[4], rb[4];
  auto gload = [&](int kt) {
    const int ko = kt * kTileK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = a_src[i] ? ld16(a_src[i] + ko) : u32x4{0, 0, 0, 0};
      rb[i] = b_src[i] ? ld16(b_src[i] + ko) : u32x4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(&sA[buf][a_lds[i]]) = ra[i];
      *reinterpret_cast<u32x4*>(&sB[buf][b_lds[i]]) = rb[i];
    }
  };

  // ---- wave sub-tile: 4 weight blocks x 4 route blocks of 16x16 ------------
  const int ww = wave & 1, wt = wave >> 1;
  int arow[4], brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (MODE == GM_GATEUP) arow[i] = (i < 2 ? 0 : 64) + 32 * ww + 16 * (i & 1);
    else arow[i] = 64 * ww + 16 * i;
    brow[i] = 64 * wt + 16 * i;
  }
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / kTileK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int fr = lane & 15, fk = lane >> 4;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra_ = arow[i] + fr;
        af[i] = *reinterpret_cast<const bf16x8*>(&sA[buf][swz(ra_, 4 * s + fk)]);
        const int rb_ = brow[i] + fr;
        bfr[i] = *reinterpret_cast<const bf16x8*>(&sB[buf][swz(rb_, 4 * s + fk)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue -------------------------------------------------------------
  // acc[i][j][v]: weight row arow[i] + 4*(lane>>4) + v, route brow[j] + (lane&15)
  const int rsub = 4 * (lane >> 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + brow[j] + (lane & 15);
    if (m >= count) continue;
    if constexpr (MODE == GM_GATEUP) {
      uint16_t* outp = shared ? reinterpret_cast<uint16_t*>(p.sout) + (size_t)m * Nw
                              : reinterpret_cast<uint16_t*>(p.out) + (size_t)(base + m) * Nw;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int f = n0 + arow[i] + rsub;   // arow[i] < 64 here: gate rows
        if (f < Nw) {
          const f32x4 gv = acc[i][j], uv = acc[i + 2][j];
          float hv[4];
#pragma unroll
          for (int v = 0; v < 4; ++v)   // the shared expert is always SwiGLU
            hv[v] = (shared ? silu_f(gv[v]) : act_f<ACT>(gv[v])) * uv[v];
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
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + arow[i] + rsub;
        if (n < Nw) {
          const f32x4 v = acc[i][j];
          u32x2 pk;
          pk[0] = pack_bf16x2(v[0], v[1]);
          pk[1] = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<u32x2*>(outp + n) = pk;
        }
      }
    } else {
      float* outp = reinterpret_cast<float*>(p.out) + (size_t)m * p.ncols;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int e = n0 + arow[i] + rsub + v;
          if (e < p.ncols) outp[e] = acc[i][j][v] + ((e < p.E && p.bias) ? p.bias[e] : 0.f);
        }
    }
  }
}

}  // namespace moe
