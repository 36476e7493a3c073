// Shared pieces of the bf16 MFMA GEMMs (prefill), and the prefill router.
//
// The expert GEMMs (gemm_big.h, gemm_dma.h) compute tiles of C^T = W . X^T
// over K with v_mfma_f32_32x32x16_bf16 and f32 accumulation (on gfx950 the
// 32x32x16 form sustains about 90% of the bf16 peak with one wave per SIMD,
// the 16x16x32 form about half of it).  Weights are the MFMA "A" operand,
// the gathered route activations the "B" operand, so each lane ends up
// holding runs of four consecutive output features of one route.  Their
// route tiles come from a flat list (group, first row) built after the
// expert grouping, so a skewed load only changes the number of tiles, not
// their shape.
//
// Modes: GATEUP: gate and up rows of the same features, epilogue
// h = act(gate) * up as bf16; DOWN: y = Wd h, bf16.
#pragma once

#include "common.h"

namespace moe {

constexpr int kTileW = 128;   // router: logit columns per tile
constexpr int kTileT = 128;   // router: tokens per tile
constexpr int kTileK = 64;    // router: K per stage

enum GemmMode : int { GM_GATEUP = 0, GM_DOWN = 1 };

struct GemmParams {
  // weights (bf16 bits)
  const uint16_t* w0;    // GATEUP: gate [E,I,H]; DOWN: down [E,H,I]
  const uint16_t* w1;    // GATEUP: up [E,I,H]
  const uint16_t* sw0;   // shared gate [Is,H] / shared down [H,Is]
  const uint16_t* sw1;   // shared up [Is,H]
  // activations (bf16 bits)
  const uint16_t* act;   // GATEUP: x [T,H]; DOWN: h [R,I]
  const uint16_t* sact;  // DOWN: hs [T,Is]
  // outputs
  void* out;             // GATEUP: h [R,I] bf16; DOWN: y [R,H] bf16
  void* sout;            // GATEUP: hs [T,Is]; DOWN: ys [T,H]
  // grouping
  const int32_t* counts;     // [G]
  const int32_t* offsets;    // [E+1]
  const int32_t* row_token;  // [R]
  const int32_t* tile_group; // [max_tiles]
  const int32_t* tile_m0;
  const int32_t* n_tiles;
  int E, T, H, I, Is;
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

// Prefill router: logits[t, c] = x[t, :] . Wr[c, :] (+ bias[c] for c < E)
// for the first nw columns of rows ncols floats apart; column E (with a
// shared expert) would be the shared gate vector, but the top-k kernel takes
// that one dot product per token itself, so nw = E and no column tile is
// spent on it.  K is split into
// nsplit equal ranges (grid z): range z writes its partial dot products to
// logits + z * split_stride (the bias goes with range 0), and the top-k
// kernel adds the ranges in order, so more workgroups share a short K loop
// and the sum stays deterministic.  Each workgroup
// computes a 128-column x 128-token tile over its K range in steps of 64 with
// v_mfma_f32_32x32x16_bf16; each wave a 64 x 64 sub-tile (2 x 2 blocks of
// 32x32).  Operand tiles are staged through LDS (double-buffered, the
// 16-byte chunks of each 128-byte row XOR-swizzled, see swz) from registers
// loaded one K-step ahead; the finished logits leave through LDS as whole
// rows.
struct RouterParams {
  const uint16_t* x;       // [T, H]
  const uint16_t* wr;      // [E, H]
  const uint16_t* wsg;     // [H] shared gate vector (column E), or null
  const float* bias;       // [E] or null
  float* logits;           // [nsplit, T, ncols] partial logits
  int T, H, E, ncols;
  int nw;                  // logit columns computed (the first nw of each row)
  int nsplit;              // K ranges (H / 64 a multiple of it)
  size_t split_stride;     // floats between the ranges' partial logits
};

constexpr int kRouterEpStride = kTileW + 4;  // floats per staged logit row
__global__ __launch_bounds__(256) void k_router_mfma(RouterParams p) {
  // the operand tiles, then (after the K loop) half a tile of logits
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (kTileW + kTileT) * kTileK * 2];
  static_assert((kTileT / 2) * kRouterEpStride * 4 <= sizeof(smem), "staged logits fit");
  auto sA = reinterpret_cast<uint16_t (*)[kTileW * kTileK]>(smem);
  auto sB = reinterpret_cast<uint16_t (*)[kTileT * kTileK]>(smem + 2 * kTileW * kTileK * 2);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.x * kTileT, n0 = blockIdx.y * kTileW;
  if (m0 >= p.T) return;
  const int K = p.H;
  const int nk = K / kTileK / p.nsplit;       // K steps of this range
  const int k0 = blockIdx.z * nk * kTileK;   // its first element

  // ---- per-thread global load assignments (4 chunks of A, 4 of B) ----------
  // Rows past the end are clamped to the last valid one (never stored), so
  // the loads need no branch.
  const uint16_t* a_src[4];
  const uint16_t* b_src[4];
  int lds_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + 256 * i;
    const int row = q >> 3, ck = q & 7;
    lds_off[i] = swz(row, ck);
    const int e = min(n0 + row, p.nw - 1);
    a_src[i] = ((e < p.E) ? p.wr + (size_t)e * K : p.wsg) + k0 + ck * 8;
    const int m = min(m0 + row, p.T - 1);
    b_src[i] = p.x + (size_t)m * K + k0 + ck * 8;
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
      *reinterpret_cast<u32x4*>(&sA[buf][lds_off[i]]) = ra[i];
      *reinterpret_cast<u32x4*>(&sB[buf][lds_off[i]]) = rb[i];
    }
  };

  // ---- wave sub-tile: columns [64ww, +64) x tokens [64wt, +64) ---------------
  const int ww = wave & 1, wt = wave >> 1;
  int arow[2], brow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    arow[i] = 64 * ww + 32 * i;
    brow[i] = 64 * wt + 32 * i;
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

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

  // ---- epilogue: acc[i][j][4q + v] = column arow[i] + 8q + 4*(lane>>5) + v,
  //      token brow[j] + (lane & 31).  Each half of the token rows goes
  //      through LDS (waves 2wt, 2wt+1 hold half wt) and out as whole rows,
  //      consecutive lanes on consecutive columns.
  const int rsub = 4 * (lane >> 5);
  float* ep = reinterpret_cast<float*>(smem);
  const bool add_bias = blockIdx.z == 0 && p.bias;
  float* outz = p.logits + blockIdx.z * p.split_stride;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (wt == h) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = 32 * j + (lane & 31), c = arow[i] + 8 * q + rsub;
            *reinterpret_cast<f32x4*>(&ep[r * kRouterEpStride + c]) =
                f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          }
    }
    __syncthreads();
    for (int idx = tid; idx < (kTileT / 2) * kTileW; idx += 256) {
      const int r = idx / kTileW, c = idx - r * kTileW;
      const int m = m0 + (kTileT / 2) * h + r, e = n0 + c;
      if (m < p.T && e < p.nw)
        outz[(size_t)m * p.ncols + e] = ep[r * kRouterEpStride + c] + ((e < p.E && add_bias) ? p.bias[e] : 0.f);
    }
    __syncthreads();
  }
}

}  // namespace moe
