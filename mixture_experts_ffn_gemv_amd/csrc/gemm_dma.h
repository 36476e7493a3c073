// bf16 MFMA grouped GEMM for experts that average many routes (prefill with
// at least kDmaMinAvgRoutes routes per expert on average): 256 weight rows x
// 256 routes per workgroup, K in steps of 64.
//
// Operands reach LDS by direct global->LDS loads (global_load_lds_dwordx4):
// no staging registers and no ds_write.  The loads are issued from inline
// assembly and their completion waits are written out: the compiler's own
// wait insertion cannot tell the ring's stages apart and drains every load
// in flight at the top of the loop.  K-steps of 64 make every load cover
// whole 128-byte lines (half as many outstanding requests per byte as steps
// of 32, whose extra ring depth measured no faster).  The route operand has
// two 32 KB LDS slots; the weight operand two or three (RA): three when its
// bytes stream from HBM once per launch (experts average fewer routes than a
// tile holds), so that two of its K-steps are in flight while one is
// multiplied.  Weight loads carry the streaming (nt) cache policy, route
// loads the default one, so that L2 keeps the gathered token rows.
//
// Each load instruction of a wave fills 1 KB of LDS, lane i writing bytes
// 16i..16i+15 of it.  A swizzled layout (16-byte chunk c of row r at slot
// c ^ ((r >> 1) & 7) for 128-byte rows) is obtained by the choice of source:
// lane i of 1-KB block b loads row b*8 + i/8, chunk (i & 7) ^ ((row >> 1) & 7).
//
// Weights may instead come packed (k_pack below): each (expert, weight tile,
// K-step) block is the 32 KB LDS image of that stage's weight operand, so a
// stage's weight loads read one contiguous 32 KB run instead of 256 rows of
// 128 bytes (a load-only stream of that pattern runs about 1.4x faster; in
// this kernel, whose time the load pipeline's latency sets, the gain is a
// few percent at most).
//
// kDmaWaves waves in a 2 (weight rows) x kDmaWaves/2 (routes) grid, each owning
// 128 weight rows x 512/kDmaWaves routes of f32 accumulators (tiles of
// v_mfma_f32_32x32x16_bf16).  Byte offsets of
// rows are 32-bit (the host checks that every operand fits).
#pragma once

#include <type_traits>

#include "common.h"
#include "gemm.h"
#include "gemm_big.h"

namespace moe {

constexpr int kDmaBT = 256;                    // routes per tile
constexpr int kDmaWaves = 8;                   // waves per workgroup (2 per SIMD)
constexpr int kDmaThreads = 64 * kDmaWaves;
constexpr int kDmaBK = 64;                     // K per stage: full 128-byte rows
constexpr int kDmaSlotsB = 2;                  // LDS slots of the route operand (32 KB each)
constexpr int kDmaGroupT = 8;                  // route tiles per tile-order group
constexpr int kDmaMinAvgRoutes = 96;           // mean routes per expert to take this kernel
constexpr int kPackRows = 256;                   // weight rows per packed block
constexpr int kPackBlock = kPackRows * kDmaBK * 2;  // bytes per packed block (32 KB)

// One 1-KB direct load per wave: lane i reads 16 bytes at sbase + voff and
// writes them to LDS byte address lds + 16 i.  M0, which carries the LDS
// address, is saved and restored around it (the compiler reserves M0).  NT:
// a streaming (non-temporal) load, for bytes read once, so that they do not
// push reused lines out of L2.
template <bool NT = false>
__device__ __forceinline__ void lds_dma16(uint32_t voff, const void* sbase, uint32_t lds) {
  uint32_t saved;
  if constexpr (NT) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lds)
        : "memory");
  } else {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lds)
        : "memory");
  }
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* q) {
  const uint64_t v = reinterpret_cast<uint64_t>(q);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

// 16-byte slot of chunk c in LDS row `row` (rows of CH chunks): XOR-ing with
// row bits spreads the 16 lanes a ds_read_b128 serves per cycle (one chunk
// of 16 consecutive rows) over 16 distinct bank groups.
template <int CH>
__device__ __forceinline__ int dma_slot(int row, int c) {
  if constexpr (CH == 4) return c ^ ((row >> 2) & 3);
  else return c ^ ((row >> 1) & 7);
}

// Logical workgroup L -> (route tile, weight tile): groups of kDmaGroupT
// route tiles x all weight tiles, route tiles varying fastest, so the
// workgroups resident on one XCD at a time share weight tiles (and route
// tiles) in its L2.
__device__ __forceinline__ void dma_tile_order(int L, int ntt, int nnt, int& tt, int& nt) {
  const int gsz = kDmaGroupT * nnt;
  const int grp = L / gsz, r = L - grp * gsz;
  const int t0 = grp * kDmaGroupT;
  const int gt = min(kDmaGroupT, ntt - t0);
  tt = t0 + r % gt;
  nt = r / gt;
}

// BKD: K per stage (32 or 64); RA: LDS slots of the weight operand (2 or 3).
template <int MODE, int ACT, int BKD, int RA>
__global__ __launch_bounds__(kDmaThreads, 1) void k_gemm_dma(GemmParams p) {
  constexpr int NW = kDmaWaves;
  constexpr int CH = BKD / 8;              // 16-byte chunks per LDS row
  constexpr int RPB = 64 / CH;             // rows per 1-KB load block
  constexpr int BLK = 256 / RPB;           // blocks per operand per stage
  constexpr int NH = BLK / NW;             // blocks per operand per wave
  constexpr int S = BKD / 16;              // k-steps of 16 per stage
  constexpr int WTR = kDmaBT / (NW / 2);   // routes per wave
  constexpr int NJ = WTR / 32;             // 32-wide route blocks per wave
  constexpr int REGION = 256 * BKD * 2;    // bytes of A (and of B) per stage
  static_assert(S % 2 == 0 && BLK % NW == 0 && 3 * NH <= 63, "tile shape");
  static_assert((RA == 2 || RA == 3) && kDmaSlotsB == 2, "the issue order below");
  // slots 0..RA-1: weight operand; RA, RA+1: route operand
  __shared__ __attribute__((aligned(1024))) uint8_t smem[(RA + kDmaSlotsB) * REGION];
  const uint32_t lds0 =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nnt = gridDim.y;
  const int ntiles = *p.n_tiles;
  const int L = xcd_valid_remap(blockIdx.y * gridDim.x + blockIdx.x, ntiles * nnt);
  if (L < 0) return;
  int ti, nt;
  dma_tile_order(L, ntiles, nnt, ti, nt);
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

  // ---- load sources: wave w fills blocks w, w+NW, ... of A and of B -----------
  const bool packed = p.pk != nullptr;  // the host passes both or neither
  const int nk = K / BKD;
  const uint8_t* a_base[NH];
  uint32_t a_off[NH], b_off[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int blk = wave + NW * h;
    const int row = blk * RPB + lane / CH;
    const int c = dma_slot<CH>(row, lane % CH);  // the XOR is its own inverse
    if (packed) {
      static_assert(BKD == kDmaBK, "packed blocks hold K-steps of kDmaBK");
      // tiles of this expert: 128 features (gate/up) or 256 outputs (down)
      const int nwt = (MODE == GM_GATEUP) ? (Nw + 127) / 128 : (Nw + 255) / 256;
      a_base[h] = uniform_ptr(shared ? p.spk : p.pk + (size_t)g * nwt * nk * kPackBlock);
      a_off[h] = (uint32_t)(nt * nk) * (uint32_t)kPackBlock + (uint32_t)blk * 1024u +
                 (uint32_t)lane * 16u;
    } else {
      const uint16_t* m;
      int wr;
      if constexpr (MODE == GM_GATEUP) {  // first half of the blocks: gate rows, then up
        m = blk < BLK / 2 ? (shared ? p.sw0 : p.w0) : (shared ? p.sw1 : p.w1);
        wr = min(n0 + (row & 127), Nw - 1);  // clamped rows are never stored
      } else {
        m = shared ? p.sw0 : p.w0;
        wr = min(n0 + row, Nw - 1);
      }
      a_base[h] = reinterpret_cast<const uint8_t*>(
          uniform_ptr(m + (shared ? (size_t)0 : (size_t)g * Nw * K)));
      a_off[h] = (uint32_t)wr * (uint32_t)K * 2u + (uint32_t)c * 16u;
    }
    const int rm = min(m0 + row, count - 1);  // clamped routes are never stored
    uint32_t br;
    if constexpr (MODE == GM_DOWN) br = (uint32_t)(shared ? rm : base + rm);
    else br = (uint32_t)(shared ? rm : p.row_token[base + rm]);
    b_off[h] = br * (uint32_t)K * 2u + (uint32_t)c * 16u;
  }
  const uint8_t* b_base = reinterpret_cast<const uint8_t*>(
      uniform_ptr((MODE == GM_DOWN && shared) ? p.sact : p.act));

  const size_t a_step = packed ? (size_t)kPackBlock : (size_t)BKD * 2;  // bytes per K-step
  auto issue_a = [&](int kt, int slot) {
    const uint32_t sb = lds0 + (uint32_t)(slot * REGION);
    const size_t koa = (size_t)kt * a_step;
    // Weight loads are streaming: they are read once a launch (RA = 3) or
    // shared only by the workgroups that run a weight tile together, while
    // the gathered route rows are re-read by every weight tile of their
    // group.  Measured: 4k tokens 525 -> 492 us a step, 16k 12.6 -> 12.45 ms
    // (streaming route loads as well: 572 us and 15.8 ms).
#pragma unroll
    for (int h = 0; h < NH; ++h)
      lds_dma16<true>(a_off[h], a_base[h] + koa, sb + (wave + NW * h) * 1024);
  };
  auto issue_b = [&](int kt, int slot) {
    const uint32_t sb = lds0 + (uint32_t)((RA + slot) * REGION);
    const size_t ko = (size_t)kt * BKD * 2;
#pragma unroll
    for (int h = 0; h < NH; ++h) lds_dma16(b_off[h], b_base + ko, sb + (wave + NW * h) * 1024);
  };

  // ---- wave sub-tile: 128 weight rows x WTR routes ----------------------------
  const int ww = wave & 1, wt = wave >> 1;
  int arow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (MODE == GM_GATEUP)  // blocks 0,1 gate, 2,3 up of the same features
      arow[i] = (i >> 1) * 128 + 64 * ww + 32 * (i & 1);
    else
      arow[i] = 128 * ww + 32 * i;
  }
  const int brow0 = WTR * wt;
  // 32-route blocks of this wave that hold routes of the tile: a tile with
  // fewer than kDmaBT routes (an expert's last tile) skips the fragment reads
  // and multiplies of the empty blocks.  Waves whose blocks are all empty
  // still load their share of the operands and join every barrier.
  const int tile_rows = min(kDmaBT, count - m0);
  const int nja = min(NJ, max(0, (tile_rows - brow0 + 31) >> 5));
  f32x16 acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  const int fr = lane & 31, fk = lane >> 5;

  // ---- pipeline ---------------------------------------------------------------
  // The route operand (gathered rows) runs one K-step ahead; the weight
  // operand RA-1 steps: with RA = 3 (3 + 2 slots of 32 KB, the whole 160 KB
  // of LDS) for weights streamed from HBM once, whose latency one step of
  // multiplies does not cover.  Issue order: A0 B0 A1 B1 [A2], then after the
  // barrier of iteration kt: B(kt+2) into kt's route slot, A(kt+RA) into kt's
  // weight slot.  So when iteration kt waits for step kt+1, the loads issued
  // after B(kt+1) are A(kt+2)'s if RA = 3 and none if RA = 2: wait until
  // (RA-2)*NH (per wave) remain.
  // Iteration kt: for each k-step of step kt, read the next k-step's
  // fragments while multiplying the current ones; before the last k-step,
  // wait for step kt+1 and synchronise (after which nobody reads kt's slots
  // any more), refill them, and read the first fragments of step kt+1 while
  // the last k-step of kt is multiplied.  Fragment reads always overlap
  // multiplies, and the barrier sits between two runs of multiplies.  The
  // last step is peeled off: a branch inside the loop body would make the
  // wait-count pass merge two paths and wait for the prefetched reads.  NA
  // (the wave's non-empty route blocks) is a template constant so that no
  // branch sits between the reads and the multiplies.
  auto pipeline = [&](auto na_c) {
    constexpr int NA = decltype(na_c)::value;
    // Fragments of k-step s (16 deep) from weight slot sa and route slot sb.
    auto frag = [&](int sa, int sb, int s, bf16x8 (&af)[4], bf16x8 (&bfr)[NJ]) {
      if constexpr (NA > 0) {
        const uint16_t* sA = reinterpret_cast<const uint16_t*>(smem + sa * REGION);
        const uint16_t* sB = reinterpret_cast<const uint16_t*>(smem + (RA + sb) * REGION);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = arow[i] + fr;
          af[i] = *reinterpret_cast<const bf16x8*>(
              &sA[r * BKD + (dma_slot<CH>(r, 2 * s + fk) << 3)]);
        }
#pragma unroll
        for (int j = 0; j < NA; ++j) {
          const int r = brow0 + 32 * j + fr;
          bfr[j] = *reinterpret_cast<const bf16x8*>(
              &sB[r * BKD + (dma_slot<CH>(r, 2 * s + fk) << 3)]);
        }
      }
    };
    auto mma = [&](const bf16x8 (&af)[4], const bf16x8 (&bfr)[NJ]) {
#pragma unroll
      for (int j = 0; j < NA; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    };
    issue_a(0, 0);
    issue_b(0, 0);
    if (nk > 1) {
      issue_a(1, 1);
      issue_b(1, 1);
    }
    if (RA == 3 && nk > 2) issue_a(2, 2);
    if (RA == 3 && nk > 2) wait_vmem<3 * NH>();  // A1 B1 A2 may stay in flight
    else if (nk > 1) wait_vmem<2 * NH>();
    else wait_vmem<0>();
    __syncthreads();
    bf16x8 fa[2][4], fb[2][NJ];
    frag(0, 0, 0, fa[0], fb[0]);
    int sa = 0;  // weight slot of step kt
    for (int kt = 0; kt + 1 < nk; ++kt) {
      const int sb = kt & 1;
#pragma unroll
      for (int s = 1; s < S; ++s) {
        frag(sa, sb, s, fa[s & 1], fb[s & 1]);
        mma(fa[(s - 1) & 1], fb[(s - 1) & 1]);
      }
      if (RA == 3 && kt + 2 < nk) wait_vmem<NH>();  // A(kt+2) may stay in flight
      else wait_vmem<0>();
      __syncthreads();
      if (kt + 2 < nk) issue_b(kt + 2, sb);
      if (kt + RA < nk) issue_a(kt + RA, sa);
      sa = sa == RA - 1 ? 0 : sa + 1;
      frag(sa, sb ^ 1, 0, fa[0], fb[0]);
      mma(fa[1], fb[1]);
    }
    {
      const int sb = (nk - 1) & 1;
#pragma unroll
      for (int s = 1; s < S; ++s) {
        frag(sa, sb, s, fa[s & 1], fb[s & 1]);
        mma(fa[(s - 1) & 1], fb[(s - 1) & 1]);
      }
      mma(fa[1], fb[1]);
    }
  };
  static_assert(NJ == 2, "one pipeline instance per count of non-empty blocks");
  if (nja == 2) pipeline(std::integral_constant<int, 2>{});
  else if (nja == 1) pipeline(std::integral_constant<int, 1>{});
  else pipeline(std::integral_constant<int, 0>{});

  // ---- epilogue: acc[i][j][4q + v] = weight row arow[i] + 8q + 4*(lane>>5) + v,
  //      route brow0 + 32 j + (lane & 31) -----------------------------------------
  const int rsub = 4 * (lane >> 5);
  if constexpr (MODE == GM_GATEUP) {
    // h = act(gate) * up straight from the accumulators: 8 bytes per route row
    // and store (staging through LDS, as below, measured slower for h)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int m = m0 + brow0 + 32 * j + (lane & 31);
      if (m >= count) continue;
      uint16_t* outp = shared ? reinterpret_cast<uint16_t*>(p.sout) + (size_t)m * Nw
                              : reinterpret_cast<uint16_t*>(p.out) + (size_t)(base + m) * Nw;
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
    }
  } else {
    // y passes through LDS (route-major rows of 128 outputs, padded to 272
    // bytes so that the 32 routes one write covers fall on distinct banks)
    // and leaves as 16-byte stores, 16 lanes covering 256 contiguous bytes of
    // a row, instead of 8 bytes in each of 32 rows per store instruction.
    constexpr int ROWB = 128 * 2 + 16;
    static_assert(256 * ROWB <= (RA + kDmaSlotsB) * REGION, "staging fits the operand slots");
    auto stage8 = [&](int row, int col, float a, float b, float c, float d) {
      u32x2 pk;
      pk[0] = pack_bf16x2(a, b);
      pk[1] = pack_bf16x2(c, d);
      *reinterpret_cast<u32x2*>(smem + row * ROWB + col * 2) = pk;
    };
    // staged rows (routes m0 ..) x 128 values -> output columns n0 + colbase + 0..127
    auto flush = [&](int colbase) {
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 256 * 16 / kDmaThreads; ++u) {
        const int ch = tid + kDmaThreads * u;
        const int row = ch >> 4, cc = ch & 15;
        const int m = m0 + row;
        const int n = n0 + colbase + 8 * cc;
        if (m < count && n < Nw) {
          uint16_t* outp = shared ? reinterpret_cast<uint16_t*>(p.sout) + (size_t)m * Nw
                                  : reinterpret_cast<uint16_t*>(p.out) + (size_t)(base + m) * Nw;
          *reinterpret_cast<u32x4*>(outp + n) =
              *reinterpret_cast<const u32x4*>(smem + row * ROWB + cc * 16);
        }
      }
    };
    __syncthreads();  // every wave is done with the operand slots
    // two passes of 128 outputs: pass h stages the waves with ww == h
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h == 1) __syncthreads();  // pass 0's rows have been read out
      if (ww == h) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              stage8(brow0 + 32 * j + (lane & 31), 32 * i + 8 * q + rsub, acc[i][j][4 * q],
                     acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
      }
      flush(128 * h);
    }
  }
}

// Weight packing for the kernel above.  Block (t, s) of an expert holds
// weight tile t at K-step s as 256 rows of 128 bytes: for gate/up, rows
// 0-127 are gate features 128t + r and rows 128-255 the up features
// 128t + r - 128; for down, row r is output 256t + r.  Row r's 16-byte chunk
// c (K elements 64s + 8c .. 64s + 8c + 7) sits in slot dma_slot<8>(r, c) of
// the row, so the block is byte for byte what the kernel's stage holds.  Rows
// past the matrix are zero.  Blocks of an expert are ordered t-major
// (t * K/64 + s) and experts follow one another.  One workgroup per block:
// blockIdx.x = t * K/64 + s, blockIdx.y = expert.
template <int MODE>
__global__ __launch_bounds__(256) void k_pack(const uint16_t* __restrict__ w0,
                                              const uint16_t* __restrict__ w1,
                                              uint8_t* __restrict__ dst, int Nw, int K, int nwt) {
  const int ks = K / kDmaBK;
  const int t = blockIdx.x / ks, s = blockIdx.x - t * ks;
  const size_t src0 = (size_t)blockIdx.y * Nw * K + (size_t)s * kDmaBK;
  uint8_t* db = dst + ((size_t)blockIdx.y * nwt * ks + blockIdx.x) * kPackBlock;
  constexpr int CH = kDmaBK / 8;  // 16-byte chunks per row
#pragma unroll
  for (int i = 0; i < kPackBlock / 16 / 256; ++i) {
    const int q = threadIdx.x + 256 * i;  // destination chunk
    const int r = q / CH;
    const int c = dma_slot<CH>(r, q % CH);  // the XOR is its own inverse
    int f;
    const uint16_t* m;
    if constexpr (MODE == GM_GATEUP) {
      f = 128 * t + (r & 127);
      m = r < 128 ? w0 : w1;
    } else {
      f = 256 * t + r;
      m = w0;
    }
    u32x4 v = {0u, 0u, 0u, 0u};
    if (f < Nw) v = *reinterpret_cast<const u32x4*>(m + src0 + (size_t)f * K + 8 * c);
    *reinterpret_cast<u32x4*>(db + (size_t)q * 16) = v;
  }
}

}  // namespace moe
