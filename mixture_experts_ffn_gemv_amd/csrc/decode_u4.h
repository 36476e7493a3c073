// Decode path for 4-bit affine weights (codes in groups of 32 along K, one
// f16 scale and one f16 min per group: w = code * scale + min), T <= 32.
//
// One workgroup per (touched expert, block of output rows).  The activations
// of the expert's routes (x for gate/up, h for down), up to kU4Routes per
// pass, are staged once in LDS and shared by every row of the block, in a
// group-contiguous layout: 16-byte piece q of 32-element group c of route r
// sits at float4 index (r*G + c)*9 + q (G groups per row, one float4 of
// padding per group), so a lane reads its group's 8 pieces at immediate
// offsets from one address, and the 144-byte stride between the lanes'
// groups keeps every 8 or 16 lanes of a ds_read_b128 on distinct banks.
// Next to them, the sum of each group's 32 activations.
//
// A group of one row is dequantised once and reused for every route:
//   sum_i (c_i*s + m) x_i = s * sum_i c_i x_i + m * sum_i x_i,
// the nibbles go to floats by byte-wise conversion, and the second term
// takes the staged group sum.  Per weight element that is about 1.25
// conversion operations plus one FMA per route.
//
// gate/up: each wave owns features f (gate row and up row of f); the epilogue
//          writes h = act(gate) * up (f32).
// down   : each wave owns output rows n; writes y[position, n] (f32, rows in
//          the expert-grouped order), summed per token with the routing
//          weights by k_combine.
#pragma once

#include "common.h"
#include "gemv.h"
#include "decode.h"

namespace moe {

constexpr int kU4Routes = 4;     // most routes staged per pass (Dec2Params::rc may be fewer)
constexpr int kU4Rows = 32;      // output rows (features) per workgroup
constexpr int kU4LdsMax = 160 * 1024 - 4096;  // LDS bytes available to the staging

// LDS bytes per staged route of row length K: activations plus group sums.
constexpr int kU4GroupF4 = 9;   // float4 slots per staged group (8 pieces + padding)
__host__ __device__ constexpr int u4_route_bytes(int K) { return (K / 32) * (kU4GroupF4 * 16 + 4); }

// Byte n of v as a float, one v_cvt_f32_ubyte{n} (written out: from the
// shifted-and-masked C expression the compiler emits a bit-field extract
// and then the byte-0 conversion, two instructions).
template <int N>
__device__ __forceinline__ float ubyte_f(uint32_t v) {
  float f;
  if constexpr (N == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(f) : "v"(v));
  else if constexpr (N == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(f) : "v"(v));
  else if constexpr (N == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(f) : "v"(v));
  else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(f) : "v"(v));
  return f;
}

// 8 nibbles of one 32-bit word -> floats, in element order (low nibble
// first): two masks, one shift and eight byte conversions.
__device__ __forceinline__ void nib8(uint32_t w, float (&f)[8]) {
  const uint32_t lo = w & 0x0F0F0F0Fu;          // elements 0, 2, 4, 6 in bytes 0..3
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // elements 1, 3, 5, 7
  f[0] = ubyte_f<0>(lo); f[1] = ubyte_f<0>(hi);
  f[2] = ubyte_f<1>(lo); f[3] = ubyte_f<1>(hi);
  f[4] = ubyte_f<2>(lo); f[5] = ubyte_f<2>(hi);
  f[6] = ubyte_f<3>(lo); f[7] = ubyte_f<3>(hi);
}

// Stage the activations of nr routes (rows[rr], f32 or bf16, length K) and
// their per-group sums.  Pieces are ordered (route, group, q) over the 256
// threads, 8 consecutive threads holding one group, so a group's sum is a
// butterfly over 8 lanes; each thread has kStageUnroll loads in flight.
constexpr int kStageUnroll = 8;
__device__ __forceinline__ void u4_stage(f32x4* __restrict__ xs, float* __restrict__ xsum, int nr,
                                         int K, int act_bf16,
                                         const void* const (&rows)[kU4Routes]) {
  const int G = K / 32;
  const int n = nr * G * 8;
  for (int base = 0; base < n; base += 256 * kStageUnroll) {
    f32x4 v[kStageUnroll];
#pragma unroll
    for (int j = 0; j < kStageUnroll; ++j) {
      const int i = min(base + 256 * j + (int)threadIdx.x, n - 1);  // clamped: loads stay unconditional
      const int q = i & 7, rc = i >> 3;
      const int rr = rc / G, c = rc - rr * G;
      const size_t off = (size_t)c * 32 + (size_t)q * 4;
      if (act_bf16) {
        const u32x2 b2 = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(rows[rr]) + off);
        v[j] = f32x4{bf16lo(b2[0]), bf16hi(b2[0]), bf16lo(b2[1]), bf16hi(b2[1])};
      } else {
        v[j] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(rows[rr]) + off);
      }
    }
#pragma unroll
    for (int j = 0; j < kStageUnroll; ++j) {
      const int i = base + 256 * j + (int)threadIdx.x;
      const bool ok = i < n;
      const int q = i & 7, rc = i >> 3;
      const int rr = rc / G, c = rc - rr * G;
      if (ok) xs[(rr * G + c) * kU4GroupF4 + q] = v[j];
      float sm = ok ? (v[j][0] + v[j][1]) + (v[j][2] + v[j][3]) : 0.f;
      sm += __shfl_xor(sm, 1, 64);
      sm += __shfl_xor(sm, 2, 64);
      sm += __shfl_xor(sm, 4, 64);
      if (ok && q == 0) xsum[rr * G + c] = sm;
    }
  }
}

// Dot products of one 32-element group of two rows (codes v0/v1, scales,
// mins) with the staged activations of nr routes:
//   acc[k][r] += sc_k * sum_i c_ki x_ri + mn_k * xsum_r.
// Each activation read from LDS serves both rows.
template <bool BATCH>
__device__ __forceinline__ void u4_group_dot2(const u32x4& v0, uint32_t sm0, const u32x4& v1,
                                              uint32_t sm1, const f32x4* __restrict__ xs,
                                              const float* __restrict__ xsum, int G, int c, int nr,
                                              float (&acc0)[kU4Routes], float (&acc1)[kU4Routes]) {
  const float sc0 = f16_to_f32((uint16_t)sm0), mn0 = f16_to_f32((uint16_t)(sm0 >> 16));
  const float sc1 = f16_to_f32((uint16_t)sm1), mn1 = f16_to_f32((uint16_t)(sm1 >> 16));
  float w0[32], w1[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float f[8], h[8];
    nib8(v0[q], f);
    nib8(v1[q], h);
#pragma unroll
    for (int j = 0; j < 8; ++j) { w0[8 * q + j] = f[j]; w1[8 * q + j] = h[j]; }
  }
#pragma unroll
  for (int r = 0; r < kU4Routes; ++r) {
    if (r < nr) {
      // BATCH: the route's 8 LDS reads are all issued before the first
      // multiply-add (read and use interleaved, each read's latency is
      // exposed), at the cost of 32 more registers; without it the reads
      // stream one by one
      const f32x4* xr = xs + ((size_t)r * G + c) * kU4GroupF4;
      const float xsr = xsum[r * G + c];
      float d0 = 0.f, d1 = 0.f;
      if constexpr (BATCH) {
        f32x4 x4[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) x4[q] = xr[q];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            d0 = fmaf(w0[4 * q + e], x4[q][e], d0);
            d1 = fmaf(w1[4 * q + e], x4[q][e], d1);
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const f32x4 x4 = xr[q];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            d0 = fmaf(w0[4 * q + e], x4[e], d0);
            d1 = fmaf(w1[4 * q + e], x4[e], d1);
          }
        }
      }
      acc0[r] = fmaf(sc0, d0, fmaf(mn0, xsr, acc0[r]));
      acc1[r] = fmaf(sc1, d1, fmaf(mn1, xsr, acc1[r]));
    }
  }
}

// One group of one row: codes (16 bytes) plus the f16 bits of its scale and
// min.  The loads are unconditional (the group index is clamped; lanes past
// the row's end skip the group): a load inside a branch, or a conversion of
// its result inside one, makes the compiler wait for it on the spot.
__device__ __forceinline__ void u4_load(const MatStack& m, size_t row, int G, int c, u32x4& v,
                                        uint32_t& sc_mn) {
  const size_t gi = row * G + min(c, G - 1);
  v = ld16_stream(m.p + gi * 16);
  sc_mn = (uint32_t)m.sc[gi] | ((uint32_t)m.mn[gi] << 16);
}

// MODE 0: gate/up (K = H, rows = I features, two matrices); 1: down (K = I,
// rows = H outputs).  LPR lanes share a row (64: the whole wave; 16: four
// rows side by side, for rows whose group count is not a multiple of 64,
// e.g. 48 groups at K = 1536 would leave a quarter of a 64-lane wave
// idle); U groups per lane cover it (LPR*U >= K/32).
template <int MODE, int ACT, int U, int LPR>
__global__ __launch_bounds__(256) void k_dec_u4(Dec2Params p) {
  constexpr int SEGS = 64 / LPR;  // rows side by side in a wave
  extern __shared__ __attribute__((aligned(16))) float u4lds[];
  const int s = blockIdx.x;
  if (s >= *p.n_active) return;
  const int R = p.T * p.k;
  const int g = ws_group(p.active[s], p.E, false);
  const int K = MODE == 0 ? p.H : p.I;
  const int N = MODE == 0 ? p.I : p.H;
  const int G = K / 32;
  const int rb = blockIdx.y * kU4Rows * SEGS;
  if (rb >= N) return;
  int count = p.counts[g], base = p.offsets[g];
  ws_span(base, count, R);
  const int rc = p.rc;  // routes per pass (<= kU4Routes), sized to the LDS
  f32x4* xs = reinterpret_cast<f32x4*>(u4lds);
  float* xsum = u4lds + (size_t)rc * G * kU4GroupF4 * 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int seg = lane / LPR, sl = lane % LPR;  // the lane's row segment, lane in it
  constexpr int RPW = kU4Rows / 4;  // rows per wave segment

  for (int r0 = 0; r0 < count; r0 += rc) {
    const int nr = min(rc, count - r0);
    __syncthreads();  // the previous pass is done with the staged rows
    const void* rows[kU4Routes];
#pragma unroll
    for (int rr = 0; rr < kU4Routes; ++rr) {
      const int route = ws_route(p.perm[base + r0 + min(rr, nr - 1)], R);
      if constexpr (MODE == 0) {
        const int t = route / p.k;
        rows[rr] = p.x_bf16 ? static_cast<const void*>(static_cast<const uint16_t*>(p.x) + (size_t)t * K)
                            : static_cast<const void*>(static_cast<const float*>(p.x) + (size_t)t * K);
      } else {
        rows[rr] = p.h + (size_t)route * K;
      }
    }
    u4_stage(xs, xsum, nr, K, MODE == 0 ? p.x_bf16 : 0, rows);
    __syncthreads();

    // Two rows per step: gate and up of feature n (gate/up), or output rows
    // n and n+1 (down); each activation read from LDS serves both.
    constexpr int STEPS = MODE == 0 ? RPW : RPW / 2;
    auto rows_of = [&](int i, size_t& ra, size_t& rb2, int& na, int& nb) {
      const int r0w = rb + (wave * SEGS + seg) * RPW;
      if constexpr (MODE == 0) {
        na = nb = r0w + i;
      } else {
        na = r0w + 2 * i;
        nb = na + 1;
      }
      ra = (size_t)g * N + min(na, N - 1);  // rows past N are clamped and never stored
      rb2 = (size_t)g * N + min(nb, N - 1);
    };
    auto load2 = [&](int i, u32x4 (&va)[U], uint32_t (&sa)[U], u32x4 (&vb)[U],
                     uint32_t (&sb)[U]) {
      size_t ra, rb2;
      int na, nb;
      rows_of(i, ra, rb2, na, nb);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = sl + LPR * u;
        if constexpr (MODE == 0) {
          u4_load(p.gate, ra, G, c, va[u], sa[u]);
          u4_load(p.up, rb2, G, c, vb[u], sb[u]);
        } else {
          u4_load(p.down, ra, G, c, va[u], sa[u]);
          u4_load(p.down, rb2, G, c, vb[u], sb[u]);
        }
      }
    };
    // weights of step i+1 are loaded while step i is multiplied (the copy at
    // the end of the step waits for them, after the multiplies)
    u32x4 va[U], vb[U], nva[U], nvb[U];
    uint32_t sa[U], sb[U], nsa[U], nsb[U];
    load2(0, va, sa, vb, sb);
#pragma unroll 1
    for (int i = 0; i < STEPS; ++i) {
      load2(min(i + 1, STEPS - 1), nva, nsa, nvb, nsb);
      float a0[kU4Routes], a1[kU4Routes];
#pragma unroll
      for (int r = 0; r < kU4Routes; ++r) { a0[r] = 0.f; a1[r] = 0.f; }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = sl + LPR * u;
        // gate/up stages more activations (fewer workgroups per CU) and has
        // registers to spare at its occupancy; down does not
        if (c < G) u4_group_dot2<MODE == 0>(va[u], sa[u], vb[u], sb[u], xs, xsum, G, c, nr, a0, a1);
      }
      size_t ra, rb2;
      int na, nb;
      rows_of(i, ra, rb2, na, nb);
#pragma unroll
      for (int r = 0; r < kU4Routes; ++r) {
        if (r < nr) {
          const float d0 = LPR == 64 ? wave_sum(a0[r]) : group_sum<LPR>(a0[r]);
          const float d1 = LPR == 64 ? wave_sum(a1[r]) : group_sum<LPR>(a1[r]);
          if (sl == 0) {
            if constexpr (MODE == 0) {
              const int route = ws_route(p.perm[base + r0 + r], R);
              if (na < N) p.h[(size_t)route * N + na] = act_f<ACT>(d0) * d1;
            } else {  // rows of y in the expert-grouped order (position, not route id)
              const size_t pos = (size_t)(base + r0 + r);
              if (na < N) p.y[pos * N + na] = d0;
              if (nb < N) p.y[pos * N + nb] = d1;
            }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) { va[u] = nva[u]; sa[u] = nsa[u]; vb[u] = nvb[u]; sb[u] = nsb[u]; }
    }
  }
}

}  // namespace moe
