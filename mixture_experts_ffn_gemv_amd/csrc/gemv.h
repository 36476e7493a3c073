// Memory-bound expert GEMVs for few tokens per expert (decode).
//
// Work item = (active expert group, block of matrix rows).  Each wave owns
// RW weight rows; the 64/RW lanes of a row split its K dimension into
// 16-byte chunks (4 f32, 8 bf16 or 32 four-bit codes), so every weight
// byte is loaded once, with 128-bit coalesced loads, and dotted with the
// activation vectors of all routes of that expert (four per pass).
//   gate/up : h[route, n] = act(Wg[e][n,:] . x_t) * (Wu[e][n,:] . x_t)
//   down    : y[route, n] = Wd[e][n,:] . h[route, :]
// The shared expert is one more group (id E) whose routes are all T tokens.
#pragma once

#include "common.h"

namespace moe {

struct MatStack {           // one weight matrix per group, [G, N, K] row-major
  const uint8_t* p;         // f32 / bf16 elements, or u4 codes
  const uint16_t* sc;       // u4: fp16 scales [G, N, K/32]
  const uint16_t* mn;       // u4: fp16 mins   [G, N, K/32]
};

template <int WF> struct WTraits;
template <> struct WTraits<WF_F32> { static constexpr int EPC = 4; };
template <> struct WTraits<WF_BF16> { static constexpr int EPC = 8; };
template <> struct WTraits<WF_U4> { static constexpr int EPC = 32; };

// Load and decode chunk c (EPC elements) of row `row` (row length K).
template <int WF>
__device__ __forceinline__ void load_w(const MatStack& m, size_t row, int K, int c,
                                       float (&w)[WTraits<WF>::EPC]) {
  if constexpr (WF == WF_F32) {
    u32x4 v = ld16_stream(m.p + (row * K + (size_t)c * 4) * 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = __uint_as_float(v[q]);
  } else if constexpr (WF == WF_BF16) {
    u32x4 v = ld16_stream(m.p + (row * K + (size_t)c * 8) * 2);
#pragma unroll
    for (int q = 0; q < 4; ++q) { w[2 * q] = bf16lo(v[q]); w[2 * q + 1] = bf16hi(v[q]); }
  } else {
    u32x4 v = ld16_stream(m.p + (row * K) / 2 + (size_t)c * 16);
    const size_t gi = row * (K / 32) + c;
    const float s = f16_to_f32(m.sc[gi]);
    const float mn = f16_to_f32(m.mn[gi]);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        w[8 * q + j] = fmaf(static_cast<float>((v[q] >> (4 * j)) & 15u), s, mn);
  }
}

// Load EPC activations starting at element c*EPC of a row.
template <typename XT, int EPC>
__device__ __forceinline__ void load_x(const XT* row, int c, float (&xv)[EPC]) {
  if constexpr (sizeof(XT) == 4) {
#pragma unroll
    for (int q = 0; q < EPC / 4; ++q) {
      u32x4 v = ld16(row + (size_t)c * EPC + 4 * q);
      xv[4 * q] = __uint_as_float(v[0]);
      xv[4 * q + 1] = __uint_as_float(v[1]);
      xv[4 * q + 2] = __uint_as_float(v[2]);
      xv[4 * q + 3] = __uint_as_float(v[3]);
    }
  } else if constexpr (EPC >= 8) {
#pragma unroll
    for (int q = 0; q < EPC / 8; ++q) {
      u32x4 v = ld16(row + (size_t)c * EPC + 8 * q);
#pragma unroll
      for (int i = 0; i < 4; ++i) { xv[8 * q + 2 * i] = bf16lo(v[i]); xv[8 * q + 2 * i + 1] = bf16hi(v[i]); }
    }
  } else {
    u32x2 v = *reinterpret_cast<const u32x2*>(row + (size_t)c * EPC);
    xv[0] = bf16lo(v[0]); xv[1] = bf16hi(v[0]); xv[2] = bf16lo(v[1]); xv[3] = bf16hi(v[1]);
  }
}

struct GroupInfo {
  const int32_t* counts;     // [G]
  const int32_t* offsets;    // [E+1]
  const int32_t* active;     // [G]
  const int32_t* n_active;   // [1]
  const int32_t* row_token;  // [R]
  int E, T;
};

struct GemvGateUpParams {
  MatStack gate, up, sgate, sup;
  const void* x;
  float* h;   // [R, I]
  float* hs;  // [T, Is]
  GroupInfo gi;
  int H, I, Is;
};

constexpr int kGemvWaves = 4;
constexpr int kRoutesPerPass = 4;

template <int WF, int ACT, typename XT, int RW>
__global__ __launch_bounds__(256) void k_dec_gateup(GemvGateUpParams p) {
  constexpr int EPC = WTraits<WF>::EPC;
  constexpr int LPR = 64 / RW;
  constexpr int FPW = RW / 2;
  constexpr int RC = kRoutesPerPass;
  const int s = blockIdx.x;
  if (s >= *p.gi.n_active) return;
  const int g = p.gi.active[s];
  const bool shared = (g == p.gi.E);
  const int N = shared ? p.Is : p.I;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int f0 = (blockIdx.y * kGemvWaves + wave) * FPW;
  if (f0 >= N) return;
  const int rl = lane / LPR, li = lane % LPR;
  const int f = f0 + (rl >> 1);
  const bool is_up = rl & 1;
  const bool fvalid = f < N;
  const MatStack& M = shared ? (is_up ? p.sup : p.sgate) : (is_up ? p.up : p.gate);
  const size_t row = shared ? (size_t)f : (size_t)g * N + f;
  const int count = shared ? p.gi.T : p.gi.counts[g];
  const int base = shared ? 0 : p.gi.offsets[g];
  const XT* x = reinterpret_cast<const XT*>(p.x);
  const int cpr = p.H / EPC;
  for (int r0 = 0; r0 < count; r0 += RC) {
    float acc[RC];
    const XT* xr[RC];
#pragma unroll
    for (int r = 0; r < RC; ++r) {
      acc[r] = 0.f;
      const int i = r0 + r;
      const int tok = (i < count) ? (shared ? i : p.gi.row_token[base + i]) : 0;
      xr[r] = x + (size_t)tok * p.H;
    }
    if (fvalid) {
#pragma unroll 2
      for (int c = li; c < cpr; c += LPR) {
        float w[EPC];
        load_w<WF>(M, row, p.H, c, w);
#pragma unroll
        for (int r = 0; r < RC; ++r) {
          if (r0 + r < count) {
            float xv[EPC];
            load_x<XT, EPC>(xr[r], c, xv);
            float sacc = 0.f;
#pragma unroll
            for (int q = 0; q < EPC; ++q) sacc = fmaf(w[q], xv[q], sacc);
            acc[r] += sacc;
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RC; ++r) {
      const float gsum = group_sum<LPR>(acc[r]);
      const float usum = __shfl(gsum, (lane + LPR) & 63, 64);
      if (!is_up && li == 0 && fvalid && r0 + r < count) {
        // the shared expert is always SwiGLU
        const float hv = (shared ? silu_f(gsum) : act_f<ACT>(gsum)) * usum;
        if (shared) p.hs[(size_t)(r0 + r) * N + f] = hv;
        else p.h[(size_t)(base + r0 + r) * N + f] = hv;
      }
    }
  }
}

struct GemvDownParams {
  MatStack down, sdown;
  const float* h;   // [R, I]
  const float* hs;  // [T, Is]
  float* y;         // [R, H]
  float* ys;        // [T, H]
  GroupInfo gi;
  int H, I, Is;
};

template <int WF, int RW>
__global__ __launch_bounds__(256) void k_dec_down(GemvDownParams p) {
  constexpr int EPC = WTraits<WF>::EPC;
  constexpr int LPR = 64 / RW;
  constexpr int RC = kRoutesPerPass;
  const int s = blockIdx.x;
  if (s >= *p.gi.n_active) return;
  const int g = p.gi.active[s];
  const bool shared = (g == p.gi.E);
  const int K = shared ? p.Is : p.I;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = (blockIdx.y * kGemvWaves + wave) * RW;
  if (n0 >= p.H) return;
  const int rl = lane / LPR, li = lane % LPR;
  const int n = n0 + rl;
  const bool nvalid = n < p.H;
  const MatStack& M = shared ? p.sdown : p.down;
  const size_t row = shared ? (size_t)n : (size_t)g * p.H + n;
  const int count = shared ? p.gi.T : p.gi.counts[g];
  const int base = shared ? 0 : p.gi.offsets[g];
  const float* hb = shared ? p.hs : p.h + (size_t)base * K;
  const int cpr = K / EPC;
  for (int r0 = 0; r0 < count; r0 += RC) {
    float acc[RC];
#pragma unroll
    for (int r = 0; r < RC; ++r) acc[r] = 0.f;
    if (nvalid) {
#pragma unroll 2
      for (int c = li; c < cpr; c += LPR) {
        float w[EPC];
        load_w<WF>(M, row, K, c, w);
#pragma unroll
        for (int r = 0; r < RC; ++r) {
          if (r0 + r < count) {
            float xv[EPC];
            load_x<float, EPC>(hb + (size_t)(r0 + r) * K, c, xv);
            float sacc = 0.f;
#pragma unroll
            for (int q = 0; q < EPC; ++q) sacc = fmaf(w[q], xv[q], sacc);
            acc[r] += sacc;
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RC; ++r) {
      const float v = group_sum<LPR>(acc[r]);
      if (li == 0 && nvalid && r0 + r < count) {
        if (shared) p.ys[(size_t)(r0 + r) * p.H + n] = v;
        else p.y[(size_t)(base + r0 + r) * p.H + n] = v;
      }
    }
  }
}

// --------------------------------------------------------------------------
// Weighted combine: out[t, :] = sum_j w[t, j] * y[pos(t, j), :]
//                               (+ sigmoid gate[t] * ys[t, :])
// in slot order j = 0..k-1, then the shared expert; no atomics.
// YT = float (decode) or uint16_t bf16 bits (prefill); 4 columns / thread.
// --------------------------------------------------------------------------
template <typename YT>
__global__ __launch_bounds__(256) void k_combine(const YT* __restrict__ y,
                                                 const YT* __restrict__ ys,
                                                 const float* __restrict__ wts,
                                                 const int32_t* __restrict__ pos_of_route,
                                                 const float* __restrict__ sgate,
                                                 float* out, const float* residual, int T,
                                                 int H, int k, int has_shared) {
  const int cols4 = H / 4;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)T * cols4) return;
  const int t = idx / cols4;
  const int c = (idx % cols4) * 4;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  for (int j = 0; j < k; ++j) {
    const float w = wts[(size_t)t * k + j];
    const size_t pos = pos_of_route[(size_t)t * k + j];
    if constexpr (sizeof(YT) == 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(y + pos * H + c);
      a0 = fmaf(w, v[0], a0); a1 = fmaf(w, v[1], a1); a2 = fmaf(w, v[2], a2); a3 = fmaf(w, v[3], a3);
    } else {
      const u32x2 v = *reinterpret_cast<const u32x2*>(y + pos * H + c);
      a0 = fmaf(w, bf16lo(v[0]), a0); a1 = fmaf(w, bf16hi(v[0]), a1);
      a2 = fmaf(w, bf16lo(v[1]), a2); a3 = fmaf(w, bf16hi(v[1]), a3);
    }
  }
  if (has_shared) {
    const float s = sgate[t];
    if constexpr (sizeof(YT) == 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(ys + (size_t)t * H + c);
      a0 = fmaf(s, v[0], a0); a1 = fmaf(s, v[1], a1); a2 = fmaf(s, v[2], a2); a3 = fmaf(s, v[3], a3);
    } else {
      const u32x2 v = *reinterpret_cast<const u32x2*>(ys + (size_t)t * H + c);
      a0 = fmaf(s, bf16lo(v[0]), a0); a1 = fmaf(s, bf16hi(v[0]), a1);
      a2 = fmaf(s, bf16lo(v[1]), a2); a3 = fmaf(s, bf16hi(v[1]), a3);
    }
  }
  if (residual) {  // may be out itself: read before the store, same thread
    const f32x4 r = *reinterpret_cast<const f32x4*>(residual + (size_t)t * H + c);
    a0 += r[0]; a1 += r[1]; a2 += r[2]; a3 += r[3];
  }
  f32x4 o = {a0, a1, a2, a3};
  *reinterpret_cast<f32x4*>(out + (size_t)t * H + c) = o;
}

// Prefill combine with bf16 y: 8 consecutive outputs per thread, so every
// y row is read in 16-byte pieces, and the k rows of a token are loaded 8 at a
// time before they are summed (slot order kept: padded slots add 0 * y).
__global__ __launch_bounds__(256) void k_combine_bf16x8(const uint16_t* __restrict__ y,
                                                        const uint16_t* __restrict__ ys,
                                                        const float* __restrict__ wts,
                                                        const int32_t* __restrict__ pos_of_route,
                                                        const float* __restrict__ sgate,
                                                        float* out, const float* residual,
                                                        int T, int H, int k, int has_shared) {
  const int cols8 = H / 8;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)T * cols8) return;
  const int t = idx / cols8;
  const int c = (idx % cols8) * 8;
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < k; j0 += 8) {
    u32x4 v[8];
    float w[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = min(j0 + jj, k - 1);
      const size_t pos = pos_of_route[(size_t)t * k + j];
      v[jj] = ld16_stream(y + pos * H + c);  // each y row is read once
      w[jj] = (j0 + jj < k) ? wts[(size_t)t * k + j] : 0.f;
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a[2 * q] = fmaf(w[jj], bf16lo(v[jj][q]), a[2 * q]);
        a[2 * q + 1] = fmaf(w[jj], bf16hi(v[jj][q]), a[2 * q + 1]);
      }
  }
  if (has_shared) {
    const float s = sgate[t];
    const u32x4 v = *reinterpret_cast<const u32x4*>(ys + (size_t)t * H + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[2 * q] = fmaf(s, bf16lo(v[q]), a[2 * q]);
      a[2 * q + 1] = fmaf(s, bf16hi(v[q]), a[2 * q + 1]);
    }
  }
  if (residual) {  // may be out itself: read before the store, same thread
    const f32x4* r = reinterpret_cast<const f32x4*>(residual + (size_t)t * H + c);
    const f32x4 r0 = r[0], r1 = r[1];
#pragma unroll
    for (int q = 0; q < 4; ++q) { a[q] += r0[q]; a[4 + q] += r1[q]; }
  }
  f32x4* o = reinterpret_cast<f32x4*>(out + (size_t)t * H + c);
  o[0] = f32x4{a[0], a[1], a[2], a[3]};
  o[1] = f32x4{a[4], a[5], a[6], a[7]};
}

}  // namespace moe
