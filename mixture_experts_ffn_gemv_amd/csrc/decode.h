// Decode path (few tokens, T <= 32): four launches per layer.
//
//   router GEMV -> k_route_small -> k_dec_gateup3 -> k_dec_down3
//
// k_route_small   one workgroup: softmax/top-k/renormalise for every token,
//                 then the stable expert grouping (counts, offsets, list of
//                 touched experts, routes grouped by expert).
// k_dec_gateup3   work item = (touched expert, block of 4 features).  Each
//                 wave owns 1 feature (its gate and up rows); its 64 lanes
//                 split K into 16-byte chunks and issue every weight load of
//                 those rows before touching the activations.  Only the
//                 touched experts' weights are read, each byte once.
// k_dec_down3     work item = block of output features; the 4 waves split
//                 the touched experts, each loading the expert's down rows
//                 once and applying them to all of the expert's routes, and
//                 the routing-weighted sum per token is formed in LDS and
//                 written straight to the output: no y buffer, no atomics.
//                 The shared expert is one more group whose routes are all
//                 tokens, weighted by sigmoid(x . shared_gate_inp).
#pragma once

#include "common.h"
#include "gemv.h"

namespace moe {

constexpr int kSmallMaxTokens = 32;
constexpr int kSmallRoutes = kSmallMaxTokens * MOE_MAX_TOP_K_DEV;

// ---------------------------------------------------------------------------
// Top-k of one token's logits by one wave.  Lane j < k returns slot j's
// expert and weight.  See k_topk for the selection and weight rules.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void wave_topk(const float* __restrict__ l, int E, int k, int normalize,
                                          int lane, int& my_id, float& my_w) {
  float v[4];
  unsigned taken = 0;  // bit q: candidate q of this lane is used up (or absent)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    v[q] = (e < E) ? l[e] : -INFINITY;
    if (e >= E) taken |= 1u << q;
  }
  my_id = 0;
  float my_val = -INFINITY;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (!((taken >> q) & 1u) && (v[q] > bv || bi == 0x7FFFFFFF)) { bv = v[q]; bi = lane + 64 * q; }
    wave_argmax(bv, bi);
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == j) { my_id = bi; my_val = bv; }
  }
  const float lmax = __shfl(my_val, 0, 64);
  const float ex = (lane < k) ? __expf(my_val - lmax) : 0.f;
  float denom;
  if (normalize) {
    denom = wave_sum(ex);
  } else {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (lane + 64 * q < E) s += __expf(v[q] - lmax);
    denom = wave_sum(s);
  }
  my_w = ex / denom;
}

constexpr int kRoutedMaxTokens = 4;
constexpr int kRoutedMaxRoutes = kRoutedMaxTokens * MOE_MAX_TOP_K_DEV;

struct RoutedLds {
  int ids[kRoutedMaxRoutes];      // expert of route r = t*k + j
  float w[kRoutedMaxRoutes];      // routing weight of route r
  int perm[kRoutedMaxRoutes];     // routes grouped by expert, stable
  int first[kRoutedMaxRoutes];    // route r is its expert's first route
  int gexp[MOE_MAX_EXPERTS_DEV];  // expert of touched slot s (ascending)
  int gstart[MOE_MAX_EXPERTS_DEV + 1];
  int nrouted;
  float sg[kRoutedMaxTokens];     // shared-expert gate per token
};

// Routing of T <= 4 tokens by one workgroup into LDS (wave t handles token t),
// then the stable grouping of the R = T*k routes by expert with O(R^2)
// rank counting: few barriers, no scan.
__device__ __forceinline__ void route_tokens_lds(const float* __restrict__ logits, int T, int E,
                                                 int k, int ncols, int normalize, int has_shared,
                                                 RoutedLds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = T * k;
  if (wave < T) {
    const float* l = logits + (size_t)wave * ncols;
    int id;
    float w;
    wave_topk(l, E, k, normalize, lane, id, w);
    if (lane < k) {
      L.ids[wave * k + lane] = id;
      L.w[wave * k + lane] = w;
    }
    if (lane == 0) L.sg[wave] = has_shared ? sigmoid_f(l[E]) : 0.f;
  }
  __syncthreads();
  // stable position of each route in expert order, and first-of-expert flags
  if (tid < R) {
    const int e = L.ids[tid];
    int less = 0, first = 1;
    for (int r2 = 0; r2 < R; ++r2) {
      const int e2 = L.ids[r2];
      less += (e2 < e) || (e2 == e && r2 < tid);
      first &= !(e2 == e && r2 < tid);
    }
    L.perm[less] = tid;
    L.first[tid] = first;
  }
  __syncthreads();
  if (tid < R && L.first[tid]) {
    const int e = L.ids[tid];
    int slot = 0, start = 0;
    for (int r2 = 0; r2 < R; ++r2) {
      const int e2 = L.ids[r2];
      slot += (e2 < e) && L.first[r2];
      start += (e2 < e);
    }
    L.gexp[slot] = e;
    L.gstart[slot] = start;
  }
  if (tid == 0) {
    int n = 0;
    for (int r2 = 0; r2 < R; ++r2) n += L.first[r2];
    L.nrouted = n;
    L.gstart[n] = R;
  }
  __syncthreads();
}

struct SmallRouteOut {
  int32_t* ids;          // [R]
  float* wts;            // [R]
  float* sgate;          // [T]
  int32_t* counts;       // [G]
  int32_t* offsets;      // [E+1]
  int32_t* active;       // [G]
  int32_t* n_active;     // [1]
  int32_t* perm;         // [R] routes grouped by expert
  int32_t* pos_of_route; // [R]
  int32_t* user_ids;
  float* user_w;
  int32_t* user_counts;
  int32_t* user_offsets;
  int32_t* user_perm;
};

__global__ __launch_bounds__(256) void k_route_small(const float* __restrict__ logits, int T, int E,
                                                     int k, int ncols, int normalize,
                                                     int has_shared, SmallRouteOut o) {
  __shared__ int s_ids[kSmallRoutes];
  __shared__ int s_cnt[256];
  __shared__ int s_sc[256];
  __shared__ int s_sa[256];
  __shared__ RoutedLds L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = T * k;
  if (T <= kRoutedMaxTokens) {
    route_tokens_lds(logits, T, E, k, ncols, normalize, has_shared, L);
    for (int r = tid; r < R; r += 256) {
      o.ids[r] = L.ids[r];
      o.wts[r] = L.w[r];
      o.perm[r] = L.perm[r];
      o.pos_of_route[L.perm[r]] = r;
      if (o.user_ids) o.user_ids[r] = L.ids[r];
      if (o.user_w) o.user_w[r] = L.w[r];
      if (o.user_perm) o.user_perm[r] = L.perm[r];
    }
    // per-expert counts and offsets over all E experts
    for (int e = tid; e <= E; e += 256) {
      int less = 0, eq = 0;
      for (int r = 0; r < R; ++r) {
        less += L.ids[r] < e;
        eq += L.ids[r] == e;
      }
      o.offsets[e] = less;
      if (o.user_offsets) o.user_offsets[e] = less;
      if (e < E) {
        o.counts[e] = eq;
        if (o.user_counts) o.user_counts[e] = eq;
      }
    }
    const int nrouted = L.nrouted;
    for (int sl = tid; sl < nrouted; sl += 256) o.active[sl] = L.gexp[sl];
    if (tid < T && has_shared) o.sgate[tid] = L.sg[tid];
    if (tid == 0) {
      int na = nrouted;
      if (has_shared) {
        o.counts[E] = T;
        o.active[na++] = E;
      }
      *o.n_active = na;
    }
    return;
  }
  s_cnt[tid] = 0;
  for (int t = wave; t < T; t += 4) {
    const float* l = logits + (size_t)t * ncols;
    int id;
    float w;
    wave_topk(l, E, k, normalize, lane, id, w);
    if (lane < k) {
      const int r = t * k + lane;
      s_ids[r] = id;
      o.ids[r] = id;
      o.wts[r] = w;
      if (o.user_ids) o.user_ids[r] = id;
      if (o.user_w) o.user_w[r] = w;
    }
    if (has_shared && lane == 0) o.sgate[t] = sigmoid_f(l[E]);
  }
  __syncthreads();
  for (int r = tid; r < R; r += 256) atomicAdd(&s_cnt[s_ids[r]], 1);
  __syncthreads();
  const int cnt = s_cnt[tid];
  const int act = (tid < E && cnt > 0) ? 1 : 0;
  // inclusive scans of counts and active flags: within each wave by
  // shuffles, then across the four waves
  int ic = cnt, ia = act;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int a = __shfl_up(ic, d, 64);
    const int b = __shfl_up(ia, d, 64);
    if (lane >= d) { ic += a; ia += b; }
  }
  if (lane == 63) { s_sc[wave] = ic; s_sa[wave] = ia; }
  __syncthreads();
  for (int w = 0; w < wave; ++w) { ic += s_sc[w]; ia += s_sa[w]; }
  __syncthreads();
  s_sc[tid] = ic;
  s_sa[tid] = ia;
  __syncthreads();
  const int off = s_sc[tid] - cnt;
  const int aoff = s_sa[tid] - act;
  const int nact = s_sa[255];
  if (tid < E) {
    o.counts[tid] = cnt;
    o.offsets[tid] = off;
    if (o.user_counts) o.user_counts[tid] = cnt;
    if (o.user_offsets) o.user_offsets[tid] = off;
    if (act) o.active[aoff] = tid;
  }
  if (tid == 0) {
    o.offsets[E] = R;
    if (o.user_offsets) o.user_offsets[E] = R;
    int na = nact;
    if (has_shared) {
      o.counts[E] = T;
      o.active[na++] = E;
    }
    *o.n_active = na;
  }
  __syncthreads();
  s_cnt[tid] = off;  // running position per expert
  __syncthreads();
  // stable placement, 64 routes per step by wave 0
  for (int base = 0; base < R; base += 64) {
    const int r = base + lane;
    const bool valid = r < R;
    int pos = 0, e = 0;
    uint64_t mask = 0;
    if (wave == 0) {
      e = valid ? s_ids[r] : 0;
      mask = __ballot(valid);
#pragma unroll
      for (int bit = 0; bit < 8; ++bit) {
        const bool set = (e >> bit) & 1;
        const uint64_t b = __ballot(set);
        mask &= set ? b : ~b;
      }
      pos = s_cnt[e] + __popcll(mask & lanemask_lt());
    }
    __syncthreads();
    if (wave == 0 && valid) {
      if ((mask >> lane) == 1ull) s_cnt[e] += __popcll(mask);
      o.perm[pos] = r;
      o.pos_of_route[r] = pos;
      if (o.user_perm) o.user_perm[pos] = r;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
struct Dec2Params {
  MatStack gate, up, sgate, sup, down, sdown;
  const void* x;
  int x_bf16;
  float* h;      // [R, I]  by route id r = t*k + j
  float* hs;     // [T, Is]
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* active;
  const int32_t* n_active;
  const int32_t* perm;
  const float* wts;
  const float* sgate_val;
  float* out;    // [T, H]
  int T, E, k, H, I, Is, rc;
};

template <int WF>
__device__ __forceinline__ const uint8_t* row_ptr(const MatStack& m, size_t row, int K) {
  if constexpr (WF == WF_F32) return m.p + row * K * 4;
  else if constexpr (WF == WF_BF16) return m.p + row * K * 2;
  else return m.p + row * K / 2;
}

// Decode chunk `v` (16 bytes) of a row into EPC floats.
template <int WF>
__device__ __forceinline__ void decode_chunk(const u32x4& v, float s, float mn,
                                             float (&w)[WTraits<WF>::EPC]) {
  if constexpr (WF == WF_F32) {
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = __uint_as_float(v[q]);
  } else if constexpr (WF == WF_BF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) { w[2 * q] = bf16lo(v[q]); w[2 * q + 1] = bf16hi(v[q]); }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        w[8 * q + j] = fmaf(static_cast<float>((v[q] >> (4 * j)) & 15u), s, mn);
  }
}

// Load chunk c of a row (16 bytes) plus, for 4-bit rows, its group's scale/min.
template <int WF>
__device__ __forceinline__ void load_chunk(const MatStack& m, size_t row, int K, int c, bool ok,
                                           u32x4& v, float& s, float& mn) {
  v = ok ? ld16_stream(row_ptr<WF>(m, row, K) + (size_t)c * 16) : u32x4{0, 0, 0, 0};
  if constexpr (WF == WF_U4) {
    const size_t gi = row * (K / 32) + c;
    s = ok ? f16_to_f32(m.sc[gi]) : 0.f;
    mn = ok ? f16_to_f32(m.mn[gi]) : 0.f;
  } else {
    s = 0.f;
    mn = 0.f;
  }
}

template <int WF>
__device__ __forceinline__ float dot_chunk(const u32x4& v, float s, float mn,
                                           const float (&xv)[WTraits<WF>::EPC]) {
  float w[WTraits<WF>::EPC];
  decode_chunk<WF>(v, s, mn, w);
  float a = 0.f;
#pragma unroll
  for (int e = 0; e < WTraits<WF>::EPC; ++e) a = fmaf(w[e], xv[e], a);
  return a;
}

// EPC activations of chunk c from a row in global memory (f32 or bf16), as f32.
template <int EPC>
__device__ __forceinline__ void load_act(const void* x, int bf16, size_t off, float (&xv)[EPC]) {
  if (bf16) {
    const uint16_t* r = reinterpret_cast<const uint16_t*>(x) + off;
#pragma unroll
    for (int q = 0; q < EPC / 4; ++q) {
      const u32x2 b = *reinterpret_cast<const u32x2*>(r + 4 * q);
      xv[4 * q] = bf16lo(b[0]); xv[4 * q + 1] = bf16hi(b[0]);
      xv[4 * q + 2] = bf16lo(b[1]); xv[4 * q + 3] = bf16hi(b[1]);
    }
  } else {
    const float* r = reinterpret_cast<const float*>(x) + off;
#pragma unroll
    for (int q = 0; q < EPC / 4; ++q) {
      const f32x4 t4 = *reinterpret_cast<const f32x4*>(r + 4 * q);
      xv[4 * q] = t4[0]; xv[4 * q + 1] = t4[1]; xv[4 * q + 2] = t4[2]; xv[4 * q + 3] = t4[3];
    }
  }
}

constexpr int kRCMax = 4;    // routes per LDS pass (gate/up with several routes per expert)
constexpr int kGUWaves = 4;  // features per gate/up workgroup (one per wave)

// gate/up: each wave owns one feature f of one touched expert: its gate row
// and its up row, full K, lane l holding chunks l, l+64, ... (U of them).
// DIRECT (every expert has exactly one route, i.e. one token): the lane's
// activation chunks are loaded straight into registers.  Otherwise the
// activations of up to rc routes are staged in LDS as f32 per pass.
template <int WF, int ACT, int U, bool DIRECT>
__global__ __launch_bounds__(256) void k_dec_gateup3(Dec2Params p) {
  constexpr int EPC = WTraits<WF>::EPC;
  extern __shared__ float xs[];  // [rc][H] (staged path only)
  const int s = blockIdx.x;
  if (s >= *p.n_active) return;
  const int g = p.active[s];
  const bool shared = (g == p.E);
  const int N = shared ? p.Is : p.I;
  const int fblk = blockIdx.y * kGUWaves;
  if (fblk >= N) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int f = fblk + wave;
  const bool fok = f < N;
  const int cpr = p.H / EPC;
  const MatStack& Mg = shared ? p.sgate : p.gate;
  const MatStack& Mu = shared ? p.sup : p.up;
  const size_t row = shared ? (size_t)f : (size_t)g * N + f;

  const int count = shared ? p.T : p.counts[g];
  const int base = shared ? 0 : p.offsets[g];

  if constexpr (DIRECT) {
    const int r = shared ? 0 : p.perm[base];
    const int t = shared ? 0 : r / p.k;
    float ag = 0.f, au = 0.f;
    for (int kb = 0; kb < cpr; kb += 64 * U) {
      // all weight loads of this wave (for this K block) first
      u32x4 wg[U], wu[U];
      float sg[U], mg[U], su[U], mu[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = kb + lane + 64 * u;
        const bool ok = fok && c < cpr;
        load_chunk<WF>(Mg, row, p.H, c, ok, wg[u], sg[u], mg[u]);
        load_chunk<WF>(Mu, row, p.H, c, ok, wu[u], su[u], mu[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = kb + lane + 64 * u;
        if (c < cpr) {
          float xv[EPC];
          load_act<EPC>(p.x, p.x_bf16, (size_t)t * p.H + (size_t)c * EPC, xv);
          ag += dot_chunk<WF>(wg[u], sg[u], mg[u], xv);
          au += dot_chunk<WF>(wu[u], su[u], mu[u], xv);
        }
      }
    }
    ag = wave_sum(ag);
    au = wave_sum(au);
    if (lane == 0 && fok) {
      // the shared expert is always SwiGLU
      const float hv = (shared ? silu_f(ag) : act_f<ACT>(ag)) * au;
      if (shared) p.hs[f] = hv;
      else p.h[(size_t)r * N + f] = hv;
    }
  } else {
    for (int r0 = 0; r0 < count; r0 += p.rc) {
      const int nr = min(p.rc, count - r0);
      float ag[kRCMax], au[kRCMax];
#pragma unroll
      for (int r = 0; r < kRCMax; ++r) { ag[r] = 0.f; au[r] = 0.f; }
      for (int kb = 0; kb < cpr; kb += 64 * U) {
        u32x4 wg[U], wu[U];
        float sg[U], mg[U], su[U], mu[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = kb + lane + 64 * u;
          const bool ok = fok && c < cpr;
          load_chunk<WF>(Mg, row, p.H, c, ok, wg[u], sg[u], mg[u]);
          load_chunk<WF>(Mu, row, p.H, c, ok, wu[u], su[u], mu[u]);
        }
        if (kb == 0) {
          // stage this pass's activations (after the weight loads are issued)
          __syncthreads();
          const int q4 = p.H / 4;
          for (int i = tid; i < nr * q4; i += 256) {
            const int r = i / q4, c4 = i - r * q4;
            const int t = shared ? (r0 + r) : (p.perm[base + r0 + r] / p.k);
            float v4[4];
            load_act<4>(p.x, p.x_bf16, (size_t)t * p.H + 4 * c4, v4);
            *reinterpret_cast<f32x4*>(&xs[r * p.H + 4 * c4]) = f32x4{v4[0], v4[1], v4[2], v4[3]};
          }
          __syncthreads();
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = kb + lane + 64 * u;
          if (c < cpr) {
#pragma unroll
            for (int r = 0; r < kRCMax; ++r) {
              if (r < nr) {
                float xv[EPC];
#pragma unroll
                for (int q = 0; q < EPC / 4; ++q) {
                  const f32x4 t4 = *reinterpret_cast<const f32x4*>(&xs[r * p.H + c * EPC + 4 * q]);
                  xv[4 * q] = t4[0]; xv[4 * q + 1] = t4[1]; xv[4 * q + 2] = t4[2]; xv[4 * q + 3] = t4[3];
                }
                ag[r] += dot_chunk<WF>(wg[u], sg[u], mg[u], xv);
                au[r] += dot_chunk<WF>(wu[u], su[u], mu[u], xv);
              }
            }
          }
        }
      }
#pragma unroll
      for (int r = 0; r < kRCMax; ++r) {
        if (r < nr) {
          const float gs = wave_sum(ag[r]);
          const float us = wave_sum(au[r]);
          if (lane == 0 && fok) {
            const float hv = (shared ? silu_f(gs) : act_f<ACT>(gs)) * us;
            if (shared) p.hs[(size_t)(r0 + r) * N + f] = hv;
            else p.h[(size_t)p.perm[base + r0 + r] * N + f] = hv;
          }
        }
      }
    }
  }
}

constexpr int kDownRPW = 4;  // output features per down+combine workgroup

// down + combine: a workgroup owns kDownRPW output features; its 4 waves take
// the touched experts in turn (s = wave, wave+4, ...), loading the next
// expert's rows while computing with the current one, and accumulate
// w_route * (Wd[e][n,:] . h_route) per token in LDS.  The shared expert is
// the last group, weighted by its sigmoid gate.  The four waves' partial
// sums are added in a fixed order and written to out: no atomics.
template <int WF, int U>
__global__ __launch_bounds__(256) void k_dec_down3(Dec2Params p) {
  constexpr int EPC = WTraits<WF>::EPC;
  constexpr int RPW = kDownRPW;
  __shared__ float part[4][kSmallMaxTokens][RPW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * RPW;
  for (int i = tid; i < 4 * kSmallMaxTokens * RPW; i += 256) (&part[0][0][0])[i] = 0.f;
  __syncthreads();
  const int na = *p.n_active;

  u32x4 wc[RPW][U], wn[RPW][U];
  float sc[RPW][U], mc[RPW][U], sn[RPW][U], mnx[RPW][U];
  auto load_group = [&](int s, u32x4 (&w)[RPW][U], float (&sv)[RPW][U], float (&mv)[RPW][U]) {
    const int g = p.active[s];
    const bool shared = (g == p.E);
    const int K = shared ? p.Is : p.I;
    const int cpr = K / EPC;
    const MatStack& M = shared ? p.sdown : p.down;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = lane + 64 * u;
#pragma unroll
      for (int q = 0; q < RPW; ++q) {
        const int n = n0 + q;
        const size_t row = shared ? (size_t)n : (size_t)g * p.H + n;
        load_chunk<WF>(M, row, K, c, n < p.H && c < cpr, w[q][u], sv[q][u], mv[q][u]);
      }
    }
  };
  int s = wave;
  if (s < na) load_group(s, wc, sc, mc);
  while (s < na) {
    const int sn_ = s + 4;
    if (sn_ < na) load_group(sn_, wn, sn, mnx);
    const int g = p.active[s];
    const bool shared = (g == p.E);
    const int K = shared ? p.Is : p.I;
    const int cpr = K / EPC;
    const int count = shared ? p.T : p.counts[g];
    const int base = shared ? 0 : p.offsets[g];
    for (int i = 0; i < count; ++i) {
      int t;
      float wgt;
      const float* hrow;
      if (shared) {
        t = i; wgt = p.sgate_val[t]; hrow = p.hs + (size_t)t * K;
      } else {
        const int r = p.perm[base + i];
        t = r / p.k; wgt = p.wts[r]; hrow = p.h + (size_t)r * K;
      }
      float acc[RPW];
#pragma unroll
      for (int q = 0; q < RPW; ++q) acc[q] = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = lane + 64 * u;
        if (c < cpr) {
          float xv[EPC];
          load_act<EPC>(hrow, 0, (size_t)c * EPC, xv);
#pragma unroll
          for (int q = 0; q < RPW; ++q) acc[q] += dot_chunk<WF>(wc[q][u], sc[q][u], mc[q][u], xv);
        }
      }
#pragma unroll
      for (int q = 0; q < RPW; ++q) {
        const float v = wave_sum(acc[q]);
        if (lane == 0) part[wave][t][q] += wgt * v;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < RPW; ++q) { wc[q][u] = wn[q][u]; sc[q][u] = sn[q][u]; mc[q][u] = mnx[q][u]; }
    s = sn_;
  }
  __syncthreads();
  for (int i = tid; i < p.T * RPW; i += 256) {
    const int t = i / RPW, q = i - t * RPW;
    const int n = n0 + q;
    if (n < p.H) p.out[(size_t)t * p.H + n] = part[0][t][q] + part[1][t][q] + part[2][t][q] + part[3][t][q];
  }
}

}  // namespace moe
