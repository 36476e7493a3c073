// Decode path (few tokens, T <= 32): three launches per layer.
//
//   T = 1, f32 or bf16 weights:  k_router_gemv  -> k_dec_gateup3<ONE> -> k_dec_down3<ONE>
//   otherwise:                   k_router_route -> k_dec_gateup3        -> k_dec_down3
//
// k_router_gemv   router logits only (one workgroup per router row).
// k_router_route  router logits (one workgroup per router row); the last
//                 workgroup to finish then does softmax/top-k/renormalise
//                 for every token and the stable expert grouping (counts,
//                 offsets, list of touched experts, routes grouped by
//                 expert).
// k_dec_gateup3   work item = (touched expert, block of 4 features).  Each
//                 wave owns 1 feature (its gate and up rows); its 64 lanes
//                 split K into 16-byte chunks and issue every weight load of
//                 those rows before touching the activations.  Only the
//                 touched experts' weights are read, each byte once.  With
//                 ONE (one token) every wave ranks the token's logits
//                 itself (route_one_token: the selection order and weights
//                 of the routing workgroup) to find its expert, and one
//                 wave of workgroup (0,0) writes the routing (and the slot
//                 table k_dec_down3<ONE> reads) for the down kernel and the
//                 caller: one token's top-k costs a wave less than a
//                 grid-wide handoff inside the router launch does.
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
#include "route.h"

namespace moe {

constexpr int kSmallMaxTokens = 32;
constexpr int kSmallRoutes = kSmallMaxTokens * MOE_MAX_TOP_K_DEV;

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
  // one token routed in the gate/up kernel: the slot table (null otherwise)
  int4* slots;
};

// Slot table of one-token decode: entry 0 = {slots in use, 0, 0, 0}; entry
// 1 + s = {expert, route, routing weight (f32 bits), 0} of slot s, the
// selected experts in ascending order, then the shared expert (route 0,
// weight its sigmoid gate).  The down kernel reads it with one load a lane.
constexpr int kSlotTab = MOE_MAX_TOP_K_DEV + 2;

// Exclusive prefix sums of two per-thread values over the 256 threads of a
// workgroup (thread order), and their totals.
__device__ __forceinline__ void block_scan2(int a, int b, int& ea, int& eb, int& ta, int& tb) {
  __shared__ int s_part[2][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int ia = a, ib = b;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(ia, d, 64);
    const int v = __shfl_up(ib, d, 64);
    if (lane >= d) { ia += u; ib += v; }
  }
  if (lane == 63) { s_part[0][wave] = ia; s_part[1][wave] = ib; }
  __syncthreads();
  ta = 0; tb = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) { ia += s_part[0][w]; ib += s_part[1][w]; }
    ta += s_part[0][w];
    tb += s_part[1][w];
  }
  ea = ia - a;
  eb = ib - b;
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Routing of T <= 32 tokens by one workgroup.  The logits of every token go
// to LDS, the k experts of each token are selected by one of two methods,
// the softmax denominators are summed by a 16-lane row per token, the
// weights formed one thread per route, and the grouping is one thread per
// expert: its routes, in token order, are its stable block.
//
// Rank selection (few pairs): pair (t, e) gets the key (order-preserving
// bits of l[t,e], ~e).  Keys of one token are distinct and order "larger
// logit first, lower expert index among equal logits", the tie rule of the
// stable descending sort.  A pair's rank is the number of larger keys of its
// token; ranks below k are the slots.  All pairs are ranked at once, E
// comparisons each, where a wave-wide arg-max needs k dependent rounds.
//
// Row selection (more pairs): a 16-lane row per token, four tokens per
// wave; k rounds of a row maximum over the same keys, built from DPP row
// operations, which need no cross-row readlane.
// ---------------------------------------------------------------------------
constexpr int kRankMaxPairs = 1024;

__device__ __forceinline__ bool rank_route_ok(int T, int E) {
  const int pairs = T * E;
  return pairs <= kRankMaxPairs && ((pairs + 255) / 256) * E <= 256;
}

// Order-preserving 32-bit image of a logit (-0 and +0 tie) and its inverse.
__device__ __forceinline__ uint32_t route_ord(float l) {
  const uint32_t u = __float_as_uint(l == 0.0f ? 0.0f : l);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord_logit(uint32_t ord) {
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}
// Rank key of (logit, expert): larger logit first, then the lower expert.
__device__ __forceinline__ uint64_t route_key(float l, int e) {
  return ((uint64_t)route_ord(l) << 32) | (uint32_t)~(uint32_t)e;
}

typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF,
                                                            0xF, true);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// k rounds of a 16-lane maximum over the rank keys per token; lane l of a
// row holds the keys of experts l, l+16, ... (CPL of them, E <= 16*CPL), and
// the lane holding a round's winner clears it.
template <int CPL>
__device__ __forceinline__ void row_select(const float* __restrict__ s_l, int T, int E, int k,
                                           int8_t* __restrict__ s_sel, int* __restrict__ s_rid) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15;
  for (int t0 = wave * 4; t0 < T; t0 += 16) {
    const int t = t0 + (lane >> 4);
    const bool tok = t < T;
    uint64_t key[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int e = l16 + 16 * c;
      key[c] = (tok && e < E) ? route_key(s_l[t * E + e], e) : 0;
    }
    for (int j = 0; j < k; ++j) {
      uint64_t m[CPL];  // pairwise tree: independent compares can overlap
#pragma unroll
      for (int c = 0; c < CPL; ++c) m[c] = key[c];
#pragma unroll
      for (int w = CPL / 2; w >= 1; w /= 2)
#pragma unroll
        for (int c = 0; c < w; ++c) m[c] = max_u64(m[c], m[c + w]);
      uint64_t b = m[0];
      b = max_u64(b, dpp_u64<kDppXor1>(b));
      b = max_u64(b, dpp_u64<kDppXor2>(b));
      b = max_u64(b, dpp_u64<kDppHalfMirror>(b));
      b = max_u64(b, dpp_u64<kDppMirror>(b));
#pragma unroll
      for (int c = 0; c < CPL; ++c) key[c] = key[c] == b ? 0 : key[c];
      const int e = (int)~(uint32_t)b;
      if (tok && (e & 15) == l16) s_sel[t * E + e] = (int8_t)j;
      if (tok && l16 == 0) s_rid[t * k + j] = e;
    }
  }
}

constexpr int kDppRowBcast15 = 0x142;  // lane 15 of each row to the next row
constexpr int kDppRowBcast31 = 0x143;  // lane 31 to rows 2 and 3

// Maximum of v over the wave, wave-uniform: the row maximum by four DPP
// steps, then two row broadcasts carry it to lane 63.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)dpp_i<kDppXor1>((int)v));
  v = max(v, (uint32_t)dpp_i<kDppXor2>((int)v));
  v = max(v, (uint32_t)dpp_i<kDppHalfMirror>((int)v));
  v = max(v, (uint32_t)dpp_i<kDppMirror>((int)v));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kDppRowBcast15, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kDppRowBcast31, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// One token's routing in one wave (E <= 64*C): the selection order and
// weights of route_small_impl at T = 1.  Lane l holds experts l, l+64, ...;
// each of k rounds takes the wave maximum M of the order images, then the
// lowest still-live expert whose image is M (ballots over the lanes, the
// live set a wave-uniform bit mask, since taken and absent experts both read
// as image 0), which is exactly the maximum of the rank keys.  Lane j < k
// returns the expert and routing weight of top-k position j; `sel` returns
// the selected experts as bit masks (expert 64c + b at bit b of sel[c]).
// Every lane must take part.
static_assert(MOE_MAX_EXPERTS_DEV <= 4 * 64, "one-token ranking holds at most 4 logits a lane");
template <int C>
__device__ __forceinline__ void route_one_token(const float* __restrict__ l, int E, int k,
                                                RouteMode rm, int& id, float& w,
                                                uint64_t (&sel)[C]) {
  const int lane = threadIdx.x & 63;
  float lv[C];
  uint32_t ord[C];
  uint64_t live[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int e = lane + 64 * c;
    const bool ok = e < E;
    lv[c] = ok ? l[e] : 0.f;
    ord[c] = ok ? route_ord(lv[c]) : 0u;
    live[c] = __ballot(ok);
    sel[c] = 0;
  }
  int my_e = 0;
  uint32_t my_ord = 0, top = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t m = ord[0];
#pragma unroll
    for (int c = 1; c < C; ++c) m = max(m, ord[c]);
    const uint32_t M = wave_max_u32(m);
    int e = 0;
    bool found = false;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const uint64_t hit = __ballot(ord[c] == M) & live[c];
      if (!found && hit != 0) {
        e = 64 * c + __ffsll((unsigned long long)hit) - 1;
        found = true;
      }
    }
    const int ce = e >> 6, le = e & 63;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const uint64_t bit = c == ce ? 1ull << le : 0ull;  // selects, no branch
      live[c] &= ~bit;
      sel[c] |= bit;
      ord[c] = (c == ce && lane == le) ? 0u : ord[c];
    }
    if (j == 0) top = M;
    if (lane == j) {
      my_e = e;
      my_ord = M;
    }
  }
  id = lane < k ? my_e : 0;
  const float li = ord_logit(my_ord);
  const float lmax = ord_logit(top);  // the top logit
  const float ex =
      lane < k ? (rm.sigmoid ? sigmoid_f(li) : __expf(li - lmax)) * expert_scale_of(rm, id) : 0.f;
  float denom;
  if (rm.normalize) {
    denom = wave_sum(ex);
  } else if (rm.sigmoid) {
    denom = 1.f;
  } else {
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c)
      if (lane + 64 * c < E) sum += __expf(lv[c] - lmax);
    denom = wave_sum(sum);
  }
  w = ex / denom * rm.scale;
}

struct RouteLds {
  float l[kSmallMaxTokens * MOE_MAX_EXPERTS_DEV];     // logits [T][E]
  int8_t sel[kSmallMaxTokens * MOE_MAX_EXPERTS_DEV];  // slot of (t, e), or -1
  int rid[kSmallRoutes];                              // expert of route t*k + j
  float den[kSmallMaxTokens];                         // softmax denominator per token
  // rank keys, rows padded to an even length with key 0 (below every real key)
  __attribute__((aligned(16))) uint64_t key[kRankMaxPairs + kSmallMaxTokens];
};

// TMAX bounds T: the per-token loops are unrolled to TMAX, so the common
// few-token case runs a short instruction stream.
template <int TMAX>
__device__ __forceinline__ void route_small_impl(const float* __restrict__ logits, int T, int E,
                                                 int k, int ncols, RouteMode rm, int has_shared,
                                                 const SmallRouteOut& o, RouteLds& L) {
  float* s_l = L.l;
  int8_t* s_sel = L.sel;
  int* s_rid = L.rid;
  float* s_den = L.den;
  uint64_t* s_key = L.key;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = T * k;
  const bool use_rank = rank_route_ok(T, E);
  const int Ep = (E + 1) & ~1;

  // 1. logits -> LDS; thread e loads column e of every token, all loads at once
  {
    const bool eok = tid < E;
    float lv[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
      lv[t] = (t < T && eok) ? logits[(size_t)t * ncols + tid] : 0.f;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t < T && eok) {
        s_l[t * E + tid] = lv[t];
        s_sel[t * E + tid] = -1;
        if (use_rank) s_key[t * Ep + tid] = route_key(lv[t], tid);
      }
    }
    if (use_rank && (E & 1) && tid < T) s_key[tid * Ep + E] = 0;
  }
  __syncthreads();

  // 2. selection
  if (use_rank) {
    for (int q = tid; q < T * E; q += 256) {
      const int t = q / E, e = q - t * E;
      const uint64_t mine = s_key[t * Ep + e];
      const u64x2* row = reinterpret_cast<const u64x2*>(&s_key[t * Ep]);
      int rank = 0;
      for (int i = 0; i < Ep / 2; ++i) {
        const u64x2 kk = row[i];
        rank += (kk[0] > mine ? 1 : 0) + (kk[1] > mine ? 1 : 0);
      }
      if (rank < k) {
        s_sel[q] = (int8_t)rank;
        s_rid[t * k + rank] = e;
      }
    }
  } else if (E <= 64) {
    row_select<4>(s_l, T, E, k, s_sel, s_rid);
  } else if (E <= 128) {
    row_select<8>(s_l, T, E, k, s_sel, s_rid);
  } else {
    row_select<16>(s_l, T, E, k, s_sel, s_rid);
  }
  __syncthreads();

  if constexpr (TMAX <= 4) {
    // 3+4. weights: wave t handles token t, lane j slot j
    if (wave < T) {
      const int t = wave;
      const float* lt = s_l + t * E;
      const int id = lane < k ? s_rid[t * k + lane] : 0;
      const float lmax = lt[s_rid[t * k]];
      const float ex = lane < k ? (rm.sigmoid ? sigmoid_f(lt[id]) : __expf(lt[id] - lmax)) *
                                      expert_scale_of(rm, id)
                                : 0.f;
      float denom;
      if (rm.normalize) {
        denom = wave_sum(ex);
      } else if (rm.sigmoid) {
        denom = 1.f;
      } else {
        float sum = 0.f;
        for (int e = lane; e < E; e += 64) sum += __expf(lt[e] - lmax);
        denom = wave_sum(sum);
      }
      if (lane < k) {
        const int r = t * k + lane;
        const float w = ex / denom * rm.scale;
        o.ids[r] = id;
        o.wts[r] = w;
        if (o.user_ids) o.user_ids[r] = id;
        if (o.user_w) o.user_w[r] = w;
      }
    }
  } else {
    // 3. denominators, a 16-lane row per token: the selected terms
    //    (renormalised weights), all E terms (plain softmax probabilities),
    //    or none (plain sigmoid scores)
    const int l16 = lane & 15;
    for (int t0 = wave * 4; t0 < T; t0 += 16) {
      const int t = t0 + (lane >> 4);
      float sum = 0.f;
      if (t < T) {
        const float* lt = s_l + t * E;
        const float lmax = lt[s_rid[t * k]];
        for (int e = l16; e < E; e += 16) {
          const bool sel = s_sel[t * E + e] >= 0;
          if (rm.sigmoid) {
            if (sel) sum += sigmoid_f(lt[e]) * expert_scale_of(rm, e);
          } else if (!rm.normalize) {
            sum += __expf(lt[e] - lmax);
          } else if (sel) {
            sum += __expf(lt[e] - lmax) * expert_scale_of(rm, e);
          }
        }
      }
      sum += dpp_f<kDppXor1>(sum);
      sum += dpp_f<kDppXor2>(sum);
      sum += dpp_f<kDppHalfMirror>(sum);
      sum += dpp_f<kDppMirror>(sum);
      if (t < T && l16 == 0) s_den[t] = (rm.sigmoid && !rm.normalize) ? 1.f : sum;
    }
    __syncthreads();
    // 4. ids and weights, one thread per route
    for (int r = tid; r < R; r += 256) {
      const int t = r / k;
      const float* lt = s_l + t * E;
      const int id = s_rid[r];
      const float sc = (rm.sigmoid ? sigmoid_f(lt[id]) : __expf(lt[id] - lt[s_rid[t * k]])) *
                       expert_scale_of(rm, id);
      const float w = sc / s_den[t] * rm.scale;
      o.ids[r] = id;
      o.wts[r] = w;
      if (o.user_ids) o.user_ids[r] = id;
      if (o.user_w) o.user_w[r] = w;
    }
  }
  if (has_shared && tid < T) o.sgate[tid] = sigmoid_f(logits[(size_t)tid * ncols + E]);

  // 5. grouping, one thread per expert
  int sel[TMAX];
  int cnt = 0;
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    sel[t] = (t < T && tid < E) ? (int)s_sel[t * E + tid] : -1;
    cnt += sel[t] >= 0 ? 1 : 0;
  }
  const int act = cnt > 0 ? 1 : 0;
  int off, aoff, total, nact;
  block_scan2(cnt, act, off, aoff, total, nact);
  if (tid < E) {
    o.counts[tid] = cnt;
    o.offsets[tid] = off;
    if (o.user_counts) o.user_counts[tid] = cnt;
    if (o.user_offsets) o.user_offsets[tid] = off;
    if (act) o.active[aoff] = tid;
    int pos = off;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (sel[t] >= 0) {
        const int r = t * k + sel[t];
        o.perm[pos] = r;
        o.pos_of_route[r] = pos;
        if (o.user_perm) o.user_perm[pos] = r;
        ++pos;
      }
    }
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
}

__device__ void route_small_body(const float* __restrict__ logits, int T, int E, int k,
                                 int ncols, RouteMode rm, int has_shared,
                                 const SmallRouteOut& o) {
  __shared__ RouteLds L;
  if (T <= 4) route_small_impl<4>(logits, T, E, k, ncols, rm, has_shared, o, L);
  else route_small_impl<kSmallMaxTokens>(logits, T, E, k, ncols, rm, has_shared, o, L);
}

// Router logits fused with the routing: workgroup e computes router row e
// (logit column e for every token), then takes a ticket.  The workgroup
// that takes the last ticket sees every column written, routes all tokens
// and sets the ticket counter back to zero for the next call.
// Publication: the logits are stored at device scope and the wave waits
// for those stores to complete before the ticket is taken; the last
// workgroup invalidates its caches (device-scope acquire) before reading
// them.  A device-scope release fence per workgroup would instead write
// back the whole L2 of its XCD, which costs far more than the GEMV.
template <typename XT, int RDT, int NC>
__global__ __launch_bounds__(256) void k_router_route(const XT* __restrict__ x,
                                                      const void* __restrict__ router,
                                                      const float* __restrict__ bias,
                                                      const void* __restrict__ shared_gate_inp,
                                                      float* __restrict__ logits, int T, int H,
                                                      int E, int k, int ncols, RouteMode rm,
                                                      int has_shared, int* __restrict__ ticket,
                                                      SmallRouteOut o) {
  if (H / (RDT ? 8 : 4) <= 256 * NC && T <= kRowTokens)
    router_row_few<XT, RDT, true, NC>(x, router, bias, shared_gate_inp, logits, T, H, E, ncols,
                                      blockIdx.x);
  else
    router_row<XT, RDT, true, NC>(x, router, bias, shared_gate_inp, logits, T, H, E, ncols,
                                  blockIdx.x);
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);  // this wave's logit stores have completed
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (int)gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (threadIdx.x == 0) __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  route_small_body(logits, T, E, k, ncols, rm, has_shared, o);
}

// Routing data read back from the workspace, clamped to the layer's ranges,
// so that the expert kernels stay in bounds whatever the workspace holds
// (for instance one whose leading counter bytes were never zeroed).
__device__ __forceinline__ int ws_group(int g, int E, bool has_shared) {
  return (g >= 0 && (g < E || (has_shared && g == E))) ? g : 0;
}
__device__ __forceinline__ void ws_span(int& base, int& count, int R) {
  base = min(max(base, 0), R);
  count = min(max(count, 0), R - base);
}
__device__ __forceinline__ int ws_route(int r, int R) { return min(max(r, 0), R - 1); }

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
  const float* residual;  // [T, H] or null, added to out (may be out)
  float* y;      // [R, H] per-route down outputs (4-bit path)
  int T, E, k, H, I, Is, rc;
  // one token routed inside the gate/up kernel: the router's logits [ncols],
  // the routing mode, and where workgroup (0, 0) writes the routing
  const float* logits;
  RouteMode rm;
  SmallRouteOut ro;
  const int4* slots;  // slot table for the down kernel (one token), or null
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
// `row` must be a row of m (callers clamp).  BRANCHLESS: lanes past the
// row's end re-read its last chunk (a line their neighbours fetch anyway)
// and keep zeros where !ok, so the loads carry no branch and a wave's loads
// issue back to back (faster for the gate/up rows; the down kernel, whose
// last chunks are mostly past the row, does better skipping them).
template <int WF, bool BRANCHLESS = false>
__device__ __forceinline__ void load_chunk(const MatStack& m, size_t row, int K, int c, bool ok,
                                           u32x4& v, float& s, float& mn) {
  const int cc = BRANCHLESS ? min(c, K / WTraits<WF>::EPC - 1) : c;
  if constexpr (BRANCHLESS) {
    const u32x4 t = ld16_stream(row_ptr<WF>(m, row, K) + (size_t)cc * 16);
    v = ok ? t : u32x4{0, 0, 0, 0};
  } else {
    v = ok ? ld16_stream(row_ptr<WF>(m, row, K) + (size_t)cc * 16) : u32x4{0, 0, 0, 0};
  }
  if constexpr (WF == WF_U4) {
    const size_t gi = row * (K / 32) + cc;
    if constexpr (BRANCHLESS) {
      const float ts = f16_to_f32(m.sc[gi]), tm = f16_to_f32(m.mn[gi]);
      s = ok ? ts : 0.f;
      mn = ok ? tm : 0.f;
    } else {
      s = ok ? f16_to_f32(m.sc[gi]) : 0.f;
      mn = ok ? f16_to_f32(m.mn[gi]) : 0.f;
    }
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

// One token, routed in the gate/up kernel: every wave ranks the router
// logits itself (route_one_token: the same result in each), so the weight
// stream waits for no routing launch.  Slot s is the s-th smallest selected
// expert, its route the expert's top-k position; slot k is the shared
// expert.
struct OneRoute {
  int id;           // lane j < k: the expert of top-k position j
  float w;          // and its routing weight
  uint64_t sel[4];  // selected experts, expert 64c + b at bit b of sel[c]
};
template <int C>
__device__ __forceinline__ void route_slot(const Dec2Params& p, int s, int& na, int& slot_g,
                                           int& route_r, OneRoute& rt) {
  const int lane = threadIdx.x & 63;
  uint64_t sel[C];
  route_one_token<C>(p.logits, p.E, p.k, p.rm, rt.id, rt.w, sel);
#pragma unroll
  for (int c = 0; c < 4; ++c) rt.sel[c] = c < C ? sel[c] : 0ull;
  na = p.k + (p.Is > 0 ? 1 : 0);
  slot_g = p.E;
  route_r = 0;
  if (s < p.k) {  // the s-th set bit of sel, on the scalar unit
    int rem = s;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      uint64_t m = sel[c];
      const int n = __popcll(m);
      if (rem >= 0 && rem < n) {
        for (int i = 0; i < rem; ++i) m &= m - 1;
        slot_g = 64 * c + __ffsll((unsigned long long)m) - 1;
      }
      rem -= n;
    }
    const uint64_t at = __ballot(lane < p.k && rt.id == slot_g);
    route_r = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)at) - 1);
  }
}

// The routing of one token for the down kernel (slot table) and the caller,
// written by one wave of the grid once its own weight loads are in flight.
__device__ __forceinline__ void route_write(const Dec2Params& p, const OneRoute& rt) {
  const int lane = threadIdx.x & 63;
  const SmallRouteOut& o = p.ro;
  const bool sh = p.Is > 0;
  const int na = p.k + (sh ? 1 : 0);
  const int id = rt.id;
  if (lane < p.k) {
    int asc = 0;  // selected experts below this lane's
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int d = id - 64 * c;
      asc += __popcll(d >= 64 ? rt.sel[c] : d <= 0 ? 0ull : rt.sel[c] & (~0ull >> (64 - d)));
    }
    o.ids[lane] = id;
    o.wts[lane] = rt.w;
    if (o.user_ids) o.user_ids[lane] = id;
    if (o.user_w) o.user_w[lane] = rt.w;
    o.active[asc] = id;
    o.perm[asc] = lane;  // route r = slot (token 0)
    o.pos_of_route[lane] = asc;
    if (o.user_perm) o.user_perm[asc] = lane;
    if (o.slots) o.slots[1 + asc] = make_int4(id, lane, __float_as_int(rt.w), 0);
  }
  const uint64_t below_lane = lanemask_lt();
  int prefix = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = 64 * c + lane;
    if (e < p.E) {
      const int cnt = (int)((rt.sel[c] >> lane) & 1ull);
      const int below = prefix + __popcll(rt.sel[c] & below_lane);
      o.counts[e] = cnt;
      o.offsets[e] = below;
      if (o.user_counts) o.user_counts[e] = cnt;
      if (o.user_offsets) o.user_offsets[e] = below;
    }
    prefix += __popcll(rt.sel[c]);
  }
  if (lane == 0) {
    o.offsets[p.E] = p.k;
    if (o.user_offsets) o.user_offsets[p.E] = p.k;
    const float sg = sh ? sigmoid_f(p.logits[p.E]) : 0.f;
    if (sh) {
      o.counts[p.E] = 1;
      o.active[p.k] = p.E;
      o.sgate[0] = sg;
    }
    *o.n_active = na;
    if (o.slots) {
      o.slots[0] = make_int4(na, 0, 0, 0);
      if (sh) o.slots[1 + p.k] = make_int4(p.E, 0, __float_as_int(sg), 0);
    }
  }
}

// gate/up: each wave owns one feature f of one touched expert: its gate row
// and its up row, full K, lane l holding chunks l, l+64, ... (U of them).
// ONE (one token, routed in this kernel: every expert has exactly one
// route): the lane's activation chunks are loaded straight into registers.
// Otherwise the activations of up to rc routes are staged in LDS as f32 per
// pass.
template <int WF, int ACT, int U, bool ONE>
__global__ __launch_bounds__(256) void k_dec_gateup3(Dec2Params p) {
  constexpr int EPC = WTraits<WF>::EPC;
  extern __shared__ float xs[];  // [rc][H] (staged path only)
  const int s = blockIdx.x;
  // The slot's expert is read together with the slot count (the active list
  // has an entry for every slot of the grid), and the first K block's weight
  // loads go out as soon as the expert is known: the route and token lookups
  // follow while they are in flight.
  int na, slot_g, route_r = 0;
  OneRoute rt;
  if constexpr (ONE) {
    if (p.E <= 128) route_slot<2>(p, s, na, slot_g, route_r, rt);
    else route_slot<4>(p, s, na, slot_g, route_r, rt);
  } else {
    na = *p.n_active;
    slot_g = p.active[s];
    // one round trip for both (and for the weight pointers), ahead of the exit test
    asm volatile("" ::"s"(na), "s"(slot_g), "s"(p.gate.p), "s"(p.up.p), "s"(p.sgate.p),
                 "s"(p.sup.p));
  }
  if (s >= na) return;
  const int R = p.T * p.k;
  const int g = ws_group(slot_g, p.E, p.Is > 0);
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
  const int fc = min(f, N - 1);  // waves past the last feature read a valid row, unused
  const size_t row = shared ? (size_t)fc : (size_t)g * N + fc;

  if constexpr (ONE) {
    int r = 0, t = 0;
    float ag = 0.f, au = 0.f;
    for (int kb = 0; kb < cpr; kb += 64 * U) {
      // all weight loads of this wave (for this K block) first
      u32x4 wg[U], wu[U];
      float sg[U], mg[U], su[U], mu[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = kb + lane + 64 * u;
        const bool ok = fok && c < cpr;
        load_chunk<WF, true>(Mg, row, p.H, c, ok, wg[u], sg[u], mg[u]);
        load_chunk<WF, true>(Mu, row, p.H, c, ok, wu[u], su[u], mu[u]);
      }
      // workgroup (0, 0) holds slot 0, a routed expert, and feature 0
      if (kb == 0 && blockIdx.x == 0 && blockIdx.y == 0 && wave == 0) route_write(p, rt);
      if (kb == 0 && !shared) {  // the expert's one route, and its token
        r = route_r;
        t = r / p.k;
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
    int count = shared ? p.T : p.counts[g];
    int base = shared ? 0 : p.offsets[g];
    if (!shared) ws_span(base, count, R);
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
          load_chunk<WF, true>(Mg, row, p.H, c, ok, wg[u], sg[u], mg[u]);
          load_chunk<WF, true>(Mu, row, p.H, c, ok, wu[u], su[u], mu[u]);
        }
        if (kb == 0) {
          // stage this pass's activations (after the weight loads are issued)
          __syncthreads();
          const int q4 = p.H / 4;
          for (int i = tid; i < nr * q4; i += 256) {
            const int r = i / q4, c4 = i - r * q4;
            const int t = shared ? (r0 + r) : (ws_route(p.perm[base + r0 + r], R) / p.k);
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
            else p.h[(size_t)ws_route(p.perm[base + r0 + r], R) * N + f] = hv;
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
// sums are added in a fixed order and written to out: no atomics.  ONE (one
// token, routed in the gate/up kernel): each slot's expert, route and weight
// come from the slot table, read with one load a lane, instead of a chain of
// dependent lookups (slot count, expert, its span, route, weight).
template <int WF, int U, bool ONE = false>
__global__ __launch_bounds__(256) void k_dec_down3(Dec2Params p) {
  constexpr int EPC = WTraits<WF>::EPC;
  constexpr int RPW = kDownRPW;
  constexpr int TMAX = ONE ? 1 : kSmallMaxTokens;
  __shared__ float part[4][TMAX][RPW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * RPW;
  const int gmax = p.E + (p.Is > 0 ? 1 : 0);
  int4 tab = make_int4(0, 0, 0, 0);
  int na;
  if constexpr (ONE) {
    if (lane < kSlotTab) tab = p.slots[lane];
    na = min(max(__builtin_amdgcn_readlane(tab.x, 0), 0), min(gmax, p.k + (p.Is > 0 ? 1 : 0)));
  }
  // ONE: each wave sums its slots in registers and stores its partials once
  // at the end, so no zeroing (and no barrier) comes first
  float osum[RPW];
#pragma unroll
  for (int q = 0; q < RPW; ++q) osum[q] = 0.f;
  if constexpr (!ONE) {
    for (int i = tid; i < 4 * TMAX * RPW; i += 256) (&part[0][0][0])[i] = 0.f;
    __syncthreads();
    na = min(*p.n_active, gmax);
  }
  const int R = p.T * p.k;
  auto slot_group = [&](int s) {
    if constexpr (ONE) return ws_group(__builtin_amdgcn_readlane(tab.x, 1 + s), p.E, p.Is > 0);
    else return ws_group(p.active[s], p.E, p.Is > 0);
  };

  u32x4 wc[RPW][U], wn[RPW][U];
  float sc[RPW][U], mc[RPW][U], sn[RPW][U], mnx[RPW][U];
  auto load_group = [&](int g, u32x4 (&w)[RPW][U], float (&sv)[RPW][U], float (&mv)[RPW][U]) {
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
        const int nc = min(n, p.H - 1);
        const size_t row = shared ? (size_t)nc : (size_t)g * p.H + nc;
        load_chunk<WF>(M, row, K, c, n < p.H && c < cpr, w[q][u], sv[q][u], mv[q][u]);
      }
    }
  };
  int s = wave;
  int g = s < na ? slot_group(s) : 0;
  if (s < na) load_group(g, wc, sc, mc);
  while (s < na) {
    const int sn_ = s + 4;
    const int gn = sn_ < na ? slot_group(sn_) : 0;
    if (sn_ < na) load_group(gn, wn, sn, mnx);
    const bool shared = (g == p.E);
    const int K = shared ? p.Is : p.I;
    const int cpr = K / EPC;
    int count = 1, base = 0;
    if constexpr (!ONE) {
      count = shared ? p.T : p.counts[g];
      base = shared ? 0 : p.offsets[g];
      if (!shared) ws_span(base, count, R);
    }
    for (int i = 0; i < count; ++i) {
      int t;
      float wgt;
      const float* hrow;
      if constexpr (ONE) {
        const int r = ws_route(__builtin_amdgcn_readlane(tab.y, 1 + s), R);
        t = 0;
        wgt = __int_as_float(__builtin_amdgcn_readlane(tab.z, 1 + s));
        hrow = shared ? p.hs : p.h + (size_t)r * K;
      } else if (shared) {
        t = i; wgt = p.sgate_val[t]; hrow = p.hs + (size_t)t * K;
      } else {
        const int r = ws_route(p.perm[base + i], R);
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
        if constexpr (ONE) osum[q] += wgt * v;
        else if (lane == 0) part[wave][t][q] += wgt * v;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < RPW; ++q) { wc[q][u] = wn[q][u]; sc[q][u] = sn[q][u]; mc[q][u] = mnx[q][u]; }
    s = sn_;
    g = gn;
  }
  if constexpr (ONE) {
    if (lane == 0) {
#pragma unroll
      for (int q = 0; q < RPW; ++q) part[wave][0][q] = osum[q];
    }
  }
  __syncthreads();
  for (int i = tid; i < p.T * RPW; i += 256) {
    const int t = i / RPW, q = i - t * RPW;
    const int n = n0 + q;
    if (n < p.H) {
      float o = part[0][t][q] + part[1][t][q] + part[2][t][q] + part[3][t][q];
      if (p.residual) o += p.residual[(size_t)t * p.H + n];
      p.out[(size_t)t * p.H + n] = o;
    }
  }
}

}  // namespace moe
