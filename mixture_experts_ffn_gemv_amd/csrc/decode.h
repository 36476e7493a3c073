// Decode path (few tokens, T <= 32): three launches per layer.
//
//   T = 1, f32 or bf16 weights:  k_router_gemv  -> k_dec_gateup3<ONE> -> k_dec_down3<ONE>
//   otherwise:                   k_router_route -> k_dec_gateup3        -> k_dec_down3
//
// k_router_gemv   router logits only (one workgroup per router row).
// k_router_route  router logits (workgroup = 4 logit columns x one K
//                 slice, every token); the last workgroup to finish then
//                 does softmax/top-k/renormalise for every token (one wave
//                 per token) and the stable expert grouping (counts,
//                 offsets, list of touched experts, routes grouped by
//                 expert).
// k_dec_gateup3   work item = (touched expert, block of 4 features).  Each
//                 wave owns 1 feature (its gate and up rows); its 64 lanes
//                 split K into 16-byte chunks and issue every weight load of
//                 those rows before touching the activations.  Only the
//                 touched experts' weights are read, each byte once.  With
//                 ONE (one token) the workgroups of column s < k take the
//                 expert at top-k position s, and each of their waves runs
//                 the first s + 1 rounds of the ranking itself to find it;
//                 one wave of column k - 1 ranks in full (route_one_token)
//                 and writes the routing (and the slot table
//                 k_dec_down3<ONE> reads) for the down kernel and the
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

// One token's routing in one wave (E <= 64*C).  Lane l holds experts l,
// l+64, ...; each of k rounds takes the wave maximum M of the order images,
// then the lowest live expert whose image is M (one ballot per logit a lane;
// taken and absent experts read as image 0 and are not live): the larger
// logit first, the lower expert among equal logits, the order of a stable
// descending sort.  The live flags stay in the lanes, so a round costs a few
// scalar operations beyond the wave maximum.  Lane j < k returns the expert
// and routing weight of top-k position j; `sel` returns the selected experts
// as bit masks (expert 64c + b at bit b of sel[c]).  Every lane must take
// part.
template <int C>
__device__ __forceinline__ void route_one_token(const float* __restrict__ l, int E, int k,
                                                RouteMode rm, int& id, float& w,
                                                uint64_t (&sel)[C]) {
  const int lane = threadIdx.x & 63;
  float lv[C];
  uint32_t ord[C];
  bool live[C];
  rank_load<C>(l, E, lv, ord, live);
  int my_e = 0;
  uint32_t my_ord = 0, top = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t M;
    const int e = rank_round<C>(ord, live, M);
    if (j == 0) top = M;
    if (lane == j) {
      my_e = e;
      my_ord = M;
    }
  }
#pragma unroll
  for (int c = 0; c < C; ++c) sel[c] = __ballot(!live[c] && lane + 64 * c < E);
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

// ---------------------------------------------------------------------------
// Router logits and routing of T <= 32 tokens in one launch.
//
// Logits: workgroup (cb, ks) computes logit columns 4cb .. 4cb+3 (column E,
// with a shared expert, is its gate vector) of every token over K slice ks.
// Its 16 waves are (group of 8 tokens) x (K part); lane l of a wave takes 4
// K elements of each 256-element piece of the slice and accumulates the
// 8 x 4 products of those elements, so each weight and activation element
// is loaded once per wave.  A reduce-scatter over the wave leaves each
// (token, column) sum in two lanes, the K parts are added through LDS in a
// fixed order, and the slice's partial logits are stored at device scope.
// The slices keep the grid near one workgroup per CU while a workgroup reads
// four weight rows and only its slice of the activations.
//
// Routing: the workgroup that takes the last ticket adds the slices in order
// (then the bias) into LDS, ranks each token with one wave
// (route_one_token), and groups the routes by expert, one thread per expert:
// its routes, in token order, are its stable block.
// ---------------------------------------------------------------------------
constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kRouteCols = 4;       // logit columns per workgroup
constexpr int kRouteTokGroup = 8;   // tokens per wave
constexpr int kRouteMaxSlices = 4;  // K slices at most
static_assert(kRouteTokGroup * kRouteCols == 32, "one reduce-scatter of 32 sums per wave");
static_assert(MOE_MAX_EXPERTS_DEV <= 4 * 64, "the grouping scan covers the first four waves");

// token groups of a workgroup for T tokens (the wave count is a multiple)
__host__ __device__ inline int route_tgroups(int T) { return T <= 8 ? 1 : T <= 16 ? 2 : 4; }

// K slices: doubled while the grid stays within one workgroup per CU and
// each wave of a slice keeps at least one 256-element piece.
inline int route_slices(int T, int H, int ncols) {
  const int ncb = (ncols + kRouteCols - 1) / kRouteCols;
  const int nkw = kRouteWaves / route_tgroups(T);
  const int pieces = (H / 4 + 63) / 64;
  int n = 1;
  while (n < kRouteMaxSlices && ncb * n * 2 <= 256 && pieces / (n * 2) >= nkw) n *= 2;
  return n;
}
// floats from one slice's partial logits to the next (16-byte aligned)
__host__ __device__ inline size_t route_slice_stride(int T, int ncols) {
  return ((size_t)T * ncols + 3) & ~(size_t)3;
}

// four consecutive elements as floats: f32 (one 16-byte load) or bf16 (8 bytes)
template <bool BF16>
__device__ __forceinline__ void ld4f(const void* p, float (&v)[4]) {
  if constexpr (BF16) {
    const u32x2 u = *reinterpret_cast<const u32x2*>(p);
    v[0] = bf16lo(u[0]); v[1] = bf16hi(u[0]); v[2] = bf16lo(u[1]); v[3] = bf16hi(u[1]);
  } else {
    const u32x4 u = ld16(p);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = __uint_as_float(u[q]);
  }
}

// Reduce-scatter of 32 values a lane over the wave: afterwards lanes 2q and
// 2q+1 hold the sum over all 64 lanes of value q.  Each level pairs lanes
// that differ in one bit (bit 5: lane ^ 32, bit 4: lane ^ 16, bit 3: mirror
// within a 16-lane row, bit 2: mirror within 8 lanes, bit 1: lane ^ 2); a
// lane keeps the half of its values picked by that bit and adds its
// partner's copy of the same half.  The last level (lane ^ 1) adds the pair.
__device__ __forceinline__ float wave_reduce_scatter32(float (&v)[32]) {
  const int lane = threadIdx.x & 63;
  {
    const bool hi = (lane & 32) != 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float send = hi ? v[i] : v[i + 16], keep = hi ? v[i + 16] : v[i];
      v[i] = keep + __shfl_xor(send, 32, 64);
    }
  }
  {
    const bool hi = (lane & 16) != 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float send = hi ? v[i] : v[i + 8], keep = hi ? v[i + 8] : v[i];
      v[i] = keep + __shfl_xor(send, 16, 64);
    }
  }
  {
    const bool hi = (lane & 8) != 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float send = hi ? v[i] : v[i + 4], keep = hi ? v[i + 4] : v[i];
      v[i] = keep + dpp_f<kDppMirror>(send);
    }
  }
  {
    const bool hi = (lane & 4) != 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float send = hi ? v[i] : v[i + 2], keep = hi ? v[i + 2] : v[i];
      v[i] = keep + dpp_f<kDppHalfMirror>(send);
    }
  }
  {
    const bool hi = (lane & 2) != 0;
    const float send = hi ? v[0] : v[1], keep = hi ? v[1] : v[0];
    v[0] = keep + dpp_f<kDppXor2>(send);
  }
  return v[0] + dpp_f<kDppXor1>(v[0]);
}

// One workgroup's partial logits (see above); part holds nks slices of
// [T][ncols] floats, sstride apart.
template <typename XT, int RDT>
__device__ __forceinline__ void route_tile(const XT* __restrict__ x, const void* __restrict__ router,
                                           const void* __restrict__ sgi, float* __restrict__ part,
                                           int nks, size_t sstride, int T, int H, int E, int ncols,
                                           int blk, float (*s_red)[32]) {
  constexpr int RB = RDT ? 2 : 4;  // router element bytes
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntg = route_tgroups(T), nkw = kRouteWaves / ntg;
  const int tg = wave % ntg, kw = wave / ntg;
  const int cb = blk / nks, ks = blk - cb * nks;
  const int nch = H >> 2;                 // 4-element chunks of a row
  const int cps = (nch + nks - 1) / nks;  // chunks of a slice
  const int c0 = ks * cps, c1 = min(c0 + cps, nch);
  const uint8_t* wr[kRouteCols];
#pragma unroll
  for (int j = 0; j < kRouteCols; ++j) {
    const int c = min(cb * kRouteCols + j, ncols - 1);
    wr[j] = c < E ? static_cast<const uint8_t*>(router) + (size_t)c * H * RB
                  : static_cast<const uint8_t*>(sgi);
  }
  const XT* xr[kRouteTokGroup];
#pragma unroll
  for (int i = 0; i < kRouteTokGroup; ++i)
    xr[i] = x + (size_t)min(tg * kRouteTokGroup + i, T - 1) * H;
  float acc[kRouteTokGroup * kRouteCols];  // [token][column]
#pragma unroll
  for (int q = 0; q < kRouteTokGroup * kRouteCols; ++q) acc[q] = 0.f;
  for (int pb = c0 + kw * 64; pb < c1; pb += nkw * 64) {
    const int ch = pb + lane;
    const bool ok = ch < c1;
    const int cc = ok ? ch : pb;  // a chunk of the slice; its products are dropped
    float w[kRouteCols][4], xv[kRouteTokGroup][4];
#pragma unroll
    for (int j = 0; j < kRouteCols; ++j) ld4f<RDT != 0>(wr[j] + (size_t)cc * 4 * RB, w[j]);
#pragma unroll
    for (int i = 0; i < kRouteTokGroup; ++i)
      ld4f<sizeof(XT) == 2>(xr[i] + (size_t)cc * 4, xv[i]);
#pragma unroll
    for (int j = 0; j < kRouteCols; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) w[j][e] = ok ? w[j][e] : 0.f;
#pragma unroll
    for (int i = 0; i < kRouteTokGroup; ++i)
#pragma unroll
      for (int j = 0; j < kRouteCols; ++j) {
        float d = acc[i * kRouteCols + j];
#pragma unroll
        for (int e = 0; e < 4; ++e) d = fmaf(xv[i][e], w[j][e], d);
        acc[i * kRouteCols + j] = d;
      }
  }
  const float v = wave_reduce_scatter32(acc);
  if ((lane & 1) == 0) s_red[wave][lane >> 1] = v;
  __syncthreads();
  if (tid < ntg * 32) {
    const int g = tid >> 5, q = tid & 31;
    const int t = g * kRouteTokGroup + (q >> 2), c = cb * kRouteCols + (q & 3);
    if (t < T && c < ncols) {
      float sm = 0.f;
      for (int kp = 0; kp < nkw; ++kp) sm += s_red[kp * ntg + g][q];
      __hip_atomic_store(part + (size_t)ks * sstride + (size_t)t * ncols + c, sm, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

struct RouteTailLds {
  float l[kSmallMaxTokens * MOE_MAX_EXPERTS_DEV];     // logits [T][E]
  int8_t pos[kSmallMaxTokens * MOE_MAX_EXPERTS_DEV];  // top-k position of a selected (t, e)
  uint32_t tok[MOE_MAX_EXPERTS_DEV];                  // bit t: token t selected expert e
  int part[4];                                        // per-wave scan totals
};

// The routing of all T tokens by the last workgroup (E <= 64 * C).
template <int C>
__device__ __forceinline__ void route_tail(const float* __restrict__ part, int nks, size_t sstride,
                                           const float* __restrict__ bias, int T, int E, int k,
                                           int ncols, RouteMode rm, int has_shared,
                                           const SmallRouteOut& o, RouteTailLds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = T * ncols;
  // 1. logits: slices added in order, then the bias; a thread takes quads of
  //    4 entries and issues all its loads before adding
  constexpr int kQuads = (kSmallMaxTokens * (MOE_MAX_EXPERTS_DEV + 1) + 4 * kRouteThreads - 1) /
                         (4 * kRouteThreads);
  u32x4 pv[kQuads][kRouteMaxSlices];
#pragma unroll
  for (int qi = 0; qi < kQuads; ++qi) {
    const int q = tid + qi * kRouteThreads;
#pragma unroll
    for (int s = 0; s < kRouteMaxSlices; ++s)
      pv[qi][s] = (4 * q < n && s < nks) ? ld16(part + s * sstride + 4 * (size_t)q) : u32x4{0, 0, 0, 0};
  }
  if (tid < E) L.tok[tid] = 0u;
#pragma unroll
  for (int qi = 0; qi < kQuads; ++qi) {
    const int q = tid + qi * kRouteThreads;
    int t = 4 * q / ncols, c = 4 * q - t * ncols;
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      if (4 * q + e4 < n) {
        float v = __uint_as_float(pv[qi][0][e4]);
#pragma unroll
        for (int s = 1; s < kRouteMaxSlices; ++s)
          if (s < nks) v += __uint_as_float(pv[qi][s][e4]);
        if (c < E) {
          if (bias) v += bias[c];
          L.l[t * E + c] = v;
        } else {
          o.sgate[t] = sigmoid_f(v);
        }
      }
      if (++c == ncols) {
        c = 0;
        ++t;
      }
    }
  }
  __syncthreads();

  // 2. top-k, weights: one wave per token
  for (int t = wave; t < T; t += kRouteWaves) {
    int id;
    float w;
    uint64_t sel[C];
    route_one_token<C>(L.l + t * E, E, k, rm, id, w, sel);
    if (lane < k) {
      const int r = t * k + lane;
      o.ids[r] = id;
      o.wts[r] = w;
      if (o.user_ids) o.user_ids[r] = id;
      if (o.user_w) o.user_w[r] = w;
      L.pos[t * E + id] = (int8_t)lane;
      atomicOr(&L.tok[id], 1u << t);
    }
  }
  __syncthreads();

  // 3. grouping, one thread per expert: counts and the active flag, packed
  //    in one word for the scan (counts stay below 2^16)
  const uint32_t tok = tid < E ? L.tok[tid] : 0u;  // bit t: token t selected this expert
  const int cnt = __popc(tok);
  const int mine = cnt | (cnt > 0 ? 1 << 16 : 0);
  int incl = 0;
  if (wave < 4) {
    incl = wave_incl_scan(mine);
    if (lane == 63) L.part[wave] = incl;
  }
  __syncthreads();
  if (tid < E) {
    int base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int pw = L.part[w];
      base += w < wave ? pw : 0;
      total += pw;
    }
    const int ex = incl + base - mine;
    const int off = ex & 0xFFFF, aoff = ex >> 16;
    o.counts[tid] = cnt;
    o.offsets[tid] = off;
    if (o.user_counts) o.user_counts[tid] = cnt;
    if (o.user_offsets) o.user_offsets[tid] = off;
    if (cnt > 0) o.active[aoff] = tid;
    int pos = off;
    for (uint32_t m = tok; m != 0u; m &= m - 1u) {
      const int t = __ffs(m) - 1;
      const int r = t * k + L.pos[t * E + tid];
      o.perm[pos] = r;
      o.pos_of_route[r] = pos;
      if (o.user_perm) o.user_perm[pos] = r;
      ++pos;
    }
    if (tid == 0) {
      const int R = T * k;
      o.offsets[E] = R;
      if (o.user_offsets) o.user_offsets[E] = R;
      int na = total >> 16;
      if (has_shared) {
        o.counts[E] = T;
        o.active[na++] = E;
      }
      *o.n_active = na;
    }
  }
}

// Publication of the partial logits: they are stored at device scope and
// each wave waits for its stores to complete before the ticket is taken;
// the last workgroup invalidates its caches (device-scope acquire) before
// reading them, and sets the counter back to zero for the next call.  A
// device-scope release fence per workgroup would instead write back the
// whole L2 of its XCD, which costs far more than the tile.
template <typename XT, int RDT>
__global__ __launch_bounds__(kRouteThreads) void k_router_route(
    const XT* __restrict__ x, const void* __restrict__ router, const float* __restrict__ bias,
    const void* __restrict__ shared_gate_inp, float* __restrict__ part, int nks, int T, int H,
    int E, int k, int ncols, RouteMode rm, int has_shared, int* __restrict__ ticket,
    SmallRouteOut o) {
  __shared__ float s_red[kRouteWaves][32];
  __shared__ RouteTailLds L;
  __shared__ int s_last;
  const size_t sstride = route_slice_stride(T, ncols);
  route_tile<XT, RDT>(x, router, shared_gate_inp, part, nks, sstride, T, H, E, ncols, blockIdx.x,
                      s_red);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores have completed
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (int)gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (threadIdx.x == 0) __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (E <= 64)
    route_tail<1>(part, nks, sstride, bias, T, E, k, ncols, rm, has_shared, o, L);
  else if (E <= 128)
    route_tail<2>(part, nks, sstride, bias, T, E, k, ncols, rm, has_shared, o, L);
  else if (E <= 192)
    route_tail<3>(part, nks, sstride, bias, T, E, k, ncols, rm, has_shared, o, L);
  else
    route_tail<4>(part, nks, sstride, bias, T, E, k, ncols, rm, has_shared, o, L);
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
// logits itself, so the weight stream waits for no routing launch.
// Workgroup column s < k takes the expert at top-k position s (its route
// s) and needs only the first s + 1 rounds of the ranking; column k is the
// shared expert (no ranking).  One wave of column k - 1, which needs all k
// rounds anyway, ranks in full (route_one_token) and writes the routing.
struct OneRoute {
  int id;           // lane j < k: the expert of top-k position j
  float w;          // and its routing weight
  uint64_t sel[4];  // selected experts, expert 64c + b at bit b of sel[c]
};
template <int C>
__device__ __forceinline__ void route_slot(const Dec2Params& p, int s, bool writer, int& na,
                                           int& slot_g, int& route_r, OneRoute& rt) {
  na = p.k + (p.Is > 0 ? 1 : 0);
  slot_g = p.E;
  route_r = 0;
  if (writer) {
    uint64_t sel[C];
    route_one_token<C>(p.logits, p.E, p.k, p.rm, rt.id, rt.w, sel);
#pragma unroll
    for (int c = 0; c < 4; ++c) rt.sel[c] = c < C ? sel[c] : 0ull;
    slot_g = __builtin_amdgcn_readlane(rt.id, s);
    route_r = s;
  } else if (s < p.k) {
    slot_g = rank_nth<C>(p.logits, p.E, s + 1);
    route_r = s;
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
  // the wave that writes the routing (column k - 1 holds a routed expert)
  const bool writer = ONE && s == p.k - 1 && blockIdx.y == 0 && threadIdx.x < 64;
  if constexpr (ONE) {
    if (p.E <= 128) route_slot<2>(p, s, writer, na, slot_g, route_r, rt);
    else route_slot<4>(p, s, writer, na, slot_g, route_r, rt);
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
      if (kb == 0 && writer) route_write(p, rt);
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
