// Host side of the MoE FFN C ABI (include/moe_ffn.h): descriptor
// validation, workspace plan, kernel selection and launches on the
// caller's stream.  The library allocates no device memory.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>
#include <type_traits>

#include "../../include/moe_ffn.h"
#include "common.h"
#include "gemm.h"
#include "gemm_big.h"
#include "gemm_dma.h"
#include "decode.h"
#include "decode_u4.h"
#include "gemv.h"
#include "norm.h"
#include "backward.h"
#include "route.h"

namespace {

using namespace moe;

thread_local std::string g_err;

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

// Largest token count that takes the GEMV (decode) path when the MFMA
// path is available.
constexpr int64_t kDecodeMaxTokens = 32;
constexpr size_t kSyncBytes = MOE_WORKSPACE_ZERO_BYTES;
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;

size_t align_up(size_t v, size_t a = 256) { return (v + a - 1) / a * a; }

struct Plan {
  int64_t T = 0, R = 0;
  int E = 0, k = 0, H = 0, I = 0, Is = 0, G = 0, ncols = 0;
  bool shared = false;
  bool mfma = false;       // prefill path (bf16 MFMA grouped GEMM)
  int ra = 2;              // direct-to-LDS GEMM: LDS slots of the weight operand
  bool small = false;      // decode path (T <= 32, GEMV kernels, one-workgroup routing)
  int rc = 0;              // decode: routes staged in LDS per pass
  int nblk = 0;            // permutation blocks
  int max_tiles = 0;       // grouped-GEMM route tiles (upper bound)
  int bt = 128;            // grouped-GEMM route-tile height
  int max_groups = 0;      // active groups (upper bound)
  int rsplit = 1;          // prefill router: K ranges (partial logits added by the top-k)
  int rks = 1;             // few-token router: K slices (partial logits added by the routing)
  // workspace offsets
  size_t o_sync, o_xn, o_logits, o_ids, o_wts, o_sgate, o_bhist, o_boff, o_counts, o_offsets, o_active,
      o_nactive, o_ntiles, o_perm, o_pos, o_rowtok, o_tgroup, o_tm0, o_h, o_hs, o_y, o_ys, o_slots;
  // 4-bit path: staged activation rows (tokens, routes), their group sums and
  // factors, and the expert work list
  size_t o_u4xs = 0, o_u4xsum = 0, o_u4xfac = 0, o_u4hs = 0, o_u4hsum = 0, o_u4hfac = 0,
      o_u4q = 0, o_u4qn = 0;
  int u4slots = 0;         // routes per work-list entry (0: the shapes do not fit)
  int u4qmax = 0;          // work-list entries (upper bound)
  size_t total = 0;
};

RouteMode route_mode(const moe_desc* d, const moe_weights* w) {
  return RouteMode{d->normalize_topk, d->gating == MOE_GATING_SIGMOID ? 1 : 0, d->routed_scale,
                   w->expert_scale};
}

int epc_of(int wf) { return wf == MOE_WEIGHTS_F32 ? 4 : (wf == MOE_WEIGHTS_BF16 ? 8 : 32); }

moe_status check_desc(const moe_desc* d) {
  if (!d) return fail(MOE_INVALID_ARGUMENT, "desc is NULL");
  if (d->hidden <= 0 || d->intermediate <= 0)
    return fail(MOE_INVALID_ARGUMENT, "hidden (%d) and intermediate (%d) must be positive",
                d->hidden, d->intermediate);
  if (d->num_experts < 1 || d->num_experts > MOE_MAX_EXPERTS)
    return fail(MOE_INVALID_ARGUMENT, "num_experts %d outside 1..%d", d->num_experts,
                MOE_MAX_EXPERTS);
  if (d->top_k < 1 || d->top_k > d->num_experts || d->top_k > MOE_MAX_TOP_K)
    return fail(MOE_INVALID_ARGUMENT, "top_k %d outside 1..min(num_experts=%d, %d)", d->top_k,
                d->num_experts, MOE_MAX_TOP_K);
  if (d->activation != MOE_ACT_SILU && d->activation != MOE_ACT_GELU_TANH)
    return fail(MOE_INVALID_ARGUMENT, "unknown activation %d", d->activation);
  if (d->weight_format < MOE_WEIGHTS_F32 || d->weight_format > MOE_WEIGHTS_U4_G32)
    return fail(MOE_INVALID_ARGUMENT, "unknown weight_format %d", d->weight_format);
  if ((d->act_dtype != MOE_F32 && d->act_dtype != MOE_BF16) ||
      (d->router_dtype != MOE_F32 && d->router_dtype != MOE_BF16))
    return fail(MOE_INVALID_ARGUMENT, "act_dtype/router_dtype must be MOE_F32 or MOE_BF16");
  if (d->normalize_topk != 0 && d->normalize_topk != 1)
    return fail(MOE_INVALID_ARGUMENT, "normalize_topk must be 0 or 1");
  if (d->gating != MOE_GATING_SOFTMAX && d->gating != MOE_GATING_SIGMOID)
    return fail(MOE_INVALID_ARGUMENT, "unknown gating %d", d->gating);
  if (!std::isfinite(d->routed_scale))
    return fail(MOE_INVALID_ARGUMENT, "routed_scale must be finite");
  if (d->pre_norm != 0 && d->pre_norm != 1)
    return fail(MOE_INVALID_ARGUMENT, "pre_norm must be 0 or 1");
  if (d->out_dtype != MOE_F32 && d->out_dtype != MOE_BF16)
    return fail(MOE_INVALID_ARGUMENT, "unknown out_dtype %d", d->out_dtype);
  if (d->out_dtype != MOE_F32)
    return fail(MOE_UNSUPPORTED, "only f32 output (out_dtype MOE_F32) is built");
  if (d->pre_norm && !(std::isfinite(d->norm_eps) && d->norm_eps > 0.f))
    return fail(MOE_INVALID_ARGUMENT, "norm_eps must be finite and positive");
  if (d->has_shared_expert != 0 && d->has_shared_expert != 1)
    return fail(MOE_INVALID_ARGUMENT, "has_shared_expert must be 0 or 1");
  if (d->has_shared_expert && d->shared_intermediate <= 0)
    return fail(MOE_INVALID_ARGUMENT, "shared_intermediate must be positive");
  if (d->has_shared_expert && d->weight_format == MOE_WEIGHTS_U4_G32)
    return fail(MOE_UNSUPPORTED, "a shared expert with 4-bit weights is not supported");
  if (d->weight_format == MOE_WEIGHTS_U4_G32 && d->group_size != 32)
    return fail(MOE_UNSUPPORTED, "4-bit weights need group_size 32 (got %d)", d->group_size);
  const int mult = 32;
  if (d->hidden % mult || d->intermediate % mult ||
      (d->has_shared_expert && d->shared_intermediate % mult))
    return fail(MOE_UNSUPPORTED, "hidden, intermediate and shared_intermediate must be multiples of %d",
                mult);
  return MOE_OK;
}

Plan make_plan(const moe_desc* d, int64_t T) {
  Plan p;
  p.T = T;
  p.E = d->num_experts;
  p.k = d->top_k;
  p.H = d->hidden;
  p.I = d->intermediate;
  p.shared = d->has_shared_expert != 0;
  p.Is = p.shared ? d->shared_intermediate : 0;
  p.R = T * p.k;
  p.G = p.E + (p.shared ? 1 : 0);
  p.ncols = p.G;
  p.mfma = d->weight_format == MOE_WEIGHTS_BF16 && d->act_dtype == MOE_BF16 &&
           d->router_dtype == MOE_BF16 && p.H % 64 == 0 && p.I % 64 == 0 &&
           (!p.shared || p.Is % 64 == 0) && T > kDecodeMaxTokens;
  p.small = !p.mfma && T <= kSmallMaxTokens &&
            std::max(p.I, p.Is) / epc_of(d->weight_format) <= 64 * 8;
  p.rc = (int)std::max<int64_t>(1, std::min<int64_t>({(int64_t)kRCMax, std::max<int64_t>(T, 1),
                                                      (int64_t)(16384 / p.H)}));
  p.nblk = (int)((p.R + kPermBlock - 1) / kPermBlock);
  // 256-route tiles (direct-to-LDS kernel) when the experts average at least
  // kDmaMinAvgRoutes routes, so that most experts fit in one route tile and
  // their weights are streamed once, and every operand's row offsets fit in
  // 32 bits
  p.bt = 128;
  if (p.mfma && p.R >= (int64_t)kDmaMinAvgRoutes * p.E) {
    const uint64_t lim = 1ull << 32;
    const uint64_t maxI = (uint64_t)std::max(p.I, p.Is);
    const bool fits = (uint64_t)T * p.H * 2 < lim && (uint64_t)p.R * maxI * 2 < lim &&
                      maxI * p.H * 2 < lim;
    if (fits) p.bt = kDmaBT;
    // Fewer routes per expert than one route tile holds: each weight byte is
    // fetched from HBM about once, and the weight operand runs two K-steps
    // ahead.  More: weights and routes both come largely from L2, and the
    // weight operand keeps the route operand's one step.
    p.ra = p.R < (int64_t)kDmaBT * p.E ? 3 : 2;
  }
  p.max_tiles = (int)((p.R + p.bt - 1) / p.bt) + p.E + (p.shared ? (int)((T + p.bt - 1) / p.bt) : 0);
  p.max_groups = (int)std::min<int64_t>(p.E, p.R) + (p.shared ? 1 : 0);
  const size_t es = p.mfma ? 2 : 4;  // h / y element size
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align_up(o + bytes); return r; };
  p.o_sync = take(kSyncBytes);  // ticket counter(s), kept at zero between calls
  p.o_xn = take(d->pre_norm ? (size_t)T * p.H * (d->act_dtype == MOE_BF16 ? 2 : 4) : 0);
  if (p.mfma) {
    // fewer router tiles than compute units: split K until there are about
    // as many workgroups (each range keeps at least 8 K steps); more tiles
    // gain nothing from it and would only give the top-k more partial rows
    const int64_t tiles = ((T + kTileT - 1) / kTileT) * ((p.E + kTileW - 1) / kTileW);
    const int nk = p.H / kTileK;
    while (tiles * p.rsplit < 256 && nk % (2 * p.rsplit) == 0 && nk / (2 * p.rsplit) >= 8)
      p.rsplit *= 2;
  }
  // few tokens routed in the router launch: partial logits of its K slices
  if (p.small) p.rks = route_slices((int)T, p.H, p.ncols);
  p.o_logits = take(std::max((size_t)p.rsplit * T * p.ncols,
                             (size_t)p.rks * route_slice_stride((int)T, p.ncols)) * 4);
  p.o_ids = take((size_t)p.R * 4);
  p.o_wts = take((size_t)p.R * 4);
  p.o_sgate = take((size_t)T * 4);
  p.o_bhist = take((size_t)p.nblk * p.E * 4);
  p.o_boff = take((size_t)p.nblk * p.E * 4);
  p.o_counts = take((size_t)p.G * 4);
  p.o_offsets = take((size_t)(p.E + 1) * 4);
  p.o_active = take((size_t)p.G * 4);
  p.o_nactive = take(4);
  p.o_ntiles = take(4);
  p.o_perm = take((size_t)p.R * 4);
  p.o_pos = take((size_t)p.R * 4);
  p.o_rowtok = take((size_t)p.R * 4);
  p.o_tgroup = take((size_t)p.max_tiles * 4);
  p.o_tm0 = take((size_t)p.max_tiles * 4);
  p.o_h = take((size_t)p.R * p.I * es);
  p.o_hs = take((size_t)T * p.Is * es);
  p.o_y = take((size_t)p.R * p.H * es);
  p.o_ys = take((size_t)(p.shared ? T : 0) * p.H * es);
  p.o_slots = take((size_t)kSlotTab * 16);
  if (d->weight_format == MOE_WEIGHTS_U4_G32) {
    const int GH = p.H / 32, GI = p.I / 32;
    // up to 4 routes a workgroup, as many as the larger row leaves LDS for
    for (int ns = 4; ns >= 1; --ns)
      if (u4_lds_bytes(p.H, kU4UGGateUp, ns) <= kU4LdsMax && u4_lds_bytes(p.I, kU4UGDown, ns) <= kU4LdsMax) {
        p.u4slots = ns;
        break;
      }
    const int ns = std::max(p.u4slots, 1);
    p.o_u4xs = take((size_t)T * GH * 128);
    p.o_u4xsum = take((size_t)T * GH * 4);
    p.o_u4xfac = take((size_t)T * 4);
    p.o_u4hs = take((size_t)p.R * GI * 128);
    p.o_u4hsum = take((size_t)p.R * GI * 4);
    p.o_u4hfac = take((size_t)p.R * 4);
    // sum over touched experts of ceil(count / ns) <= (R + (ns - 1) min(E, R)) / ns
    p.u4qmax = (int)((p.R + (ns - 1) * std::min<int64_t>(p.E, p.R) + ns - 1) / ns);
    p.o_u4q = take((size_t)p.u4qmax * 4);
    p.o_u4qn = take(4);
  }
  p.total = o;
  return p;
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

// ---------------------------------------------------------------- timing
struct TimingRec {
  const char* name;
  hipEvent_t a, b;
};
std::mutex g_tmu;
bool g_timing = false;
std::vector<TimingRec> g_pending;
std::vector<hipEvent_t> g_evpool;
std::map<std::string, std::pair<int64_t, double>> g_tsum;

hipEvent_t ev_get() {
  if (!g_evpool.empty()) {
    hipEvent_t e = g_evpool.back();
    g_evpool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  // timing-only events: without the system-scope fence an event record
  // costs no cache writeback, so the bracket stays close to the kernel
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

template <class F>
moe_status launch(const char* name, hipStream_t s, F&& f) {
  hipEvent_t a = nullptr, b = nullptr;
  if (g_timing) {
    std::lock_guard<std::mutex> lk(g_tmu);
    a = ev_get();
    b = ev_get();
    if (a) (void)hipEventRecord(a, s);
  }
  f();
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MOE_HIP_ERROR, "launch of %s failed: %s", name, hipGetErrorString(e));
  if (g_timing && a && b) {
    (void)hipEventRecord(b, s);
    std::lock_guard<std::mutex> lk(g_tmu);
    g_pending.push_back({name, a, b});
  }
  return MOE_OK;
}

#define MOE_TRY(x)                      \
  do {                                  \
    moe_status st__ = (x);              \
    if (st__ != MOE_OK) return st__;    \
  } while (0)

template <typename T>
T* wsp(void* ws, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<uint8_t*>(ws) + off);
}

// ------------------------------------------------------------ launch steps
// Calls go(XT{}, integral_constant<RDT>, integral_constant<NC>) for the
// activation type, router dtype and chunks-per-thread of a router launch.
template <class F>
void dispatch_router(bool xb, bool rb, int nc, F&& go) {
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  auto by_nc = [&](auto xt, auto rt) {
    if (nc == 1) go(xt, rt, std::integral_constant<int, 1>{});
    else if (nc == 2) go(xt, rt, std::integral_constant<int, 2>{});
    else go(xt, rt, std::integral_constant<int, 4>{});
  };
  if (xb) { if (rb) by_nc(uint16_t{}, I1{}); else by_nc(uint16_t{}, I0{}); }
  else { if (rb) by_nc(float{}, I1{}); else by_nc(float{}, I0{}); }
}
moe_status run_router(const moe_desc* d, const Plan& p, const void* x, const moe_weights* w,
                      void* ws, hipStream_t s) {
  float* logits = wsp<float>(ws, p.o_logits);
  const int T = (int)p.T;
  if (p.mfma) {
    RouterParams rp{static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w->router),
                    static_cast<const uint16_t*>(w->shared_gate_inp), w->router_bias, logits,
                    T, p.H, p.E, p.ncols, p.E, p.rsplit, (size_t)T * p.ncols};
    dim3 grid((T + kTileT - 1) / kTileT, (p.E + kTileW - 1) / kTileW, p.rsplit);
    return launch("router_mfma", s, [&] { k_router_mfma<<<grid, 256, 0, s>>>(rp); });
  }
  const bool xb = d->act_dtype == MOE_BF16, rb = d->router_dtype == MOE_BF16;
  dim3 grid(p.ncols);
  const int nc = router_nc(p.H / (rb ? 8 : 4));
  return launch("router_gemv", s, [&] {
    auto go = [&](auto xtag, auto rtag, auto nctag) {
      using XT = decltype(xtag);
      constexpr int RDT = decltype(rtag)::value, NC = decltype(nctag)::value;
      if (T == 1)
        k_router_gemv<XT, RDT, NC, 1><<<grid, 256, 0, s>>>(static_cast<const XT*>(x), w->router,
            w->router_bias, w->shared_gate_inp, logits, T, p.H, p.E, p.ncols);
      else
        k_router_gemv<XT, RDT, NC><<<grid, 256, 0, s>>>(static_cast<const XT*>(x), w->router,
            w->router_bias, w->shared_gate_inp, logits, T, p.H, p.E, p.ncols);
    };
    dispatch_router(xb, rb, nc, go);
  });
}

moe_status run_route_small(const moe_desc* d, const Plan& p, const void* x, const moe_weights* w,
                           void* ws, int32_t* user_ids, float* user_w, int32_t* user_counts,
                           int32_t* user_offsets, int32_t* user_perm, hipStream_t s) {
  const int T = (int)p.T;
  SmallRouteOut o{};
  o.ids = wsp<int32_t>(ws, p.o_ids);
  o.wts = wsp<float>(ws, p.o_wts);
  o.sgate = wsp<float>(ws, p.o_sgate);
  o.counts = wsp<int32_t>(ws, p.o_counts);
  o.offsets = wsp<int32_t>(ws, p.o_offsets);
  o.active = wsp<int32_t>(ws, p.o_active);
  o.n_active = wsp<int32_t>(ws, p.o_nactive);
  o.perm = wsp<int32_t>(ws, p.o_perm);
  o.pos_of_route = wsp<int32_t>(ws, p.o_pos);
  o.user_ids = user_ids;
  o.user_w = user_w;
  o.user_counts = user_counts;
  o.user_offsets = user_offsets;
  o.user_perm = user_perm;
  float* logits = wsp<float>(ws, p.o_logits);
  int* ticket = wsp<int>(ws, p.o_sync);
  const bool xb = d->act_dtype == MOE_BF16, rb = d->router_dtype == MOE_BF16;
  const int sh = p.shared ? 1 : 0;
  const RouteMode rm = route_mode(d, w);
  const dim3 grid((p.ncols + kRouteCols - 1) / kRouteCols * p.rks);
  return launch("router_route", s, [&] {
    auto go = [&](auto xtag, auto rtag) {
      using XT = decltype(xtag);
      constexpr int RDT = decltype(rtag)::value;
      k_router_route<XT, RDT><<<grid, kRouteThreads, 0, s>>>(static_cast<const XT*>(x),
          w->router, w->router_bias, w->shared_gate_inp, logits, p.rks, T, p.H, p.E, p.k,
          p.ncols, rm, sh, ticket, o);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    if (xb) { if (rb) go(uint16_t{}, I1{}); else go(uint16_t{}, I0{}); }
    else { if (rb) go(float{}, I1{}); else go(float{}, I0{}); }
  });
}

// x: the rows the router read; with the MFMA router the top-k kernel takes
// the shared gate's logit from them (the router computes the E expert
// columns only).
moe_status run_route_and_group(const moe_desc* d, const Plan& p, const void* x,
                               const moe_weights* w, void* ws, int32_t* user_ids,
                               float* user_w, int32_t* user_counts, int32_t* user_offsets,
                               int32_t* user_perm, hipStream_t s) {
  const int T = (int)p.T, R = (int)p.R;
  MOE_TRY(launch("topk", s, [&] {
    k_topk<<<(T + 3) / 4, 256, 0, s>>>(wsp<float>(ws, p.o_logits), p.rsplit, (size_t)T * p.ncols,
                                       T, p.E, p.k, p.ncols,
                                       route_mode(d, w), p.shared ? 1 : 0,
                                       p.mfma && p.shared ? static_cast<const uint16_t*>(x) : nullptr,
                                       static_cast<const uint16_t*>(w->shared_gate_inp), p.H,
                                       wsp<int32_t>(ws, p.o_ids), wsp<float>(ws, p.o_wts),
                                       user_ids, user_w, wsp<float>(ws, p.o_sgate));
  }));
  MOE_TRY(launch("perm_hist", s, [&] {
    k_perm_hist<<<p.nblk, 256, 0, s>>>(wsp<int32_t>(ws, p.o_ids), R, p.E, wsp<int32_t>(ws, p.o_bhist));
  }));
  ScanOut so;
  so.counts = wsp<int32_t>(ws, p.o_counts);
  so.offsets = wsp<int32_t>(ws, p.o_offsets);
  so.block_off = wsp<int32_t>(ws, p.o_boff);
  so.active = wsp<int32_t>(ws, p.o_active);
  so.n_active = wsp<int32_t>(ws, p.o_nactive);
  so.tile_group = wsp<int32_t>(ws, p.o_tgroup);
  so.tile_m0 = wsp<int32_t>(ws, p.o_tm0);
  so.n_tiles = wsp<int32_t>(ws, p.o_ntiles);
  so.user_counts = user_counts;
  so.user_offsets = user_offsets;
  MOE_TRY(launch("perm_scan", s, [&] {
    k_perm_scan<<<1, 256 * kScanParts, 0, s>>>(wsp<int32_t>(ws, p.o_bhist), p.nblk, p.E, T, p.shared ? 1 : 0,
                                  p.bt, p.mfma ? 1 : 0, so);
  }));
  return launch("perm_scatter", s, [&] {
    k_perm_scatter<<<p.nblk, 64 * kScatterWaves, 0, s>>>(wsp<int32_t>(ws, p.o_ids), R, p.E, p.k,
                                         wsp<int32_t>(ws, p.o_boff), wsp<int32_t>(ws, p.o_perm),
                                         wsp<int32_t>(ws, p.o_pos), wsp<int32_t>(ws, p.o_rowtok),
                                         user_perm);
  });
}

MatStack mat_of(const moe_desc* d, const void* dense, const moe_u4_matrix& q) {
  MatStack m{};
  if (d->weight_format == MOE_WEIGHTS_U4_G32) {
    m.p = q.codes;
    m.sc = q.scales;
    m.mn = q.mins;
  } else {
    m.p = static_cast<const uint8_t*>(dense);
  }
  return m;
}

// rows per wave for a GEMV whose rows have `cpr` 16-byte chunks: the most
// lanes per row that still leave each lane >= 8 chunks (8 lanes minimum).
int pick_rw(int cpr, bool pairs) {
  const int opts[4] = {1, 2, 4, 8};
  for (int i = pairs ? 1 : 0; i < 4; ++i) {
    const int lpr = 64 / opts[i];
    if (cpr / lpr >= 8) return opts[i];
  }
  return 8;
}

template <int WF, int ACT, typename XT>
void launch_gateup_rw(int rw, dim3 grid, hipStream_t s, const GemvGateUpParams& gp) {
  switch (rw) {
    case 2: k_dec_gateup<WF, ACT, XT, 2><<<grid, 256, 0, s>>>(gp); break;
    case 4: k_dec_gateup<WF, ACT, XT, 4><<<grid, 256, 0, s>>>(gp); break;
    default: k_dec_gateup<WF, ACT, XT, 8><<<grid, 256, 0, s>>>(gp); break;
  }
}
template <int WF, typename XT>
void launch_gateup_act(int act, int rw, dim3 grid, hipStream_t s, const GemvGateUpParams& gp) {
  if (act == MOE_ACT_SILU) launch_gateup_rw<WF, ACT_SILU, XT>(rw, grid, s, gp);
  else launch_gateup_rw<WF, ACT_GELU_TANH, XT>(rw, grid, s, gp);
}
template <int WF>
void launch_gateup_x(bool xbf16, int act, int rw, dim3 grid, hipStream_t s,
                     const GemvGateUpParams& gp) {
  if (xbf16) launch_gateup_act<WF, uint16_t>(act, rw, grid, s, gp);
  else launch_gateup_act<WF, float>(act, rw, grid, s, gp);
}
template <int WF>
void launch_down_rw(int rw, dim3 grid, hipStream_t s, const GemvDownParams& dp) {
  switch (rw) {
    case 1: k_dec_down<WF, 1><<<grid, 256, 0, s>>>(dp); break;
    case 2: k_dec_down<WF, 2><<<grid, 256, 0, s>>>(dp); break;
    case 4: k_dec_down<WF, 4><<<grid, 256, 0, s>>>(dp); break;
    default: k_dec_down<WF, 8><<<grid, 256, 0, s>>>(dp); break;
  }
}

moe_status run_experts_gemv(const moe_desc* d, const Plan& p, const void* x,
                            const moe_weights* w, float* out, const float* residual, void* ws,
                            hipStream_t s) {
  const int wf = d->weight_format;
  const int epc = epc_of(wf);
  GroupInfo gi;
  gi.counts = wsp<int32_t>(ws, p.o_counts);
  gi.offsets = wsp<int32_t>(ws, p.o_offsets);
  gi.active = wsp<int32_t>(ws, p.o_active);
  gi.n_active = wsp<int32_t>(ws, p.o_nactive);
  gi.row_token = wsp<int32_t>(ws, p.o_rowtok);
  gi.E = p.E;
  gi.T = (int)p.T;

  GemvGateUpParams gp;
  gp.gate = mat_of(d, w->gate, w->gate_u4);
  gp.up = mat_of(d, w->up, w->up_u4);
  gp.sgate = MatStack{static_cast<const uint8_t*>(w->shared_gate), nullptr, nullptr};
  gp.sup = MatStack{static_cast<const uint8_t*>(w->shared_up), nullptr, nullptr};
  gp.x = x;
  gp.h = wsp<float>(ws, p.o_h);
  gp.hs = wsp<float>(ws, p.o_hs);
  gp.gi = gi;
  gp.H = p.H;
  gp.I = p.I;
  gp.Is = p.Is;
  const int rw_gu = pick_rw(p.H / epc, true);
  const int maxN = std::max(p.I, p.Is);
  dim3 g1(p.max_groups, (maxN + kGemvWaves * (rw_gu / 2) - 1) / (kGemvWaves * (rw_gu / 2)));
  const bool xb = d->act_dtype == MOE_BF16;
  MOE_TRY(launch("gemv_gateup", s, [&] {
    if (wf == MOE_WEIGHTS_F32) launch_gateup_x<WF_F32>(xb, d->activation, rw_gu, g1, s, gp);
    else if (wf == MOE_WEIGHTS_BF16) launch_gateup_x<WF_BF16>(xb, d->activation, rw_gu, g1, s, gp);
    else launch_gateup_x<WF_U4>(xb, d->activation, rw_gu, g1, s, gp);
  }));

  GemvDownParams dp;
  dp.down = mat_of(d, w->down, w->down_u4);
  dp.sdown = MatStack{static_cast<const uint8_t*>(w->shared_down), nullptr, nullptr};
  dp.h = gp.h;
  dp.hs = gp.hs;
  dp.y = wsp<float>(ws, p.o_y);
  dp.ys = wsp<float>(ws, p.o_ys);
  dp.gi = gi;
  dp.H = p.H;
  dp.I = p.I;
  dp.Is = p.Is;
  const int minK = p.shared ? std::min(p.I, p.Is) : p.I;
  const int rw_d = pick_rw(minK / epc, false);
  dim3 g2(p.max_groups, (p.H + kGemvWaves * rw_d - 1) / (kGemvWaves * rw_d));
  MOE_TRY(launch("gemv_down", s, [&] {
    if (wf == MOE_WEIGHTS_F32) launch_down_rw<WF_F32>(rw_d, g2, s, dp);
    else if (wf == MOE_WEIGHTS_BF16) launch_down_rw<WF_BF16>(rw_d, g2, s, dp);
    else launch_down_rw<WF_U4>(rw_d, g2, s, dp);
  }));

  const size_t nthr = (size_t)p.T * (p.H / 4);
  return launch("combine", s, [&] {
    k_combine<float><<<(unsigned)((nthr + 255) / 256), 256, 0, s>>>(
        dp.y, dp.ys, wsp<float>(ws, p.o_wts), wsp<int32_t>(ws, p.o_pos), wsp<float>(ws, p.o_sgate),
        out, residual, (int)p.T, p.H, p.k, p.shared ? 1 : 0);
  });
}

// chunks per lane per K block for the decode GEMVs: the smallest supported
// count covering a row of `cpr` 16-byte chunks, at most 8
int pick_u(int cpr) {
  const int need = (cpr + 63) / 64;
  const int opts[6] = {1, 2, 3, 4, 6, 8};
  for (int o : opts)
    if (o >= need) return o;
  return 8;
}

template <int WF, int ACT, bool ONE>
void launch_gu3_u(int u, dim3 grid, size_t lds, hipStream_t s, const Dec2Params& dp) {
  switch (u) {
    case 1: k_dec_gateup3<WF, ACT, 1, ONE><<<grid, 256, lds, s>>>(dp); break;
    case 2: k_dec_gateup3<WF, ACT, 2, ONE><<<grid, 256, lds, s>>>(dp); break;
    case 3: k_dec_gateup3<WF, ACT, 3, ONE><<<grid, 256, lds, s>>>(dp); break;
    case 4: k_dec_gateup3<WF, ACT, 4, ONE><<<grid, 256, lds, s>>>(dp); break;
    case 6: k_dec_gateup3<WF, ACT, 6, ONE><<<grid, 256, lds, s>>>(dp); break;
    default: k_dec_gateup3<WF, ACT, 8, ONE><<<grid, 256, lds, s>>>(dp); break;
  }
}
// one: one token, ranked in the kernel (no LDS); else the routes' activations staged
template <int WF, int ACT>
void launch_gu3(bool one, int u, dim3 grid, size_t lds, hipStream_t s, const Dec2Params& dp) {
  if (one) launch_gu3_u<WF, ACT, true>(u, grid, 0, s, dp);
  else launch_gu3_u<WF, ACT, false>(u, grid, lds, s, dp);
}
template <int WF, bool ONE>
void launch_dn3_u(int u, dim3 grid, hipStream_t s, const Dec2Params& dp) {
  switch (u) {
    case 1: k_dec_down3<WF, 1, ONE><<<grid, 256, 0, s>>>(dp); break;
    case 2: k_dec_down3<WF, 2, ONE><<<grid, 256, 0, s>>>(dp); break;
    case 3: k_dec_down3<WF, 3, ONE><<<grid, 256, 0, s>>>(dp); break;
    case 4: k_dec_down3<WF, 4, ONE><<<grid, 256, 0, s>>>(dp); break;
    case 6: k_dec_down3<WF, 6, ONE><<<grid, 256, 0, s>>>(dp); break;
    default: k_dec_down3<WF, 8, ONE><<<grid, 256, 0, s>>>(dp); break;
  }
}
// one: one token whose routing the gate/up kernel wrote as a slot table
template <int WF>
void launch_dn3(bool one, int u, dim3 grid, hipStream_t s, const Dec2Params& dp) {
  if (one) launch_dn3_u<WF, true>(u, grid, s, dp);
  else launch_dn3_u<WF, false>(u, grid, s, dp);
}

// Raises a kernel's dynamic-LDS limit to the full 160 KB, once per device
// and kernel (launches then need no attribute call).
std::mutex g_lds_mu;
std::map<std::pair<int, const void*>, bool> g_lds_set;
moe_status allow_full_lds(const void* kern, const char* name) {
  int dev = 0;
  (void)hipGetDevice(&dev);
  std::lock_guard<std::mutex> lk(g_lds_mu);
  auto key = std::make_pair(dev, kern);
  if (g_lds_set.count(key)) return MOE_OK;
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     kU4LdsMax);
  if (e != hipSuccess)
    return fail(MOE_HIP_ERROR, "allowing %d bytes of LDS for %s failed: %s", kU4LdsMax, name,
                hipGetErrorString(e));
  g_lds_set[key] = true;
  return MOE_OK;
}

// One expert kernel of the 4-bit path: the vector-scale form when the row's
// group count allows it.
template <int MODE, int ACT, int UG, int PW>
moe_status launch_u4_experts(const char* name, int qmax, hipStream_t s, const U4Experts& ep) {
  const int K = MODE == 0 ? ep.d.H : ep.d.I, N = MODE == 0 ? ep.d.I : ep.d.H;
  const int rows = kU4Waves * PW * (MODE == 0 ? 4 : 8);
  const dim3 grid(qmax, (N + rows - 1) / rows);
  const size_t lds = (size_t)u4_lds_bytes(K, UG, ep.nslot);
  auto go = [&](auto kern) -> moe_status {
    MOE_TRY(allow_full_lds(reinterpret_cast<const void*>(kern), name));
    return launch(name, s, [&] { kern<<<grid, kU4Threads, lds, s>>>(ep); });
  };
  if ((K / 32) % (4 * UG) == 0) return go(k_u4_mfma<MODE, ACT, UG, PW, true>);
  return go(k_u4_mfma<MODE, ACT, UG, PW, false>);
}

// 4-bit weights: the tokens' rows staged (with the expert work list), gate/up
// on the MFMA, the routes' h rows staged, down, then the weighted combine.
moe_status run_experts_u4(const moe_desc* d, const Plan& p, Dec2Params dp, float* out,
                          const float* residual, void* ws, hipStream_t s) {
  dp.y = wsp<float>(ws, p.o_y);
  U4Stage sx{};
  sx.src = dp.x;
  sx.src_bf16 = dp.x_bf16;
  sx.K = p.H;
  sx.rows = (int)p.T;
  sx.stage = wsp<uint8_t>(ws, p.o_u4xs);
  sx.gsum = wsp<float>(ws, p.o_u4xsum);
  sx.fac = wsp<float>(ws, p.o_u4xfac);
  sx.counts = dp.counts;
  sx.active = dp.active;
  sx.n_active = dp.n_active;
  sx.qlist = wsp<int32_t>(ws, p.o_u4q);
  sx.qn = wsp<int32_t>(ws, p.o_u4qn);
  sx.E = p.E;
  sx.qmax = p.u4qmax;
  sx.nslot = p.u4slots;
  MOE_TRY(launch("stage_x", s, [&] {
    k_u4_stage<<<(unsigned)p.T + 1, kU4StageThreads, 0, s>>>(sx);
  }));
  U4Experts ep{};
  ep.d = dp;
  ep.stage = sx.stage;
  ep.gsum = sx.gsum;
  ep.fac = sx.fac;
  ep.qlist = sx.qlist;
  ep.qn = sx.qn;
  ep.nslot = p.u4slots;
  if (d->activation == MOE_ACT_SILU)
    MOE_TRY((launch_u4_experts<0, ACT_SILU, kU4UGGateUp, kU4PWGateUp>("gemv_gateup", p.u4qmax, s, ep)));
  else
    MOE_TRY((launch_u4_experts<0, ACT_GELU_TANH, kU4UGGateUp, kU4PWGateUp>("gemv_gateup", p.u4qmax, s, ep)));

  U4Stage sh{};
  sh.src = dp.h;
  sh.K = p.I;
  sh.rows = (int)p.R;
  sh.stage = wsp<uint8_t>(ws, p.o_u4hs);
  sh.gsum = wsp<float>(ws, p.o_u4hsum);
  sh.fac = wsp<float>(ws, p.o_u4hfac);
  MOE_TRY(launch("stage_h", s, [&] {
    k_u4_stage<<<(unsigned)p.R, kU4StageThreads, 0, s>>>(sh);
  }));
  U4Experts ed = ep;
  ed.stage = sh.stage;
  ed.gsum = sh.gsum;
  ed.fac = sh.fac;
  MOE_TRY((launch_u4_experts<1, 0, kU4UGDown, kU4PWDown>("gemv_down", p.u4qmax, s, ed)));
  const size_t nthr = (size_t)p.T * (p.H / 4);
  return launch("combine", s, [&] {
    k_combine<float><<<(unsigned)((nthr + 255) / 256), 256, 0, s>>>(
        dp.y, nullptr, dp.wts, wsp<int32_t>(ws, p.o_pos), dp.sgate_val, out, residual, (int)p.T,
        p.H, p.k, 0);
  });
}

// route: one token with f32/bf16 weights, routed inside the gate/up kernel
// from the logits the router GEMV left in the workspace (user_ids/user_w:
// the caller's routing outputs, or null)
moe_status run_experts_small(const moe_desc* d, const Plan& p, const void* x,
                             const moe_weights* w, float* out, const float* residual, void* ws,
                             hipStream_t s, bool route = false, int32_t* user_ids = nullptr,
                             float* user_w = nullptr) {
  const int wf = d->weight_format;
  const int epc = epc_of(wf);
  Dec2Params dp;
  dp.gate = mat_of(d, w->gate, w->gate_u4);
  dp.up = mat_of(d, w->up, w->up_u4);
  dp.down = mat_of(d, w->down, w->down_u4);
  dp.sgate = MatStack{static_cast<const uint8_t*>(w->shared_gate), nullptr, nullptr};
  dp.sup = MatStack{static_cast<const uint8_t*>(w->shared_up), nullptr, nullptr};
  dp.sdown = MatStack{static_cast<const uint8_t*>(w->shared_down), nullptr, nullptr};
  dp.x = x;
  dp.x_bf16 = d->act_dtype == MOE_BF16 ? 1 : 0;
  dp.h = wsp<float>(ws, p.o_h);
  dp.hs = wsp<float>(ws, p.o_hs);
  dp.counts = wsp<int32_t>(ws, p.o_counts);
  dp.offsets = wsp<int32_t>(ws, p.o_offsets);
  dp.active = wsp<int32_t>(ws, p.o_active);
  dp.n_active = wsp<int32_t>(ws, p.o_nactive);
  dp.perm = wsp<int32_t>(ws, p.o_perm);
  dp.wts = wsp<float>(ws, p.o_wts);
  dp.sgate_val = wsp<float>(ws, p.o_sgate);
  dp.out = out;
  dp.residual = residual;
  dp.T = (int)p.T; dp.E = p.E; dp.k = p.k; dp.H = p.H; dp.I = p.I; dp.Is = p.Is; dp.rc = p.rc;
  dp.logits = wsp<float>(ws, p.o_logits);
  dp.rm = route_mode(d, w);
  dp.ro = SmallRouteOut{wsp<int32_t>(ws, p.o_ids), wsp<float>(ws, p.o_wts),
                        wsp<float>(ws, p.o_sgate), wsp<int32_t>(ws, p.o_counts),
                        wsp<int32_t>(ws, p.o_offsets), wsp<int32_t>(ws, p.o_active),
                        wsp<int32_t>(ws, p.o_nactive), wsp<int32_t>(ws, p.o_perm),
                        wsp<int32_t>(ws, p.o_pos), user_ids, user_w, nullptr, nullptr, nullptr,
                        route ? wsp<int4>(ws, p.o_slots) : nullptr};
  dp.slots = dp.ro.slots;

  if (wf == MOE_WEIGHTS_U4_G32) return run_experts_u4(d, p, dp, out, residual, ws, s);

  const int u1 = pick_u(p.H / epc);
  const int maxN = std::max(p.I, p.Is);
  dim3 g1(p.max_groups, (maxN + kGUWaves - 1) / kGUWaves);
  const size_t lds = (size_t)p.rc * p.H * 4;
  MOE_TRY(launch("gemv_gateup", s, [&] {
    const bool silu = d->activation == MOE_ACT_SILU;
    if (wf == MOE_WEIGHTS_F32) {
      if (silu) launch_gu3<WF_F32, ACT_SILU>(route, u1, g1, lds, s, dp);
      else launch_gu3<WF_F32, ACT_GELU_TANH>(route, u1, g1, lds, s, dp);
    } else {
      if (silu) launch_gu3<WF_BF16, ACT_SILU>(route, u1, g1, lds, s, dp);
      else launch_gu3<WF_BF16, ACT_GELU_TANH>(route, u1, g1, lds, s, dp);
    }
  }));
  const int maxK = std::max(p.I, p.Is);
  const int u2 = pick_u(maxK / epc);
  dim3 g2((p.H + kDownRPW - 1) / kDownRPW);
  return launch("gemv_down_combine", s, [&] {
    if (wf == MOE_WEIGHTS_F32) launch_dn3<WF_F32>(route, u2, g2, s, dp);
    else launch_dn3<WF_BF16>(route, u2, g2, s, dp);
  });
}

moe_status run_experts_mfma(const moe_desc* d, const Plan& p, const void* x,
                            const moe_weights* w, float* out, const float* residual, void* ws,
                            hipStream_t s) {
  GemmParams g{};
  g.counts = wsp<int32_t>(ws, p.o_counts);
  g.offsets = wsp<int32_t>(ws, p.o_offsets);
  g.row_token = wsp<int32_t>(ws, p.o_rowtok);
  g.tile_group = wsp<int32_t>(ws, p.o_tgroup);
  g.tile_m0 = wsp<int32_t>(ws, p.o_tm0);
  g.n_tiles = wsp<int32_t>(ws, p.o_ntiles);
  g.E = p.E; g.T = (int)p.T; g.H = p.H; g.I = p.I; g.Is = p.Is;

  GemmParams gu = g;
  gu.w0 = static_cast<const uint16_t*>(w->gate);
  gu.w1 = static_cast<const uint16_t*>(w->up);
  gu.sw0 = static_cast<const uint16_t*>(w->shared_gate);
  gu.sw1 = static_cast<const uint16_t*>(w->shared_up);
  gu.act = static_cast<const uint16_t*>(x);
  gu.out = wsp<uint16_t>(ws, p.o_h);
  gu.sout = wsp<uint16_t>(ws, p.o_hs);
  if (p.bt == kDmaBT && w->gate_up_packed) {
    gu.pk = static_cast<const uint8_t*>(w->gate_up_packed);
    gu.spk = static_cast<const uint8_t*>(w->shared_gate_up_packed);
  }
  const int maxN = std::max(p.I, p.Is);
  // The kernels deal the existing tiles to the XCDs in 8 equal ranges of
  // ceil(n / 8) workgroup slots each, so the grid needs a whole multiple of
  // 8 columns: max_tiles columns alone leave the last ranges short whenever
  // max_tiles * rows < 8 * ceil(n / 8), and those tiles would never run.
  const int gx = (p.max_tiles + 7) / 8 * 8;
  dim3 g1(gx, (maxN + kBW / 2 - 1) / (kBW / 2));
  MOE_TRY(launch("gemm_gateup", s, [&] {
    const bool silu = d->activation == MOE_ACT_SILU;
    if (p.bt == kDmaBT && p.ra == 3) {
      if (silu) k_gemm_dma<GM_GATEUP, ACT_SILU, kDmaBK, 3><<<g1, kDmaThreads, 0, s>>>(gu);
      else k_gemm_dma<GM_GATEUP, ACT_GELU_TANH, kDmaBK, 3><<<g1, kDmaThreads, 0, s>>>(gu);
    } else if (p.bt == kDmaBT) {
      if (silu) k_gemm_dma<GM_GATEUP, ACT_SILU, kDmaBK, 2><<<g1, kDmaThreads, 0, s>>>(gu);
      else k_gemm_dma<GM_GATEUP, ACT_GELU_TANH, kDmaBK, 2><<<g1, kDmaThreads, 0, s>>>(gu);
    } else {
      if (silu) k_gemm_big<GM_GATEUP, ACT_SILU, 128><<<g1, 256, 0, s>>>(gu);
      else k_gemm_big<GM_GATEUP, ACT_GELU_TANH, 128><<<g1, 256, 0, s>>>(gu);
    }
  }));

  GemmParams gd = g;
  gd.w0 = static_cast<const uint16_t*>(w->down);
  gd.sw0 = static_cast<const uint16_t*>(w->shared_down);
  gd.act = wsp<uint16_t>(ws, p.o_h);
  gd.sact = wsp<uint16_t>(ws, p.o_hs);
  gd.out = wsp<uint16_t>(ws, p.o_y);
  gd.sout = wsp<uint16_t>(ws, p.o_ys);
  if (p.bt == kDmaBT && w->down_packed) {
    gd.pk = static_cast<const uint8_t*>(w->down_packed);
    gd.spk = static_cast<const uint8_t*>(w->shared_down_packed);
  }
  dim3 g2(gx, (p.H + kBW - 1) / kBW);
  MOE_TRY(launch("gemm_down", s, [&] {
    if (p.bt == kDmaBT && p.ra == 3) k_gemm_dma<GM_DOWN, 0, kDmaBK, 3><<<g2, kDmaThreads, 0, s>>>(gd);
    else if (p.bt == kDmaBT) k_gemm_dma<GM_DOWN, 0, kDmaBK, 2><<<g2, kDmaThreads, 0, s>>>(gd);
    else k_gemm_big<GM_DOWN, 0, 128><<<g2, 256, 0, s>>>(gd);
  }));

  const size_t nthr = (size_t)p.T * (p.H / 8);
  return launch("combine", s, [&] {
    k_combine_bf16x8<<<(unsigned)((nthr + 255) / 256), 256, 0, s>>>(
        wsp<uint16_t>(ws, p.o_y), wsp<uint16_t>(ws, p.o_ys), wsp<float>(ws, p.o_wts),
        wsp<int32_t>(ws, p.o_pos), wsp<float>(ws, p.o_sgate), out, residual, (int)p.T, p.H, p.k,
        p.shared ? 1 : 0);
  });
}

// The layer's input: x, or its RMSNorm rows written to the workspace first.
moe_status layer_input(const moe_desc* d, const Plan& p, const void* x, const moe_weights* w,
                       void* ws, hipStream_t s, const void** xin) {
  *xin = x;
  if (!d->pre_norm) return MOE_OK;
  void* xn = static_cast<uint8_t*>(ws) + p.o_xn;
  *xin = xn;
  return launch("rmsnorm", s, [&] {
    if (d->act_dtype == MOE_BF16)
      k_rmsnorm<uint16_t><<<(unsigned)p.T, 256, 0, s>>>(static_cast<const uint16_t*>(x),
          w->norm_weight, d->norm_eps, p.H, static_cast<uint16_t*>(xn));
    else
      k_rmsnorm<float><<<(unsigned)p.T, 256, 0, s>>>(static_cast<const float*>(x),
          w->norm_weight, d->norm_eps, p.H, static_cast<float*>(xn));
  });
}

// Sizes of the packed weight arrays (the direct-to-LDS GEMM's layout).
struct PackSizes {
  size_t gu = 0, dn = 0, sgu = 0, sdn = 0;
};

moe_status pack_sizes(const moe_desc* d, PackSizes* o) {
  MOE_TRY(check_desc(d));
  if (d->weight_format != MOE_WEIGHTS_BF16)
    return fail(MOE_UNSUPPORTED, "packed weights exist for bf16 weights only");
  const int H = d->hidden, I = d->intermediate;
  const int Is = d->has_shared_expert ? d->shared_intermediate : 0;
  if (H % kDmaBK || I % kDmaBK || Is % kDmaBK)
    return fail(MOE_UNSUPPORTED, "packed weights need hidden and intermediate sizes that are "
                "multiples of %d", kDmaBK);
  auto gu = [&](int n) { return (size_t)((n + 127) / 128) * (H / kDmaBK) * kPackBlock; };
  auto dn = [&](int n) { return (size_t)((H + kPackRows - 1) / kPackRows) * (n / kDmaBK) * kPackBlock; };
  const int n = std::max(I, Is);
  if (gu(n) > UINT32_MAX || dn(n) > UINT32_MAX)
    return fail(MOE_UNSUPPORTED, "one expert's packed weights exceed 4 GiB");
  o->gu = (size_t)d->num_experts * gu(I);
  o->dn = (size_t)d->num_experts * dn(I);
  if (Is) {
    o->sgu = gu(Is);
    o->sdn = dn(Is);
  }
  return MOE_OK;
}

moe_status check_packed(const moe_desc* d, const moe_weights* w) {
  const void* pp[4] = {w->gate_up_packed, w->down_packed, w->shared_gate_up_packed,
                       w->shared_down_packed};
  if (!pp[0] && !pp[1] && !pp[2] && !pp[3]) return MOE_OK;
  PackSizes ps;
  MOE_TRY(pack_sizes(d, &ps));
  for (const void* q : pp)
    if (!aligned16(q)) return fail(MOE_UNSUPPORTED, "packed weights must be 16-byte aligned");
  if (d->has_shared_expert && ((!pp[0] != !pp[2]) || (!pp[1] != !pp[3])))
    return fail(MOE_INVALID_ARGUMENT, "routed and shared packed weights go together");
  if (!d->has_shared_expert && (pp[2] || pp[3]))
    return fail(MOE_INVALID_ARGUMENT, "shared packed weights given without a shared expert");
  return MOE_OK;
}

// own_scratch: the call runs on the library's static scratch (ws is not
// checked; the plan must fit kScratchBytes instead).
moe_status check_common(const moe_desc* d, int64_t T, const void* x, const moe_weights* w,
                        void* ws, size_t ws_bytes, bool full, Plan* plan,
                        bool own_scratch = false) {
  MOE_TRY(check_desc(d));
  if (T < 0) return fail(MOE_INVALID_ARGUMENT, "num_tokens %lld is negative", (long long)T);
  if (T * d->top_k > INT32_MAX || T > INT32_MAX / 4)
    return fail(MOE_UNSUPPORTED, "num_tokens %lld too large", (long long)T);
  if (!w) return fail(MOE_INVALID_ARGUMENT, "weights is NULL");
  *plan = make_plan(d, T);
  if (T == 0) return MOE_OK;
  if (!x) return fail(MOE_INVALID_ARGUMENT, "x is NULL");
  if (!w->router) return fail(MOE_INVALID_ARGUMENT, "weights->router is NULL");
  if (d->has_shared_expert && !w->shared_gate_inp)
    return fail(MOE_INVALID_ARGUMENT, "weights->shared_gate_inp is NULL");
  if (full) {
    if (d->weight_format == MOE_WEIGHTS_U4_G32) {
      const moe_u4_matrix* ms[3] = {&w->gate_u4, &w->up_u4, &w->down_u4};
      for (const moe_u4_matrix* m : ms) {
        if (!m->codes || !m->scales || !m->mins)
          return fail(MOE_INVALID_ARGUMENT, "a 4-bit weight pointer is NULL");
        if (!aligned16(m->codes)) return fail(MOE_UNSUPPORTED, "4-bit codes must be 16-byte aligned");
      }
      if (plan->u4slots < 1)
        return fail(MOE_UNSUPPORTED, "hidden %d / intermediate %d: a 4-bit workgroup stages one "
                    "activation row in at most %d bytes of LDS", d->hidden, d->intermediate,
                    kU4LdsMax);
    } else {
      if (!w->gate || !w->up || !w->down)
        return fail(MOE_INVALID_ARGUMENT, "gate/up/down weight pointer is NULL");
      if (!aligned16(w->gate) || !aligned16(w->up) || !aligned16(w->down))
        return fail(MOE_UNSUPPORTED, "expert weights must be 16-byte aligned");
    }
    if (d->has_shared_expert) {
      if (!w->shared_gate || !w->shared_up || !w->shared_down)
        return fail(MOE_INVALID_ARGUMENT, "shared expert weight pointer is NULL");
      if (!aligned16(w->shared_gate) || !aligned16(w->shared_up) || !aligned16(w->shared_down))
        return fail(MOE_UNSUPPORTED, "shared expert weights must be 16-byte aligned");
    }
  }
  if (full) MOE_TRY(check_packed(d, w));
  if (d->pre_norm && (!w->norm_weight || !aligned16(w->norm_weight)))
    return fail(w->norm_weight ? MOE_UNSUPPORTED : MOE_INVALID_ARGUMENT,
                "pre_norm needs weights->norm_weight, 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(w->expert_scale) & 3u)
    return fail(MOE_UNSUPPORTED, "expert_scale must be 4-byte aligned");
  if (!aligned16(x) || !aligned16(w->router) ||
      (d->has_shared_expert && !aligned16(w->shared_gate_inp)))
    return fail(MOE_UNSUPPORTED, "x, router and shared_gate_inp must be 16-byte aligned");
  if (!plan->mfma && d->hidden > 16384)
    return fail(MOE_UNSUPPORTED, "hidden %d > 16384 needs bf16 weights and activations and more "
                "than %d tokens", d->hidden, (int)kDecodeMaxTokens);
  if (own_scratch) {
    if (plan->total > kScratchBytes)
      return fail(MOE_UNSUPPORTED, "%lld tokens need %zu bytes of scratch; the library's static "
                  "scratch holds %zu (call moe_ffn_forward with a workspace instead)",
                  (long long)T, plan->total, kScratchBytes);
    return MOE_OK;
  }
  if (!ws) return fail(MOE_INVALID_ARGUMENT, "workspace is NULL");
  if (!aligned16(ws)) return fail(MOE_UNSUPPORTED, "workspace must be 16-byte aligned");
  if (ws_bytes < plan->total)
    return fail(MOE_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", ws_bytes, plan->total);
  return MOE_OK;
}

// The whole layer once the arguments have passed check_common.
moe_status forward_body(const moe_desc* desc, const Plan& p, int64_t num_tokens, const void* x,
                        const moe_weights* weights, float* out, const float* residual,
                        int32_t* topk_ids_out, float* topk_w_out, void* ws, hipStream_t s) {
  MOE_TRY(layer_input(desc, p, x, weights, ws, s, &x));
  if (p.small) {
    if (num_tokens == 1 && desc->weight_format != MOE_WEIGHTS_U4_G32) {
      // one token: the router kernel writes only the logits; the gate/up
      // kernel ranks them itself and writes the routing (no routing tail)
      MOE_TRY(run_router(desc, p, x, weights, ws, s));
      return run_experts_small(desc, p, x, weights, out, residual, ws, s, true, topk_ids_out,
                               topk_w_out);
    }
    MOE_TRY(run_route_small(desc, p, x, weights, ws, topk_ids_out, topk_w_out, nullptr, nullptr,
                            nullptr, s));
    return run_experts_small(desc, p, x, weights, out, residual, ws, s);
  }
  MOE_TRY(run_router(desc, p, x, weights, ws, s));
  MOE_TRY(run_route_and_group(desc, p, x, weights, ws, topk_ids_out, topk_w_out, nullptr, nullptr,
                              nullptr, s));
  if (p.mfma) return run_experts_mfma(desc, p, x, weights, out, residual, ws, s);
  return run_experts_gemv(desc, p, x, weights, out, residual, ws, s);
}

// ------------------------------------------------- library-owned scratch
// moe_ffn_forward_noalloc runs on this array instead of a caller workspace.
// Host code never uses its name as an address: each device's copy is found
// with hipGetSymbolAddress once, with that device current, and that
// pointer is what kernels and fills receive.
__global__ void k_zero_words(uint32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
bool g_scratch_zeroed[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

// The current device's scratch.  Its leading MOE_WORKSPACE_ZERO_BYTES (the
// routing ticket) must be zero before its first use: until a call made
// outside graph capture has zeroed them, each call first enqueues a small
// fill kernel on its stream (under capture that kernel becomes part of the
// graph, so every replay starts from zero too).
moe_status scratch_for_device(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_HIP_ERROR, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_UNSUPPORTED, "device %d: at most %d devices have library scratch", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* q = nullptr;
    e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !q)
      return fail(MOE_HIP_ERROR, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = q;
  }
  if (!g_scratch_zeroed[dev]) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(s, &cs);
    if (e != hipSuccess)
      return fail(MOE_HIP_ERROR, "hipStreamIsCapturing failed: %s", hipGetErrorString(e));
    MOE_TRY(launch("zero_scratch_counters", s, [&] {
      k_zero_words<<<1, 64, 0, s>>>(static_cast<uint32_t*>(g_scratch_ptr[dev]),
                                    MOE_WORKSPACE_ZERO_BYTES / 4);
    }));
    if (cs == hipStreamCaptureStatusNone) g_scratch_zeroed[dev] = true;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_FFN_ABI_VERSION; }

const char* moe_last_error(void) { return g_err.c_str(); }

moe_status moe_workspace_size(const moe_desc* desc, int64_t num_tokens, size_t* bytes) {
  g_err.clear();
  MOE_TRY(check_desc(desc));
  if (num_tokens < 0) return fail(MOE_INVALID_ARGUMENT, "num_tokens is negative");
  if (!bytes) return fail(MOE_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = make_plan(desc, num_tokens).total;
  return MOE_OK;
}

moe_status moe_route(const moe_desc* desc, int64_t num_tokens, const void* x,
                     const moe_weights* weights, int32_t* topk_ids, float* topk_w,
                     int32_t* expert_counts, int32_t* expert_offsets, int32_t* route_perm,
                     void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  Plan p;
  MOE_TRY(check_common(desc, num_tokens, x, weights, ws, ws_bytes, false, &p));
  if (num_tokens == 0) return MOE_OK;
  if (!topk_ids || !topk_w) return fail(MOE_INVALID_ARGUMENT, "topk_ids/topk_w is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_TRY(layer_input(desc, p, x, weights, ws, s, &x));
  if (p.small)
    return run_route_small(desc, p, x, weights, ws, topk_ids, topk_w, expert_counts,
                           expert_offsets, route_perm, s);
  MOE_TRY(run_router(desc, p, x, weights, ws, s));
  return run_route_and_group(desc, p, x, weights, ws, topk_ids, topk_w, expert_counts,
                             expert_offsets, route_perm, s);
}

moe_status moe_ffn_forward(const moe_desc* desc, int64_t num_tokens, const void* x,
                           const moe_weights* weights, float* out, const float* residual,
                           int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes,
                           void* stream) {
  g_err.clear();
  Plan p;
  MOE_TRY(check_common(desc, num_tokens, x, weights, ws, ws_bytes, true, &p));
  if (num_tokens == 0) return MOE_OK;
  if (!out) return fail(MOE_INVALID_ARGUMENT, "out is NULL");
  if (!aligned16(out) || !aligned16(residual))
    return fail(MOE_UNSUPPORTED, "out and residual must be 16-byte aligned");
  return forward_body(desc, p, num_tokens, x, weights, out, residual, topk_ids_out, topk_w_out,
                      ws, static_cast<hipStream_t>(stream));
}

moe_status moe_ffn_forward_noalloc(const moe_desc* desc, int64_t num_tokens, const void* x,
                                   const moe_weights* weights, float* out, const float* residual,
                                   int32_t* topk_ids_out, float* topk_w_out, void* stream) {
  g_err.clear();
  Plan p;
  MOE_TRY(check_common(desc, num_tokens, x, weights, nullptr, 0, true, &p, true));
  if (num_tokens == 0) return MOE_OK;
  if (!out) return fail(MOE_INVALID_ARGUMENT, "out is NULL");
  if (!aligned16(out) || !aligned16(residual))
    return fail(MOE_UNSUPPORTED, "out and residual must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  MOE_TRY(scratch_for_device(s, &ws));
  return forward_body(desc, p, num_tokens, x, weights, out, residual, topk_ids_out, topk_w_out,
                      ws, s);
}

moe_status moe_packed_weight_bytes(const moe_desc* desc, size_t* gate_up_bytes,
                                   size_t* down_bytes, size_t* shared_gate_up_bytes,
                                   size_t* shared_down_bytes) {
  g_err.clear();
  PackSizes ps;
  MOE_TRY(pack_sizes(desc, &ps));
  if (gate_up_bytes) *gate_up_bytes = ps.gu;
  if (down_bytes) *down_bytes = ps.dn;
  if (shared_gate_up_bytes) *shared_gate_up_bytes = ps.sgu;
  if (shared_down_bytes) *shared_down_bytes = ps.sdn;
  return MOE_OK;
}

moe_status moe_pack_weights(const moe_desc* desc, const moe_weights* w, void* gate_up_packed,
                            void* down_packed, void* shared_gate_up_packed,
                            void* shared_down_packed, void* stream) {
  g_err.clear();
  PackSizes ps;
  MOE_TRY(pack_sizes(desc, &ps));
  if (!w) return fail(MOE_INVALID_ARGUMENT, "weights is NULL");
  const bool sh = desc->has_shared_expert != 0;
  const void* src[6] = {w->gate, w->up, w->down, sh ? w->shared_gate : w->gate,
                        sh ? w->shared_up : w->gate, sh ? w->shared_down : w->gate};
  void* dst[4] = {gate_up_packed, down_packed, sh ? shared_gate_up_packed : gate_up_packed,
                  sh ? shared_down_packed : gate_up_packed};
  for (const void* q : src)
    if (!q) return fail(MOE_INVALID_ARGUMENT, "a weight matrix to pack is NULL");
  for (void* q : dst)
    if (!q) return fail(MOE_INVALID_ARGUMENT, "a packed destination is NULL");
  for (const void* q : src)
    if (!aligned16(q)) return fail(MOE_UNSUPPORTED, "weights must be 16-byte aligned");
  for (void* q : dst)
    if (!aligned16(q)) return fail(MOE_UNSUPPORTED, "packed destinations must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int H = desc->hidden, E = desc->num_experts;
  auto pack_gu = [&](const void* g, const void* u, void* o, int n, int ne) {
    const int nwt = (n + 127) / 128;
    dim3 grid(nwt * (H / kDmaBK), ne);
    return launch("pack_gate_up", s, [&] {
      k_pack<GM_GATEUP><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(g),
          static_cast<const uint16_t*>(u), static_cast<uint8_t*>(o), n, H, nwt);
    });
  };
  auto pack_dn = [&](const void* dn, void* o, int n, int ne) {
    const int nwt = (H + kPackRows - 1) / kPackRows;
    dim3 grid(nwt * (n / kDmaBK), ne);
    return launch("pack_down", s, [&] {
      k_pack<GM_DOWN><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(dn), nullptr,
          static_cast<uint8_t*>(o), H, n, nwt);
    });
  };
  MOE_TRY(pack_gu(w->gate, w->up, gate_up_packed, desc->intermediate, E));
  MOE_TRY(pack_dn(w->down, down_packed, desc->intermediate, E));
  if (sh) {
    MOE_TRY(pack_gu(w->shared_gate, w->shared_up, shared_gate_up_packed,
                    desc->shared_intermediate, 1));
    MOE_TRY(pack_dn(w->shared_down, shared_down_packed, desc->shared_intermediate, 1));
  }
  return MOE_OK;
}

moe_status moe_weighted_sum_backward(int64_t num_tokens, int32_t top_k, int32_t hidden,
                                     const float* w, const float* y, const float* dout,
                                     float* dy, float* dw, void* stream) {
  g_err.clear();
  if (num_tokens < 0) return fail(MOE_INVALID_ARGUMENT, "num_tokens is negative");
  if (top_k < 1 || top_k > MOE_MAX_TOP_K)
    return fail(MOE_INVALID_ARGUMENT, "top_k %d outside 1..%d", top_k, MOE_MAX_TOP_K);
  if (hidden <= 0) return fail(MOE_INVALID_ARGUMENT, "hidden must be positive");
  if (hidden % 4) return fail(MOE_UNSUPPORTED, "hidden must be a multiple of 4");
  if ((num_tokens + 7) / 8 * 8 * top_k > INT32_MAX)
    return fail(MOE_UNSUPPORTED, "num_tokens * top_k too large");
  if (num_tokens == 0 || (!dy && !dw)) return MOE_OK;
  if (!w || !dout || (dw && !y)) return fail(MOE_INVALID_ARGUMENT, "w, y or dout is NULL");
  if (!aligned16(y) || !aligned16(dout) || !aligned16(dy))
    return fail(MOE_UNSUPPORTED, "y, dout and dy must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  // whole groups of 8 tokens (one per XCD); the blocks past T return at once
  const unsigned grid = (unsigned)((num_tokens + 7) / 8 * 8 * top_k);
  const int64_t T = num_tokens;
  return launch("wsum_backward", s, [&] {
    if (dy && dw)
      k_wsum_backward<true, true><<<grid, 256, 0, s>>>(w, y, dout, dy, dw, top_k, hidden, T);
    else if (dy)
      k_wsum_backward<true, false><<<grid, 256, 0, s>>>(w, y, dout, dy, dw, top_k, hidden, T);
    else
      k_wsum_backward<false, true><<<grid, 256, 0, s>>>(w, y, dout, dy, dw, top_k, hidden, T);
  });
}

moe_status moe_glu_backward(int64_t rows, int32_t intermediate, int32_t activation,
                            const float* gate_up, const float* dh, float* d_gate_up,
                            void* stream) {
  g_err.clear();
  if (rows < 0) return fail(MOE_INVALID_ARGUMENT, "rows is negative");
  if (intermediate <= 0) return fail(MOE_INVALID_ARGUMENT, "intermediate must be positive");
  if (intermediate % 4) return fail(MOE_UNSUPPORTED, "intermediate must be a multiple of 4");
  if (activation != MOE_ACT_SILU && activation != MOE_ACT_GELU_TANH)
    return fail(MOE_INVALID_ARGUMENT, "unknown activation %d", activation);
  if (rows == 0) return MOE_OK;
  if (!gate_up || !dh || !d_gate_up) return fail(MOE_INVALID_ARGUMENT, "a pointer is NULL");
  if (!aligned16(gate_up) || !aligned16(dh) || !aligned16(d_gate_up))
    return fail(MOE_UNSUPPORTED, "gate_up, dh and d_gate_up must be 16-byte aligned");
  const uint64_t n = (uint64_t)rows * (uint64_t)(intermediate / 4);
  if ((n + 255) / 256 > 0x7FFFFFFFull) return fail(MOE_UNSUPPORTED, "rows too large");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned grid = (unsigned)((n + 255) / 256);
  return launch("glu_backward", s, [&] {
    if (activation == MOE_ACT_SILU)
      k_glu_backward<ACT_SILU><<<grid, 256, 0, s>>>(gate_up, dh, d_gate_up, rows, intermediate);
    else
      k_glu_backward<ACT_GELU_TANH><<<grid, 256, 0, s>>>(gate_up, dh, d_gate_up, rows, intermediate);
  });
}

moe_status moe_timing_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timing = enable != 0;
  return MOE_OK;
}

static void drain_pending() {
  for (auto& r : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      auto& e = g_tsum[r.name];
      e.first += 1;
      e.second += ms;
    }
    g_evpool.push_back(r.a);
    g_evpool.push_back(r.b);
  }
  g_pending.clear();
}

int32_t moe_timing_read(char* names, int32_t name_stride, int64_t* launches, double* total_ms,
                        int32_t max_entries) {
  std::lock_guard<std::mutex> lk(g_tmu);
  if (!names || name_stride < 2 || !launches || !total_ms || max_entries < 0) return -1;
  drain_pending();
  int32_t n = 0;
  for (auto& kv : g_tsum) {
    if (n >= max_entries) break;
    std::snprintf(names + (size_t)n * name_stride, name_stride, "%s", kv.first.c_str());
    launches[n] = kv.second.first;
    total_ms[n] = kv.second.second;
    ++n;
  }
  return n;
}

moe_status moe_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_tmu);
  drain_pending();
  g_tsum.clear();
  return MOE_OK;
}

}  // extern "C"
