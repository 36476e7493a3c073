// Router logits (GEMV form), softmax/top-k/renormalise, and the stable
// expert grouping of the routes (histogram -> exclusive scan -> scatter).
#pragma once

#include "common.h"

namespace moe {

// --------------------------------------------------------------------------
// Router logits for few tokens: l[t, e] = x[t,:] . Wr[e,:] (+ b[e]).
// One workgroup per router row; threads split H into 16-byte weight chunks
// and loop over the tokens four at a time.  Row E (when the layer has a
// shared expert) is the shared expert's gate vector, whose logit lands in
// column E.
// --------------------------------------------------------------------------
// RDT: 0 = f32 router, 1 = bf16 router.  NC: chunks per thread per block of
// the row; TB: tokens per step (1 for one token, so the activation row is
// read once, else 4); all loads of a (TB-token, block) step are issued
// before the first is used, with clamped indices so that none sits behind a
// branch.
template <typename XT, int RDT, int NC = 1, int TB = 4>
__device__ __forceinline__ void router_row(const XT* __restrict__ x, const void* __restrict__ router,
                                           const float* __restrict__ bias,
                                           const void* __restrict__ shared_gate_inp,
                                           float* __restrict__ logits, int T, int H, int E,
                                           int ncols, int e) {
  constexpr int EPC = RDT ? 8 : 4;  // router elements per 16-byte chunk
  const int tid = threadIdx.x;
  const uint8_t* row = (e < E)
      ? reinterpret_cast<const uint8_t*>(router) + (size_t)e * H * (RDT ? 2 : 4)
      : reinterpret_cast<const uint8_t*>(shared_gate_inp);
  const int cpr = H / EPC;
  __shared__ float red[4][TB];
  for (int t0 = 0; t0 < T; t0 += TB) {
    float acc[TB];
#pragma unroll
    for (int r = 0; r < TB; ++r) acc[r] = 0.f;
    for (int cb = 0; cb < cpr; cb += 256 * NC) {
      u32x4 wv[NC];
      float xv[NC][TB][EPC];
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const int c = min(cb + tid + 256 * j, cpr - 1);
        wv[j] = ld16(row + (size_t)c * 16);
#pragma unroll
        for (int r = 0; r < TB; ++r) {
          const XT* xr = x + (size_t)min(t0 + r, T - 1) * H + (size_t)c * EPC;
#pragma unroll
          for (int q = 0; q < EPC; ++q) {
            if constexpr (sizeof(XT) == 4) xv[j][r][q] = xr[q];
            else xv[j][r][q] = bf16_to_f32(xr[q]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        if (cb + tid + 256 * j < cpr) {
          float w[EPC];
          if constexpr (RDT) {
#pragma unroll
            for (int q = 0; q < 4; ++q) { w[2 * q] = bf16lo(wv[j][q]); w[2 * q + 1] = bf16hi(wv[j][q]); }
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) w[q] = __uint_as_float(wv[j][q]);
          }
#pragma unroll
          for (int r = 0; r < TB; ++r) {
            float sdot = 0.f;
#pragma unroll
            for (int q = 0; q < EPC; ++q) sdot = fmaf(w[q], xv[j][r][q], sdot);
            acc[r] += sdot;
          }
        }
      }
    }
    const int wv2 = tid >> 6, ln = tid & 63;
#pragma unroll
    for (int r = 0; r < TB; ++r) {
      float sm = wave_sum(acc[r]);
      if (ln == 0) red[wv2][r] = sm;
    }
    __syncthreads();
    if (tid < TB && t0 + tid < T) {
      float sm = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
      if (e < E && bias) sm += bias[e];
      logits[(size_t)(t0 + tid) * ncols + e] = sm;
    }
    __syncthreads();
  }
}

// chunks per thread for a row of `cpr` 16-byte chunks (one block when it fits in 4)
inline int router_nc(int cpr) { return cpr <= 256 ? 1 : cpr <= 512 ? 2 : 4; }

template <typename XT, int RDT, int NC, int TB = 4>
__global__ __launch_bounds__(256) void k_router_gemv(
    const XT* __restrict__ x, const void* __restrict__ router,
    const float* __restrict__ bias, const void* __restrict__ shared_gate_inp,
    float* __restrict__ logits, int T, int H, int E, int ncols) {
  router_row<XT, RDT, NC, TB>(x, router, bias, shared_gate_inp, logits, T, H, E, ncols,
                              blockIdx.x);
}

// How the selected experts' weights follow from their logits:
//   softmax gating: p = softmax(l) over all E experts;
//   sigmoid gating: p_e = sigmoid(l_e), each expert on its own;
//   escale:         [E] or null: a selected expert's score p_j becomes
//                   p_j * escale[e_j] (selection looks at p alone);
//   normalize:      w_j = p_j / (sum of the k selected p), else w_j = p_j;
//   scale:          every w_j is multiplied by it.
struct RouteMode {
  int normalize;
  int sigmoid;
  float scale;
  const float* escale;
};
__device__ __forceinline__ float expert_scale_of(const RouteMode& rm, int e) {
  return rm.escale ? rm.escale[e] : 1.f;
}

// --------------------------------------------------------------------------
// Ranking of one token's logits by one wave.
// --------------------------------------------------------------------------
// Order-preserving 32-bit image of a logit (-0 and +0 tie) and its inverse.
__device__ __forceinline__ uint32_t route_ord(float l) {
  const uint32_t u = __float_as_uint(l == 0.0f ? 0.0f : l);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord_logit(uint32_t ord) {
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

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

static_assert(MOE_MAX_EXPERTS_DEV <= 4 * 64, "one-token ranking holds at most 4 logits a lane");
template <int C>
__device__ __forceinline__ void rank_load(const float* __restrict__ l, int E, float (&lv)[C],
                                          uint32_t (&ord)[C], bool (&live)[C]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int e = lane + 64 * c;
    const bool ok = e < E;
    lv[c] = ok ? l[e] : 0.f;
    ord[c] = ok ? route_ord(lv[c]) : 0u;
    live[c] = ok;
  }
}
// One round: the wave maximum M of the images and the lowest live expert e
// whose image is M, which is then taken (wave-uniform results).
template <int C>
__device__ __forceinline__ int rank_round(uint32_t (&ord)[C], bool (&live)[C], uint32_t& M) {
  const int lane = threadIdx.x & 63;
  uint32_t m = ord[0];
#pragma unroll
  for (int c = 1; c < C; ++c) m = max(m, ord[c]);
  M = wave_max_u32(m);
  int e = 0;
#pragma unroll
  for (int c = C - 1; c >= 0; --c) {
    const uint64_t hit = __ballot(live[c] && ord[c] == M);
    e = hit != 0 ? 64 * c + __ffsll((unsigned long long)hit) - 1 : e;
  }
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const bool taken = lane + 64 * c == e;
    live[c] = live[c] && !taken;
    ord[c] = taken ? 0u : ord[c];
  }
  return e;
}
// The expert at top-k position n - 1 (n >= 1): the first n rounds alone.
template <int C>
__device__ __forceinline__ int rank_nth(const float* __restrict__ l, int E, int n) {
  float lv[C];
  uint32_t ord[C], M;
  bool live[C];
  rank_load<C>(l, E, lv, ord, live);
  int e = 0;
  for (int j = 0; j < n; ++j) e = rank_round<C>(ord, live, M);
  return e;
}

// --------------------------------------------------------------------------
// Softmax (or sigmoid) -> top-k -> renormalise, one wave per token.
// Selection is on the logits: softmax is monotone, so the k most probable
// experts are the k largest logits, with the lower index first on a tie.
// The renormalised weights are exp(l_j - l_max) / sum over the selected
// exp(l - l_max), which equals p_j / sum(p_selected).  Without
// renormalisation the denominator runs over all E experts.  Sigmoid scores
// are increasing in the logit too, so selection is the same; their weights
// are sigmoid(l_j) over the selected sum, or sigmoid(l_j) alone.  A
// per-expert scale multiplies the selected numerators (and so the
// renormalising sum) only.
// --------------------------------------------------------------------------
// One token's routing in one wave: l points at the token's logits (global
// or LDS), column E holding the shared expert's gate logit when there is
// one.  Lane j < k writes top-k position j.
// l: the token's logits row, or the first of nsplit partial rows sstride
// floats apart (added in order).
__device__ __forceinline__ float split_sum(const float* l, int e, int nsplit, size_t sstride) {
  float v = l[e];
  for (int z = 1; z < nsplit; ++z) v += l[z * sstride + e];
  return v;
}
// The shared expert's gate logit is column E of the logits, or, when gx is
// set (bf16 rows x and gate vector gw of length H, a multiple of 8), the dot
// product taken here by the wave: lane l takes 8-element chunks l, l + 64, ...
template <int C>
__device__ __forceinline__ void topk_token(const float* l, int nsplit, size_t sstride, int t, int E,
                                           int k, RouteMode rm, int has_shared,
                                           const uint16_t* __restrict__ gx,
                                           const uint16_t* __restrict__ gw, int H,
                                           int32_t* __restrict__ ids, float* __restrict__ wts,
                                           int32_t* __restrict__ user_ids,
                                           float* __restrict__ user_w, float* __restrict__ sgate) {
  const int lane = threadIdx.x & 63;
  float v[C];
  uint32_t ord[C];
  bool live[C];
#pragma unroll
  for (int q = 0; q < C; ++q) {
    const int e = lane + 64 * q;
    live[q] = e < E;
    v[q] = live[q] ? split_sum(l, e, nsplit, sstride) : 0.f;
    ord[q] = live[q] ? route_ord(v[q]) : 0u;
  }
  int my_id = 0;
  uint32_t my_ord = 0, top = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t M;
    const int e = rank_round<C>(ord, live, M);
    if (j == 0) top = M;
    if (lane == j) {
      my_id = e;
      my_ord = M;
    }
  }
  const float my_val = ord_logit(my_ord), lmax = ord_logit(top);
  const float ex = (lane < k) ? (rm.sigmoid ? sigmoid_f(my_val) : __expf(my_val - lmax)) *
                                    expert_scale_of(rm, my_id)
                              : 0.f;
  float denom;
  if (rm.normalize) {
    denom = wave_sum(ex);
  } else if (rm.sigmoid) {
    denom = 1.f;
  } else {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < C; ++q)
      if (lane + 64 * q < E) s += __expf(v[q] - lmax);
    denom = wave_sum(s);
  }
  if (lane < k) {
    const float w = ex / denom * rm.scale;
    ids[(size_t)t * k + lane] = my_id;
    wts[(size_t)t * k + lane] = w;
    if (user_ids) user_ids[(size_t)t * k + lane] = my_id;
    if (user_w) user_w[(size_t)t * k + lane] = w;
  }
  if (has_shared) {
    float g;
    if (gx) {
      const uint16_t* xr = gx + (size_t)t * H;
      float d = 0.f;
      constexpr int U = 4;  // chunks a lane loads at once (clamped, so no load is behind a branch)
      for (int c0 = lane * 8; c0 < H; c0 += U * 64 * 8) {
        u32x4 a[U], b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = min(c0 + u * 64 * 8, H - 8);
          a[u] = ld16(xr + c);
          b[u] = ld16(gw + c);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (c0 + u * 64 * 8 < H) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              d = fmaf(bf16lo(a[u][q]), bf16lo(b[u][q]), d);
              d = fmaf(bf16hi(a[u][q]), bf16hi(b[u][q]), d);
            }
          }
        }
      }
      g = wave_sum(d);
    } else {
      g = split_sum(l, E, nsplit, sstride);
    }
    if (lane == 0) sgate[t] = sigmoid_f(g);
  }
}

__global__ __launch_bounds__(256) void k_topk(
    const float* __restrict__ logits, int nsplit, size_t sstride, int T, int E, int k, int ncols,
    RouteMode rm, int has_shared, const uint16_t* __restrict__ gx,
    const uint16_t* __restrict__ gw, int H, int32_t* __restrict__ ids,
    float* __restrict__ wts, int32_t* __restrict__ user_ids,
    float* __restrict__ user_w, float* __restrict__ sgate) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* l = logits + (size_t)t * ncols;
#define MOE_TOPK(C) \
  topk_token<C>(l, nsplit, sstride, t, E, k, rm, has_shared, gx, gw, H, ids, wts, user_ids, user_w, sgate)
  if (E <= 64) MOE_TOPK(1);
  else if (E <= 128) MOE_TOPK(2);
  else if (E <= 192) MOE_TOPK(3);
  else MOE_TOPK(4);
#undef MOE_TOPK
}

// --------------------------------------------------------------------------
// Expert grouping.  Routes r = t*k + j are cut into blocks of kPermBlock;
// pass 1 counts each block's routes per expert, pass 2 turns the counts
// into per-(block, expert) starting positions (an exclusive scan over
// (expert, block) order), pass 3 places every route at its position,
// stably: within a block, routes to the same expert keep their order.
// --------------------------------------------------------------------------
constexpr int kPermBlock = 1024;

__global__ __launch_bounds__(256) void k_perm_hist(const int32_t* __restrict__ ids, int R, int E,
                                                   int32_t* __restrict__ block_hist) {
  __shared__ int hist[MOE_MAX_EXPERTS_DEV];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int r0 = blockIdx.x * kPermBlock;
  const int r1 = min(R, r0 + kPermBlock);
  for (int r = r0 + threadIdx.x; r < r1; r += 256) atomicAdd(&hist[ids[r]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) block_hist[(size_t)blockIdx.x * E + e] = hist[e];
}

struct ScanOut {
  int32_t* counts;        // [G]   routes per group (group E = shared: T)
  int32_t* offsets;       // [G+1] start of each routed group (routed only)
  int32_t* block_off;     // [nblk, E]
  int32_t* active;        // [G]   groups with routes, ascending, shared last
  int32_t* n_active;      // [1]
  int32_t* tile_group;    // [max_tiles]
  int32_t* tile_m0;       // [max_tiles]
  int32_t* n_tiles;       // [1]
  int32_t* user_counts;   // [E] or null
  int32_t* user_offsets;  // [E+1] or null
};

// One workgroup of 1024 threads: thread (part, e) = (tid / 256, tid % 256)
// owns expert e (E <= 256) over a quarter of the blocks (a contiguous
// range), so each thread reads a quarter of the column of per-block counts;
// the quarters' sums meet in LDS.  Every quarter's four waves then scan the
// expert totals themselves (DPP wave scans, one exchange of wave totals), so
// each thread has its expert's offset without a further barrier, and writes
// the starting positions of its blocks.  The per-block counts of a range
// are read kScanBatch at a time, every load of a batch issued before any is
// added (indices clamped, so the loads need no branch).
constexpr int kScanBatch = 16;
constexpr int kScanParts = 4;
__global__ __launch_bounds__(256 * kScanParts) void k_perm_scan(
    const int32_t* __restrict__ block_hist, int nblk, int E, int T, int has_shared, int tile_rows,
    int build_tiles, ScanOut o) {
  __shared__ int s_cnt[kScanParts][256];
  __shared__ int s_tot[kScanParts][4][3];
  const int tid = threadIdx.x, e = tid & 255, part = tid >> 8;
  const int lane = tid & 63, w4 = (tid >> 6) & 3;
  const int ec = min(e, E - 1);
  const int per = (nblk + kScanParts - 1) / kScanParts;
  const int b0 = part * per, b1 = min(b0 + per, nblk);
  auto batch = [&](int bb, int (&v)[kScanBatch]) {
#pragma unroll
    for (int j = 0; j < kScanBatch; ++j)
      v[j] = block_hist[(size_t)min(bb + j, nblk - 1) * E + ec];
  };
  int mine = 0;  // this quarter's routes to expert e
  for (int bb = b0; bb < b1; bb += kScanBatch) {
    int v[kScanBatch];
    batch(bb, v);
#pragma unroll
    for (int j = 0; j < kScanBatch; ++j) mine += (bb + j < b1) ? v[j] : 0;
  }
  s_cnt[part][e] = mine;
  __syncthreads();
  int cnt = 0, before = 0;  // expert total; routes of the quarters before this one
#pragma unroll
  for (int q = 0; q < kScanParts; ++q) {
    const int v = s_cnt[q][e];
    cnt += v;
    before += q < part ? v : 0;
  }
  if (e >= E) cnt = 0;
  const int act = (e < E && cnt > 0) ? 1 : 0;
  const int tiles = (e < E) ? (cnt + tile_rows - 1) / tile_rows : 0;
  const int ic = wave_incl_scan(cnt), ia = wave_incl_scan(act), it = wave_incl_scan(tiles);
  if (lane == 63) {
    s_tot[part][w4][0] = ic;
    s_tot[part][w4][1] = ia;
    s_tot[part][w4][2] = it;
  }
  __syncthreads();
  int off = ic - cnt, aoff = ia - act, toff = it - tiles, total = 0, nact = 0, ntile = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int tc = s_tot[part][w][0], ta = s_tot[part][w][1], tt = s_tot[part][w][2];
    off += w < w4 ? tc : 0;
    aoff += w < w4 ? ta : 0;
    toff += w < w4 ? tt : 0;
    total += tc;
    nact += ta;
    ntile += tt;
  }
  if (e < E) {
    if (part == 0) {
      o.counts[e] = cnt;
      o.offsets[e] = off;
      if (o.user_counts) o.user_counts[e] = cnt;
      if (o.user_offsets) o.user_offsets[e] = off;
      if (act) o.active[aoff] = e;
      if (build_tiles)
        for (int i = 0; i < tiles; ++i) {
          o.tile_group[toff + i] = e;
          o.tile_m0[toff + i] = i * tile_rows;
        }
    }
    int run = off + before;
    for (int bb = b0; bb < b1; bb += kScanBatch) {
      int v[kScanBatch];
      batch(bb, v);
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) {
        if (bb + j < b1) {
          o.block_off[(size_t)(bb + j) * E + e] = run;
          run += v[j];
        }
      }
    }
  }
  if (tid == 0) {
    o.offsets[E] = total;
    if (o.user_offsets) o.user_offsets[E] = total;
    int na = nact, nt = ntile;
    if (has_shared) {
      o.counts[E] = T;
      o.active[na++] = E;
      if (build_tiles) {
        const int stiles = (T + tile_rows - 1) / tile_rows;
        for (int i = 0; i < stiles; ++i) {
          o.tile_group[nt + i] = E;
          o.tile_m0[nt + i] = i * tile_rows;
        }
        nt += stiles;
      }
    }
    *o.n_active = na;
    *o.n_tiles = nt;
  }
}

// Four waves per block; wave w places the routes of the block's w-th
// quarter, 64 at a time.  Lanes with the same expert find each other with
// eight ballots over the expert id bits; a lane's rank is the number of
// lower lanes in its group.  The waves first count their quarter's routes
// per expert, and each starts from the block's offset plus the counts of the
// quarters before it, so the block stays stable.
constexpr int kScatterWaves = 4;
constexpr int kScatterSteps = kPermBlock / (64 * kScatterWaves);
__global__ __launch_bounds__(64 * kScatterWaves) void k_perm_scatter(
    const int32_t* __restrict__ ids, int R, int E, int k, const int32_t* __restrict__ block_off,
    int32_t* __restrict__ perm, int32_t* __restrict__ pos_of_route,
    int32_t* __restrict__ row_token, int32_t* __restrict__ user_perm) {
  __shared__ int run[kScatterWaves][MOE_MAX_EXPERTS_DEV];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kScatterWaves * MOE_MAX_EXPERTS_DEV; i += 64 * kScatterWaves)
    (&run[0][0])[i] = 0;
  const int r0 = blockIdx.x * kPermBlock + wave * (kPermBlock / kScatterWaves);
  int ev[kScatterSteps];
  bool valid[kScatterSteps];
#pragma unroll
  for (int s = 0; s < kScatterSteps; ++s) {
    const int r = r0 + 64 * s + lane;
    valid[s] = r < R;
    ev[s] = ids[min(r, R - 1)];
  }
  uint64_t grp[kScatterSteps];  // lanes of the same expert in step s
#pragma unroll
  for (int s = 0; s < kScatterSteps; ++s) {
    const int e = valid[s] ? ev[s] : 0;
    uint64_t mask = __ballot(valid[s]);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool set = (e >> bit) & 1;
      const uint64_t b = __ballot(set);
      mask &= set ? b : ~b;
    }
    grp[s] = mask;
  }
  __syncthreads();
  // counts of the wave's quarter: the highest lane of each group adds its size
#pragma unroll
  for (int s = 0; s < kScatterSteps; ++s)
    if (valid[s] && (grp[s] >> lane) == 1ull) run[wave][ev[s]] += __popcll(grp[s]);
  __syncthreads();
  for (int e = tid; e < E; e += 64 * kScatterWaves) {
    int b = block_off[(size_t)blockIdx.x * E + e];
#pragma unroll
    for (int w = 0; w < kScatterWaves; ++w) {
      const int c = run[w][e];
      run[w][e] = b;
      b += c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < kScatterSteps; ++s) {
    const int r = r0 + 64 * s + lane;
    const int e = valid[s] ? ev[s] : 0;
    const int pos = run[wave][e] + __popcll(grp[s] & lanemask_lt());  // read by every lane ...
    if (valid[s]) {
      if ((grp[s] >> lane) == 1ull) run[wave][e] += __popcll(grp[s]);  // ... before the update
      perm[pos] = r;
      pos_of_route[r] = pos;
      row_token[pos] = r / k;
      if (user_perm) user_perm[pos] = r;
    }
  }
}

}  // namespace moe
