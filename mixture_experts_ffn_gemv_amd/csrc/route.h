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
// RDT: 0 = f32 router, 1 = bf16 router.  COHERENT: logits are stored at
// device scope (written through to the point of coherence of all XCDs), so
// that another workgroup may read them within the same launch.  NC: chunks
// per thread per block of the row; TB: tokens per step (1 for one token, so
// the activation row is read once, else 4); all loads of a (TB-token, block)
// step are issued before the first is used, with clamped indices so that
// none sits behind a branch.
template <typename XT, int RDT, bool COHERENT = false, int NC = 1, int TB = 4>
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
      float* dst = logits + (size_t)(t0 + tid) * ncols + e;
      if constexpr (COHERENT) __hip_atomic_store(dst, sm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else *dst = sm;
    }
    __syncthreads();
  }
}

// Router row e for at most kRowTokens tokens when the row fits one block of
// NC chunks a thread: the weight chunks are loaded once, every token's
// partial dot product stays in a register, and one reduction at the end
// (one barrier) gives all the token's logits; tokens are walked in steps of
// 4 with all activation loads of a step issued together.  COHERENT as in
// router_row.
constexpr int kRowTokens = 32;
template <typename XT, int RDT, bool COHERENT, int NC>
__device__ __forceinline__ void router_row_few(const XT* __restrict__ x, const void* __restrict__ router,
                                               const float* __restrict__ bias,
                                               const void* __restrict__ shared_gate_inp,
                                               float* __restrict__ logits, int T, int H, int E,
                                               int ncols, int e) {
  constexpr int EPC = RDT ? 8 : 4;  // router elements per 16-byte chunk
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint8_t* row = (e < E)
      ? reinterpret_cast<const uint8_t*>(router) + (size_t)e * H * (RDT ? 2 : 4)
      : reinterpret_cast<const uint8_t*>(shared_gate_inp);
  const int cpr = H / EPC;
  __shared__ float red[4][kRowTokens];
  float w[NC][EPC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c = min(tid + 256 * j, cpr - 1);
    const u32x4 v = ld16(row + (size_t)c * 16);
    const bool ok = tid + 256 * j < cpr;
    if constexpr (RDT) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w[j][2 * q] = ok ? bf16lo(v[q]) : 0.f;
        w[j][2 * q + 1] = ok ? bf16hi(v[q]) : 0.f;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) w[j][q] = ok ? __uint_as_float(v[q]) : 0.f;
    }
  }
  float acc[kRowTokens];
#pragma unroll
  for (int t0 = 0; t0 < kRowTokens; t0 += 4) {
    if (t0 < T) {
      float xv[4][NC][EPC];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const XT* xr = x + (size_t)min(t0 + r, T - 1) * H;
#pragma unroll
        for (int j = 0; j < NC; ++j) {
          const int c = min(tid + 256 * j, cpr - 1);
#pragma unroll
          for (int q = 0; q < EPC; ++q) {
            if constexpr (sizeof(XT) == 4) xv[r][j][q] = xr[(size_t)c * EPC + q];
            else xv[r][j][q] = bf16_to_f32(xr[(size_t)c * EPC + q]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float sdot = 0.f;
#pragma unroll
        for (int j = 0; j < NC; ++j)
#pragma unroll
          for (int q = 0; q < EPC; ++q) sdot = fmaf(w[j][q], xv[r][j][q], sdot);
        acc[t0 + r] = sdot;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[t0 + r] = 0.f;
    }
  }
#pragma unroll
  for (int t = 0; t < kRowTokens; ++t) {
    if (t < T) {
      const float sm = wave_sum(acc[t]);
      if (lane == 0) red[wave][t] = sm;
    }
  }
  __syncthreads();
  if (tid < T) {
    float sm = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
    if (e < E && bias) sm += bias[e];
    float* dst = logits + (size_t)tid * ncols + e;
    if constexpr (COHERENT) __hip_atomic_store(dst, sm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *dst = sm;
  }
}

// chunks per thread for a row of `cpr` 16-byte chunks (one block when it fits in 4)
inline int router_nc(int cpr) { return cpr <= 256 ? 1 : cpr <= 512 ? 2 : 4; }

template <typename XT, int RDT, int NC, int TB = 4>
__global__ __launch_bounds__(256) void k_router_gemv(
    const XT* __restrict__ x, const void* __restrict__ router,
    const float* __restrict__ bias, const void* __restrict__ shared_gate_inp,
    float* __restrict__ logits, int T, int H, int E, int ncols) {
  router_row<XT, RDT, false, NC, TB>(x, router, bias, shared_gate_inp, logits, T, H, E, ncols,
                                 blockIdx.x);
}

// How the selected experts' weights follow from their logits:
//   softmax gating: p = softmax(l) over all E experts;
//   sigmoid gating: p_e = sigmoid(l_e), each expert on its own;
//   normalize:      w_j = p_j / (sum of the k selected p), else w_j = p_j;
//   scale:          every w_j is multiplied by it.
struct RouteMode {
  int normalize;
  int sigmoid;
  float scale;
};

// --------------------------------------------------------------------------
// Softmax (or sigmoid) -> top-k -> renormalise, one wave per token.
// Selection is on the logits: softmax is monotone, so the k most probable
// experts are the k largest logits, with the lower index first on a tie.
// The renormalised weights are exp(l_j - l_max) / sum over the selected
// exp(l - l_max), which equals p_j / sum(p_selected).  Without
// renormalisation the denominator runs over all E experts.  Sigmoid scores
// are increasing in the logit too, so selection is the same; their weights
// are sigmoid(l_j) over the selected sum, or sigmoid(l_j) alone.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_topk(
    const float* __restrict__ logits, int T, int E, int k, int ncols,
    RouteMode rm, int has_shared, int32_t* __restrict__ ids,
    float* __restrict__ wts, int32_t* __restrict__ user_ids,
    float* __restrict__ user_w, float* __restrict__ sgate) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* l = logits + (size_t)t * ncols;
  float v[4];
  unsigned taken = 0;  // bit q: candidate q of this lane is used up (or absent)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    v[q] = (e < E) ? l[e] : -INFINITY;
    if (e >= E) taken |= 1u << q;
  }
  int my_id = 0;
  float my_val = -INFINITY;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (!((taken >> q) & 1u) && (v[q] > bv || bi == 0x7FFFFFFF)) { bv = v[q]; bi = lane + 64 * q; }
    }
    wave_argmax(bv, bi);
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == j) { my_id = bi; my_val = bv; }
  }
  const float lmax = __shfl(my_val, 0, 64);
  const float ex = (lane < k) ? (rm.sigmoid ? sigmoid_f(my_val) : __expf(my_val - lmax)) : 0.f;
  float denom;
  if (rm.normalize) {
    denom = wave_sum(ex);
  } else if (rm.sigmoid) {
    denom = 1.f;
  } else {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
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
  if (has_shared && lane == 0) sgate[t] = sigmoid_f(l[E]);
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

// One workgroup of 256 threads; thread e owns expert e (E <= 256).  The
// per-block counts of a column are read kScanBatch at a time, every load of
// a batch issued before any is added (indices clamped, so the loads need no
// branch): read one by one, each load's latency would add up over the
// blocks.
constexpr int kScanBatch = 16;
__global__ __launch_bounds__(256) void k_perm_scan(const int32_t* __restrict__ block_hist,
                                                   int nblk, int E, int T, int has_shared,
                                                   int tile_rows, int build_tiles, ScanOut o) {
  __shared__ int sc[256];
  __shared__ int sa[256];
  __shared__ int st[256];
  const int e = threadIdx.x;
  const int ec = min(e, E - 1);
  auto batch = [&](int b0, int (&v)[kScanBatch]) {
#pragma unroll
    for (int j = 0; j < kScanBatch; ++j) v[j] = block_hist[(size_t)min(b0 + j, nblk - 1) * E + ec];
  };
  int cnt = 0;
  for (int b0 = 0; b0 < nblk; b0 += kScanBatch) {
    int v[kScanBatch];
    batch(b0, v);
#pragma unroll
    for (int j = 0; j < kScanBatch; ++j) cnt += (b0 + j < nblk) ? v[j] : 0;
  }
  if (e >= E) cnt = 0;
  const int act = (e < E && cnt > 0) ? 1 : 0;
  const int tiles = (e < E) ? (cnt + tile_rows - 1) / tile_rows : 0;
  sc[e] = cnt;
  sa[e] = act;
  st[e] = tiles;
  __syncthreads();
  // inclusive Hillis-Steele scans over 256 entries
  for (int o2 = 1; o2 < 256; o2 <<= 1) {
    int a = (e >= o2) ? sc[e - o2] : 0;
    int b = (e >= o2) ? sa[e - o2] : 0;
    int c = (e >= o2) ? st[e - o2] : 0;
    __syncthreads();
    sc[e] += a;
    sa[e] += b;
    st[e] += c;
    __syncthreads();
  }
  const int off = sc[e] - cnt;  // exclusive
  const int aoff = sa[e] - act;
  const int toff = st[e] - tiles;
  const int total = sc[255];
  const int nact = sa[255];
  const int ntile = st[255];
  if (e < E) {
    o.counts[e] = cnt;
    o.offsets[e] = off;
    if (o.user_counts) o.user_counts[e] = cnt;
    if (o.user_offsets) o.user_offsets[e] = off;
    if (act) o.active[aoff] = e;
    int run = off;
    for (int b0 = 0; b0 < nblk; b0 += kScanBatch) {
      int v[kScanBatch];
      batch(b0, v);
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) {
        if (b0 + j < nblk) {
          o.block_off[(size_t)(b0 + j) * E + e] = run;
          run += v[j];
        }
      }
    }
    if (build_tiles)
      for (int i = 0; i < tiles; ++i) {
        o.tile_group[toff + i] = e;
        o.tile_m0[toff + i] = i * tile_rows;
      }
  }
  if (e == 0) {
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

// One wave per block, 64 routes per step.  Lanes with the same expert find
// each other with eight ballots over the expert id bits; a lane's rank is
// the number of lower lanes in its group.
__global__ __launch_bounds__(64) void k_perm_scatter(const int32_t* __restrict__ ids, int R,
                                                     int E, int k,
                                                     const int32_t* __restrict__ block_off,
                                                     int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ pos_of_route,
                                                     int32_t* __restrict__ row_token,
                                                     int32_t* __restrict__ user_perm) {
  __shared__ int run[MOE_MAX_EXPERTS_DEV];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) run[e] = block_off[(size_t)blockIdx.x * E + e];
  __syncthreads();
  const int r0 = blockIdx.x * kPermBlock;
  const int r1 = min(R, r0 + kPermBlock);
  for (int base = r0; base < r1; base += 64) {
    const int r = base + lane;
    const bool valid = r < r1;
    const int e = valid ? ids[r] : 0;
    uint64_t mask = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool set = (e >> bit) & 1;
      const uint64_t b = __ballot(set);
      mask &= set ? b : ~b;
    }
    const int rank = __popcll(mask & lanemask_lt());
    const int pos = valid ? run[e] + rank : 0;
    __syncthreads();
    if (valid) {
      if ((mask >> lane) == 1ull) run[e] += __popcll(mask);  // highest lane of its group
      perm[pos] = r;
      pos_of_route[r] = pos;
      row_token[pos] = r / k;
      if (user_perm) user_perm[pos] = r;
    }
    __syncthreads();
  }
}

}  // namespace moe
