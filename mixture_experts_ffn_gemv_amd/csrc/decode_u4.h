// Decode path for 4-bit affine weights (codes in groups of 32 along K, one
// f16 scale and one f16 min per group: w = code * scale + min), T <= 32 (any
// T runs, in chunks of up to 4 routes per expert).
//
// The dot products run on the 4x4x4 (16-block) f16 MFMA with the codes
// exact.  Per group g of a weight row and route r:
//   sum_i (c_i s + m) x_ri = s * sum_i c_i x_ri + m * sum_i x_ri,
// the first sum on the MFMA, the second from a staged per-group sum.  The
// codes enter as the f16 integers 0..15 (normal numbers, so the products are
// exact); each activation as two f16 terms hi + lo of the route's row scaled
// by a power of two, about 22 significant bits, and the MFMA accumulates in
// f32.
//
// Launches: k_u4_stage (each token's x row, and the expert work list), the
// gate/up kernel, k_u4_stage again (each route's h row), the down kernel,
// then the weighted combine.
//
// Lane layout of v_mfma_f32_4x4x4f16 (16 blocks of 4x4 outputs, 4 k each):
// lane l = 4b + j of block b holds row j of A (here: staged route slot j)
// and column j of B (here: row j of a quad of weight rows), 4 k values each;
// output D[b][i][j] comes back in lane 4b + j, register i.  Block b takes
// groups b + 16u of the weight row, so one MFMA step covers one 8-element
// word of 16 groups for 4 weight rows and 4 routes.
#pragma once

#include "common.h"
#include "gemv.h"
#include "decode.h"

namespace moe {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr int kU4Waves = 8;                     // waves per expert-kernel workgroup
constexpr int kU4Threads = 64 * kU4Waves;
constexpr int kU4LdsMax = 160 * 1024 - 4096;    // dynamic LDS an expert kernel may take
constexpr int kU4StageThreads = 256;
// groups per lane per step (UG) and row pairs per wave (PW) of the two
// expert kernels: gate/up 128 features a workgroup, down 256 output rows
constexpr int kU4UGGateUp = 2, kU4PWGateUp = 4;
constexpr int kU4UGDown = 1, kU4PWDown = 8;

// Staged activation row (one token of x, or one route of h), row length K,
// G = K / 32 groups.  Value v of the row is multiplied by the row's power of
// two sigma (largest |v| sigma < 2^15), the odd elements of each 8-element
// word also by 1/16 (their codes enter as 16 c), and split into f16
// hi = f16(v') and lo = f16(v' - hi).  Group c takes 128 bytes: word q gives
// two 16-byte pieces, even elements (0, 4, 2, 6) and odd elements
// (1, 5, 3, 7), each hi[4] then lo[4]; piece p sits at slot p ^ u4_swz(c).
// Beside the rows: each group's plain f32 sum, and the row's factor
// 1 / sigma.
__host__ __device__ constexpr size_t u4_row_bytes(int G) { return (size_t)G * 128; }
__device__ __forceinline__ int u4_swz(int c) { return (c ^ (c >> 1)) & 1; }

// Expert-kernel LDS: staged route slot r at r * (RS + 32), RS a multiple of
// 256 with room for the 96-byte shift of slot 3; the group sums of 4 slots
// as float4[G]; 16 floats of slot factors; per wave 512 UG bytes for the
// step's scales and mins.  The group swizzle together with the 32-byte slot
// shift keeps the A-operand reads (lane 4b + j: slot j, group b + 16u, one
// piece) on distinct banks for every 8 and 16 lanes.
__host__ __device__ constexpr int u4_route_stride(int G) { return (G * 128 + 96 + 255) / 256 * 256; }
__host__ __device__ constexpr int u4_lds_bytes(int K, int UG, int nslot) {
  return nslot * u4_route_stride(K / 32) + (K / 32) * 16 + 64 + kU4Waves * 512 * UG;
}

// (w & mask) | magic: one v_and_or_b32.  It is plain code, not inline
// assembly, so that the compiler knows which registers it writes and keeps
// the wait states the MFMAs need around them (an asm block that overwrote a
// register an MFMA still reads would go unseen).  The VOP3 form takes no
// literal: the two constants come from registers the compiler cannot fold
// (opaque_s, opaque_v), the mask scalar and the magic vector.
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic) {
  return (w & mask) | magic;
}
// A constant in a scalar or vector register, hidden from constant folding.
// Only ALU instructions read these, so the asm blocks meet no MFMA hazard.
__device__ __forceinline__ uint32_t opaque_s(uint32_t v) {
  uint32_t r;
  asm volatile("s_mov_b32 %0, %1" : "=s"(r) : "i"(v));
  return r;
}
__device__ __forceinline__ uint32_t opaque_v(uint32_t v) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
  return r;
}

// Masked nibbles with the exponent of 1024 or-ed in (f16 values 1024 + v,
// v < 2^10) -> the f16 values v exactly, by one packed f16 subtraction.
__device__ __forceinline__ f16x4 codes4(uint32_t lo, uint32_t hi) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f16x2 k = {(_Float16)1024.f, (_Float16)1024.f};
  const f16x2 a = __builtin_bit_cast(f16x2, lo) - k;
  const f16x2 b = __builtin_bit_cast(f16x2, hi) - k;
  return f16x4{a[0], a[1], b[0], b[1]};
}

// 8 consecutive values of an f32 or bf16 row.
__device__ __forceinline__ void load8(const void* row, int bf16, size_t off, float (&v)[8]) {
  if (bf16) {
    const u32x4 b = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(row) + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[2 * e] = bf16lo(b[e]); v[2 * e + 1] = bf16hi(b[e]); }
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(row) + off);
    const f32x4 c = *reinterpret_cast<const f32x4*>(static_cast<const float*>(row) + off + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = c[e]; }
  }
}

__device__ __forceinline__ uint32_t pack_h2(_Float16 a, _Float16 b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

struct U4Stage {
  const void* src;     // rows [rows, K], f32 or bf16
  int src_bf16;
  int K, rows;
  uint8_t* stage;      // [rows, G * 128]
  float* gsum;         // [rows, G]
  float* fac;          // [rows]
  // the expert kernels' work list, built by one extra workgroup when qlist
  // is set: for each active slot s, ceil(count / nslot) entries
  // s | chunk << 16, in slot order; qn = their number
  const int32_t* counts;
  const int32_t* active;
  const int32_t* n_active;
  int32_t* qlist;
  int32_t* qn;
  int E, qmax, nslot;
};

// One workgroup per row (plus, with qlist set, one for the work list).
__global__ __launch_bounds__(kU4StageThreads) void k_u4_stage(U4Stage p) {
  constexpr int NT = kU4StageThreads;
  __shared__ float wmax[NT / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x;
  if (row >= p.rows) {
    if (!p.qlist || wave != 0) return;
    const int na = min(max(*p.n_active, 0), p.E + 1);
    int total = 0;
    for (int s0 = 0; s0 < na; s0 += 64) {
      const int s = s0 + lane;
      int nq = 0;
      if (s < na) nq = (max(p.counts[ws_group(p.active[s], p.E, false)], 0) + p.nslot - 1) / p.nslot;
      int inc = nq;  // inclusive scan over the wave
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(inc, o, 64);
        if (lane >= o) inc += t;
      }
      const int first = total + inc - nq;
      for (int q = 0; q < nq; ++q)
        if (first + q < p.qmax) p.qlist[first + q] = s | (q << 16);
      total += __shfl(inc, 63, 64);
    }
    if (lane == 0) *p.qn = min(total, p.qmax);
    return;
  }
  const int K = p.K, G = K / 32;
  const void* src = p.src_bf16 ? static_cast<const void*>(static_cast<const uint16_t*>(p.src) + (size_t)row * K)
                               : static_cast<const void*>(static_cast<const float*>(p.src) + (size_t)row * K);
  const int n = G * 4;  // 8-element words
  float mx = 0.f;
  for (int i = tid; i < n; i += NT) {
    float v[8];
    load8(src, p.src_bf16, (size_t)i * 8, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(v[e]));
  }
  mx = wave_max(mx);
  if (lane == 0) wmax[wave] = mx;
  __syncthreads();
  float m = 0.f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) m = fmaxf(m, wmax[w]);
  int e = 0;  // m < 2^e; rows of zeros or non-finite values keep sigma 2^15
  if (m > 0.f && m <= 3.4e38f) (void)frexpf(m, &e);
  e = max(-100, e);
  const float sg = ldexpf(1.f, 15 - e);
  if (tid == 0) p.fac[row] = ldexpf(1.f, e - 15);
  uint8_t* dst = p.stage + (size_t)row * u4_row_bytes(G);
  for (int base = 0; base < n; base += NT) {  // uniform trip count: all lanes shuffle
    const int i = base + tid;
    const bool ok = i < n;
    const int ii = ok ? i : n - 1;
    const int c = ii >> 2, q = ii & 3;
    float v[8];
    load8(src, p.src_bf16, (size_t)ii * 8, v);
    float sm = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    sm += __shfl_xor(sm, 1, 64);  // the group's 4 words are 4 consecutive threads
    sm += __shfl_xor(sm, 2, 64);
    if (!ok) continue;
    const int sw = u4_swz(c);
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const float f = par ? sg * 0.0625f : sg;
      _Float16 hi[4], lo[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float a = v[par + ((k & 1) << 2) + ((k >> 1) << 1)] * f;  // elements 0, 4, 2, 6
        hi[k] = (_Float16)a;
        lo[k] = (_Float16)(a - (float)hi[k]);
      }
      const u32x4 pc = {pack_h2(hi[0], hi[1]), pack_h2(hi[2], hi[3]), pack_h2(lo[0], lo[1]),
                        pack_h2(lo[2], lo[3])};
      *reinterpret_cast<u32x4*>(dst + (size_t)c * 128 + (((2 * q + par) ^ sw) * 16)) = pc;
    }
    if (q == 0) p.gsum[(size_t)row * G + c] = sm;
  }
}

// The step's scales and mins for one lane: 8 UG bytes.
template <int UG> struct U4ScaleVec { typedef u32x2 type; };
template <> struct U4ScaleVec<2> { typedef u32x4 type; };

struct U4Experts {
  Dec2Params d;
  const uint8_t* stage;  // staged rows: tokens (gate/up) or routes (down)
  const float* gsum;
  const float* fac;
  const int32_t* qlist;
  const int32_t* qn;
  int nslot;             // routes per work-list entry, 1..4
};

// MODE 0: gate/up (K = H, N = I features; row sets: the gate and the up row
// of feature j of the quad); MODE 1: down (K = I, N = H outputs; row sets:
// two quads of output rows).  One workgroup per (work-list entry, block of
// rows).  UG groups per lane per step, PW row pairs per wave.  SV: the
// step's scales and mins (16 UG groups of the 8 rows, both arrays) come in as
// one coalesced load of 8 UG bytes per lane and reach the lanes that use
// them through a per-wave LDS slot (needs G a multiple of 4 UG); otherwise
// each lane loads its own 2-byte values.
template <int MODE, int ACT, int UG, int PW, bool SV>
__global__ __launch_bounds__(kU4Threads) __attribute__((amdgpu_waves_per_eu(4)))
void k_u4_mfma(U4Experts ep) {
  static_assert(!SV || UG == 1 || UG == 2, "vector scale loads cover 1 or 2 groups per lane");
  constexpr int NT = kU4Threads;
  constexpr int RPS = MODE == 0 ? 4 : 8;  // weight rows per pair step
  typedef typename U4ScaleVec<UG>::type SVec;
  extern __shared__ __attribute__((aligned(16))) uint8_t u4lds[];
  const Dec2Params& p = ep.d;
  const int wi = blockIdx.x;
  if (wi >= *ep.qn) return;
  const int qe = ep.qlist[wi];
  const int s = qe & 0xFFFF, chunk = qe >> 16;
  const int R = p.T * p.k;
  const int g = ws_group(p.active[s], p.E, false);
  const int K = MODE == 0 ? p.H : p.I;
  const int N = MODE == 0 ? p.I : p.H;
  const int G = K / 32;
  const int rb = blockIdx.y * (kU4Waves * PW * RPS);
  if (rb >= N) return;
  int count = p.counts[g], base = p.offsets[g];
  ws_span(base, count, R);
  const int r0 = ep.nslot * chunk;
  if (r0 >= count) return;
  const int nr = min(ep.nslot, count - r0);
  const int RS = u4_route_stride(G);
  uint8_t* xs = u4lds;
  f32x4* xsum4 = reinterpret_cast<f32x4*>(u4lds + ep.nslot * RS);
  float* rfac = reinterpret_cast<float*>(xsum4 + G);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint8_t* sbuf = reinterpret_cast<uint8_t*>(rfac + 16) + wave * (512 * UG);
  const int b = lane >> 2, j = lane & 3;
  const int NU = (G + 15) / 16, NCH = (NU + UG - 1) / UG;
  const int nsteps = PW * NCH;
  const MatStack& ma = MODE == 0 ? p.gate : p.down;
  const MatStack& mb = MODE == 0 ? p.up : p.down;

  // staged row of slot i (i < nr)
  auto srow = [&](int i) __attribute__((always_inline)) -> int {
    const int route = ws_route(p.perm[base + r0 + i], R);
    return MODE == 0 ? route / p.k : route;
  };

  // ---- the slots' staged rows into LDS (plain copies), the first batch
  // issued before the first step's weights
  const size_t rowb = u4_row_bytes(G);
  const int n16 = (int)(rowb / 16);
  const int ncopy = nr * n16;
  constexpr int kCopy = 8;  // 16-byte pieces in flight per thread
  u32x4 cp[kCopy];
  int cdst[kCopy];
  auto copy_load = [&](int it) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kCopy; ++k) {
      const int i = min((it * kCopy + k) * NT + tid, ncopy - 1);  // clamped: loads stay unconditional
      const int slot = i / n16, pc = i - slot * n16;
      cp[k] = *reinterpret_cast<const u32x4*>(ep.stage + (size_t)srow(slot) * rowb + (size_t)pc * 16);
      cdst[k] = slot * (RS + 32) + pc * 16;
    }
  };
  auto copy_store = [&](int it) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kCopy; ++k)
      if ((it * kCopy + k) * NT + tid < ncopy) *reinterpret_cast<u32x4*>(xs + cdst[k]) = cp[k];
  };
  copy_load(0);

  auto rows_of = [&](int pw, int jj, int& n0, int& n1) __attribute__((always_inline)) {
    const int q0 = rb + (wave * PW + pw) * RPS + jj;
    n0 = q0;
    n1 = MODE == 0 ? q0 : q0 + 4;
  };
  // codes of the step's groups for the lane's two rows (and their scales)
  auto load = [&](int st, u32x4 (&va)[UG], u32x4 (&vb)[UG], uint32_t (&sa)[UG],
                  uint32_t (&sb)[UG], SVec& sv) __attribute__((always_inline)) {
    const int pw = st / NCH, ch = st - pw * NCH;
    int n0, n1;
    rows_of(pw, j, n0, n1);
    const size_t ra = (size_t)g * N + min(n0, N - 1), rbb = (size_t)g * N + min(n1, N - 1);
#pragma unroll
    for (int uu = 0; uu < UG; ++uu) {
      const int c = min(b + 16 * (ch * UG + uu), G - 1);  // clamped groups contribute zero
      const size_t ga = ra * G + c, gb = rbb * G + c;
      va[uu] = ld16_stream(ma.p + ga * 16);
      vb[uu] = ld16_stream(mb.p + gb * 16);
      if constexpr (!SV) {
        sa[uu] = (uint32_t)ma.sc[ga] | ((uint32_t)ma.mn[ga] << 16);
        sb[uu] = (uint32_t)mb.sc[gb] | ((uint32_t)mb.mn[gb] << 16);
      }
    }
    if constexpr (SV) {
      // segment (row set rs, array kind, row jj): 16 UG groups, 4 lanes each
      const int sg = lane >> 2, part = lane & 3;
      const int rs = sg >> 3, kind = (sg >> 2) & 1, jj = sg & 3;
      int m0, m1;
      rows_of(pw, jj, m0, m1);
      const int n = min(rs ? m1 : m0, N - 1);
      const MatStack& m = rs ? mb : ma;
      const uint16_t* arr = kind ? m.mn : m.sc;
      int gs = 16 * UG * ch + 4 * UG * part;
      gs = gs < G ? gs : 0;  // past the row's end: any in-bounds groups (unused)
      sv = *reinterpret_cast<const SVec*>(arr + ((size_t)g * N + n) * G + gs);
    }
  };
  u32x4 va[UG], vb[UG], nva[UG], nvb[UG];
  uint32_t sa[UG], sb[UG], nsa[UG], nsb[UG];
  SVec sv, nsv;
  load(0, va, vb, sa, sb, sv);
  copy_store(0);
  for (int it = 1; it * kCopy * NT < ncopy; ++it) {
    copy_load(it);
    copy_store(it);
  }
  for (int i = tid; i < G * 4; i += NT) {
    const int c = i >> 2, r = i & 3;
    reinterpret_cast<float*>(xsum4)[i] = r < nr ? ep.gsum[(size_t)srow(r) * G + c] : 0.f;
  }
  if (tid < 4) rfac[tid] = ep.fac[srow(min(tid, nr - 1))];
  __syncthreads();

  const int jr = min(j, nr - 1);  // A rows past the slots repeat the last (never stored)
  const uint8_t* xa = xs + (size_t)jr * (RS + 32);
  const int fo = u4_swz(b);       // swizzle of the lane's groups b + 16u
  float fac[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) fac[i] = rfac[i];
  const uint32_t magic = opaque_v(0x64006400u);
  const uint32_t mlo = opaque_s(0x000F000Fu), mhi = opaque_s(0x00F000F0u);

  // per route: sum over groups of s * D (aS) and of m * group sum (aM)
  float aS0[4], aM0[4], aS1[4], aM1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { aS0[i] = aM0[i] = aS1[i] = aM1[i] = 0.f; }
#pragma unroll 1
  for (int st = 0; st < nsteps; ++st) {
    load(min(st + 1, nsteps - 1), nva, nvb, nsa, nsb, nsv);
    const int pw = st / NCH, ch = st - pw * NCH;
    if constexpr (SV) *reinterpret_cast<SVec*>(sbuf + lane * (8 * UG)) = sv;
#pragma unroll
    for (int uu = 0; uu < UG; ++uu) {
      const int c = b + 16 * (ch * UG + uu);
      const int cc = min(c, G - 1);
      const uint8_t* xg = xa + (size_t)cc * 128;
      f32x4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 pe = *reinterpret_cast<const u32x4*>(xg + (((2 * q) ^ fo) << 4));
        const u32x4 po = *reinterpret_cast<const u32x4*>(xg + (((2 * q + 1) ^ fo) << 4));
        const uint32_t w0 = va[uu][q], w1 = vb[uu][q];
        const uint32_t w08 = w0 >> 8, w18 = w1 >> 8;
        // codes (0, 4, 2, 6) and 16 x codes (1, 5, 3, 7) of word q
        const f16x4 b0e = codes4(and_or(w0, mlo, magic), and_or(w08, mlo, magic));
        const f16x4 b0o = codes4(and_or(w0, mhi, magic), and_or(w08, mhi, magic));
        const f16x4 b1e = codes4(and_or(w1, mlo, magic), and_or(w18, mlo, magic));
        const f16x4 b1o = codes4(and_or(w1, mhi, magic), and_or(w18, mhi, magic));
        const f16x4 ahe = __builtin_bit_cast(f16x4, u32x2{pe[0], pe[1]});
        const f16x4 ale = __builtin_bit_cast(f16x4, u32x2{pe[2], pe[3]});
        const f16x4 aho = __builtin_bit_cast(f16x4, u32x2{po[0], po[1]});
        const f16x4 alo = __builtin_bit_cast(f16x4, u32x2{po[2], po[3]});
        d0 = __builtin_amdgcn_mfma_f32_4x4x4f16(ahe, b0e, d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_4x4x4f16(ahe, b1e, d1, 0, 0, 0);
        d0 = __builtin_amdgcn_mfma_f32_4x4x4f16(aho, b0o, d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_4x4x4f16(aho, b1o, d1, 0, 0, 0);
        d0 = __builtin_amdgcn_mfma_f32_4x4x4f16(ale, b0e, d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_4x4x4f16(ale, b1e, d1, 0, 0, 0);
        d0 = __builtin_amdgcn_mfma_f32_4x4x4f16(alo, b0o, d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_4x4x4f16(alo, b1o, d1, 0, 0, 0);
      }
      uint32_t scm0, scm1;  // scale | min << 16 of row sets 0 and 1
      if constexpr (SV) {
        const uint16_t* sp = reinterpret_cast<const uint16_t*>(sbuf);
        const int gl = b + 16 * uu;
        constexpr int SEG = 16 * UG;  // u16 per segment
        scm0 = (uint32_t)sp[(0 + j) * SEG + gl] | ((uint32_t)sp[(4 + j) * SEG + gl] << 16);
        scm1 = (uint32_t)sp[(8 + j) * SEG + gl] | ((uint32_t)sp[(12 + j) * SEG + gl] << 16);
      } else {
        scm0 = sa[uu];
        scm1 = sb[uu];
      }
      // groups past the row's end contribute zero (scale and min +0); the
      // f16 values enter the FMAs directly (mixed-precision FMA)
      const bool ok = c < G;
      scm0 = ok ? scm0 : 0u;
      scm1 = ok ? scm1 : 0u;
      const _Float16 s0 = __builtin_bit_cast(_Float16, (uint16_t)scm0);
      const _Float16 m0 = __builtin_bit_cast(_Float16, (uint16_t)(scm0 >> 16));
      const _Float16 s1 = __builtin_bit_cast(_Float16, (uint16_t)scm1);
      const _Float16 m1 = __builtin_bit_cast(_Float16, (uint16_t)(scm1 >> 16));
      const f32x4 xsm = xsum4[cc];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        aS0[i] = fmaf((float)s0, d0[i], aS0[i]);
        aM0[i] = fmaf((float)m0, xsm[i], aM0[i]);
        aS1[i] = fmaf((float)s1, d1[i], aS1[i]);
        aM1[i] = fmaf((float)m1, xsm[i], aM1[i]);
      }
    }
    if (ch == NCH - 1) {
      // the pair's rows are done: sum the 16 blocks (lanes j, j+4, ..., j+60)
      float t0[4], t1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float a = fmaf(aS0[i], fac[i], aM0[i]);
        float c2 = fmaf(aS1[i], fac[i], aM1[i]);
        a += dpp_f<kDppRowRor4>(a);
        a += dpp_f<kDppRowRor8>(a);
        a += __shfl_xor(a, 16, 64);
        a += __shfl_xor(a, 32, 64);
        c2 += dpp_f<kDppRowRor4>(c2);
        c2 += dpp_f<kDppRowRor8>(c2);
        c2 += __shfl_xor(c2, 16, 64);
        c2 += __shfl_xor(c2, 32, 64);
        t0[i] = a;
        t1[i] = c2;
        aS0[i] = aM0[i] = aS1[i] = aM1[i] = 0.f;
      }
      if (b == 0) {
        int n0, n1;
        rows_of(pw, j, n0, n1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i < nr) {
            if constexpr (MODE == 0) {
              const int route = ws_route(p.perm[base + r0 + i], R);
              if (n0 < N) p.h[(size_t)route * N + n0] = act_f<ACT>(t0[i]) * t1[i];
            } else {  // rows of y in the expert-grouped order (position, not route id)
              const size_t pos = (size_t)(base + r0 + i);
              if (n0 < N) p.y[pos * N + n0] = t0[i];
              if (n1 < N) p.y[pos * N + n1] = t1[i];
            }
          }
        }
      }
    }
#pragma unroll
    for (int uu = 0; uu < UG; ++uu) { va[uu] = nva[uu]; sa[uu] = nsa[uu]; vb[uu] = nvb[uu]; sb[uu] = nsb[uu]; }
    sv = nsv;
  }
}

}  // namespace moe
