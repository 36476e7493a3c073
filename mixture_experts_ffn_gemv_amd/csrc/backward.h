// Backward kernels of two steps of the layer, for training: the
// routing-weighted combine and the gated activation (the pair of backward
// kernels mlx-native's moe_dispatch.rs adds for moe_weighted_sum_seq and
// moe_swiglu_seq).  Both are streaming passes over f32 arrays, bound by
// HBM: every input element is read once and every output written once.
#pragma once

#include "common.h"

namespace moe {

// Combine backward, one workgroup per (token t, slot j):
//   dy[t,j,:] = w[t,j] * dout[t,:]     dw[t,j] = y[t,j,:] . dout[t,:]
// dout[t] is read by the k workgroups of token t.  Workgroups are handed
// to the 8 XCDs round-robin (block b to XCD b % 8), so block b serves
// token 8 * (q / k) + b % 8, slot q % k (q = b / 8): the k workgroups of a
// token share one XCD and its L2, and start together, so dout[t] comes
// from HBM once.  The dot product is summed per thread in a fixed order,
// then over the wave and over the 4 waves in wave order: repeat runs agree.
template <bool DY, bool DW>
__global__ __launch_bounds__(256) void k_wsum_backward(const float* __restrict__ w,
                                                       const float* __restrict__ y,
                                                       const float* __restrict__ dout,
                                                       float* __restrict__ dy,
                                                       float* __restrict__ dw, int k, int H,
                                                       int64_t T) {
  __shared__ float s_part[4];
  const size_t q = blockIdx.x >> 3;
  const size_t t = (q / (size_t)k) * 8 + (blockIdx.x & 7);
  if (t >= (size_t)T) return;
  const size_t tj = t * (size_t)k + q % (size_t)k;
  const float wt = w[tj];
  const float* dr = dout + t * H;
  const float* yr = y + tj * H;
  float* dyr = dy + tj * H;
  float acc = 0.f;
  for (int c0 = threadIdx.x * 4; c0 < H; c0 += 2048) {
    // two chunks per pass, both loads issued before either is used
    const int c1 = c0 + 1024;
    const bool ok1 = c1 < H;
    const f32x4 d0 = *reinterpret_cast<const f32x4*>(dr + c0);
    const f32x4 d1 = *reinterpret_cast<const f32x4*>(dr + (ok1 ? c1 : c0));
    f32x4 y0, y1;
    if constexpr (DW) {
      y0 = *reinterpret_cast<const f32x4*>(yr + c0);
      y1 = *reinterpret_cast<const f32x4*>(yr + (ok1 ? c1 : c0));
    }
    if constexpr (DY) {
      *reinterpret_cast<f32x4*>(dyr + c0) = f32x4{wt * d0[0], wt * d0[1], wt * d0[2], wt * d0[3]};
      if (ok1)
        *reinterpret_cast<f32x4*>(dyr + c1) = f32x4{wt * d1[0], wt * d1[1], wt * d1[2], wt * d1[3]};
    }
    if constexpr (DW) {
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = fmaf(y0[q], d0[q], acc);
      if (ok1) {
#pragma unroll
        for (int q = 0; q < 4; ++q) acc = fmaf(y1[q], d1[q], acc);
      }
    }
  }
  if constexpr (DW) {
    acc = wave_sum(acc);
    if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) dw[tj] = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
  }
}

// d/dz of the two activations, with act(z) itself (same forms as act_f):
//   silu:  s = sigmoid(z), act = z s, act' = s (1 + z (1 - s))
//   gelu:  u = c (z + a z^3), th = tanh(u), act = z (1 + th) / 2,
//          act' = (1 + th) / 2 + z (1 - th^2) c (1 + 3 a z^2) / 2
template <int ACT>
__device__ __forceinline__ void act_and_grad(float z, float& a, float& da) {
  if constexpr (ACT == ACT_SILU) {
    const float s = 1.0f / (1.0f + __expf(-z));
    a = z * s;
    da = s * (1.0f + z * (1.0f - s));
  } else {
    const float c = 0.7978845608f, k3 = 0.044715f;
    const float u = c * (z + k3 * z * z * z);
    const float th = 1.0f - 2.0f / (1.0f + __expf(2.0f * u));
    a = 0.5f * z * (1.0f + th);
    da = 0.5f * (1.0f + th) + 0.5f * z * (1.0f - th * th) * c * (1.0f + 3.0f * k3 * z * z);
  }
}

// Gated-activation backward: thread per 4 consecutive features of a row.
template <int ACT>
__global__ __launch_bounds__(256) void k_glu_backward(const float* __restrict__ gate_up,
                                                      const float* __restrict__ dh,
                                                      float* __restrict__ dgu, int64_t rows,
                                                      int I) {
  const int c4 = I / 4;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)rows * c4) return;
  const size_t r = idx / c4;
  const int c = (int)(idx - r * c4) * 4;
  const float* gr = gate_up + r * 2 * I;
  const f32x4 g = *reinterpret_cast<const f32x4*>(gr + c);
  const f32x4 u = *reinterpret_cast<const f32x4*>(gr + I + c);
  const f32x4 d = *reinterpret_cast<const f32x4*>(dh + r * I + c);
  f32x4 dg, du;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float a, da;
    act_and_grad<ACT>(g[q], a, da);
    dg[q] = d[q] * u[q] * da;
    du[q] = d[q] * a;
  }
  float* o = dgu + r * 2 * I;
  *reinterpret_cast<f32x4*>(o + c) = dg;
  *reinterpret_cast<f32x4*>(o + I + c) = du;
}

}  // namespace moe
