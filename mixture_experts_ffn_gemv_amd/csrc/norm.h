// Optional pre-FFN RMSNorm: the layer's input rows replaced by
// x[t] / sqrt(mean(x[t]^2) + eps) * w, stored in the activation type
// (bf16 rounded to nearest even), so every later kernel reads the
// normalised rows unchanged.  One workgroup per token; each thread sums
// the squares of its 4-element chunks in a fixed order, and the waves'
// sums are added in wave order, so the result does not depend on timing.
#pragma once

#include "common.h"

namespace moe {

template <typename XT>
__global__ __launch_bounds__(256) void k_rmsnorm(const XT* __restrict__ x,
                                                 const float* __restrict__ w, float eps, int H,
                                                 XT* __restrict__ y) {
  __shared__ float s_part[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const XT* xr = x + (size_t)t * H;
  XT* yr = y + (size_t)t * H;
  auto load4 = [&](int c, float (&v)[4]) {
    if constexpr (sizeof(XT) == 2) {
      const u32x2 b = *reinterpret_cast<const u32x2*>(xr + c);
      v[0] = bf16lo(b[0]); v[1] = bf16hi(b[0]); v[2] = bf16lo(b[1]); v[3] = bf16hi(b[1]);
    } else {
      const f32x4 f = *reinterpret_cast<const f32x4*>(xr + c);
      v[0] = f[0]; v[1] = f[1]; v[2] = f[2]; v[3] = f[3];
    }
  };
  float ss = 0.f;
  for (int c = tid * 4; c < H; c += 1024) {
    float v[4];
    load4(c, v);
#pragma unroll
    for (int q = 0; q < 4; ++q) ss = fmaf(v[q], v[q], ss);
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) s_part[tid >> 6] = ss;
  __syncthreads();
  const float mean = (s_part[0] + s_part[1] + s_part[2] + s_part[3]) / (float)H;
  const float r = 1.0f / sqrtf(mean + eps);
  for (int c = tid * 4; c < H; c += 1024) {
    float v[4];
    load4(c, v);
    const f32x4 wv = *reinterpret_cast<const f32x4*>(w + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = v[q] * r * wv[q];
    if constexpr (sizeof(XT) == 2) {
      u32x2 o;
      o[0] = pack_bf16x2(v[0], v[1]);
      o[1] = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<u32x2*>(yr + c) = o;
    } else {
      *reinterpret_cast<f32x4*>(yr + c) = f32x4{v[0], v[1], v[2], v[3]};
    }
  }
}

}  // namespace moe
