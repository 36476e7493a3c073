// Shared device helpers for the gfx950 MoE FFN kernels: storage decode,
// activations, wave-level reductions and the workspace plan shared by the
// host launcher and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_MAX_EXPERTS_DEV 256
#define MOE_MAX_TOP_K_DEV 32

namespace moe {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

enum WeightFormat : int { WF_F32 = 0, WF_BF16 = 1, WF_U4 = 2 };
enum Act : int { ACT_SILU = 0, ACT_GELU_TANH = 1 };

// ------------------------------------------------------------ storage decode
__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}
// f32 -> bf16 bits, round to nearest even (finite values).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}
__device__ __forceinline__ float f16_to_f32(uint16_t v) {
  return static_cast<float>(__builtin_bit_cast(_Float16, v));
}

// ---------------------------------------------------------------- activations
__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }
__device__ __forceinline__ float gelu_tanh_f(float z) {
  // 0.5 z (1 + tanh(u)) with tanh(u) = 1 - 2 / (1 + e^{2u})
  const float u = 0.7978845608f * (z + 0.044715f * z * z * z);
  const float t = 1.0f - 2.0f / (1.0f + __expf(2.0f * u));
  return 0.5f * z * (1.0f + t);
}
template <int ACT>
__device__ __forceinline__ float act_f(float z) {
  if constexpr (ACT == ACT_SILU) return silu_f(z);
  else return gelu_tanh_f(z);
}
__device__ __forceinline__ float sigmoid_f(float z) { return 1.0f / (1.0f + __expf(-z)); }

// ------------------------------------------------------------ wave reductions
// Sum over aligned groups of `width` lanes (width a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
// DPP row operations: xor-1 and xor-2 quad permutes, then the 8-lane
// half-mirror and the 16-lane mirror leave every lane of a 16-lane row with
// the row's reduction; four readlanes combine the rows.  All lanes must be
// active.  The result is wave-uniform.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppRowRor4 = 0x124;   // row_ror:4 (rotate within 16-lane rows)
constexpr int kDppRowRor8 = 0x128;   // row_ror:8
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

constexpr int kDppRowBcast15 = 0x142;  // lane 15 of each row to the next row
constexpr int kDppRowBcast31 = 0x143;  // lane 31 to rows 2 and 3

// Inclusive prefix sum over the wave's lanes (row shifts, then the row
// broadcasts that carry row totals forward).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast15, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast31, 0xC, 0xF, false);
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = threadIdx.x & 63;
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// ------------------------------------------------------------------ loads
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

}  // namespace moe
