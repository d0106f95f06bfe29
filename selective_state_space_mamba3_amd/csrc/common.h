// Device helpers shared by the gfx950 kernels of the Mamba-3 forward path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m3 {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// v_mfma_f32_16x16x4_f32, one 16x16 block, fp32 in / fp32 accumulate.
// Lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16]; register r of the
// result in lane l is D[4 * (l / 16) + r][l % 16].
__device__ __forceinline__ floatx4 mfma16(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float sigmoidf_acc(float u) {
  // 1 / (1 + e^-u) without overflow for large |u|.
  if (u >= 0.f) return 1.f / (1.f + expf(-u));
  const float e = expf(u);
  return e / (1.f + e);
}

__device__ __forceinline__ float siluf_acc(float u) { return u * sigmoidf_acc(u); }

__device__ __forceinline__ float softplusf_acc(float u) {
  // max(u, 0) + log1p(e^-|u|): exact for large |u|, no overflow.
  return fmaxf(u, 0.f) + log1pf(expf(-fabsf(u)));
}

__device__ __forceinline__ floatx4 lds_read4(const float* p) {
  return *reinterpret_cast<const floatx4*>(p);
}

// Map a hardware workgroup id to a logical work unit so that consecutive
// logical units land on the same XCD: the dispatcher hands workgroup i to
// XCD i % 8, so logical units are dealt out in eight contiguous runs.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t i, uint32_t n) {
  const uint32_t per = n / 8u, rem = n % 8u;
  const uint32_t xcd = i % 8u, j = i / 8u;
  return xcd < rem ? xcd * (per + 1u) + j : rem * (per + 1u) + (xcd - rem) * per + j;
}

}  // namespace m3
