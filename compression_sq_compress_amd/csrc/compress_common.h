// Device helpers shared by the compress kernels: the bf16 x3 split of fp32
// values and the 16x16x32 bf16 MFMA.
#pragma once
#include "devcommon.h"

namespace sq {

__device__ __forceinline__ void split3(const float *v, uint4 &p0, uint4 &p1, uint4 &p2) {
  uint16_t a[8], b[8], c[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float x = v[e];
    a[e] = f32_to_bf16_rne(x);
    x -= __uint_as_float((uint32_t)a[e] << 16);
    b[e] = f32_to_bf16_rne(x);
    x -= __uint_as_float((uint32_t)b[e] << 16);
    c[e] = f32_to_bf16_rne(x);
  }
  p0 = make_uint4(a[0] | (a[1] << 16), a[2] | (a[3] << 16), a[4] | (a[5] << 16), a[6] | (a[7] << 16));
  p1 = make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16));
  p2 = make_uint4(c[0] | (c[1] << 16), c[2] | (c[3] << 16), c[4] | (c[5] << 16), c[6] | (c[7] << 16));
}

__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

}  // namespace sq
