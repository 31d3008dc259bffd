// Weight-only FP8 (OCP E4M3) copies of the decode projections: the per-output-channel
// quantiser and the export of its codes.  Generation is bandwidth bound, and 8-bit
// weights halve the bytes each decode step streams (Chapter 11 "System Architecture &
// Infrastructure at Scale", section "The Generation Bottleneck: Quantitative
// Analysis", Table 11.4 and the optimisation list after it).
#include "common.h"
#include "kernels.h"

namespace he {

// E4M3 code of y by round-to-nearest-even, saturating at +-448 (E4M3 has no
// infinity; 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals
// k 2^-9).  From the format: below 2^-6 the grid step is 2^-9 and the code is the
// count of steps (count 8 is the smallest normal, code 8); above, the step is
// 2^(e - 3) for |y| in [2^e, 2^(e+1)) and the code is (e + 7) << 3 | (mantissa).
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  if (!(a < 464.f)) return sign | 0x7Eu;                 // 448 and beyond saturate to 448
  if (a < 0x1p-6f) return sign | (uint32_t)__builtin_rintf(a * 0x1p9f);
  int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;
  uint32_t r = (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 3 - e));   // 8 .. 16, exact scaling
  if (r == 16u) { r = 8u; ++e; }
  return sign | ((uint32_t)(e + 7) << 3) | (r - 8u);
}

// One block of 256 threads per row n: amax over the row (any order gives the same
// maximum), scale = amax / 448 in float32 (1 for a zero row), codes of W / scale.
// W is bf16 in layout w_il (il_off); each thread takes runs of 8 consecutive k.
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const bf16* __restrict__ W, int K, int w_il,
                                                           uint8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ float red[4];
  const int n = blockIdx.x, tid = threadIdx.x;
  float amax = 0.f;
  for (int k = tid * 8; k < K; k += 256 * 8) {
    const uint4 u = *reinterpret_cast<const uint4*>(W + il_off(n, k, K, w_il));
    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(w4[i] << 16)), fabsf(__uint_as_float(w4[i] & 0xffff0000u))));
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax > 0.f ? amax / 448.f : 1.f;       // correctly rounded division
  for (int k = tid * 8; k < K; k += 256 * 8) {
    const uint4 u = *reinterpret_cast<const uint4*>(W + il_off(n, k, K, w_il));
    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
    uint32_t c[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[2 * i] = f32_to_e4m3(__uint_as_float(w4[i] << 16) / s);
      c[2 * i + 1] = f32_to_e4m3(__uint_as_float(w4[i] & 0xffff0000u) / s);
    }
    uint2 o;
    o.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    o.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    *reinterpret_cast<uint2*>(q + f8_off(n, k, K)) = o;   // 8 consecutive k: 8 consecutive bytes
  }
  if (tid == 0) scale[n] = s;
}

void launch_quantize_fp8(const void* W, int N, int K, int w_il, uint8_t* q, float* scale, hipStream_t st) {
  quantize_fp8_kernel<<<N, 256, 0, st>>>((const bf16*)W, K, w_il, q, scale);
}

// Codes back to row-major [N][K] (one thread per 8 consecutive k).
__global__ __launch_bounds__(256) void fp8_rowmajor_kernel(const uint8_t* __restrict__ q, int N, int K,
                                                           uint8_t* __restrict__ out) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x, units = (size_t)N * (K / 8);
  if (i >= units) return;
  const int n = (int)(i / (K / 8)), k = (int)(i % (K / 8)) * 8;
  *reinterpret_cast<uint2*>(out + (size_t)n * K + k) = *reinterpret_cast<const uint2*>(q + f8_off(n, k, K));
}

void launch_fp8_rowmajor(const uint8_t* q, int N, int K, uint8_t* out, hipStream_t st) {
  const size_t units = (size_t)N * (K / 8);
  fp8_rowmajor_kernel<<<(unsigned)((units + 255) / 256), 256, 0, st>>>(q, N, K, out);
}

}  // namespace he
