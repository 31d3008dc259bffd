// Device-side helpers shared by the HIP kernels of libhe (gfx950, wave64).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace he {

typedef uint16_t bf16;   // bfloat16 bit pattern

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(bf16 b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16 f2bf(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(bf16, h);
}

// Storage-type load/store: T is float (fp32 models) or bf16 (bf16 models).
__device__ __forceinline__ float ld(const float* p) { return *p; }
__device__ __forceinline__ float ld(const bf16* p) { return bf2f(*p); }
__device__ __forceinline__ void st(float* p, float v) { *p = v; }
__device__ __forceinline__ void st(bf16* p, float v) { *p = f2bf(v); }

template <typename T> __device__ __forceinline__ T to_store(float v);
template <> __device__ __forceinline__ float to_store<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 to_store<bf16>(float v) { return f2bf(v); }

// Eight consecutive storage elements widened to float.
__device__ __forceinline__ void load8(const bf16* p, float* out) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  out[0] = __uint_as_float(u.x << 16); out[1] = __uint_as_float(u.x & 0xffff0000u);
  out[2] = __uint_as_float(u.y << 16); out[3] = __uint_as_float(u.y & 0xffff0000u);
  out[4] = __uint_as_float(u.z << 16); out[5] = __uint_as_float(u.z & 0xffff0000u);
  out[6] = __uint_as_float(u.w << 16); out[7] = __uint_as_float(u.w & 0xffff0000u);
}
__device__ __forceinline__ void load8(const float* p, float* out) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}
__device__ __forceinline__ void store8(bf16* p, const float* v) {
  uint4 u;
  u.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
  u.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
  u.z = (uint32_t)f2bf(v[4]) | ((uint32_t)f2bf(v[5]) << 16);
  u.w = (uint32_t)f2bf(v[6]) | ((uint32_t)f2bf(v[7]) << 16);
  *reinterpret_cast<uint4*>(p) = u;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Reductions over the 64 lanes of a wave (all lanes active), the same bits in every
// lane: DPP moves within each row of 16 lanes (swap neighbours, swap pairs, mirror
// within 8, mirror within 16), then the gfx950 lane swaps between rows 16 and 32
// apart.  Each step combines two values with a commutative operation, so partner lanes
// compute the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = op(v, dpp_move<0xB1>(v));     // quad_perm [1,0,3,2]
  v = op(v, dpp_move<0x4E>(v));     // quad_perm [2,3,0,1]
  v = op(v, dpp_move<0x141>(v));    // row_half_mirror
  v = op(v, dpp_move<0x140>(v));    // row_mirror
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}

// ---------------------------------------------------------------------------------
// Inference layout of a bf16 weight W[N][K] (N % 16 == 0, K % 32 == 0).  W is cut into
// blocks of 16 rows x BW columns, BW = 2^il the largest power of two <= 512 dividing
// K.  A block keeps its place in memory (16 row segments of BW elements), but its
// 16-byte units are reordered so that the 16 x 32 slice feeding one MFMA
// (v_mfma_f32_16x16x32_bf16 A operand: lane l holds row l % 16, k 8 (l / 16) .. + 8)
// is 1 KB of consecutive bytes, lane-ordered.  Unit (row j, unit column u) of a block
// goes to position p = (u / 4) * 64 + (u % 4) * 16 + j, which is stored at block row
// p / (BW / 8), unit column p % (BW / 8).  il == 0 means plain row-major.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ size_t il_off(int n, int k, int K, int il) {
  if (il == 0) return (size_t)n * K + k;
  const int bw = 1 << il, lgu = il - 3;
  const int j = n & 15, kb = k & (bw - 1), u = kb >> 3;
  const int p = ((u >> 2) << 6) | ((u & 3) << 4) | j;
  return (size_t)((n & ~15) + (p >> lgu)) * K + (k - kb) + ((p & ((1 << lgu) - 1)) << 3) + (k & 7);
}

// Offset of lane l's 8 elements of MFMA fragment (row block rb, k-step s): rows
// 16 rb + l % 16, k = 32 s + 8 (l / 16) .. + 8, in the inference layout or, for
// il == 0, row-major (then a fragment is 16 row pieces of 64 bytes).
__device__ __forceinline__ size_t il_frag(int rb, int s, int lane, int K, int il) {
  if (il == 0) return (size_t)(rb * 16 + (lane & 15)) * K + s * 32 + ((lane >> 4) << 3);
  const int lgu = il - 3, fpb = 1 << (il - 5);         // units per block row, fragments per block
  const int q = s & (fpb - 1), p = (q << 6) | lane;
  return (size_t)(rb * 16 + (p >> lgu)) * K + ((s >> (il - 5)) << il) + ((p & ((1 << lgu) - 1)) << 3);
}

// Fragment-tiled activations X[M][K] (M <= 16 mt): the B operand of one MFMA k-step s
// and row tile t (rows 16 t .. + 16, k 32 s .. + 32) is 1 KB at ((s * mt + t) * 512),
// lane l holding row 16 t + l % 16, k 32 s + 8 (l / 16) .. + 8.
__device__ __forceinline__ size_t xt_off(int m, int k, int mt) {
  return ((size_t)((k >> 5) * mt + (m >> 4)) << 9) + (((m & 15) | (((k >> 3) & 3) << 4)) << 3) + (k & 7);
}

// 16 bytes read once (a weight or KV stream): a non-temporal load, which does not keep
// the line in the caches.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_once(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// FP8 (E4M3) decode-weight layout of W [N][K] (N % 16 == 0, K % 64 == 0): blocks of
// 16 rows x 64 k, 1 KB each, row block major then k, so a row block's whole K range
// is contiguous.  Lane l of a block holds row l % 16 and, in its 16 bytes, k 8 (l / 16)
// .. + 8 of the block's first 32-wide k-step (bytes 0..7) and of its second (bytes
// 8..15): one 16-byte load per lane gives the MFMA A operands of two k-steps.
__device__ __forceinline__ size_t f8_off(int n, int k, int K) {
  return ((size_t)(n >> 4) * (K >> 6) + (k >> 6)) * 1024 + (((n & 15) + 16 * ((k & 31) >> 3)) << 4) +
         (k & 7) + 8 * ((k >> 5) & 1);
}

// Activation layout code of a [M][K] storage-type matrix: 0 row-major; mt > 0 the
// decode fragment tiling with mt row tiles (xt_off); -il < 0 the inference layout with
// block width 2^il over K (il_off, as for weights), the prompt-pass GEMM operand.
__device__ __forceinline__ size_t act_off(int m, int k, int K, int lay) {
  return lay > 0 ? xt_off(m, k, lay) : il_off(m, k, K, -lay);
}

// Counter-based generator Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011): ten rounds of the 4 x 64-bit bijection on the
// counter, the key advanced by the Weyl increments after every round.
__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(M0, c[0]), lo0 = M0 * c[0];
    const uint64_t hi1 = __umul64hi(M1, c[2]), lo1 = M1 * c[2];
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
    k0 += W0; k1 += W1;
  }
}

// Gumbel noise G = -log(-log U) of vocabulary columns 4 n4 .. 4 n4 + 3 for batch row
// `row` generating the token at `position`: one generator block at counter
// (n4, row, position, 0), key (seed, 0); column 4 n4 + w takes word w, and
// U = (its top 23 bits + 1/2) / 2^23, exact in float32 and inside [2^-24, 1 - 2^-24]
// (24 bits would round the largest value up to U = 1, an infinite G).
__device__ __forceinline__ void gumbel4(uint64_t seed, int row, int position, int n4, float g[4]) {
  uint64_t c[4] = {(uint64_t)n4, (uint64_t)row, (uint64_t)position, 0ull};
  philox4x64_10(c, seed, 0ull);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float u = ((float)(uint32_t)(c[w] >> 41) + 0.5f) * 0x1p-23f;
    g[w] = -logf(-logf(u));
  }
}

// Sum over the block in a fixed order (deterministic).  `red` holds >= nwaves floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int nw = (blockDim.x + kWave - 1) / kWave;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

}  // namespace he
