// Decode-step projections of libhe: Y[M,N] = X[M,K] W[N,K]^T with M = batch.
//
// Generation streams every weight once per token (paper summary, "Inference Mode:
// Generation Phase Optimizations": generation is bound by memory bandwidth, the
// kernels are laid out for sequential weight access).  Each wave owns 16 rows of
// W and streams them with 16-byte loads straight into the A operand of
// v_mfma_f32_16x16x32_bf16 (a lane holds 8 consecutive k of one row, four lanes
// cover 64 contiguous bytes); the small activation X (B rows) is the B operand,
// read from L2 and shared by the WG's waves through the L1.  Column blocks of
// WAVES*16 rows and an optional split over K give enough WGs to fill the chip.
// Outputs: split-K partials (reduced later in a fixed order by the consumer
// kernel), bias+ReLU, or a per-block greedy argmax (+ optional logits).
#include "common.h"
#include "kernels.h"

namespace he {

constexpr int kGvWaves = 4;                   // 64 output rows per WG
constexpr int kGvRows = kGvWaves * 16;

int gemv_argmax_blocks(int /*dt*/, int N) { return (N + kGvRows - 1) / kGvRows; }

__device__ __forceinline__ bool gv_better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Per-row (m) argmax over this WG's columns; values[r] are columns n0w + 4*g + r.
template <int MT>
__device__ __forceinline__ void argmax_epilogue(const f32x4 (&acc)[MT], int n_wave0, int N, int M,
                                                const GemvArgs& g) {
  __shared__ float sv[kGvWaves][MT * 16];
  __shared__ int si[kGvWaves][MT * 16];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, grp = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + (lane & 15);
    float bv = -INFINITY;
    int bi = min(n_wave0 + grp * 4, N - 1);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = n_wave0 + grp * 4 + r;
      if (n < N) {
        float v = acc[mt][r];
        if (g.logits && m < M) g.logits[(size_t)m * N + n] = v;
        if (gv_better(v, n, bv, bi)) { bv = v; bi = n; }
      }
    }
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
      float ov = __shfl_xor(bv, o, 64);
      int oi = __shfl_xor(bi, o, 64);
      if (gv_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (grp == 0) { sv[wv][mt * 16 + (lane & 15)] = bv; si[wv][mt * 16 + (lane & 15)] = bi; }
  }
  __syncthreads();
  for (int m = threadIdx.x; m < MT * 16; m += blockDim.x) {
    float bv = sv[0][m];
    int bi = si[0][m];
    for (int w = 1; w < kGvWaves; ++w)
      if (gv_better(sv[w][m], si[w][m], bv, bi)) { bv = sv[w][m]; bi = si[w][m]; }
    if (m < M) {
      g.best_val[(size_t)m * g.n_blocks + blockIdx.x] = bv;
      g.best_idx[(size_t)m * g.n_blocks + blockIdx.x] = bi;
    }
  }
  if (g.bump && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *g.bump += 1;
}

template <int MT, int OUT>
__global__ __launch_bounds__(kGvWaves * 64) void gemv_bf16_kernel(const bf16* __restrict__ X,
                                                                  const bf16* __restrict__ W,
                                                                  int M, int N, int K,
                                                                  GemvArgs g) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n_wave0 = blockIdx.x * kGvRows + wv * 16;
  const int row = min(n_wave0 + (lane & 15), N - 1);   // clamp: ragged last block
  const int ko = (lane >> 4) * 8;
  const int steps = K / 32;
  const int s0 = (int)((long)blockIdx.y * steps / gridDim.y);
  const int s1 = (int)((long)(blockIdx.y + 1) * steps / gridDim.y);

  const bf16* wp = W + (size_t)row * K + ko;
  const bf16* xp = X + (size_t)(lane & 15) * K + ko;

  f32x4 acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll 4
  for (int s = s0; s < s1; ++s) {
    const int k = s * 32;
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(wp + k);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(xp + (size_t)mt * 16 * K + k);
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[mt], 0, 0, 0);
    }
  }

  // acc[mt][r] = Y[m = mt*16 + lane%16][n = n_wave0 + 4*(lane/16) + r]
  if (OUT == GV_ARGMAX) {
    argmax_epilogue<MT>(acc, n_wave0, N, M, g);
    return;
  }
  const int nb = n_wave0 + (lane >> 4) * 4;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + (lane & 15);
    if (m >= M) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = nb + r;
      if (n >= N) continue;
      if (OUT == GV_PARTIAL) {
        g.parts[((size_t)blockIdx.y * M + m) * N + n] = acc[mt][r];
      } else {   // GV_RELU
        float v = acc[mt][r] + bf2f(((const bf16*)g.bias)[n]);
        ((bf16*)g.out)[(size_t)m * N + n] = f2bf(fmaxf(v, 0.f));
      }
    }
  }
}

// fp32 models: one thread per (m, n), 64 columns per WG (same blocking as above).
template <int OUT>
__global__ __launch_bounds__(64) void gemv_f32_kernel(const float* __restrict__ X,
                                                      const float* __restrict__ W, int M, int N,
                                                      int K, GemvArgs g) {
  const int n = blockIdx.x * kGvRows + threadIdx.x;
  const int m = blockIdx.z;
  const int s0 = (int)((long)blockIdx.y * K / gridDim.y), s1 = (int)((long)(blockIdx.y + 1) * K / gridDim.y);
  float acc = 0.f;
  if (n < N)
    for (int k = s0; k < s1; ++k) acc = fmaf(X[(size_t)m * K + k], W[(size_t)n * K + k], acc);
  if (OUT == GV_PARTIAL) {
    if (n < N) g.parts[((size_t)blockIdx.y * M + m) * N + n] = acc;
  } else if (OUT == GV_RELU) {
    if (n < N) ((float*)g.out)[(size_t)m * N + n] = fmaxf(acc + ((const float*)g.bias)[n], 0.f);
  } else {
    if (n < N && g.logits) g.logits[(size_t)m * N + n] = acc;
    float bv = n < N ? acc : -INFINITY;
    int bi = n < N ? n : N - 1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      float ov = __shfl_xor(bv, o, 64);
      int oi = __shfl_xor(bi, o, 64);
      if (gv_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (threadIdx.x == 0) {
      g.best_val[(size_t)m * g.n_blocks + blockIdx.x] = bv;
      g.best_idx[(size_t)m * g.n_blocks + blockIdx.x] = bi;
      if (g.bump && blockIdx.x == 0 && m == 0) *g.bump += 1;
    }
  }
}

template <int OUT>
static void gemv_dispatch(int dt, const void* X, const void* W, int M, int N, int K,
                          const GemvArgs& g, hipStream_t st) {
  const int nblk = (N + kGvRows - 1) / kGvRows;
  const int splits = OUT == GV_PARTIAL ? g.splits : 1;
  if (dt == DT_BF16) {
    dim3 grid(nblk, splits);
    const int mt = (M + 15) / 16;
    if (mt <= 1) gemv_bf16_kernel<1, OUT><<<grid, kGvWaves * 64, 0, st>>>((const bf16*)X, (const bf16*)W, M, N, K, g);
    else if (mt <= 2) gemv_bf16_kernel<2, OUT><<<grid, kGvWaves * 64, 0, st>>>((const bf16*)X, (const bf16*)W, M, N, K, g);
    else if (mt <= 4) gemv_bf16_kernel<4, OUT><<<grid, kGvWaves * 64, 0, st>>>((const bf16*)X, (const bf16*)W, M, N, K, g);
    else gemv_bf16_kernel<8, OUT><<<grid, kGvWaves * 64, 0, st>>>((const bf16*)X, (const bf16*)W, M, N, K, g);
  } else {
    dim3 grid(nblk, splits, M);
    gemv_f32_kernel<OUT><<<grid, 64, 0, st>>>((const float*)X, (const float*)W, M, N, K, g);
  }
}

void launch_gemv(int dt, const void* X, const void* W, int M, int N, int K, const GemvArgs& g,
                 hipStream_t st) {
  switch (g.out_mode) {
    case GV_RELU: gemv_dispatch<GV_RELU>(dt, X, W, M, N, K, g, st); break;
    case GV_ARGMAX: gemv_dispatch<GV_ARGMAX>(dt, X, W, M, N, K, g, st); break;
    default: gemv_dispatch<GV_PARTIAL>(dt, X, W, M, N, K, g, st); break;
  }
}

}  // namespace he
