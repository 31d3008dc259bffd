// Decode-step projections of libhe: Y[M,N] = X[M,K] W[N,K]^T with M = batch <= 128.
//
// Generation streams every weight once per token (paper summary, "Inference Mode:
// Generation Phase Optimizations": generation is bound by memory bandwidth; the
// inference kernels lay weights out for sequential access).  The kernel is built
// around that stream:
//  * Each wave owns FR x 16 rows of W and loads them straight from HBM into the A
//    operand of v_mfma_f32_16x16x32_bf16 with 16-byte loads (a lane holds 8
//    consecutive k of one row; four lanes cover 64 contiguous bytes), one K-chunk
//    ahead of the MFMAs (register double buffering).
//  * The activation X (B rows, L2 resident) is the B operand.  The WG stages each
//    K-chunk of X in LDS once and its four waves read it from there, so the vector
//    memory path carries W plus only M/(64 FR) of its bytes in X.
//  * Column blocks of 64 FR rows and an optional split over K (partials reduced
//    later, in a fixed order, by the consuming kernel) give enough WGs to cover the
//    256 CUs.
// Outputs: split-K partials, bias+ReLU (rounded), or a per-block greedy argmax
// (+ optional fp32 logits).
#include "common.h"
#include "kernels.h"

namespace he {

constexpr int kCS = 4;                     // 32-wide k-steps per staged chunk
constexpr int kKC = kCS * 32;              // k per chunk
constexpr int kLDX = kKC + 8;              // LDS row stride (bf16): 272 B, conflict-free b128 reads

int gemv_argmax_blocks(int /*dt*/, int N) { return (N + 127) / 128; }   // FR = 2 for the head

// Work split of one decode projection: FR (16-row frags per wave) and K splits.
GemvPlan gemv_plan(int M, int N, int K, bool allow_split) {
  const int mpad = (M + 15) / 16 * 16;
  const int steps = K / 32;
  int smax = 1;
  if (allow_split) {
    smax = std::max(1, K / (16 * mpad));            // partial bytes <= 1/8 of weight bytes
    smax = std::min(smax, std::max(1, steps / (2 * kCS)));
  }
  GemvPlan best{2, 1};
  long best_wg = -1;
  for (int fr = 2; fr >= 1; --fr) {
    const int nb = (N + 64 * fr - 1) / (64 * fr);
    const int s = std::min(smax, std::max(1, (512 + nb - 1) / nb));
    const long wg = (long)nb * s;
    if (wg >= 256) return GemvPlan{fr, s};
    if (wg > best_wg) { best_wg = wg; best = GemvPlan{fr, s}; }
  }
  return best;
}

__device__ __forceinline__ bool gv_better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

template <int MT, int FR>
__device__ __forceinline__ void argmax_epilogue(const f32x4 (&acc)[FR][MT], int n_wave0, int N,
                                                int M, const GemvArgs& g) {
  __shared__ float sv[4][MT * 16];
  __shared__ int si[4][MT * 16];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, grp = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + (lane & 15);
    float bv = -INFINITY;
    int bi = min(n_wave0 + grp * 4, N - 1);
#pragma unroll
    for (int f = 0; f < FR; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = n_wave0 + f * 16 + grp * 4 + r;
        if (n < N) {
          const float v = acc[f][mt][r];
          if (g.logits && m < M) g.logits[(size_t)m * N + n] = v;
          if (gv_better(v, n, bv, bi)) { bv = v; bi = n; }
        }
      }
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (gv_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (grp == 0) { sv[wv][mt * 16 + (lane & 15)] = bv; si[wv][mt * 16 + (lane & 15)] = bi; }
  }
  __syncthreads();
  for (int m = threadIdx.x; m < MT * 16; m += blockDim.x) {
    float bv = sv[0][m];
    int bi = si[0][m];
#pragma unroll
    for (int w = 1; w < 4; ++w)
      if (gv_better(sv[w][m], si[w][m], bv, bi)) { bv = sv[w][m]; bi = si[w][m]; }
    if (m < M) {
      g.best_val[(size_t)m * g.n_blocks + blockIdx.x] = bv;
      g.best_idx[(size_t)m * g.n_blocks + blockIdx.x] = bi;
    }
  }
  if (g.bump && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *g.bump += 1;
}

template <int MT, int FR, int OUT>
__global__ __launch_bounds__(256) void gemv_bf16_kernel(const bf16* __restrict__ X,
                                                        const bf16* __restrict__ W, int M, int N,
                                                        int K, GemvArgs g) {
  constexpr int XR = MT * 16;                 // staged X rows
  constexpr int XCH = XR * (kKC / 8);         // 16-byte pieces per staged chunk
  constexpr int XPT = (XCH + 255) / 256;      // pieces per thread
  __shared__ __attribute__((aligned(16))) bf16 Xs[2][XR * kLDX];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n_wave0 = blockIdx.x * (64 * FR) + wv * 16 * FR;
  const int ko = (lane >> 4) * 8;
  const int steps = K / 32;
  const int s0 = (int)((long)blockIdx.y * steps / gridDim.y);
  const int s1 = (int)((long)(blockIdx.y + 1) * steps / gridDim.y);
  const int nch = (s1 - s0 + kCS - 1) / kCS;

  const bf16* wp[FR];
#pragma unroll
  for (int f = 0; f < FR; ++f)
    wp[f] = W + (size_t)min(n_wave0 + f * 16 + (lane & 15), N - 1) * K + ko;   // clamp ragged block

  f32x4 acc[FR][MT];
#pragma unroll
  for (int f = 0; f < FR; ++f)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[f][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 wr0[FR][kCS], wr1[FR][kCS];
  uint4 xr[XPT];

  auto load_w = [&](int c, bf16x8 (&wr)[FR][kCS]) {
#pragma unroll
    for (int i = 0; i < kCS; ++i) {
      const int s = s0 + c * kCS + i;
#pragma unroll
      for (int f = 0; f < FR; ++f)
        wr[f][i] = (s < s1) ? *reinterpret_cast<const bf16x8*>(wp[f] + (size_t)s * 32) : bf16x8{};
    }
  };
  auto load_x = [&](int c) {
    const int kb = (s0 + c * kCS) * 32, ke = s1 * 32;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int idx = tid + i * 256;
      const int row = idx / (kKC / 8), col = (idx % (kKC / 8)) * 8;
      xr[i] = (idx < XCH && kb + col < ke)
                  ? *reinterpret_cast<const uint4*>(X + (size_t)row * K + kb + col)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_x = [&](int b) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int idx = tid + i * 256;
      if (idx < XCH) {
        const int row = idx / (kKC / 8), col = (idx % (kKC / 8)) * 8;
        *reinterpret_cast<uint4*>(&Xs[b][row * kLDX + col]) = xr[i];
      }
    }
  };
  auto compute = [&](int c, int b, const bf16x8 (&wr)[FR][kCS]) {
#pragma unroll
    for (int i = 0; i < kCS; ++i) {
      if (s0 + c * kCS + i < s1) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const bf16x8 xb = *reinterpret_cast<const bf16x8*>(&Xs[b][(mt * 16 + (lane & 15)) * kLDX + i * 32 + ko]);
#pragma unroll
          for (int f = 0; f < FR; ++f)
            acc[f][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wr[f][i], xb, acc[f][mt], 0, 0, 0);
        }
      }
    }
  };

  load_w(0, wr0);
  load_x(0);
  store_x(0);
  __syncthreads();
  for (int c = 0; c < nch; c += 2) {
    // even chunk: compute from buffer 0 while chunk c+1 streams into buffer 1
    if (c + 1 < nch) { load_w(c + 1, wr1); load_x(c + 1); }
    compute(c, 0, wr0);
    if (c + 1 < nch) store_x(1);
    __syncthreads();
    if (c + 1 >= nch) break;
    if (c + 2 < nch) { load_w(c + 2, wr0); load_x(c + 2); }
    compute(c + 1, 1, wr1);
    if (c + 2 < nch) store_x(0);
    __syncthreads();
  }

  // acc[f][mt][r] = Y[m = mt*16 + lane%16][n = n_wave0 + 16 f + 4 (lane/16) + r]
  if (OUT == GV_ARGMAX) {
    argmax_epilogue<MT, FR>(acc, n_wave0, N, M, g);
    return;
  }
#pragma unroll
  for (int f = 0; f < FR; ++f) {
    const int nb = n_wave0 + f * 16 + (lane >> 4) * 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + (lane & 15);
      if (m >= M) continue;
      if (OUT == GV_PARTIAL) {
        float* dst = g.parts + ((size_t)blockIdx.y * M + m) * N + nb;
        if (nb + 3 < N) {
          *reinterpret_cast<float4*>(dst) = make_float4(acc[f][mt][0], acc[f][mt][1], acc[f][mt][2], acc[f][mt][3]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (nb + r < N) dst[r] = acc[f][mt][r];
        }
      } else {   // GV_RELU
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = nb + r;
          if (n < N) {
            const float v = acc[f][mt][r] + bf2f(((const bf16*)g.bias)[n]);
            ((bf16*)g.out)[(size_t)m * N + n] = f2bf(fmaxf(v, 0.f));
          }
        }
      }
    }
  }
}

// fp32 models: one thread per (m, n), 128 columns per WG, same output blocking.
template <int OUT>
__global__ __launch_bounds__(128) void gemv_f32_kernel(const float* __restrict__ X,
                                                       const float* __restrict__ W, int M, int N,
                                                       int K, GemvArgs g) {
  __shared__ float sv[2];
  __shared__ int si[2];
  const int n = blockIdx.x * 128 + threadIdx.x;
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
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (gv_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = bv; si[threadIdx.x >> 6] = bi; }
    __syncthreads();
    if (threadIdx.x == 0) {
      if (gv_better(sv[1], si[1], bv, bi)) { bv = sv[1]; bi = si[1]; }
      g.best_val[(size_t)m * g.n_blocks + blockIdx.x] = bv;
      g.best_idx[(size_t)m * g.n_blocks + blockIdx.x] = bi;
      if (g.bump && blockIdx.x == 0 && m == 0) *g.bump += 1;
    }
  }
}

template <int OUT, int FR>
static void gemv_bf16_launch(const void* X, const void* W, int M, int N, int K, const GemvArgs& g,
                             int splits, hipStream_t st) {
  dim3 grid((N + 64 * FR - 1) / (64 * FR), splits);
  const int mt = (M + 15) / 16;
  const bf16* x = (const bf16*)X;
  const bf16* w = (const bf16*)W;
  if (mt <= 1) gemv_bf16_kernel<1, FR, OUT><<<grid, 256, 0, st>>>(x, w, M, N, K, g);
  else if (mt <= 2) gemv_bf16_kernel<2, FR, OUT><<<grid, 256, 0, st>>>(x, w, M, N, K, g);
  else if (mt <= 4) gemv_bf16_kernel<4, FR, OUT><<<grid, 256, 0, st>>>(x, w, M, N, K, g);
  else gemv_bf16_kernel<8, FR, OUT><<<grid, 256, 0, st>>>(x, w, M, N, K, g);
}

template <int OUT>
static void gemv_dispatch(int dt, const void* X, const void* W, int M, int N, int K,
                          const GemvArgs& g, hipStream_t st) {
  if (dt == DT_BF16) {
    const int splits = OUT == GV_PARTIAL ? g.splits : 1;
    const int fr = OUT == GV_ARGMAX ? 2 : g.fr;
    if (fr == 2) gemv_bf16_launch<OUT, 2>(X, W, M, N, K, g, splits, st);
    else gemv_bf16_launch<OUT, 1>(X, W, M, N, K, g, splits, st);
  } else {
    const int splits = OUT == GV_PARTIAL ? g.splits : 1;
    dim3 grid((N + 127) / 128, splits, M);
    gemv_f32_kernel<OUT><<<grid, 128, 0, st>>>((const float*)X, (const float*)W, M, N, K, g);
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
