// Prompt-pass projections of libhe: Y[M,N] = X[M,K] W[N,K]^T with fused epilogues.
//
// bf16 models: MFMA (v_mfma_f32_16x16x32_bf16) GEMM with 128 x 128 macro tiles,
// BK = 32, LDS double buffering; four waves each own a 64 x 64 sub-tile (4 x 4
// MFMA tiles).  fp32 models (the tiny workload only): a plain tiled FMA kernel.
// Both end in the same epilogue: bias, q scaling + KV-cache scatter (the prompt's
// keys and values enter the cache here), residual add, ReLU, position add.  bf16
// weights are read row-major or in the inference layout (EpiArgs::w_il, il_off):
// a 16-byte chunk is 8 consecutive k of one row in both.
#include "common.h"
#include "kernels.h"

namespace he {

// ---------------------------------------------------------------------------------
// epilogue: one output element (m, n) with fp32 accumulator acc
// ---------------------------------------------------------------------------------
template <typename T, int MODE>
__device__ __forceinline__ void epi_store(const EpiArgs& e, int m, int n, int N, float acc) {
  if (MODE == EPI_QKV) {
    const int part = n / e.d, within = n - part * e.d;
    const int head = within / e.D, dd = within - head * e.D;
    const int b = m / e.seq_len, t = m - b * e.seq_len;
    float v = acc + ld((const T*)e.bias + n);
    if (part == 0) {
      st((T*)e.q_out + (size_t)m * e.d + within, v * e.q_scale);
    } else {
      T* cache = (T*)(part == 1 ? e.k_cache : e.v_cache);
      st(cache + (((size_t)b * e.H + head) * e.S_max + e.pos0 + t) * e.D + dd, v);
    }
  } else if (MODE == EPI_RESID) {
    float bv = e.bias ? ld((const T*)e.bias + n) : 0.f;
    e.h[(size_t)m * N + n] += acc + bv;
  } else if (MODE == EPI_RELU) {
    float v = acc + ld((const T*)e.bias + n);
    st((T*)e.out + (size_t)m * N + n, fmaxf(v, 0.f));
  } else if (MODE == EPI_POSADD) {
    const int t = m % e.seq_len;
    float v = acc + ld((const T*)e.pos_emb + (size_t)(e.pos0 + t + 2) * N + n);
    e.h[(size_t)m * N + n] = v;
    st((T*)e.out + (size_t)m * N + n, v);
  } else {
    float bv = e.bias ? ld((const T*)e.bias + n) : 0.f;
    e.out_f32[(size_t)m * N + n] = acc + bv;
  }
}

// ---------------------------------------------------------------------------------
// bf16 MFMA GEMM
// ---------------------------------------------------------------------------------
constexpr int BM = 128, BN = 128, BK = 32, LDK = BK + 8;   // +8 bf16 pad: fewer bank conflicts

template <int MODE>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const bf16* __restrict__ X,
                                                        const bf16* __restrict__ W, int M, int N,
                                                        int K, EpiArgs e) {
  __shared__ __attribute__((aligned(16))) bf16 As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][BN * LDK];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;

  // global -> register staging: each thread moves 2 x 16 B of A and of B per k-tile
  const int lr = tid >> 2, lc = (tid & 3) * 8;      // row 0..63 (+64), column chunk
  uint4 ra[2], rb[2];
  auto gload = [&](int kt) {
    const int k = kt * BK + lc;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = lr + 64 * i;
      const int gm = m0 + r, gn = n0 + r;
      ra[i] = (gm < M && k < K) ? *reinterpret_cast<const uint4*>(X + (size_t)gm * K + k)
                                : make_uint4(0, 0, 0, 0);
      rb[i] = (gn < N && k < K) ? *reinterpret_cast<const uint4*>(W + il_off(gn, k, K, e.w_il))
                                : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = lr + 64 * i;
      *reinterpret_cast<uint4*>(&As[buf][r * LDK + lc]) = ra[i];
      *reinterpret_cast<uint4*>(&Bs[buf][r * LDK + lc]) = rb[i];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    bf16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *reinterpret_cast<const bf16x8*>(&As[cur][(wm * 64 + i * 16 + fr) * LDK + fk]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = *reinterpret_cast<const bf16x8*>(&Bs[cur][(wn * 64 + j * 16 + fr) * LDK + fk]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // D tile layout: lane holds rows 4*(lane/16)+r (r = 0..3) of column lane%16
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r;
        const int n = n0 + wn * 64 + j * 16 + (lane & 15);
        if (m < M && n < N) epi_store<bf16, MODE>(e, m, n, N, acc[i][j][r]);
      }
}

// ---------------------------------------------------------------------------------
// bf16 MFMA GEMM, large tiles: 256 x 256 macro tile, BK = 64, 8 waves (2 x 4), each
// wave 128 x 64 (8 x 4 MFMA tiles, 128 accumulators).  LDS holds two stages of A and
// B (128 KB) in an XOR-swizzled layout (16-byte chunk c of row r sits at c ^ (r & 7)),
// so the fragment reads of 8 consecutive rows hit distinct banks without padding.
// Tiles are handed to XCDs in contiguous runs (WG w runs on XCD w % 8) and walked in
// groups of 4 tile rows, so the WGs an XCD runs together share A and B panels in its L2.
// ---------------------------------------------------------------------------------
constexpr int LBM = 256, LBN = 256, LBK = 64;

__device__ __forceinline__ int swz(int row, int chunk) { return row * LBK + ((chunk ^ (row & 7)) << 3); }

template <int MODE>
__global__ __launch_bounds__(512) void gemm_bf16_big_kernel(const bf16* __restrict__ X,
                                                            const bf16* __restrict__ W, int M,
                                                            int N, int K, EpiArgs e) {
  __shared__ __attribute__((aligned(16))) bf16 As[2][LBM * LBK];
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][LBN * LBK];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 2, wn = wv & 3;

  // XCD-aware tile order
  const int nm = (M + LBM - 1) / LBM, nn = (N + LBN - 1) / LBN, T = nm * nn;
  const int per = (T + 7) / 8;
  const int t = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (t >= T) return;
  constexpr int GM = 4;
  const int group = t / (GM * nn), first_m = group * GM;
  const int gsz = min(nm - first_m, GM);
  const int tm = first_m + (t % (GM * nn)) % gsz, tn = (t % (GM * nn)) / gsz;
  const int m0 = tm * LBM, n0 = tn * LBN;

  // global -> LDS: 2048 16-byte chunks per operand and stage, 4 per thread
  uint4 ra[4], rb[4];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + i * 512, r = id >> 3, c = id & 7;
      const int k = kt * LBK + c * 8;
      const int gm = m0 + r, gn = n0 + r;
      ra[i] = (gm < M && k < K) ? *reinterpret_cast<const uint4*>(X + (size_t)gm * K + k) : make_uint4(0, 0, 0, 0);
      rb[i] = (gn < N && k < K) ? *reinterpret_cast<const uint4*>(W + il_off(gn, k, K, e.w_il)) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + i * 512, r = id >> 3, c = id & 7;
      *reinterpret_cast<uint4*>(&As[buf][swz(r, c)]) = ra[i];
      *reinterpret_cast<uint4*>(&Bs[buf][swz(r, c)]) = rb[i];
    }
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + LBK - 1) / LBK;
  gload(0);
  sstore(0);
  __syncthreads();
  const int fr = lane & 15, fg = lane >> 4;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ch = kk * 4 + fg;
      bf16x8 b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(&Bs[cur][swz(wn * 64 + j * 16 + fr, ch)]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&As[cur][swz(wm * 128 + i * 16 + fr, ch)]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[j], acc[i][j], 0, 0, 0);
      }
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 128 + i * 16 + fg * 4 + r;
        const int n = n0 + wn * 64 + j * 16 + fr;
        if (m < M && n < N) epi_store<bf16, MODE>(e, m, n, N, acc[i][j][r]);
      }
}

// ---------------------------------------------------------------------------------
// fp32 tiled FMA GEMM (16 x 16 threads, 64 x 64 tile, 4 x 4 outputs per thread)
// ---------------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ X,
                                                       const float* __restrict__ W, int M, int N,
                                                       int K, EpiArgs e) {
  __shared__ float Xs[16][64 + 1];
  __shared__ float Ws[16][64 + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int i = threadIdx.x; i < 16 * 64; i += 256) {
      int r = i / 16, c = i % 16;
      Xs[c][r] = (m0 + r < M && k0 + c < K) ? X[(size_t)(m0 + r) * K + k0 + c] : 0.f;
      Ws[c][r] = (n0 + r < N && k0 + c < K) ? W[(size_t)(n0 + r) * K + k0 + c] : 0.f;
    }
    __syncthreads();
    for (int c = 0; c < 16; ++c) {
      float xa[4], wb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { xa[i] = Xs[c][ty + 16 * i]; wb[i] = Ws[c][tx + 16 * i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xa[i], wb[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty + 16 * i, n = n0 + tx + 16 * j;
      if (m < M && n < N) epi_store<float, MODE>(e, m, n, N, acc[i][j]);
    }
}

template <int MODE>
static void gemm_dispatch(int dt, const void* X, const void* W, int M, int N, int K,
                          const EpiArgs& e, hipStream_t st) {
  if (dt == DT_BF16) {
    const long big_tiles = (long)((M + LBM - 1) / LBM) * ((N + LBN - 1) / LBN);
    if (big_tiles >= 256) {       // enough 256 x 256 tiles to cover the CUs
      const int blocks = (int)((big_tiles + 7) / 8 * 8);
      gemm_bf16_big_kernel<MODE><<<blocks, 512, 0, st>>>((const bf16*)X, (const bf16*)W, M, N, K, e);
      return;
    }
    dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
    gemm_bf16_kernel<MODE><<<grid, 256, 0, st>>>((const bf16*)X, (const bf16*)W, M, N, K, e);
  } else {
    dim3 grid((N + 63) / 64, (M + 63) / 64);
    gemm_f32_kernel<MODE><<<grid, 256, 0, st>>>((const float*)X, (const float*)W, M, N, K, e);
  }
}

void launch_gemm(int dt, const void* X, const void* W, int M, int N, int K, const EpiArgs& e,
                 hipStream_t st) {
  switch (e.mode) {
    case EPI_QKV: gemm_dispatch<EPI_QKV>(dt, X, W, M, N, K, e, st); break;
    case EPI_RESID: gemm_dispatch<EPI_RESID>(dt, X, W, M, N, K, e, st); break;
    case EPI_RELU: gemm_dispatch<EPI_RELU>(dt, X, W, M, N, K, e, st); break;
    case EPI_POSADD: gemm_dispatch<EPI_POSADD>(dt, X, W, M, N, K, e, st); break;
    default: gemm_dispatch<EPI_F32>(dt, X, W, M, N, K, e, st); break;
  }
}

}  // namespace he
