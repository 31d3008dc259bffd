// Bandwidth-bound element-wise and row kernels of libhe: LoRA fold, embeddings,
// LayerNorm with residual updates, argmax reduction, reward head.
#include "common.h"
#include "kernels.h"

namespace he {

// ---------------------------------------------------------------------------------
// LoRA fold: W <- round(W + sign * s * (B A)).  The update B A of a rank-r adapter
// (paper summary, "Training Mode: ZeRO and LoRA Optimizations") is accumulated in
// float32 over j = 0..r-1 in that order, so the fold and the unfold subtract the
// bitwise-same update.  A WG owns a 32 x TK tile of W; the A and B slices it
// needs are staged in LDS once, so HBM sees W read once and written once.
// ---------------------------------------------------------------------------------
template <typename T, int kLoraTK>
__global__ __launch_bounds__(256) void lora_kernel(T* __restrict__ W, const T* __restrict__ A,
                                                   const T* __restrict__ Bm, int N, int K, int r,
                                                   float s, float sign) {
  constexpr int CPR = kLoraTK / 8;            // 8-column chunks per row
  constexpr int RG = 256 / CPR;               // row groups, 4 rows each
  constexpr int TN = 4 * RG;                  // rows per tile
  extern __shared__ float lds[];
  float* As = lds;                            // [r][kLoraTK]
  float* Bs = lds + r * kLoraTK;              // [r][TN]  (transposed: 4 rows per float4)
  const int k0 = blockIdx.x * kLoraTK, n0 = blockIdx.y * TN;
  const int tid = threadIdx.x;
  const int c8 = tid % CPR, rg = tid / CPR;
  const int k = k0 + c8 * 8;
  // this thread's four rows of W, loaded before the update is formed
  float w[4][8];
  const bool kin = k < K;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = n0 + rg * 4 + i;
    if (kin && n < N) load8(W + (size_t)n * K + k, w[i]);
  }
  for (int i = tid; i < r * CPR; i += 256) {       // A slice, 16-byte chunks
    const int j = i / CPR, c = (i % CPR) * 8;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (k0 + c < K) load8(A + (size_t)j * K + k0 + c, v);
    *reinterpret_cast<float4*>(As + j * kLoraTK + c) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(As + j * kLoraTK + c + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
  for (int i = tid; i < TN * r; i += 256) {
    const int n = i / r, j = i % r;
    Bs[j * TN + n] = (n0 + n < N) ? ld(Bm + (size_t)(n0 + n) * r + j) : 0.f;
  }
  __syncthreads();
  if (!kin) return;
  float acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[i][q] = 0.f;
  for (int j = 0; j < r; ++j) {
    const float4 a0 = *reinterpret_cast<const float4*>(As + j * kLoraTK + c8 * 8);
    const float4 a1 = *reinterpret_cast<const float4*>(As + j * kLoraTK + c8 * 8 + 4);
    const float4 b4 = *reinterpret_cast<const float4*>(Bs + j * TN + rg * 4);
    const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const float b[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[i][q] = fmaf(b[i], a[q], acc[i][q]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = n0 + rg * 4 + i;
    if (n >= N) break;
#pragma unroll
    for (int q = 0; q < 8; ++q) w[i][q] = w[i][q] + sign * (s * acc[i][q]);
    store8(W + (size_t)n * K + k, w[i]);
  }
}

template <int TK>
static void lora_launch(void* W, const void* A, const void* B, int N, int K, int r, float s,
                        float sign, hipStream_t st) {
  constexpr int TN = 4 * (256 / (TK / 8));
  dim3 grid((K + TK - 1) / TK, (N + TN - 1) / TN);
  size_t lds = (size_t)(r * TK + TN * r) * sizeof(float);   // <= 48 KB for r <= 64
  lora_kernel<float, TK><<<grid, 256, lds, st>>>((float*)W, (const float*)A, (const float*)B, N, K, r, s, sign);
}

// ---------------------------------------------------------------------------------
// bf16 models: the same fold, fused with the switch between the row-major layout
// and the inference layout (common.h, il_off).  FOLD: read row-major, write
// W + s B A in the inference layout; !FOLD: read the inference layout, write
// W' - s B A row-major.  r == 0: the layout switch alone (weights without adapter).
// A WG owns one BW-wide column block, stages A's slice once, and walks 16-row
// blocks: each thread updates one 16-byte unit in each of four rows (the A values
// serve all four), the block is re-ordered in LDS, then written with contiguous
// 16-byte stores.  Each block is read completely before it is overwritten, and only
// by its WG.  The update is accumulated exactly as in lora_kernel.
// ---------------------------------------------------------------------------------
template <bool FOLD>
__global__ __launch_bounds__(256) void lora_il_kernel(bf16* __restrict__ W, const bf16* __restrict__ A,
                                                      const bf16* __restrict__ Bm, int N, int K, int r,
                                                      float s, float sign, int il) {
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  const int bw = 1 << il, upr = bw >> 3, lgu = il - 3;
  bf16* stage = reinterpret_cast<bf16*>(lds_raw);          // [16][bw]
  bf16* As = stage + 16 * bw;                              // [r][bw]
  float* Bs = reinterpret_cast<float*>(As + r * bw);       // [r][16]
  const int tid = threadIdx.x, c0 = blockIdx.x * bw, nrb = N >> 4;
  for (int i = tid; i < r * upr; i += 256) {
    const int j = i / upr, u = i - j * upr;
    *reinterpret_cast<uint4*>(As + j * bw + u * 8) = *reinterpret_cast<const uint4*>(A + (size_t)j * K + c0 + u * 8);
  }
  for (int rb = blockIdx.y; rb < nrb; rb += gridDim.y) {
    __syncthreads();                                       // stage and Bs free again
    for (int i = tid; i < 16 * r; i += 256) {
      const int row = i / r, j = i - row * r;
      Bs[j * 16 + row] = bf2f(Bm[(size_t)(rb * 16 + row) * r + j]);
    }
    __syncthreads();
    for (int it = tid; it < 4 * upr; it += 256) {
      const int jq = it / upr, u = it - jq * upr;          // rows 4 jq .. 4 jq + 3, unit u
      float v[4][8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = jq * 4 + q;
        const int p = ((u >> 2) << 6) | ((u & 3) << 4) | j;   // inference-layout position
        const int src = FOLD ? j * upr + u : p;
        load8(W + (size_t)(rb * 16 + (src >> lgu)) * K + c0 + ((src & (upr - 1)) << 3), v[q]);
      }
      if (r > 0) {
        float acc[4][8];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[q][e] = 0.f;
        for (int j = 0; j < r; ++j) {
          float a[8];
          load8(As + j * bw + u * 8, a);
          const float4 b4 = *reinterpret_cast<const float4*>(Bs + j * 16 + jq * 4);
          const float b[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[q][e] = fmaf(b[q], a[e], acc[q][e]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 8; ++e) v[q][e] = v[q][e] + sign * (s * acc[q][e]);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = jq * 4 + q;
        const int p = ((u >> 2) << 6) | ((u & 3) << 4) | j;
        store8(stage + (FOLD ? p : j * upr + u) * 8, v[q]);
      }
    }
    __syncthreads();
    for (int i = tid; i < 16 * upr; i += 256)
      *reinterpret_cast<uint4*>(W + (size_t)(rb * 16 + (i >> lgu)) * K + c0 + ((i & (upr - 1)) << 3)) =
          *reinterpret_cast<const uint4*>(stage + i * 8);
  }
}

void launch_lora(int dt, void* W, const void* A, const void* B, int N, int K, int r, float s,
                 float sign, int il, hipStream_t st) {
  if (dt != DT_BF16) {
    if (r <= 0) return;
    if (r <= 32) lora_launch<256>(W, A, B, N, K, r, s, sign, st);
    else lora_launch<128>(W, A, B, N, K, r, s, sign, st);
    return;
  }
  const int bw = 1 << il, ncb = K / bw, nrb = N / 16;
  const int gy = std::max(1, std::min(nrb, 2048 / ncb));
  const size_t lds = (size_t)16 * bw * 2 + (size_t)r * bw * 2 + (size_t)r * 16 * 4;
  dim3 grid(ncb, gy);
  if (sign > 0)
    lora_il_kernel<true><<<grid, 256, lds, st>>>((bf16*)W, (const bf16*)A, (const bf16*)B, N, K, r, s, sign, il);
  else
    lora_il_kernel<false><<<grid, 256, lds, st>>>((bf16*)W, (const bf16*)A, (const bf16*)B, N, K, r, s, sign, il);
}

// ---------------------------------------------------------------------------------
// Row LayerNorm: one WG per row, each thread owns up to two chunks of 4 consecutive
// elements (d <= 8 * blockDim, d % 4 == 0).  Mean and biased variance are two
// fixed-order block reductions (deterministic).  Wide WGs (up to 1024 threads) keep
// many loads in flight: at decode a step has only `batch` rows.
// ---------------------------------------------------------------------------------
constexpr int kLnChunks = 2;

__device__ __forceinline__ void ld4(const float* p, float* o) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
}
__device__ __forceinline__ void ld4(const bf16* p, float* o) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  o[0] = __uint_as_float(u.x << 16); o[1] = __uint_as_float(u.x & 0xffff0000u);
  o[2] = __uint_as_float(u.y << 16); o[3] = __uint_as_float(u.y & 0xffff0000u);
}
__device__ __forceinline__ void st4(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st4(bf16* p, const float* v) {
  uint2 u;
  u.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
  u.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}

// x row `row` of the GEMM input in layout x_lay (act_off): row-major [.][d], decode
// fragment tiles, or the inference layout.
template <typename T>
__device__ __forceinline__ T* x_at(T* x, int row, int k, int d, int x_lay) {
  return x + act_off(row, k, d, x_lay);
}

// LayerNorm of one row held by the block (up to kLnChunks chunks of 4 per thread),
// written rounded to x (and to the stream for post-LN).  Mean, then the biased
// variance around it, as two fixed-order block reductions; gamma and beta are
// fetched before the reductions so their latency overlaps them.
template <typename T>
__device__ __forceinline__ void ln_write_pre(const float (&v)[kLnChunks][4], const float (&gv)[kLnChunks][4],
                                             const float (&bv)[kLnChunks][4], int d, float eps, T* x,
                                             int row, int x_lay, float* hrow_post, float* red) {
  const int tid = threadIdx.x, nch = d / 4, nt = blockDim.x;
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kLnChunks; ++c)
    if (tid + c * nt < nch)
#pragma unroll
      for (int q = 0; q < 4; ++q) s += v[c][q];
  const float mean = block_sum(s, red) / (float)d;
  float s2 = 0.f;
#pragma unroll
  for (int c = 0; c < kLnChunks; ++c)
    if (tid + c * nt < nch)
#pragma unroll
      for (int q = 0; q < 4; ++q) { const float t = v[c][q] - mean; s2 += t * t; }
  const float var = block_sum(s2, red + 32) / (float)d;
  const float rstd = 1.f / sqrtf(var + eps);
#pragma unroll
  for (int c = 0; c < kLnChunks; ++c) {
    const int ch = tid + c * nt;
    if (ch < nch) {
      float y[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) y[q] = (v[c][q] - mean) * rstd * gv[c][q] + bv[c][q];
      if (hrow_post) st4(hrow_post + ch * 4, y);   // post-LN: the stream is the norm
      st4(x_at(x, row, ch * 4, d, x_lay), y);         // GEMM input: rounded
    }
  }
}

template <typename T>
__device__ __forceinline__ void ln_write(const float (&v)[kLnChunks][4], int d, float eps,
                                         const T* g, const T* b, T* x, int row, int x_lay,
                                         float* hrow_post, float* red) {
  const int tid = threadIdx.x, nch = d / 4, nt = blockDim.x;
  float gv[kLnChunks][4], bv[kLnChunks][4];
#pragma unroll
  for (int c = 0; c < kLnChunks; ++c)
    if (tid + c * nt < nch) {
      ld4(g + (tid + c * nt) * 4, gv[c]);
      ld4(b + (tid + c * nt) * 4, bv[c]);
    }
  ln_write_pre<T>(v, gv, bv, d, eps, x, row, x_lay, hrow_post, red);
}

// Threads per row: two chunks of 4 each (measured fastest at decode shapes), whole waves.
static int ln_threads(int d) {
  int t = (d / 8 + 63) / 64 * 64;
  return t < 64 ? 64 : (t > 1024 ? 1024 : t);
}

// h[m] = E[id] + P[pos + 2]; x[m] = round(LN(h[m])) (or round(h[m]) without LN).
// Position table row pos + 2: OPT's learned positions are offset by two rows.
// E may be in the inference layout (e_il > 0, it is the LM head's weight too).
template <typename T>
__global__ __launch_bounds__(1024) void embed_norm_kernel(const int32_t* __restrict__ ids,
                                                          const int32_t* __restrict__ pos_dev,
                                                          int seq_len, const T* __restrict__ E,
                                                          const T* __restrict__ P,
                                                          const T* __restrict__ g,
                                                          const T* __restrict__ b, float eps,
                                                          float* __restrict__ h, T* __restrict__ x,
                                                          int d, int vocab, int e_il, int x_lay) {
  __shared__ float red[64];
  const int m = blockIdx.x, tid = threadIdx.x, nch = d / 4, nt = blockDim.x;
  int id = ids[m];
  id = id < 0 ? 0 : (id >= vocab ? vocab - 1 : id);   // memory safety for bad ids
  const int pos = pos_dev ? *pos_dev : (m % seq_len);
  const T* pr = P + (size_t)(pos + 2) * d;
  float v[kLnChunks][4];
#pragma unroll
  for (int c = 0; c < kLnChunks; ++c) {
    const int ch = tid + c * nt;
    if (ch < nch) {
      float e[4], p[4];
      ld4(E + il_off(id, ch * 4, d, e_il), e);
      ld4(pr + ch * 4, p);
#pragma unroll
      for (int q = 0; q < 4; ++q) v[c][q] = e[q] + p[q];
      st4(h + (size_t)m * d + ch * 4, v[c]);
    }
  }
  if (g) {
    ln_write<T>(v, d, eps, g, b, x, m, x_lay, nullptr, red);
  } else {
#pragma unroll
    for (int c = 0; c < kLnChunks; ++c) {
      const int ch = tid + c * nt;
      if (ch < nch) st4(x_at(x, m, ch * 4, d, x_lay), v[c]);
    }
  }
}

void launch_embed_norm(int dt, const int32_t* ids, const int32_t* pos_dev, int seq_len,
                       const void* E, const void* P, const void* g, const void* b, float eps,
                       float* h, void* x, int M, int d, int vocab, int e_il, int x_lay, hipStream_t st) {
  const int nt = ln_threads(d);
  if (dt == DT_BF16)
    embed_norm_kernel<bf16><<<M, nt, 0, st>>>(ids, pos_dev, seq_len, (const bf16*)E, (const bf16*)P,
                                              (const bf16*)g, (const bf16*)b, eps, h, (bf16*)x, d, vocab,
                                              e_il, x_lay);
  else
    embed_norm_kernel<float><<<M, nt, 0, st>>>(ids, pos_dev, seq_len, (const float*)E, (const float*)P,
                                               (const float*)g, (const float*)b, eps, h, (float*)x, d, vocab,
                                               0, 0);
}

template <typename T>
__global__ __launch_bounds__(256) void embed_gather_kernel(const int32_t* __restrict__ ids,
                                                           const T* __restrict__ E,
                                                           T* __restrict__ xe, int de, int vocab) {
  const int m = blockIdx.x;
  int id = ids[m];
  id = id < 0 ? 0 : (id >= vocab ? vocab - 1 : id);
  for (int ch = threadIdx.x; ch < de / 8; ch += 256) {
    float v[8];
    load8(E + (size_t)id * de + ch * 8, v);
    store8(xe + (size_t)m * de + ch * 8, v);
  }
}

void launch_embed_gather(int dt, const int32_t* ids, const void* E, void* xe, int M, int de,
                         int vocab, hipStream_t st) {
  if (dt == DT_BF16)
    embed_gather_kernel<bf16><<<M, 256, 0, st>>>(ids, (const bf16*)E, (bf16*)xe, de, vocab);
  else
    embed_gather_kernel<float><<<M, 256, 0, st>>>(ids, (const float*)E, (float*)xe, de, vocab);
}

// Residual update (sum of split-K partials + bias, fixed order) and LayerNorm.  Every
// load of the row (gamma, beta, the stream, up to kNormSplits partials and the bias)
// is issued before any arithmetic, so the row costs one memory round trip.
constexpr int kNormSplits = 8;
template <typename T>
__global__ __launch_bounds__(1024) void norm_kernel(float* __restrict__ h,
                                                    const float* __restrict__ parts, int nsplit,
                                                    const T* __restrict__ bias,
                                                    const T* __restrict__ g,
                                                    const T* __restrict__ b, float eps,
                                                    T* __restrict__ x, int M, int d, int row_stride,
                                                    int row_offset, int post, int x_lay, int row_group) {
  __shared__ float red[64];
  const int r = blockIdx.x, tid = threadIdx.x, nch = d / 4, nt = blockDim.x;
  const size_t row = (size_t)(r / row_group) * row_stride + row_offset + r % row_group;
  float* hr = h + row * d;
  float v[kLnChunks][4], gv[kLnChunks][4], bv[kLnChunks][4];
  const bool pre = parts && nsplit <= kNormSplits;
  float pp[kLnChunks][kNormSplits][4], bb[kLnChunks][4];
#pragma unroll
  for (int c = 0; c < kLnChunks; ++c) {
    const int ch = tid + c * nt;
    if (ch < nch) {
      ld4(g + ch * 4, gv[c]);
      ld4(b + ch * 4, bv[c]);
      ld4(hr + ch * 4, v[c]);
      if (pre) {
        ld4(bias + ch * 4, bb[c]);
#pragma unroll
        for (int s = 0; s < kNormSplits; ++s)
          if (s < nsplit) ld4(parts + ((size_t)s * M + r) * d + ch * 4, pp[c][s]);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < kLnChunks; ++c) {
    const int ch = tid + c * nt;
    if (ch < nch && parts) {
      float add[4] = {0.f, 0.f, 0.f, 0.f};
      if (pre) {
#pragma unroll
        for (int s = 0; s < kNormSplits; ++s)
          if (s < nsplit)
#pragma unroll
            for (int q = 0; q < 4; ++q) add[q] += pp[c][s][q];
      } else {                                    // more splits than registers: in order
        ld4(bias + ch * 4, bb[c]);
        for (int s = 0; s < nsplit; ++s) {
          float p0[4];
          ld4(parts + ((size_t)s * M + r) * d + ch * 4, p0);
#pragma unroll
          for (int q = 0; q < 4; ++q) add[q] += p0[q];
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) v[c][q] += add[q] + bb[c][q];
      st4(hr + ch * 4, v[c]);
    }
  }
  ln_write_pre<T>(v, gv, bv, d, eps, x, r, x_lay, post ? hr : nullptr, red);
}

// LayerNorm of many rows with no split-K sum to add (the prompt pass, scoring, the
// reward model): one wave per row, lane l holding chunks of 4 at l, l + 64, ...  The
// row's mean and variance are wave reductions, with no block barrier, so the four
// waves of a WG and the WGs of a CU run their rows independently and keep HBM busy.
template <typename T, int NC>
__global__ __launch_bounds__(256, NC <= 16 ? 4 : 3) void norm_rows_kernel(float* __restrict__ h, const T* __restrict__ g,
                                                        const T* __restrict__ b, float eps,
                                                        T* __restrict__ x, int M, int d, int row_stride,
                                                        int row_offset, int post, int x_lay,
                                                        int row_group) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= M) return;
  const size_t row = (size_t)(r / row_group) * row_stride + row_offset + r % row_group;
  float* hr = h + row * d;
  const int nch = d / 4;
  float v[NC][4];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = lane + c * kWave;
    if (ch < nch) {                              // the stream row is read once here
      const uint4 u = ld_once(hr + ch * 4);
      v[c][0] = __uint_as_float(u.x); v[c][1] = __uint_as_float(u.y);
      v[c][2] = __uint_as_float(u.z); v[c][3] = __uint_as_float(u.w);
    } else {
      v[c][0] = v[c][1] = v[c][2] = v[c][3] = 0.f;
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q) s += v[c][q];
  const float mean = wave_sum(s) / (float)d;
  float s2 = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (lane + c * kWave < nch)
#pragma unroll
      for (int q = 0; q < 4; ++q) { const float t = v[c][q] - mean; s2 += t * t; }
  const float var = wave_sum(s2) / (float)d;
  const float rstd = 1.f / sqrtf(var + eps);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = lane + c * kWave;
    if (ch < nch) {
      float gv[4], bv[4], y[4];
      ld4(g + ch * 4, gv);
      ld4(b + ch * 4, bv);
#pragma unroll
      for (int q = 0; q < 4; ++q) y[q] = (v[c][q] - mean) * rstd * gv[q] + bv[q];
      if (post) st4(hr + ch * 4, y);                // post-LN: the stream is the norm
      st4(x_at(x, r, ch * 4, d, x_lay), y);         // GEMM input: rounded
    }
  }
}

// LayerNorm of the rows of one 16-row block of the inference layout (bf16 GEMM input,
// x_lay < 0), one wave per row.  In that layout the block's rows keep their 16 row
// segments in memory and only the 16-byte units inside each block of 16 rows x BW
// columns move, so a column chunk of whole blocks is 16 contiguous row pieces.  The
// rounded outputs of one chunk are staged in LDS row-major (rows padded by 16 bytes,
// so the gathers below hit distinct banks), then each thread fetches the unit that
// belongs at its place of the chunk's memory and writes it: every HBM line is written
// whole, where one wave per row would write 8 bytes into each of 64 lines.
constexpr int kNbCols = 2048;     // columns per staged chunk (16 x 2056 bf16, 64.25 KB)
template <int NC>
__global__ __launch_bounds__(1024) void norm_block_kernel(float* __restrict__ h, const bf16* __restrict__ g,
                                                          const bf16* __restrict__ b, float eps,
                                                          bf16* __restrict__ x, int M, int d, int row_stride,
                                                          int row_offset, int post, int il, int row_group) {
  __shared__ __attribute__((aligned(16))) bf16 tile[16 * (kNbCols + 8)];
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x >> 6;
  const int r0 = blockIdx.x * 16, r = r0 + w;
  const bool live = r < M;
  const size_t row = live ? (size_t)(r / row_group) * row_stride + row_offset + r % row_group : 0;
  float* hr = h + row * d;
  const int nch = d / 4;
  float v[NC][4];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = lane + c * kWave;
    if (live && ch < nch) {                      // the stream row is read once here
      const uint4 u = ld_once(hr + ch * 4);
      v[c][0] = __uint_as_float(u.x); v[c][1] = __uint_as_float(u.y);
      v[c][2] = __uint_as_float(u.z); v[c][3] = __uint_as_float(u.w);
    } else {
      v[c][0] = v[c][1] = v[c][2] = v[c][3] = 0.f;
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q) s += v[c][q];
  const float mean = wave_sum(s) / (float)d;
  float s2 = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (lane + c * kWave < nch)
#pragma unroll
      for (int q = 0; q < 4; ++q) { const float t = v[c][q] - mean; s2 += t * t; }
  const float var = wave_sum(s2) / (float)d;
  const float rstd = 1.f / sqrtf(var + eps);
  const int lgu = il - 3, umask = (1 << lgu) - 1;   // 16-byte units per block row
  constexpr int TS = kNbCols + 8;                  // staged row stride (elements)
  for (int c0 = 0; c0 < d; c0 += kNbCols) {
    const int cw = min(kNbCols, d - c0);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int k = (lane + c * kWave) * 4;
      if (live && k < d && k >= c0 && k < c0 + cw) {
        float gv[4], bv[4], y[4];
        ld4(g + k, gv);
        ld4(b + k, bv);
#pragma unroll
        for (int q = 0; q < 4; ++q) y[q] = (v[c][q] - mean) * rstd * gv[q] + bv[q];
        if (post) st4(hr + k, y);                  // post-LN: the stream is the norm
        st4(tile + w * TS + (k - c0), y);
      }
    }
    __syncthreads();
    // memory unit (block row sr, unit column sc / 8 of the chunk) holds, by il_off, unit
    // (row j, unit column u) of its block with position p = (u / 4) 64 + (u % 4) 16 + j.
    // A block's rows are spread over all 16 of its memory rows, so a block that is only
    // partly filled (M % 16 != 0) writes the units of its live rows, wherever they lie
    // (the buffer holds whole 16-row blocks).
    const int per_row = cw / 8;
    for (int i = threadIdx.x; i < 16 * per_row; i += 1024) {
      const int sr = i / per_row, sc = (i - sr * per_row) * 8;
      const int ub = sc >> il << il;                     // the layout block's first column in the chunk
      const int p = (sr << lgu) | ((sc >> 3) & umask);   // position inside that block
      const int j = p & 15, u = ((p >> 6) << 2) | ((p >> 4) & 3);
      if (r0 + j < M)
        *reinterpret_cast<uint4*>(x + (size_t)(r0 + sr) * d + c0 + sc) =
            *reinterpret_cast<const uint4*>(tile + j * TS + ub + u * 8);
    }
    __syncthreads();
  }
}

// LayerNorm of 8 consecutive rows per WG into the inference layout with 512-column
// blocks (d = 512 UPL), one wave per row.  In that layout each 128-byte line holds the
// same 16-byte unit column of 8 consecutive rows of a 16-row block (positions j0 .. j0 + 7
// of p = (u / 4) 64 + (u % 4) 16 + j, j0 = 0 or 8), so the WG's rows fill whole lines.
// Lane l holds the 8 consecutive columns of unit column l of each 512-column block (two
// 16-byte loads per block).  The rounded units go to LDS in the order of the output lines,
// the row's slot XOR-swizzled by (u / 2) % 8 so that both the row-wise writes and the
// line-wise reads hit distinct banks; after one barrier every lane copies whole units out.
// Writing the layout one row at a time puts 16 bytes into each of a row's 512 lines,
// which measured 1.5x slower at 16384 x 4096 (122.7 against 81.0 us).  Two WGs share a
// CU (at most 80 KB of LDS and 128 VGPRs each), so one reads while the other writes.
template <int UPL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void norm_line_kernel(float* __restrict__ h, const bf16* __restrict__ g,
                                                        const bf16* __restrict__ b, float eps,
                                                        bf16* __restrict__ x, int M, int row_stride,
                                                        int row_offset, int post, int row_group) {
  constexpr int D = 512 * UPL;
  __shared__ uint4 stage[8 * 64 * UPL];
  const int lane = threadIdx.x & (kWave - 1), t = threadIdx.x >> 6;
  const int r0 = blockIdx.x * 8, r = r0 + t;
  const bool live = r < M;
  const size_t row = live ? (size_t)(r / row_group) * row_stride + row_offset + r % row_group : 0;
  float* hr = h + row * D;
  float v[UPL][8];
#pragma unroll
  for (int c = 0; c < UPL; ++c) {
    const int e = 8 * (lane + c * kWave);
    if (live) {                                  // the stream row is read once here
      const uint4 u0 = ld_once(hr + e), u1 = ld_once(hr + e + 4);
      v[c][0] = __uint_as_float(u0.x); v[c][1] = __uint_as_float(u0.y);
      v[c][2] = __uint_as_float(u0.z); v[c][3] = __uint_as_float(u0.w);
      v[c][4] = __uint_as_float(u1.x); v[c][5] = __uint_as_float(u1.y);
      v[c][6] = __uint_as_float(u1.z); v[c][7] = __uint_as_float(u1.w);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) v[c][q] = 0.f;
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < UPL; ++c)
#pragma unroll
    for (int q = 0; q < 8; ++q) s += v[c][q];
  const float mean = wave_sum(s) / (float)D;
  float s2 = 0.f;
#pragma unroll
  for (int c = 0; c < UPL; ++c)
#pragma unroll
    for (int q = 0; q < 8; ++q) { const float dv = v[c][q] - mean; s2 += dv * dv; }
  const float rstd = 1.f / sqrtf(wave_sum(s2) / (float)D + eps);
#pragma unroll
  for (int c = 0; c < UPL; ++c) {
    const int e = 8 * (lane + c * kWave);
    float gv[8], bv[8], y[8];
    load8(g + e, gv);
    load8(b + e, bv);
#pragma unroll
    for (int q = 0; q < 8; ++q) y[q] = (v[c][q] - mean) * rstd * gv[q] + bv[q];
    if (post && live) store8(hr + e, y);         // post-LN: the stream is the norm
    uint4 u;
    u.x = (uint32_t)f2bf(y[0]) | ((uint32_t)f2bf(y[1]) << 16);
    u.y = (uint32_t)f2bf(y[2]) | ((uint32_t)f2bf(y[3]) << 16);
    u.z = (uint32_t)f2bf(y[4]) | ((uint32_t)f2bf(y[5]) << 16);
    u.w = (uint32_t)f2bf(y[6]) | ((uint32_t)f2bf(y[7]) << 16);
    stage[(c * kWave + lane) * 8 + (t ^ ((lane >> 1) & 7))] = u;   // block c, unit column lane, row t
  }
  __syncthreads();
  // output unit S of the WG: line k = S / 8 (block cb = k / 64, unit column u = k % 64),
  // row j0 + S % 8; a block that is only partly filled (M % 16 != 0) writes the units of
  // its live rows (the buffer holds whole 16-row blocks)
  const int j0 = r0 & 15, rb = r0 & ~15;
#pragma unroll
  for (int i = 0; i < UPL; ++i) {
    const int S = i * 512 + (int)threadIdx.x, k = S >> 3, tt = S & 7, cb = k >> 6, u = k & 63;
    if (r0 + tt < M) {
      const uint4 val = stage[k * 8 + (tt ^ ((u >> 1) & 7))];
      const int p = ((u >> 2) << 6) | ((u & 3) << 4) | (j0 + tt);
      *reinterpret_cast<uint4*>(x + (size_t)(rb + (p >> 6)) * D + cb * 512 + (p & 63) * 8) = val;
    }
  }
}

template <typename T>
static bool launch_norm_rows(float* h, const T* g, const T* b, float eps, T* x, int M, int d,
                             int row_stride, int row_offset, int post, int x_lay, int row_group,
                             hipStream_t st) {
  const int per_lane = (d / 4 + kWave - 1) / kWave;
  if constexpr (sizeof(T) == 2) {
    // rows of up to 1024 into the inference layout: 16-row blocks staged through LDS
    // (measured at 16384 rows: d = 1024 31.2 -> 21.8 us; at d = 4096 one WG per CU
    // serialises load, staging and stores and loses, 104.7 -> 114.1 us)
    if (x_lay < 0 && per_lane <= 4) {
      norm_block_kernel<4><<<(M + 15) / 16, 1024, 0, st>>>(h, (const bf16*)g, (const bf16*)b, eps, (bf16*)x,
                                                            M, d, row_stride, row_offset, post, -x_lay, row_group);
      return true;
    }
    // 512-column layout blocks and rows of 2048 .. 5120: 8 rows per WG, whole lines
    if (x_lay == -9 && d % 512 == 0) {
      const dim3 grid((M + 7) / 8), block(512);
      const bf16 *gb = (const bf16*)g, *bb = (const bf16*)b;
      bf16* xb = (bf16*)x;
      switch (d / 512) {
        case 4: norm_line_kernel<4><<<grid, block, 0, st>>>(h, gb, bb, eps, xb, M, row_stride, row_offset, post, row_group); return true;
        case 8: norm_line_kernel<8><<<grid, block, 0, st>>>(h, gb, bb, eps, xb, M, row_stride, row_offset, post, row_group); return true;
        case 10: norm_line_kernel<10><<<grid, block, 0, st>>>(h, gb, bb, eps, xb, M, row_stride, row_offset, post, row_group); return true;
        default: break;
      }
    }
  }
  const dim3 grid((M + 3) / 4), block(256);
#define HE_NORM_ROWS(NC)                                                                          \
  norm_rows_kernel<T, NC><<<grid, block, 0, st>>>(h, g, b, eps, x, M, d, row_stride, row_offset, \
                                                  post, x_lay, row_group)
  if (per_lane <= 4) HE_NORM_ROWS(4);
  else if (per_lane <= 8) HE_NORM_ROWS(8);
  else if (per_lane <= 16) HE_NORM_ROWS(16);
  else if (per_lane <= 20) HE_NORM_ROWS(20);
  else return false;
#undef HE_NORM_ROWS
  return true;
}

// Rows at or above which a norm with no partials to sum takes one wave per row.
constexpr int kNormRowsMin = 256;

void launch_norm(int dt, float* h, const float* parts, int nsplit, const void* bias, const void* g,
                 const void* b, float eps, void* x, int M, int d, int row_stride, int row_offset,
                 int post, int x_lay, hipStream_t st, int row_group) {
  if (!parts && M >= kNormRowsMin) {
    const bool done =
        dt == DT_BF16
            ? launch_norm_rows<bf16>(h, (const bf16*)g, (const bf16*)b, eps, (bf16*)x, M, d, row_stride,
                                     row_offset, post, x_lay, row_group, st)
            : launch_norm_rows<float>(h, (const float*)g, (const float*)b, eps, (float*)x, M, d,
                                      row_stride, row_offset, post, 0, row_group, st);
    if (done) return;
  }
  const int nt = ln_threads(d);
  if (dt == DT_BF16)
    norm_kernel<bf16><<<M, nt, 0, st>>>(h, parts, nsplit, (const bf16*)bias, (const bf16*)g,
                                        (const bf16*)b, eps, (bf16*)x, M, d, row_stride, row_offset, post,
                                        x_lay, row_group);
  else
    norm_kernel<float><<<M, nt, 0, st>>>(h, parts, nsplit, (const float*)bias, (const float*)g,
                                         (const float*)b, eps, (float*)x, M, d, row_stride, row_offset, post,
                                         0, row_group);
}

// ---------------------------------------------------------------------------------
// teacher-forced log-probabilities
// ---------------------------------------------------------------------------------
// (m, s) pairs stand for s * exp(m): the running maximum and the sum of exp(l - m).
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mx = fmaxf(m, m2);
  if (mx == -INFINITY) return;                     // both empty
  s = s * expf(m - mx) + s2 * expf(m2 - mx);
  m = mx;
}

__global__ __launch_bounds__(256) void logprob_gather_kernel(const float* __restrict__ logits, int V,
                                                             const int32_t* __restrict__ seq, int S,
                                                             int S_p, int n, int r0,
                                                             float* __restrict__ out) {
  __shared__ float sm[256], ss[256];
  const int r = blockIdx.x, tid = threadIdx.x;
  const int g = r0 + r, b = g / n, j = g - b * n;
  const float* L = logits + (size_t)r * V;
  float m = -INFINITY, s = 0.f;
  const int V4 = (V & 3) == 0 ? V >> 2 : 0;        // rows are 16-byte aligned when V % 4 == 0
  for (int i = tid; i < V4; i += 256) {
    const float4 v = reinterpret_cast<const float4*>(L)[i];
    const float mx = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
    if (mx > m) {
      s *= expf(m - mx);
      m = mx;
    }
    s += (expf(v.x - m) + expf(v.y - m)) + (expf(v.z - m) + expf(v.w - m));
  }
  for (int i = 4 * V4 + tid; i < V; i += 256) {
    const float x = L[i];
    if (x > m) {
      s *= expf(m - x);
      m = x;
    }
    s += expf(x - m);
  }
  sm[tid] = m;
  ss[tid] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {             // fixed tree: thread t takes t + w
    if (tid < w) {
      float a = sm[tid], c = ss[tid];
      lse_merge(a, c, sm[tid + w], ss[tid + w]);
      sm[tid] = a;
      ss[tid] = c;
    }
    __syncthreads();
  }
  if (tid == 0) {
    const int t = seq[(size_t)b * S + S_p + j];
    out[g] = (t >= 0 && t < V) ? L[t] - (sm[0] + logf(ss[0])) : __int_as_float(0x7fc00000);
  }
}

void launch_logprob_gather(const float* logits, int rows, int V, const int32_t* seq, int S, int S_p,
                           int n, int r0, float* out, hipStream_t st) {
  if (rows <= 0) return;
  logprob_gather_kernel<<<rows, 256, 0, st>>>(logits, V, seq, S, S_p, n, r0, out);
}

// ---------------------------------------------------------------------------------
// Pick: reduce the per-block (pick value, index) pairs of a row, greedy or sampled;
// the lowest index wins ties; optionally the log-probability.  One wave per row.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__global__ __launch_bounds__(64) void argmax_finalize_kernel(
    const float* __restrict__ best_val, const int32_t* __restrict__ best_idx, SampleArgs smp, int nb,
    int32_t* __restrict__ ids_cur, int32_t* __restrict__ tokens, float* __restrict__ logp, int tok_stride,
    const int32_t* __restrict__ pos_next, int32_t* __restrict__ pos_dev, int32_t* __restrict__ d_next) {
  const int m = blockIdx.x, l = threadIdx.x;
  const bool lse = logp && smp.blk_max;
  float bv = -INFINITY, bl = -INFINITY, mx = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = l; i < nb; i += 64) {
    const size_t o = (size_t)m * nb + i;
    const float v = best_val[o];
    const int ix = best_idx[o];
    if (better(v, ix, bv, bi)) { bv = v; bi = ix; if (lse) bl = smp.best_lg[o]; }
    if (lse) mx = fmaxf(mx, smp.blk_max[o]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64), ol = __shfl_xor(bl, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; bl = ol; }
    mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  }
  float sum = 0.f;
  if (lse) {
    // sum over blocks of blk_sum * exp(blk_max - mx): each lane its blocks in order,
    // then a fixed butterfly; lane 0's value is used
    for (int i = l; i < nb; i += 64) {
      const size_t o = (size_t)m * nb + i;
      sum += smp.blk_sum[o] * expf(smp.blk_max[o] - mx);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
  }
  if (l == 0) {
    const int p = *pos_next;
    const size_t oi = tok_stride ? (size_t)m * tok_stride + p : (size_t)m;
    if (bi == 0x7fffffff) bi = 0;
    if (ids_cur) ids_cur[m] = bi;
    if (tokens) tokens[oi] = bi;
    if (lse) logp[oi] = bl - (mx + logf(sum));
    if (d_next) d_next[m] = bi;
    if (m == 0 && pos_dev) *pos_dev = p;
  }
}

void launch_argmax_finalize(const float* best_val, const int32_t* best_idx, const SampleArgs& smp,
                            int n_blocks, int M, int32_t* ids_cur, int32_t* tokens, float* logp,
                            int tok_stride, const int32_t* pos_next, int32_t* pos_dev, int32_t* d_next,
                            hipStream_t st) {
  argmax_finalize_kernel<<<M, 64, 0, st>>>(best_val, best_idx, smp, n_blocks, ids_cur, tokens, logp,
                                           tok_stride, pos_next, pos_dev, d_next);
}

// ---------------------------------------------------------------------------------
// Top-p (nucleus) pick (Holtzman et al., ICLR 2020) from a row of fp32 logits, one
// block of 1024 threads per row.  s = logit * inv_temp and e = exp(s - max) stay in
// registers (kToppGroups groups of 4 columns per thread).  The nucleus threshold is
// the largest order key c (an order-preserving map of s to 32 bits) whose mass
// sum(e : key >= c) still reaches top_p * sum(e): found bit by bit from the top, each
// test one fixed-order block sum, so the decision is the same on every run.  The pick
// is the Gumbel-max rule over {key >= c} with the same Philox uniforms as the LM
// head's epilogue; the log-probability is that of the untruncated softmax(s).
// ---------------------------------------------------------------------------------
constexpr int kToppThreads = 1024, kToppGroups = 13;

__device__ __forceinline__ uint32_t ord_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float block_max(float v, float* red) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int nw = (blockDim.x + kWave - 1) / kWave;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = -INFINITY;
  for (int i = 0; i < nw; ++i) t = fmaxf(t, red[i]);
  return t;
}

__global__ __launch_bounds__(kToppThreads) void topp_finalize_kernel(
    const float* __restrict__ logits, int V, SampleArgs smp, float top_p, int32_t* __restrict__ ids_cur,
    int32_t* __restrict__ tokens, float* __restrict__ logp, int tok_stride,
    const int32_t* __restrict__ pos_next, int32_t* __restrict__ pos_dev) {
  __shared__ float red[64];
  __shared__ float bvs[kToppThreads / kWave];
  __shared__ int bis[kToppThreads / kWave];
  const int m = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const int p = *pos_next;
  const float* L = logits + (size_t)m * V;
  const int ng = (V + 3) >> 2;
  float sv[kToppGroups][4], ev[kToppGroups][4];
  float mx = -INFINITY;
#pragma unroll
  for (int g = 0; g < kToppGroups; ++g) {
    const int gi = tid + g * nt;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int col = 4 * gi + w;
      sv[g][w] = (gi < ng && col < V) ? L[col] * smp.inv_temp : -INFINITY;
      mx = fmaxf(mx, sv[g][w]);
    }
  }
  mx = block_max(mx, red);
  float z = 0.f;
#pragma unroll
  for (int g = 0; g < kToppGroups; ++g)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      ev[g][w] = sv[g][w] == -INFINITY ? 0.f : expf(sv[g][w] - mx);
      z += ev[g][w];
    }
  const float Z = block_sum(z, red);
  const float need = top_p * Z;
  uint32_t c = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = c | (1u << bit);
    float part = 0.f;
#pragma unroll
    for (int g = 0; g < kToppGroups; ++g)
#pragma unroll
      for (int w = 0; w < 4; ++w)
        if (sv[g][w] != -INFINITY && ord_key(sv[g][w]) >= cand) part += ev[g][w];
    if (block_sum(part, red + 32) >= need) c = cand;   // the same value in every thread
  }
  // the pick re-reads the row (from L2) rather than index the register copy by a
  // loop counter the compiler keeps rolled
  float bv = -INFINITY;
  int bi = 0x7fffffff;
#pragma unroll 1
  for (int gi = tid; gi < ng; gi += nt) {
    float gu[4];
    gumbel4(smp.seed, m, p, gi, gu);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int col = 4 * gi + w;
      if (col < V) {
        const float sw = L[col] * smp.inv_temp;
        if (ord_key(sw) >= c) {
          const float y = sw + gu[w];
          if (better(y, col, bv, bi)) { bv = y; bi = col; }
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, kWave);
    const int oi = __shfl_xor(bi, o, kWave);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  if ((tid & (kWave - 1)) == 0) { bvs[tid / kWave] = bv; bis[tid / kWave] = bi; }
  __syncthreads();
  if (tid == 0) {
    for (int i = 1; i < nt / kWave; ++i)
      if (better(bvs[i], bis[i], bv, bi)) { bv = bvs[i]; bi = bis[i]; }
    const size_t oi = tok_stride ? (size_t)m * tok_stride + p : (size_t)m;
    if (bi == 0x7fffffff) bi = 0;
    if (ids_cur) ids_cur[m] = bi;
    if (tokens) tokens[oi] = bi;
    if (logp) logp[oi] = L[bi] * smp.inv_temp - (mx + logf(Z));
    if (m == 0 && pos_dev) *pos_dev = p;
  }
}

int topp_max_vocab() { return kToppThreads * kToppGroups * 4; }

void launch_topp_finalize(const float* logits, int M, int V, const SampleArgs& smp, float top_p,
                          int32_t* ids_cur, int32_t* tokens, float* logp, int tok_stride,
                          const int32_t* pos_next, int32_t* pos_dev, hipStream_t st) {
  topp_finalize_kernel<<<M, kToppThreads, 0, st>>>(logits, V, smp, top_p, ids_cur, tokens, logp, tok_stride,
                                                   pos_next, pos_dev);
}

// ---------------------------------------------------------------------------------
// Reward head: reward[b] = (x[b, S-1] Pout^T) . w, fp32 accumulation, fixed order.
// ---------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void score_kernel(const T* __restrict__ x,
                                                    const T* __restrict__ Pout,
                                                    const T* __restrict__ w,
                                                    float* __restrict__ reward, float* __restrict__ y,
                                                    int S, int d, int de) {
  extern __shared__ float sm[];
  float* xs = sm;          // [d]
  float* ys = sm + d;      // [de]
  __shared__ float red[64];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const T* xr = x + ((size_t)b * S + S - 1) * d;
  for (int i = tid; i < d; i += 256) xs[i] = ld(xr + i);
  __syncthreads();
  if (Pout) {
    for (int j = wv; j < de; j += 4) {
      const T* pr = Pout + (size_t)j * d;
      float acc = 0.f;
      for (int k = lane; k < d; k += 64) acc = fmaf(xs[k], ld(pr + k), acc);
      acc = wave_sum(acc);
      if (lane == 0) ys[j] = acc;
    }
  } else {   // no output projection: y is the state itself (de == d)
    for (int j = tid; j < de; j += 256) ys[j] = xs[j];
  }
  __syncthreads();
  if (y)
    for (int j = tid; j < de; j += 256) y[(size_t)b * de + j] = ys[j];
  float part = 0.f;
  for (int j = tid; j < de; j += 256) part = fmaf(ys[j], ld(w + j), part);
  float tot = block_sum(part, red);
  if (tid == 0) reward[b] = tot;
}

void launch_score(int dt, const void* x, const void* proj_out, const void* w, float* reward, float* y,
                  int B, int S, int d, int de, hipStream_t st) {
  size_t lds = (size_t)(d + de) * sizeof(float);
  if (dt == DT_BF16)
    score_kernel<bf16><<<B, 256, lds, st>>>((const bf16*)x, (const bf16*)proj_out, (const bf16*)w,
                                            reward, y, S, d, de);
  else
    score_kernel<float><<<B, 256, lds, st>>>((const float*)x, (const float*)proj_out, (const float*)w,
                                             reward, y, S, d, de);
}

__global__ void set_i32_kernel(int32_t* p, int32_t v) { *p = v; }

void launch_set_i32(int32_t* p, int32_t v, hipStream_t st) { set_i32_kernel<<<1, 1, 0, st>>>(p, v); }

}  // namespace he
