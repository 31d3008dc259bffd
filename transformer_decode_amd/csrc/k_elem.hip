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
constexpr int kLoraTN = 32;

template <typename T, int kLoraTK>
__global__ __launch_bounds__(256) void lora_kernel(T* __restrict__ W, const T* __restrict__ A,
                                                   const T* __restrict__ Bm, int N, int K, int r,
                                                   float s, float sign) {
  extern __shared__ float lds[];
  float* As = lds;                    // [r][kLoraTK]
  float* Bs = lds + r * kLoraTK;      // [kLoraTN][r]
  const int k0 = blockIdx.x * kLoraTK, n0 = blockIdx.y * kLoraTN;
  const int tid = threadIdx.x;
  for (int i = tid; i < r * kLoraTK; i += 256) {
    int j = i / kLoraTK, c = i % kLoraTK;
    As[i] = (k0 + c < K) ? ld(A + (size_t)j * K + k0 + c) : 0.f;
  }
  for (int i = tid; i < kLoraTN * r; i += 256) {
    int n = i / r, j = i % r;
    Bs[i] = (n0 + n < N) ? ld(Bm + (size_t)(n0 + n) * r + j) : 0.f;
  }
  __syncthreads();
  constexpr int CPR = kLoraTK / 8;            // 8-column chunks per row
  constexpr int RPP = 256 / CPR;              // rows per pass
  const int c8 = tid % CPR, sub = tid / CPR;
  const int k = k0 + c8 * 8;
  if (k >= K) return;
#pragma unroll
  for (int i = 0; i < kLoraTN / RPP; ++i) {
    const int nl = sub + RPP * i, n = n0 + nl;
    if (n >= N) break;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < r; ++j) {
      const float b = Bs[nl * r + j];
      const float* a = As + j * kLoraTK + c8 * 8;
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = fmaf(b, a[q], acc[q]);
    }
    T* wp = W + (size_t)n * K + k;
    float w[8];
    load8(wp, w);
#pragma unroll
    for (int q = 0; q < 8; ++q) w[q] = w[q] + sign * (s * acc[q]);
    store8(wp, w);
  }
}

template <int TK>
static void lora_launch(int dt, void* W, const void* A, const void* B, int N, int K, int r, float s,
                        float sign, hipStream_t st) {
  dim3 grid((K + TK - 1) / TK, (N + kLoraTN - 1) / kLoraTN);
  size_t lds = (size_t)(r * TK + kLoraTN * r) * sizeof(float);   // <= 41 KB for r <= 64
  if (dt == DT_BF16)
    lora_kernel<bf16, TK><<<grid, 256, lds, st>>>((bf16*)W, (const bf16*)A, (const bf16*)B, N, K, r, s, sign);
  else
    lora_kernel<float, TK><<<grid, 256, lds, st>>>((float*)W, (const float*)A, (const float*)B, N, K, r, s, sign);
}

void launch_lora(int dt, void* W, const void* A, const void* B, int N, int K, int r, float s,
                 float sign, hipStream_t st) {
  if (r <= 32) lora_launch<256>(dt, W, A, B, N, K, r, s, sign, st);
  else lora_launch<128>(dt, W, A, B, N, K, r, s, sign, st);
}

// ---------------------------------------------------------------------------------
// Row LayerNorm helpers: one WG of 256 threads per row, each thread owns up to
// kMaxChunks chunks of 8 consecutive elements (d <= 8192, d % 8 == 0).  Mean and
// biased variance are two fixed-order block reductions (deterministic).
// ---------------------------------------------------------------------------------
constexpr int kMaxChunks = 4;

template <typename T>
__device__ __forceinline__ void ln_write(const float (&v)[kMaxChunks][8], int d, float eps,
                                         const T* g, const T* b, T* xrow, float* hrow_post,
                                         float* red) {
  const int tid = threadIdx.x, nch = d / 8;
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    int ch = tid + c * 256;
    if (ch < nch)
#pragma unroll
      for (int q = 0; q < 8; ++q) s += v[c][q];
  }
  const float mean = block_sum(s, red) / (float)d;
  float s2 = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    int ch = tid + c * 256;
    if (ch < nch)
#pragma unroll
      for (int q = 0; q < 8; ++q) { float t = v[c][q] - mean; s2 += t * t; }
  }
  const float var = block_sum(s2, red + 32) / (float)d;
  const float rstd = 1.f / sqrtf(var + eps);
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    int ch = tid + c * 256;
    if (ch < nch) {
      float gv[8], bv[8], y[8];
      load8(g + ch * 8, gv);
      load8(b + ch * 8, bv);
#pragma unroll
      for (int q = 0; q < 8; ++q) y[q] = (v[c][q] - mean) * rstd * gv[q] + bv[q];
      if (hrow_post) store8(hrow_post + ch * 8, y);   // post-LN: the stream is the norm
      store8(xrow + ch * 8, y);                           // GEMM input: rounded
    }
  }
}

// h[m] = E[id] + P[pos + 2]; x[m] = round(LN(h[m])) (or round(h[m]) without LN).
// Position table row pos + 2: OPT's learned positions are offset by two rows.
template <typename T>
__global__ __launch_bounds__(256) void embed_norm_kernel(const int32_t* __restrict__ ids,
                                                         const int32_t* __restrict__ pos_dev,
                                                         int seq_len, const T* __restrict__ E,
                                                         const T* __restrict__ P,
                                                         const T* __restrict__ g,
                                                         const T* __restrict__ b, float eps,
                                                         float* __restrict__ h, T* __restrict__ x,
                                                         int d, int vocab) {
  __shared__ float red[64];
  const int m = blockIdx.x, tid = threadIdx.x, nch = d / 8;
  int id = ids[m];
  id = id < 0 ? 0 : (id >= vocab ? vocab - 1 : id);   // memory safety for bad ids
  const int pos = pos_dev ? *pos_dev : (m % seq_len);
  const T* er = E + (size_t)id * d;
  const T* pr = P + (size_t)(pos + 2) * d;
  float v[kMaxChunks][8];
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    int ch = tid + c * 256;
    if (ch < nch) {
      float e[8], p[8];
      load8(er + ch * 8, e);
      load8(pr + ch * 8, p);
#pragma unroll
      for (int q = 0; q < 8; ++q) v[c][q] = e[q] + p[q];
      store8(h + (size_t)m * d + ch * 8, v[c]);
    }
  }
  if (g) {
    ln_write<T>(v, d, eps, g, b, x + (size_t)m * d, nullptr, red);
  } else {
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      int ch = tid + c * 256;
      if (ch < nch) store8(x + (size_t)m * d + ch * 8, v[c]);
    }
  }
}

void launch_embed_norm(int dt, const int32_t* ids, const int32_t* pos_dev, int seq_len,
                       const void* E, const void* P, const void* g, const void* b, float eps,
                       float* h, void* x, int M, int d, int vocab, hipStream_t st) {
  if (dt == DT_BF16)
    embed_norm_kernel<bf16><<<M, 256, 0, st>>>(ids, pos_dev, seq_len, (const bf16*)E, (const bf16*)P,
                                               (const bf16*)g, (const bf16*)b, eps, h, (bf16*)x, d,
                                               vocab);
  else
    embed_norm_kernel<float><<<M, 256, 0, st>>>(ids, pos_dev, seq_len, (const float*)E, (const float*)P,
                                                (const float*)g, (const float*)b, eps, h, (float*)x, d,
                                                vocab);
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

// Residual update (sum of split-K partials + bias, fixed order) and LayerNorm.
template <typename T>
__global__ __launch_bounds__(256) void norm_kernel(float* __restrict__ h,
                                                   const float* __restrict__ parts, int nsplit,
                                                   const T* __restrict__ bias,
                                                   const T* __restrict__ g,
                                                   const T* __restrict__ b, float eps,
                                                   T* __restrict__ x, int M, int d, int row_stride,
                                                   int row_offset, int post) {
  __shared__ float red[64];
  const int r = blockIdx.x, tid = threadIdx.x, nch = d / 8;
  const size_t row = (size_t)r * row_stride + row_offset;
  float* hr = h + row * d;
  float v[kMaxChunks][8];
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    int ch = tid + c * 256;
    if (ch < nch) {
      load8(hr + ch * 8, v[c]);
      if (parts) {
        float add[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int s = 0; s < nsplit; ++s) {
          float pv[8];
          load8(parts + ((size_t)s * M + r) * d + ch * 8, pv);
#pragma unroll
          for (int q = 0; q < 8; ++q) add[q] += pv[q];
        }
        float bv[8];
        load8(bias + ch * 8, bv);
#pragma unroll
        for (int q = 0; q < 8; ++q) v[c][q] += add[q] + bv[q];
        store8(hr + ch * 8, v[c]);
      }
    }
  }
  ln_write<T>(v, d, eps, g, b, x + (size_t)r * d, post ? hr : nullptr, red);
}

void launch_norm(int dt, float* h, const float* parts, int nsplit, const void* bias, const void* g,
                 const void* b, float eps, void* x, int M, int d, int row_stride, int row_offset,
                 int post, hipStream_t st) {
  if (dt == DT_BF16)
    norm_kernel<bf16><<<M, 256, 0, st>>>(h, parts, nsplit, (const bf16*)bias, (const bf16*)g,
                                         (const bf16*)b, eps, (bf16*)x, M, d, row_stride, row_offset, post);
  else
    norm_kernel<float><<<M, 256, 0, st>>>(h, parts, nsplit, (const float*)bias, (const float*)g,
                                          (const float*)b, eps, (float*)x, M, d, row_stride, row_offset, post);
}

// ---------------------------------------------------------------------------------
// Greedy pick: reduce the per-block (max, index) pairs of a row; the lowest index
// wins ties.  One wave per row.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__global__ __launch_bounds__(64) void argmax_finalize_kernel(
    const float* __restrict__ best_val, const int32_t* __restrict__ best_idx, int nb,
    int32_t* __restrict__ ids_cur, int32_t* __restrict__ tokens, int tok_stride,
    const int32_t* __restrict__ pos_dev, int32_t* __restrict__ d_next) {
  const int m = blockIdx.x, l = threadIdx.x;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = l; i < nb; i += 64) {
    float v = best_val[(size_t)m * nb + i];
    int ix = best_idx[(size_t)m * nb + i];
    if (better(v, ix, bv, bi)) { bv = v; bi = ix; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(bv, o, 64);
    int oi = __shfl_xor(bi, o, 64);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  if (l == 0) {
    if (bi == 0x7fffffff) bi = 0;
    if (ids_cur) ids_cur[m] = bi;
    if (tokens) tokens[(size_t)m * tok_stride + *pos_dev] = bi;
    if (d_next) d_next[m] = bi;
  }
}

void launch_argmax_finalize(const float* best_val, const int32_t* best_idx, int n_blocks, int M,
                            int32_t* ids_cur, int32_t* tokens, int tok_stride,
                            const int32_t* pos_dev, int32_t* d_next, hipStream_t st) {
  argmax_finalize_kernel<<<M, 64, 0, st>>>(best_val, best_idx, n_blocks, ids_cur, tokens,
                                           tok_stride, pos_dev, d_next);
}

// ---------------------------------------------------------------------------------
// Reward head: reward[b] = (x[b, S-1] Pout^T) . w, fp32 accumulation, fixed order.
// ---------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void score_kernel(const T* __restrict__ x,
                                                    const T* __restrict__ Pout,
                                                    const T* __restrict__ w,
                                                    float* __restrict__ reward, int S, int d,
                                                    int de) {
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
  float part = 0.f;
  for (int j = tid; j < de; j += 256) part = fmaf(ys[j], ld(w + j), part);
  float tot = block_sum(part, red);
  if (tid == 0) reward[b] = tot;
}

void launch_score(int dt, const void* x, const void* proj_out, const void* w, float* reward, int B,
                  int S, int d, int de, hipStream_t st) {
  size_t lds = (size_t)(d + de) * sizeof(float);
  if (dt == DT_BF16)
    score_kernel<bf16><<<B, 256, lds, st>>>((const bf16*)x, (const bf16*)proj_out, (const bf16*)w,
                                            reward, S, d, de);
  else
    score_kernel<float><<<B, 256, lds, st>>>((const float*)x, (const float*)proj_out, (const float*)w,
                                             reward, S, d, de);
}

__global__ void set_i32_kernel(int32_t* p, int32_t v) { *p = v; }

void launch_set_i32(int32_t* p, int32_t v, hipStream_t st) { set_i32_kernel<<<1, 1, 0, st>>>(p, v); }

}  // namespace he
