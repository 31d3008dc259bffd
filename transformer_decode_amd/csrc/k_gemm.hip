// Prompt-pass projections of libhe: Y[M,N] = X[M,K] W[N,K]^T with fused epilogues.
//
// bf16 models: for M, N multiples of 256 an MFMA GEMM on 32 x 32 x 16 tiles with
// 256 x 256 macro tiles staged by LDS DMA, one persistent WG per CU (gemm_pers_kernel,
// K a multiple of 128: every model the library accepts); other shapes run a
// 256 x 256 (8 waves) or 128 x 128 (4 waves) kernel on 16 x 16 x 32 tiles with
// register-staged loads.  fp32 models (the tiny workload only): a plain tiled FMA
// kernel.  All end in the same epilogue: bias, q scaling + KV-cache scatter (the
// prompt's keys and values enter the cache here), residual add, ReLU, position add.
// bf16 weights and activations are read row-major or in the inference layout
// (EpiArgs::w_il / x_il, il_off), and ReLU / position-add outputs written in either
// (o_il): a 16-byte chunk is 8 consecutive k of one row in both.
#include <algorithm>
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
    st((T*)e.out + il_off(m, n, N, e.o_il), fmaxf(v, 0.f));
  } else if (MODE == EPI_POSADD) {
    const int t = m % e.seq_len;
    float v = acc + ld((const T*)e.pos_emb + (size_t)(e.pos0 + t + 2) * N + n);
    e.h[(size_t)m * N + n] = v;
    st((T*)e.out + il_off(m, n, N, e.o_il), v);
  } else {
    float bv = e.bias ? ld((const T*)e.bias + n) : 0.f;
    e.out_f32[(size_t)m * (e.ldo ? e.ldo : N) + n] = acc + bv;
  }
}

// Four consecutive output columns n .. n + 3 of row m (bf16 storage, n % 4 == 0),
// the same arithmetic as epi_store element by element, with vector accesses.
__device__ __forceinline__ void ld_bf4(const bf16* p, float* o) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  o[0] = __uint_as_float(u.x << 16); o[1] = __uint_as_float(u.x & 0xffff0000u);
  o[2] = __uint_as_float(u.y << 16); o[3] = __uint_as_float(u.y & 0xffff0000u);
}
__device__ __forceinline__ void st_bf4(bf16* p, const float* v) {
  uint2 u;
  u.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
  u.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}

template <int MODE>
__device__ __forceinline__ void epi_store4(const EpiArgs& e, int m, int n, int N, const float (&acc)[4]) {
  float b[4] = {0.f, 0.f, 0.f, 0.f}, v[4];
  if (MODE != EPI_POSADD && e.bias) ld_bf4((const bf16*)e.bias + n, b);
  if (MODE == EPI_QKV) {
    const int part = n / e.d, within = n - part * e.d;
    const int head = within / e.D, dd = within - head * e.D;
    const int bb = m / e.seq_len, t = m - bb * e.seq_len;
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = acc[c] + b[c];
    if (part == 0) {
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] *= e.q_scale;
      st_bf4((bf16*)e.q_out + (size_t)m * e.d + within, v);
    } else {
      bf16* cache = (bf16*)(part == 1 ? e.k_cache : e.v_cache);
      st_bf4(cache + (((size_t)bb * e.H + head) * e.S_max + e.pos0 + t) * e.D + dd, v);
    }
  } else if (MODE == EPI_RESID) {
    float4* hp = reinterpret_cast<float4*>(e.h + (size_t)m * N + n);
    float4 h = *hp;
    h.x += acc[0] + b[0]; h.y += acc[1] + b[1]; h.z += acc[2] + b[2]; h.w += acc[3] + b[3];
    *hp = h;
  } else if (MODE == EPI_RELU) {
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = fmaxf(acc[c] + b[c], 0.f);
    st_bf4((bf16*)e.out + il_off(m, n, N, e.o_il), v);
  } else if (MODE == EPI_POSADD) {
    const int t = m % e.seq_len;
    float p[4];
    ld_bf4((const bf16*)e.pos_emb + (size_t)(e.pos0 + t + 2) * N + n, p);
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = acc[c] + p[c];
    *reinterpret_cast<float4*>(e.h + (size_t)m * N + n) = make_float4(v[0], v[1], v[2], v[3]);
    st_bf4((bf16*)e.out + il_off(m, n, N, e.o_il), v);
  } else {
    *reinterpret_cast<float4*>(e.out_f32 + (size_t)m * (e.ldo ? e.ldo : N) + n) =
        make_float4(acc[0] + b[0], acc[1] + b[1], acc[2] + b[2], acc[3] + b[3]);
  }
}

// Eight consecutive output columns n .. n + 7 of row m (bf16 storage, n % 8 == 0).
template <int MODE>
__device__ __forceinline__ void epi_store8(const EpiArgs& e, int m, int n, int N, const float (&acc)[8]) {
  float b[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, v[8];
  if (MODE != EPI_POSADD && e.bias) load8((const bf16*)e.bias + n, b);
  if (MODE == EPI_QKV) {
    const int part = n / e.d, within = n - part * e.d;
    const int head = within / e.D, dd = within - head * e.D;
    const int bb = m / e.seq_len, t = m - bb * e.seq_len;
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = acc[c] + b[c];
    if (part == 0) {
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c] *= e.q_scale;
      store8((bf16*)e.q_out + (size_t)m * e.d + within, v);
    } else {
      bf16* cache = (bf16*)(part == 1 ? e.k_cache : e.v_cache);
      store8(cache + (((size_t)bb * e.H + head) * e.S_max + e.pos0 + t) * e.D + dd, v);
    }
  } else if (MODE == EPI_RESID) {
    float* hp = e.h + (size_t)m * N + n;
    float h[8];
    load8(hp, h);
#pragma unroll
    for (int c = 0; c < 8; ++c) h[c] += acc[c] + b[c];
    store8(hp, h);
  } else if (MODE == EPI_RELU) {
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = fmaxf(acc[c] + b[c], 0.f);
    store8((bf16*)e.out + il_off(m, n, N, e.o_il), v);
  } else if (MODE == EPI_POSADD) {
    const int t = m % e.seq_len;
    float p[8];
    load8((const bf16*)e.pos_emb + (size_t)(e.pos0 + t + 2) * N + n, p);
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = acc[c] + p[c];
    store8(e.h + (size_t)m * N + n, v);
    store8((bf16*)e.out + il_off(m, n, N, e.o_il), v);
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = acc[c] + b[c];
    store8(e.out_f32 + (size_t)m * (e.ldo ? e.ldo : N) + n, v);
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
      ra[i] = (gm < M && k < K) ? *reinterpret_cast<const uint4*>(X + il_off(gm, k, K, e.x_il))
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
      ra[i] = (gm < M && k < K) ? *reinterpret_cast<const uint4*>(X + il_off(gm, k, K, e.x_il)) : make_uint4(0, 0, 0, 0);
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
// bf16 MFMA GEMM on 32 x 32 x 16 tiles staged by LDS DMA (M, N multiples of 256,
// K of 32).  256 x 256 macro tile.  The 32 x 32 x 16 instruction sustains about
// 2.1 PFLOP/s on constant operands (1.65 to 1.7 on random ones, where power sets the
// clock) where the 16 x 16 x 32 one stops near 1.3 with one wave per SIMD (measured).
// An operand fragment is 32 rows x 16 k = 1 KB, lane l holding row l % 32, k 8 (l / 32)
// .. + 8.  A stage is 32 k, staged as 16 fragments of X and 16 of W in the 16 x 32
// shape of the weights' inference layout (1 KB each, lane l at row l % 16, k 8 (l / 16)),
// filled with buffer_load_dwordx4 ... lds: each lane's 16 bytes (8 consecutive k of one
// row) land at slot + 16 l.  A W fragment in the inference layout is 1 KB of
// consecutive bytes (whole cache lines); row-major X is 16 rows x 64 bytes.  The
// 32 x 32 x 16 operands are read back from pairs of fragments with ds_read_b128 free of
// bank conflicts, and never pass through VGPRs on the way in.  Four stages (128 KB of
// LDS) rotate: loads run three stages ahead of the MFMAs.
// ---------------------------------------------------------------------------------
constexpr int FBM = 256, FBN = 256, FST = 4;
typedef __attribute__((address_space(3))) void lds_void;
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Raw buffer resource over `bytes` bytes from `base` (gfx9 descriptor word 3: 32-bit
// data format, no swizzle), for buffer_load_dwordx4 ... lds.  The buffer form of the
// LDS DMA takes a scalar offset per access and one VGPR per lane, and unlike the
// global_load_lds form it is not taken by the compiler for a possible out-of-order LDS
// access, so its LDS reads keep precise lgkmcnt waits.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void buf_dma16(__amdgpu_buffer_rsrc_t r, bf16* lds_slot, uint32_t voff,
                                          uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_slot, 16, voff, soff, 0, 0);
}

// s_waitcnt with vmcnt = n (n < 64), expcnt and lgkmcnt left open (gfx9 encoding).
#define HE_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// Workgroup barrier without __syncthreads' release fence (which waits for every
// outstanding load, the prefetch DMA included).  LDS reads before it have completed
// (each was waited for by the MFMA that used it); the asm memory clobber keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_keep_loads() { asm volatile("s_barrier" ::: "memory"); }

// Offsets of the 16 x 32 fragment (16-row tile, k-step s) of a [rows][K] operand in
// layout il (0 row-major, else the inference layout, il_off).  The address of lane l
// splits into a part fixed for the kernel and a wave-uniform part per k-step.  Row-major:
// row l % 16, k 8 (l / 16) + 32 s (16 rows x 64 bytes).  Inference layout with block
// width BW = 2^il: the fragment is 512 / BW row pieces of BW / 8 units (1 KB of
// consecutive bytes for BW = 512): lane part (l / (BW / 8)) K + 8 (l mod BW / 8), k-step
// part the block row and column of k 32 s (il_frag).
__device__ __forceinline__ uint32_t frag_lane_part(int lane, int K, int il) {
  if (il == 0) return (uint32_t)((lane & 15) * K + ((lane >> 4) << 3));
  const int lgu = il - 3;
  return (uint32_t)((lane >> lgu) * K + ((lane & ((1 << lgu) - 1)) << 3));
}
__device__ __forceinline__ uint32_t frag_step_part(int s, int K, int il) {
  if (il == 0) return (uint32_t)(32 * s);
  const int q = s & ((1 << (il - 5)) - 1);
  return (uint32_t)(((q << 6) >> (il - 3)) * K + ((s >> (il - 5)) << il));
}

// Eight waves (2 x 4), each owning 128 x 64 of the macro tile as 4 x 2 32 x 32 tiles:
// 128 accumulator registers per wave, so two waves share each SIMD and one issues MFMAs
// while the other waits at the stage barrier or for its LDS reads (measured 3 to 4%
// faster than four waves of 128 x 128 with one wave per SIMD on the 6.7B prompt-pass
// shapes, 11% on K = 1024 shapes).  Each wave loads two X and two W fragments per stage;
// per 16-wide k-step it reads 2 W and 4 X operands for 8 MFMAs.  Operand g of k-step ks
// of a stage: g < 2 column tile 2 wn + g of W, else row tile 4 wm + g - 2 of X; the
// 32 x 32 x 16 operand (lane l: row l % 32, k 8 (l / 32) .. + 8 of the step) of 32-row
// tile t is gathered from the 16-row fragments 2t and 2t + 1 (row r in fragment
// 2t + r / 16 at lane (r mod 16) + 16 (2 ks + l / 32)), so each 16 lanes read 256
// consecutive bytes, free of bank conflicts.
//
// The loop body is straight-line so the accumulators stay in place.  Each half-stage is
// four groups of one DMA issue, one or two LDS reads and two MFMAs, in that order, so
// the DMA issues and the reads of the next k-step are spread between the MFMAs rather
// than queued in front of them.  r0 holds the first 16-wide k-step of a stage, r1 the
// second; each is read one half-stage before its MFMAs.
//
// Persistent: one WG per CU walks its tiles (the same tiles, in the same order, as a
// launch of one WG per tile would give that CU).  The stage stream runs on across tiles: the
// last three k-stages of tile r issue the DMA of tile r + 1's stages 0..2 (K / 32 is a
// multiple of 4, so stage s of every tile keeps buffer s mod 4), and the epilogue of tile
// r runs while they land.  The epilogue parks 32 x 32 blocks in the fourth buffer (held
// by tile r's last stage, free after its last barrier): 4 KB per wave, 16-byte chunks
// XOR-swizzled by row so that the parking writes and the row-wise reads hit distinct
// banks.  Against one WG per tile (the same arithmetic, bit-identical results), measured
// at the OPT-6.7B prompt-pass shapes: QKV 1196.5 -> 1151.2 us, FC1 1587.1 -> 1522.1, out
// 458.4 -> 447.0.
template <int MODE, bool WIL, bool XIL>
__global__ __launch_bounds__(512) void gemm_pers_kernel(const bf16* __restrict__ X,
                                                         const bf16* __restrict__ W, int M, int N,
                                                         int K, EpiArgs e) {
  __shared__ __attribute__((aligned(1024))) bf16 fsm[FST * 2 * 16 * 512];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 2, wn = wv & 3;

  const int nm = M / FBM, nn = N / FBN, T = nm * nn;
  const int per = (T + 7) / 8;
  const int xcd = blockIdx.x & 7, jw = blockIdx.x >> 3, nj = gridDim.x >> 3;
  auto tile_of = [&](int r) -> int {       // tile r of this WG, or -1
    const int tl = jw + r * nj;
    if (tl >= per) return -1;
    const int t = xcd * per + tl;
    return t < T ? t : -1;
  };
  constexpr int GM = 4;
  auto tile_m0 = [&](int t) {
    const int group = t / (GM * nn), first_m = group * GM, gsz = min(nm - first_m, GM);
    return (first_m + (t % (GM * nn)) % gsz) * FBM;
  };
  auto tile_n0 = [&](int t) {
    const int group = t / (GM * nn), first_m = group * GM, gsz = min(nm - first_m, GM);
    return ((t % (GM * nn)) / gsz) * FBN;
  };
  int t = tile_of(0);
  if (t < 0) return;
  const int ilx = XIL ? e.x_il : 0, ilw = WIL ? e.w_il : 0;
  const uint32_t tile_bytes = (uint32_t)(FBM * K * 2);
  int m0 = tile_m0(t), n0 = tile_n0(t);
  __amdgpu_buffer_rsrc_t rx = buf_rsrc(X + (size_t)m0 * K, tile_bytes);
  __amdgpu_buffer_rsrc_t rw = buf_rsrc(W + (size_t)n0 * K, tile_bytes);
  const uint32_t lane_x = frag_lane_part(lane, K, ilx), lane_w = frag_lane_part(lane, K, ilw);
  uint32_t vx[2], vw[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint32_t rows = (uint32_t)((wv * 2 + q) * 16 * K);
    vx[q] = (lane_x + rows) * 2;
    vw[q] = (lane_w + rows) * 2;
  }
  auto dma = [&](__amdgpu_buffer_rsrc_t ax, __amdgpu_buffer_rsrc_t aw, int g, int s, int buf) {
    bf16* sa = fsm + (size_t)buf * 2 * 16 * 512 + (wv * 2 + (g >> 1)) * 512;
    if ((g & 1) == 0)
      buf_dma16(ax, sa, vx[g >> 1], frag_step_part(s, K, ilx) * 2);
    else
      buf_dma16(aw, sa + 16 * 512, vw[g >> 1], frag_step_part(s, K, ilw) * 2);
  };
  const int rl = lane & 31;
  const uint32_t lane_lds = (uint32_t)((rl >> 4) * 512 + ((rl & 15) + ((lane >> 5) << 4)) * 8);
  auto read_frag = [&](int s, int ks, int g) -> bf16x8 {
    const bf16* sa = fsm + (size_t)(s & (FST - 1)) * 2 * 16 * 512 + ks * 256 + lane_lds;
    return g < 2 ? *reinterpret_cast<const bf16x8*>(sa + 16 * 512 + (wn * 2 + g) * 1024)
                 : *reinterpret_cast<const bf16x8*>(sa + (wm * 4 + g - 2) * 1024);
  };
  f32x16 acc[4][2];
  auto mma2 = [&](const bf16x8 (&r)[6], int g) {
    acc[g][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[0], r[2 + g], acc[g][0], 0, 0, 0);
    acc[g][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r[1], r[2 + g], acc[g][1], 0, 0, 0);
  };
  auto reads = [&](bf16x8 (&r)[6], int s, int ks, int g) {
    if (g < 2) {
      r[g] = read_frag(s, ks, g);
    } else {
      r[2 * g - 2] = read_frag(s, ks, 2 * g - 2);
      r[2 * g - 1] = read_frag(s, ks, 2 * g - 1);
    }
  };

  const int ns = K / 32;                   // a multiple of 4
#pragma unroll
  for (int s = 0; s < FST - 1; ++s)
#pragma unroll
    for (int g = 0; g < 4; ++g) dma(rx, rw, g, min(s, ns - 1), s);
  HE_WAIT_VMCNT(4 * (FST - 2));
  barrier_keep_loads();
  bf16x8 r0[6], r1[6];
#pragma unroll
  for (int g = 0; g < 4; ++g) reads(r0, 0, 0, g);

  float* park = reinterpret_cast<float*>(fsm + (size_t)(FST - 1) * 2 * 16 * 512) + wv * 1024;
  for (int r = 0; t >= 0; ++r) {
    const int tn = tile_of(r + 1);
    const bool more = tn >= 0;
    const int m1 = more ? tile_m0(tn) : m0, n1 = more ? tile_n0(tn) : n0;
    const __amdgpu_buffer_rsrc_t rx1 = more ? buf_rsrc(X + (size_t)m1 * K, tile_bytes) : rx;
    const __amdgpu_buffer_rsrc_t rw1 = more ? buf_rsrc(W + (size_t)n1 * K, tile_bytes) : rw;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
    for (int s = 0; s < ns; ++s) {
      // half A: DMA of stage s + 3 (past the end: the next tile's stage s + 3 - ns, or
      // after the last tile a repeat of this tile's last stage into the free buffer),
      // read the second k-step of stage s, multiply the first
      const int sa = s + FST - 1, bd = sa & (FST - 1);
      const bool own = sa < ns;
      const __amdgpu_buffer_rsrc_t ax = own || !more ? rx : rx1, aw = own || !more ? rw : rw1;
      const int sd = own ? sa : (more ? sa - ns : ns - 1);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        dma(ax, aw, g, sd, bd);
        reads(r1, s, 1, g);
        mma2(r0, g);
        __builtin_amdgcn_sched_barrier(0);
      }
      HE_WAIT_VMCNT(4 * (FST - 2));
      barrier_keep_loads();
      // half B: read the first k-step of stage s + 1 (after the last stage: the next
      // tile's stage 0, in buffer 0), multiply the second of stage s
      const int sn = s + 1 < ns ? s + 1 : (more ? ns : s);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        reads(r0, sn, 0, g);
        mma2(r1, g);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // The last stage's buffer becomes the park: every wave's reads of it have completed
    // (its MFMAs waited for them) before any wave parks.  After the last tile the
    // repeated loads are drained.
    if (!more) HE_WAIT_VMCNT(0);
    barrier_keep_loads();

    // Epilogue, one 32 x 32 block (row tile i, column tile j) at a time: lane l holds
    // row l % 32, columns 8 q + 4 (l / 32) + c of register 4 q + c; read back, lane l
    // takes row l / 4 (+ 16) and columns 8 (l mod 4) .. + 8.
    auto park_block = [&](int i, int j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int pc = (2 * q + (lane >> 5)) ^ (rl & 7);
        *reinterpret_cast<f32x4*>(park + rl * 32 + pc * 4) =
            f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0)
    };
    auto read_block = [&](int hh, float (&v)[8]) {
      const int row = (lane >> 2) + 16 * hh, c0 = 2 * (lane & 3);
      const float4 a = *reinterpret_cast<const float4*>(park + row * 32 + ((c0 ^ (row & 7)) << 2));
      const float4 b = *reinterpret_cast<const float4*>(park + row * 32 + (((c0 + 1) ^ (row & 7)) << 2));
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    };
    const int colq = (lane & 3) << 3;
    if constexpr (MODE == EPI_RESID) {
      // h += acc + bias; the stream values of block b + 1 are fetched while block b is
      // added and stored
      float bias[2][8];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (e.bias) load8((const bf16*)e.bias + n0 + wn * 64 + j * 32 + colq, bias[j]);
        else
#pragma unroll
          for (int c = 0; c < 8; ++c) bias[j][c] = 0.f;
      }
      auto hptr = [&](int b, int hh) {
        return e.h + (size_t)(m0 + wm * 128 + (b >> 1) * 32 + (lane >> 2) + 16 * hh) * N + n0 + wn * 64 +
               (b & 1) * 32 + colq;
      };
      float hc[2][8], hn[2][8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) load8(hptr(0, hh), hc[hh]);
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        park_block(b >> 1, b & 1);
        if (b < 7)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) load8(hptr(b + 1, hh), hn[hh]);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          float v[8], hv[8];
          read_block(hh, v);
#pragma unroll
          for (int c = 0; c < 8; ++c) hv[c] = hc[hh][c] + (v[c] + bias[b & 1][c]);
          store8(hptr(b, hh), hv);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);   // this block's park reads are done
        if (b < 7)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int c = 0; c < 8; ++c) hc[hh][c] = hn[hh][c];
      }
    } else {
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        park_block(b >> 1, b & 1);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          float v[8];
          read_block(hh, v);
          epi_store8<MODE>(e, m0 + wm * 128 + (b >> 1) * 32 + (lane >> 2) + 16 * hh,
                           n0 + wn * 64 + (b & 1) * 32 + colq, N, v);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
      }
    }
    // every wave is done with the park buffer before the next tile's DMA refills it
    barrier_keep_loads();
    t = tn; m0 = m1; n0 = n1; rx = rx1; rw = rw1;
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

// Compute units of the current device (cached per device): the persistent GEMM puts at
// most one WG on each.
static int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

template <int MODE>
static void gemm_dispatch(int dt, const void* X, const void* W, int M, int N, int K,
                          const EpiArgs& e, hipStream_t st) {
  if (dt == DT_BF16) {
    if (M % FBM == 0 && N % FBN == 0 && K % (32 * FST) == 0) {
      // one WG per CU, a multiple of 8 (WG i runs on XCD i mod 8), each walking its
      // XCD's tiles with stride pb / 8
      const int per = ((M / FBM) * (N / FBN) + 7) / 8;
      const int pb = 8 * std::min(per, std::max(1, device_cus() / 8));
      const bf16 *x = (const bf16*)X, *w = (const bf16*)W;
      if (e.w_il && e.x_il)
        gemm_pers_kernel<MODE, true, true><<<pb, 512, 0, st>>>(x, w, M, N, K, e);
      else if (e.w_il)
        gemm_pers_kernel<MODE, true, false><<<pb, 512, 0, st>>>(x, w, M, N, K, e);
      else if (e.x_il)
        gemm_pers_kernel<MODE, false, true><<<pb, 512, 0, st>>>(x, w, M, N, K, e);
      else
        gemm_pers_kernel<MODE, false, false><<<pb, 512, 0, st>>>(x, w, M, N, K, e);
      return;
    }
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
