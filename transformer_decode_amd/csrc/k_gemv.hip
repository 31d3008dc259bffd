// Decode-step projections of libhe: Y[M,N] = X[M,K] W[N,K]^T with M = batch <= 128.
//
// Generation streams every weight once per token (paper summary, "Inference Mode:
// Generation Phase Optimizations": generation is bound by memory bandwidth, and the
// inference kernels lay the weights out for sequential access).  bf16 models read W
// in the inference layout (common.h, il_off) while the adapters are folded in: every
// 16 x 32 MFMA A operand is 1 KB of consecutive bytes, so one 16-byte load per lane
// fetches a whole fragment with fully used HBM bursts.  Unfused base weights
// (row-major) go through the same kernel with 64-byte pieces per row.  The activations arrive fragment-tiled too (xt_off): the B
// operand of a k-step is 1 KB per 16 batch rows, read from L2.
//
//  * A wave owns FR 16-row fragments of W and a K range of kr; it keeps PD k-steps
//    of W and X loads in flight (a register ring) ahead of its MFMAs.
//  * The NWK waves of a WG share the rows and take consecutive K ranges; at the end
//    they reduce through LDS in a fixed wave order, so split-K leaves K / (kr NWK)
//    partial groups (often one) for the consumer to sum, also in a fixed order.
//  * Epilogues: fp32 partials; bias + ReLU rounded into the next projection's tiled
//    activations (one group only); bias, q scaling and rounding with the k and v of
//    the step appended to the KV cache (one group only); per-WG greedy argmax (+
//    optional logits).
// fp32 models (the tiny workload) use a plain FMA kernel on row-major weights.
#include <utility>

#include "common.h"
#include "kernels.h"

namespace he {

namespace {
int pow2_ceil(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}
}  // namespace

int il_of(int K) {
  int il = 9;
  while (il > 5 && K % (1 << il)) --il;
  return il;
}

int decode_mt(int M) { return pow2_ceil((M + 15) / 16); }

// Work split of one decode projection.  bf16 rules, from timing every (fr, nwk, kr)
// on the decode shapes: long K ranges win (each wave streams one long run of W; up
// to 1024 k), then the most rows per wave (fewer activation loads per weight byte)
// that still puts >= 512 waves in flight, then as many waves per WG (fewer partials)
// as keeps the WG count a multiple of the 256 CUs or >= 1024.  `whole` asks for a
// single partial group (the fused bias+ReLU and argmax epilogues).  `f8` (E4M3
// weights) asks for K ranges that are multiples of 256 (eight k-steps per loop
// iteration).  65-128 batch rows (bf16 weights) follow their own rules, below.
// fp32: a split over K.
GemvPlan decode_plan(int dt, int M, int N, int K, bool allow_split, bool whole, bool f8) {
  GemvPlan p;
  if (dt != DT_BF16) {
    p.splits = allow_split ? std::max(1, std::min(K / 256, 8)) : 1;
    return p;
  }
  p.mt = decode_mt(M);
  const int nrb = N / 16, frmax = p.mt <= 4 ? 4 : 2;
  if (p.mt >= 8 && !f8) {
    // 65..128 batch rows: each k-step a wave reads 2 KB of activations from L2 per 16
    // weight rows it owns, so waves take 48-80 rows (accumulators in up to 160
    // registers, one wave per SIMD) and the grid one WG per CU.  Measured at the 13B
    // decode shapes, batch 128 (per launch, from the plans for up to 64 rows): QKV
    // 58.6 -> 43.4 us, out 24.8 -> 19.2, FC1 77.2 -> 47.0, FC2 88.8 -> 47.1.
    auto rows = [&](int fr) { return (long)(nrb + fr - 1) / fr; };
    if (whole && rows(2) >= 1024) {        // the LM head: 64 rows and the whole K per wave
      p.fr = 4; p.nwk = 1; p.kr = K; p.splits = 1;   // (batch 128, K 5120: 199.5 -> 141.1 us)
      return p;
    }
    if (whole || N > K) {                  // QKV (fused epilogue) and FC1 (ReLU epilogue): whole K
      int fr = 5;                          // the fewest rounds of 256 WGs times rows per wave
      long best = -1;
      for (int f : {5, 4, 3}) {
        const long cost = (rows(f) + 255) / 256 * f;
        if (best < 0 || cost < best) { best = cost; fr = f; }
      }
      int nwk = 1;
      while (nwk < 4 && rows(fr) * nwk < 1024 && K % (128 * nwk * 2) == 0) nwk *= 2;
      if (K % (128 * nwk) == 0) {
        p.fr = fr; p.nwk = nwk; p.kr = K / nwk; p.splits = 1;
        return p;
      }
    } else if (allow_split) {              // out-proj, FC2: the fewest partial groups that
      const long rg = rows(5);             // give 256 WGs, each with the most waves that divide K
      for (int sp = (int)std::max<long>(1, (256 + rg - 1) / rg); sp <= 64; ++sp)
        for (int nwk : {4, 2, 1})
          if (K % (sp * nwk * 128) == 0) {
            p.fr = 5; p.nwk = nwk; p.kr = K / (sp * nwk); p.splits = sp;
            return p;
          }
    }
  }
  auto choose = [&](int kr, bool need_waves) {
    const int slices = K / kr;
    for (int fr = frmax; fr >= 1; fr >>= 1) {
      const long rg = (nrb + fr - 1) / fr;
      if (need_waves && fr > 1 && rg * slices < 512) continue;
      for (int nwk = 4; nwk >= 1; nwk >>= 1) {
        if (slices % nwk) continue;
        if (whole && slices != nwk) continue;
        const long wgs = rg * (slices / nwk);
        if (nwk > 1 && !(wgs % 256 == 0 || wgs >= 1024)) continue;
        if (need_waves && rg * slices < 512) return false;
        p.fr = fr; p.nwk = nwk; p.kr = kr; p.splits = slices / nwk;
        return true;
      }
    }
    return false;
  };
  if (whole) {   // one group, a K range of K / nwk per wave
    auto rows = [&](int fr) { return (long)(nrb + fr - 1) / fr; };
    if (rows(frmax) >= 512) {         // enough WGs (the LM head): two waves split K
      const int kq = f8 ? 256 : 128;
      p.fr = frmax; p.nwk = K % (2 * kq) == 0 ? 2 : 1; p.kr = K / p.nwk; p.splits = 1;
      return p;
    }
    // few row groups (QKV): fill the 256 CUs evenly -- the fewest rounds of 256 WGs
    // times rows per wave, ties to more rows per wave (3 rows per wave fits 768 row
    // blocks to 256 WGs exactly) -- with waves per WG up to 4 toward 1024 waves
    int best_fr = frmax;
    long best_cost = -1;
    for (int fr : {4, 3, 2, 1}) {
      if (fr > frmax || (fr == 3 && p.mt > 4)) continue;
      const long cost = (rows(fr) + 255) / 256 * fr;
      if (best_cost < 0 || cost < best_cost) { best_cost = cost; best_fr = fr; }
    }
    const int kq = f8 ? 256 : 128;
    int nwk = 1;
    while (nwk < 4 && rows(best_fr) * nwk < 1024 && K % (kq * nwk * 2) == 0) nwk *= 2;
    if (K % (kq * nwk) == 0) {
      p.fr = best_fr; p.nwk = nwk; p.kr = K / nwk; p.splits = 1;
      return p;
    }
  }
  if (allow_split) {
    for (int kr = 1024; kr >= (f8 ? 256 : 128); kr >>= 1)
      if (K % kr == 0 && choose(kr, true)) return p;
  }
  // small matrices: as many waves as the shortest K range gives (K % 128 == 0 is
  // required of bf16 models, K % 256 == 0 of E4M3 weights)
  p.fr = 1; p.nwk = 1;
  p.kr = allow_split ? (f8 ? 256 : 128) : K;
  p.splits = K / p.kr;
  return p;
}

int gemv_argmax_blocks(int dt, const GemvPlan& p, int N) {
  if (dt == DT_BF16 && p.splits == 1) return (N / 16 + p.fr - 1) / p.fr;
  return (N + 127) / 128;
}

__device__ __forceinline__ bool gv_better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Compile-time loop: f(integral_constant<0>) ... f(integral_constant<N-1>).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

struct IlArgs {
  int M, N, K, il, ns;            // ns: k-steps per wave (a multiple of 4, >= 4)
  float* parts;                   // PARTIAL: [splits][M][N]
  const bf16* bias;               // RELU
  bf16* out;                      // RELU: tiled activations (mt tiles)
  float* logits;                  // ARGMAX (nullable): [M][N]
  float* best_val;                // ARGMAX: [M][n_blocks]
  int32_t* best_idx;
  int n_blocks;
  int32_t* pos_next;              // ARGMAX: gets *pos_dev + 1, the picked token's position
  float inv_temp;                 // ARGMAX: pick rule (SampleArgs)
  uint64_t seed;
  float* best_lg;
  float* blk_max;
  float* blk_sum;
  bf16* q_out;                    // QKV
  bf16* k_cache;
  bf16* v_cache;
  const int32_t* pos_dev;
  int d, H, D, S_max;
  float q_scale;
  const float* wscale;            // FP8 weights: per-row scales (W is then E4M3 in f8_off layout)
};

constexpr int kPD = 3;            // k-steps of loads in flight ahead of the MFMAs
constexpr int kNB = kPD + 1;      // ring slots

// Weights are read once per decode step: non-temporal loads, which do not keep them in
// the caches (the activations, re-read by every wave, stay there).  Measured on the
// decode kernels: the streams run markedly faster this way.
__device__ __forceinline__ bf16x8 ld_stream(const bf16* p) { return __builtin_bit_cast(bf16x8, ld_once(p)); }
__device__ __forceinline__ uint4 ld_stream_u4(const uint8_t* p) { return ld_once(p); }

// Eight E4M3 codes (two words) as the bf16 A operand of one k-step: exact, since
// every E4M3 value is a bf16 value (gfx950 packed conversion, scale 1).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, false);
  const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, true);
  const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, false);
  const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, true);
  const auto q0 = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  const auto q1 = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int MT, int FR, int NWK, int OUT, bool F8 = false>
__global__ __launch_bounds__(NWK * 64) void gemv_il_kernel(const bf16* __restrict__ X,
                                                           const bf16* __restrict__ W, IlArgs a) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nrb = a.N >> 4, rb0 = blockIdx.x * FR;
  const int s0 = (blockIdx.y * NWK + wv) * a.ns;
  int wrb[FR];
#pragma unroll
  for (int f = 0; f < FR; ++f) wrb[f] = min(rb0 + f, nrb - 1);
  f32x4 acc[FR][MT];
#pragma unroll
  for (int f = 0; f < FR; ++f)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[f][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (F8) {
    // E4M3 weights: one 16-byte load per lane and fragment covers k-steps 2u and 2u + 1
    // (double step u), so W is loaded with every other k-step.  Activations keep the
    // k-step ring of kNB slots; double steps rotate through 4 slots.  Eight k-steps per
    // iteration (a.ns % 8 == 0) keep every slot index fixed: at step i of an iteration
    // the loads of step i + kPD are issued (its activations, and for even steps the
    // double step), then step i multiplies from slot i % 4 and double slot i / 2.
    const uint8_t* W8 = reinterpret_cast<const uint8_t*>(W);
    const size_t k64 = (size_t)(a.K >> 6);
    bf16x8 xs[kNB][MT];
    uint4 w8[4][FR];
    auto load_x = [&](int j, auto slot) {
      const int s = s0 + j;
#pragma unroll
      for (int t = 0; t < MT; ++t)
        xs[slot][t] = *reinterpret_cast<const bf16x8*>(X + ((size_t)(s * MT + t) << 9) + lane * 8);
    };
    auto load_w = [&](int j, auto slot) {     // the double step holding k-step j (j even)
      const size_t u = (size_t)((s0 + j) >> 1);
#pragma unroll
      for (int f = 0; f < FR; ++f)
        w8[slot][f] = ld_stream_u4(W8 + ((size_t)wrb[f] * k64 + u) * 1024 + lane * 16);
    };
    auto mma8 = [&](auto xslot, auto wslot, auto half) {
#pragma unroll
      for (int f = 0; f < FR; ++f) {
        const uint4 q = w8[wslot][f];
        const bf16x8 wa = half ? e4m3x8_to_bf16(q.z, q.w) : e4m3x8_to_bf16(q.x, q.y);
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, xs[xslot][t], acc[f][t], 0, 0, 0);
      }
    };
    load_w(0, std::integral_constant<int, 0>{});
    load_x(0, std::integral_constant<int, 0>{});
    load_x(1, std::integral_constant<int, 1>{});
    load_w(2, std::integral_constant<int, 1>{});
    load_x(2, std::integral_constant<int, 2>{});
    int j0 = 0;
    for (; j0 + 8 < a.ns; j0 += 8) {
      static_for<8>([&](auto i) {
        constexpr int la = i + kPD;                          // step whose loads go now
        if constexpr ((la & 1) == 0) load_w(j0 + la, std::integral_constant<int, (la / 2) % 4>{});
        load_x(j0 + la, std::integral_constant<int, la % kNB>{});
        __builtin_amdgcn_sched_barrier(0);
        mma8(std::integral_constant<int, i % kNB>{}, std::integral_constant<int, (i / 2) % 4>{},
             std::integral_constant<int, i & 1>{});
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    static_for<8>([&](auto i) {                                // the last eight steps
      constexpr int la = i + kPD;
      if constexpr (la < 8) {
        if constexpr ((la & 1) == 0) load_w(j0 + la, std::integral_constant<int, (la / 2) % 4>{});
        load_x(j0 + la, std::integral_constant<int, la % kNB>{});
      }
      mma8(std::integral_constant<int, i % kNB>{}, std::integral_constant<int, (i / 2) % 4>{},
           std::integral_constant<int, i & 1>{});
    });
    // per-row scales: the fragment's lane holds rows 16 rb + 4 (lane / 16) + r
#pragma unroll
    for (int f = 0; f < FR; ++f) {
      const f32x4 sc = *reinterpret_cast<const f32x4*>(a.wscale + wrb[f] * 16 + (lane >> 4) * 4);
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[f][t] *= sc;
    }
  } else {
  bf16x8 w[kNB][FR], x[kNB][MT];
  // QKV (up to 64 batch rows) starts each WG's K range at a different k-step (7 per WG,
  // mod the range): its activations were just written by the LayerNorm, so every XCD
  // fetches them cold, and waves that all start on the same lines wait on the same
  // misses.  Measured in the 6.7B decode loop: 1376.0 -> 1369.4 ms per generation (the
  // other projections measured slower this way).  Each WG still sums its K range in one
  // fixed order.
  const int rot = OUT == GV_QKV && MT <= 4 ? (int)((blockIdx.x * 7u) % (unsigned)a.ns) : 0;
  auto load = [&](int j, auto slot) {      // k-step s0 + (j + rot mod ns) into ring slot `slot`
    int jj = j + rot;
    if (jj >= a.ns) jj -= a.ns;
    const int s = s0 + jj;
#pragma unroll
    for (int f = 0; f < FR; ++f)
      w[slot][f] = ld_stream(W + il_frag(wrb[f], s, lane, a.K, a.il));
#pragma unroll
    for (int t = 0; t < MT; ++t)
      x[slot][t] = *reinterpret_cast<const bf16x8*>(X + ((size_t)(s * MT + t) << 9) + lane * 8);
  };
  auto mma = [&](auto slot) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int f = 0; f < FR; ++f)
        acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[slot][f], x[slot][t], acc[f][t], 0, 0, 0);
  };
  // Steps j0 .. j0 + 3 per iteration, each issuing the loads of step j + 3 first.
  // The last group is peeled (its single remaining load, no clamping), which keeps
  // the ring in fixed registers and the loop's waits at "this step's loads only".
  static_for<kPD>([&](auto i) { load(i, i); });
  int j0 = 0;
  for (; j0 + kNB < a.ns; j0 += kNB) {
    static_for<kNB>([&](auto i) {
      load(j0 + i + kPD, std::integral_constant<int, (i + kPD) % kNB>{});
      __builtin_amdgcn_sched_barrier(0);
      mma(i);
      __builtin_amdgcn_sched_barrier(0);
    });
  }
  load(j0 + kPD, std::integral_constant<int, kPD>{});
  static_for<kNB>([&](auto i) { mma(i); });
  }

  // D fragment: lane holds rows n = 16 rb + 4 (lane / 16) + r of batch row 16 t + lane % 16.
  __shared__ f32x4 red[NWK > 1 || OUT == GV_ARGMAX ? NWK : 1][FR * MT][64];
  auto emit = [&](int f, int t, f32x4 v) {
    const int rb = rb0 + f;
    const int n = rb * 16 + (lane >> 4) * 4, m = t * 16 + (lane & 15);
    if (rb >= nrb || m >= a.M) return;
    if (OUT == GV_PARTIAL) {
      *reinterpret_cast<f32x4*>(a.parts + ((size_t)blockIdx.y * a.M + m) * a.N + n) = v;
    } else if (OUT == GV_RELU) {
      const uint2 bb = *reinterpret_cast<const uint2*>(a.bias + n);
      const float b4[4] = {__uint_as_float(bb.x << 16), __uint_as_float(bb.x & 0xffff0000u),
                           __uint_as_float(bb.y << 16), __uint_as_float(bb.y & 0xffff0000u)};
      uint2 u;
      u.x = (uint32_t)f2bf(fmaxf(v[0] + b4[0], 0.f)) | ((uint32_t)f2bf(fmaxf(v[1] + b4[1], 0.f)) << 16);
      u.y = (uint32_t)f2bf(fmaxf(v[2] + b4[2], 0.f)) | ((uint32_t)f2bf(fmaxf(v[3] + b4[3], 0.f)) << 16);
      *reinterpret_cast<uint2*>(a.out + xt_off(m, n, MT)) = u;
    } else if (OUT == GV_QKV) {
      // four consecutive columns of one of q, k, v (D % 4 == 0): one head, one 8-byte store
      const uint2 bb = *reinterpret_cast<const uint2*>(a.bias + n);
      float w[4] = {v[0] + __uint_as_float(bb.x << 16), v[1] + __uint_as_float(bb.x & 0xffff0000u),
                    v[2] + __uint_as_float(bb.y << 16), v[3] + __uint_as_float(bb.y & 0xffff0000u)};
      const int part = n / a.d, within = n - part * a.d;
      bf16* dst;
      if (part == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) w[c] *= a.q_scale;
        dst = a.q_out + (size_t)m * a.d + within;
      } else {
        const int head = within / a.D, dd = within - head * a.D;
        dst = (part == 1 ? a.k_cache : a.v_cache) + (((size_t)m * a.H + head) * a.S_max + *a.pos_dev) * a.D + dd;
      }
      uint2 u;
      u.x = (uint32_t)f2bf(w[0]) | ((uint32_t)f2bf(w[1]) << 16);
      u.y = (uint32_t)f2bf(w[2]) | ((uint32_t)f2bf(w[3]) << 16);
      *reinterpret_cast<uint2*>(dst) = u;
    } else {
      if (a.logits) *reinterpret_cast<f32x4*>(a.logits + (size_t)m * a.N + n) = v;
    }
  };
  if (NWK > 1) {
#pragma unroll
    for (int f = 0; f < FR; ++f)
#pragma unroll
      for (int t = 0; t < MT; ++t) red[wv][f * MT + t][lane] = acc[f][t];
    __syncthreads();
    for (int idx = wv; idx < FR * MT; idx += NWK) {
      f32x4 v = red[0][idx][lane];
#pragma unroll
      for (int q = 1; q < NWK; ++q) v += red[q][idx][lane];
      emit(idx / MT, idx % MT, v);
      if (OUT == GV_ARGMAX) red[0][idx][lane] = v;   // only this wave touches slot idx of wave 0 now
    }
  } else {
#pragma unroll
    for (int f = 0; f < FR; ++f)
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        emit(f, t, acc[f][t]);
        if (OUT == GV_ARGMAX) red[0][f * MT + t][lane] = acc[f][t];
      }
  }
  if (OUT == GV_ARGMAX) {
    // per batch row over this WG's FR * 16 rows of W: the pick (largest logit, or
    // tempered logit + Gumbel noise; lowest index on ties), its tempered logit, and the
    // block's largest tempered logit and sum of exponentials, each in a fixed order
    __syncthreads();
    const bool samp = a.inv_temp > 0.f;
    const float sc = samp ? a.inv_temp : 1.f;
    const int gpos = a.pos_dev ? *a.pos_dev + 1 : 0;
    for (int m = threadIdx.x; m < MT * 16; m += NWK * 64) {
      const int t = m >> 4, c = m & 15;
      float bv = -INFINITY, blg = -INFINITY, mx = -INFINITY;
      int bi = min(rb0 * 16, a.N - 1);
      for (int f = 0; f < FR && rb0 + f < nrb; ++f)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v = red[0][f * MT + t][g * 16 + c];
          const int n0 = (rb0 + f) * 16 + g * 4;
          float gn[4] = {0.f, 0.f, 0.f, 0.f};
          if (samp) gumbel4(a.seed, m, gpos, n0 >> 2, gn);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float lg = v[r] * sc, y = lg + gn[r];
            if (y > bv) { bv = y; bi = n0 + r; blg = lg; }   // n increases: the first maximum stays
            mx = fmaxf(mx, lg);
          }
        }
      float sum = 0.f;
      if (a.blk_max)
        for (int f = 0; f < FR && rb0 + f < nrb; ++f)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 v = red[0][f * MT + t][g * 16 + c];
#pragma unroll
            for (int r = 0; r < 4; ++r) sum += expf(v[r] * sc - mx);
          }
      if (m < a.M) {
        const size_t o = (size_t)m * a.n_blocks + blockIdx.x;
        a.best_val[o] = bv;
        a.best_idx[o] = bi;
        if (a.blk_max) { a.best_lg[o] = blg; a.blk_max[o] = mx; a.blk_sum[o] = sum; }
      }
    }
    if (a.pos_next && blockIdx.x == 0 && threadIdx.x == 0) *a.pos_next = gpos;
  }
}

thread_local LaunchTimer g_launch_timer;

template <class Kern>
static void timed_launch(Kern k, dim3 grid, dim3 block, hipStream_t st, const bf16* X, const bf16* W,
                         const IlArgs& a) {
  if (g_launch_timer.start) {
    hipExtLaunchKernelGGL(k, grid, block, 0, st, g_launch_timer.start, g_launch_timer.stop, 0, X, W, a);
    g_launch_timer = LaunchTimer{};
  } else {
    k<<<grid, block, 0, st>>>(X, W, a);
  }
}

template <int MT, int FR, int NWK>
static void il_launch(int out, const bf16* X, const bf16* W, const IlArgs& a, int splits,
                      hipStream_t st) {
  dim3 grid((a.N / 16 + FR - 1) / FR, splits);
  const dim3 block(NWK * 64);
  if (a.wscale) {                 // E4M3 weights (no LM head: it keeps bf16)
    if (out == GV_PARTIAL) timed_launch(gemv_il_kernel<MT, FR, NWK, GV_PARTIAL, true>, grid, block, st, X, W, a);
    else if (out == GV_RELU) timed_launch(gemv_il_kernel<MT, FR, NWK, GV_RELU, true>, grid, block, st, X, W, a);
    else timed_launch(gemv_il_kernel<MT, FR, NWK, GV_QKV, true>, grid, block, st, X, W, a);
    return;
  }
  if (out == GV_PARTIAL) timed_launch(gemv_il_kernel<MT, FR, NWK, GV_PARTIAL>, grid, block, st, X, W, a);
  else if (out == GV_RELU) timed_launch(gemv_il_kernel<MT, FR, NWK, GV_RELU>, grid, block, st, X, W, a);
  else if (out == GV_QKV) timed_launch(gemv_il_kernel<MT, FR, NWK, GV_QKV>, grid, block, st, X, W, a);
  else timed_launch(gemv_il_kernel<MT, FR, NWK, GV_ARGMAX>, grid, block, st, X, W, a);
}

template <int MT, int FR>
static void il_launch_nwk(int out, const bf16* X, const bf16* W, const IlArgs& a, const GemvPlan& p,
                          hipStream_t st) {
  if (p.nwk == 4) il_launch<MT, FR, 4>(out, X, W, a, p.splits, st);
  else if (p.nwk == 2) il_launch<MT, FR, 2>(out, X, W, a, p.splits, st);
  else il_launch<MT, FR, 1>(out, X, W, a, p.splits, st);
}

template <int MT>
static void il_launch_fr(int out, const bf16* X, const bf16* W, const IlArgs& a, const GemvPlan& p,
                         hipStream_t st) {
  if constexpr (MT == 8) {            // five fragments per wave: the 65-128-row plans only
    if (p.fr == 5) {
      il_launch_nwk<MT, 5>(out, X, W, a, p, st);
      return;
    }
  }
  if (p.fr == 4) il_launch_nwk<MT, 4>(out, X, W, a, p, st);
  else if (p.fr == 3) il_launch_nwk<MT, 3>(out, X, W, a, p, st);
  else if (p.fr >= 2) il_launch_nwk<MT, 2>(out, X, W, a, p, st);
  else il_launch_nwk<MT, 1>(out, X, W, a, p, st);
}

// ---------------------------------------------------------------------------------
// partial reductions
// ---------------------------------------------------------------------------------
// a[m][n] = round(relu(sum_s parts[s][m][n] + bias[n])), fixed order over s; written
// fragment-tiled (mt tiles) for the next decode projection.
__global__ __launch_bounds__(256) void reduce_relu_kernel(const float* __restrict__ parts, int S,
                                                          const bf16* __restrict__ bias,
                                                          bf16* __restrict__ out, int M, int N, int mt) {
  const size_t i4 = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const size_t total = (size_t)M * N;
  if (i4 >= total) return;
  const int n = (int)(i4 % N), m = (int)(i4 / N);
  float a[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) {
    const float4 p = *reinterpret_cast<const float4*>(parts + (size_t)s * total + i4);
    a[0] += p.x; a[1] += p.y; a[2] += p.z; a[3] += p.w;
  }
  uint2 u;
  float v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = fmaxf(a[q] + bf2f(bias[n + q]), 0.f);
  u.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
  u.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
  *reinterpret_cast<uint2*>(out + (mt ? xt_off(m, n, mt) : i4)) = u;
}

// One 128-column block of row m under the pick rule of SampleArgs: the thread holds
// column n's logit v (ok: n < N).  Writes the block's pick value and index (lowest
// index on ties) and, with blk_max, the pick's tempered logit, the largest tempered
// logit and the sum of exp(tempered logit - that maximum); the two waves are merged in
// a fixed order through `sh` (8 floats, 2 ints).
__device__ __forceinline__ void pick_block128(bool ok, float v, int n, int m, int nb, float inv_temp,
                                              uint64_t seed, int gpos, float* best_val, int32_t* best_idx,
                                              float* best_lg, float* blk_max, float* blk_sum,
                                              float* sh, int* shi) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const bool samp = inv_temp > 0.f;
  const float lg = ok ? v * (samp ? inv_temp : 1.f) : -INFINITY;
  float y = lg, blg = lg;
  if (ok && samp) {
    float g4[4];
    gumbel4(seed, m, gpos, n >> 2, g4);
    y = lg + g4[n & 3];
  }
  int idx = n;
  float mx = lg;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float ov = __shfl_xor(y, o, 64), ol = __shfl_xor(blg, o, 64);
    const int oi = __shfl_xor(idx, o, 64);
    if (gv_better(ov, oi, y, idx)) { y = ov; idx = oi; blg = ol; }
    mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  }
  if (lane == 0) { sh[wv] = y; shi[wv] = idx; sh[2 + wv] = blg; sh[4 + wv] = mx; }
  __syncthreads();
  const float bmx = fmaxf(sh[4], sh[5]);
  float e = ok ? expf(lg - bmx) : 0.f;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) e += __shfl_xor(e, o, 64);
  if (lane == 0) sh[6 + wv] = e;
  __syncthreads();
  if (threadIdx.x == 0) {
    float by = sh[0], bl = sh[2];
    int bi = shi[0];
    if (gv_better(sh[1], shi[1], by, bi)) { by = sh[1]; bi = shi[1]; bl = sh[3]; }
    const size_t o = (size_t)m * nb + blockIdx.x;
    best_val[o] = by;
    best_idx[o] = bi;
    if (blk_max) { best_lg[o] = bl; blk_max[o] = bmx; blk_sum[o] = sh[6] + sh[7]; }
  }
}

// logits[m][n] = sum_s parts[s][m][n]; per (m, block of 128 columns) the pick rule.
__global__ __launch_bounds__(128) void reduce_argmax_kernel(const float* __restrict__ parts, int S,
                                                            int M, int N, float* __restrict__ logits,
                                                            float* __restrict__ best_val,
                                                            int32_t* __restrict__ best_idx, int nb,
                                                            const int32_t* __restrict__ pos_dev,
                                                            int32_t* __restrict__ pos_next, SampleArgs smp) {
  __shared__ float sh[8];
  __shared__ int shi[2];
  const int m = blockIdx.y, n = blockIdx.x * 128 + threadIdx.x;
  const size_t total = (size_t)M * N;
  float a = 0.f;
  if (n < N) {
    for (int s = 0; s < S; ++s) a += parts[(size_t)s * total + (size_t)m * N + n];
    if (logits) logits[(size_t)m * N + n] = a;
  }
  const int gpos = pos_dev ? *pos_dev + 1 : 0;
  pick_block128(n < N, a, n, m, nb, smp.inv_temp, smp.seed, gpos, best_val, best_idx, smp.best_lg,
                smp.blk_max, smp.blk_sum, sh, shi);
  if (pos_next && blockIdx.x == 0 && m == 0 && threadIdx.x == 0) *pos_next = gpos;
}

void launch_reduce_relu(const float* parts, int S, const void* bias, void* out, int M, int N, int mt,
                        hipStream_t st) {
  const size_t n4 = ((size_t)M * N + 3) / 4;
  reduce_relu_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, st>>>(parts, S, (const bf16*)bias,
                                                                  (bf16*)out, M, N, mt);
}

void launch_reduce_argmax(const float* parts, int S, int M, int N, float* logits, float* best_val,
                          int32_t* best_idx, int nb, const int32_t* pos_dev, int32_t* pos_next,
                          const SampleArgs& smp, hipStream_t st) {
  dim3 grid((N + 127) / 128, M);
  reduce_argmax_kernel<<<grid, 128, 0, st>>>(parts, S, M, N, logits, best_val, best_idx, nb, pos_dev,
                                             pos_next, smp);
}

// ---------------------------------------------------------------------------------
// fp32 models: one thread per (m, n), 128 columns per WG, 128-column argmax blocks.
// ---------------------------------------------------------------------------------
template <int OUT>
__global__ __launch_bounds__(128) void gemv_f32_kernel(const float* __restrict__ X,
                                                       const float* __restrict__ W, int M, int N,
                                                       int K, GemvArgs g) {
  __shared__ float sh[8];
  __shared__ int shi[2];
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
  } else {   // one split (the whole K): the pick rule per 128-column block
    if (n < N && g.logits) g.logits[(size_t)m * N + n] = acc;
    const int gpos = g.pos_dev ? *g.pos_dev + 1 : 0;
    pick_block128(n < N, acc, n, m, g.n_blocks, g.smp.inv_temp, g.smp.seed, gpos, g.best_val, g.best_idx,
                  g.smp.best_lg, g.smp.blk_max, g.smp.blk_sum, sh, shi);
    if (g.pos_next && blockIdx.x == 0 && m == 0 && threadIdx.x == 0) *g.pos_next = gpos;
  }
}

void launch_gemv(int dt, const void* X, const void* W, int M, int N, int K, const GemvPlan& p,
                 const GemvArgs& g, hipStream_t st) {
  if (dt == DT_BF16) {
    IlArgs a;
    a.M = M; a.N = N; a.K = K; a.il = g.w_il; a.ns = p.kr / 32;
    a.parts = g.parts; a.bias = (const bf16*)g.bias; a.out = (bf16*)g.out;
    a.logits = g.logits; a.best_val = g.best_val; a.best_idx = g.best_idx;
    a.n_blocks = g.n_blocks; a.pos_next = g.pos_next;
    a.inv_temp = g.smp.inv_temp; a.seed = g.smp.seed;
    a.best_lg = g.smp.best_lg; a.blk_max = g.smp.blk_max; a.blk_sum = g.smp.blk_sum;
    a.q_out = (bf16*)g.q_out; a.k_cache = (bf16*)g.k_cache; a.v_cache = (bf16*)g.v_cache;
    a.pos_dev = g.pos_dev; a.d = g.d; a.H = g.H; a.D = g.D; a.S_max = g.S_max; a.q_scale = g.q_scale;
    a.wscale = g.w_scale;
    const bf16* x = (const bf16*)X;
    const bf16* w = (const bf16*)W;
    switch (p.mt) {
      case 1: il_launch_fr<1>(g.out_mode, x, w, a, p, st); break;
      case 2: il_launch_fr<2>(g.out_mode, x, w, a, p, st); break;
      case 4: il_launch_fr<4>(g.out_mode, x, w, a, p, st); break;
      default: il_launch_fr<8>(g.out_mode, x, w, a, p, st); break;
    }
    return;
  }
  const int splits = g.out_mode == GV_PARTIAL ? p.splits : 1;
  dim3 grid((N + 127) / 128, splits, M);
  switch (g.out_mode) {
    case GV_RELU: gemv_f32_kernel<GV_RELU><<<grid, 128, 0, st>>>((const float*)X, (const float*)W, M, N, K, g); break;
    case GV_ARGMAX: gemv_f32_kernel<GV_ARGMAX><<<grid, 128, 0, st>>>((const float*)X, (const float*)W, M, N, K, g); break;
    default: gemv_f32_kernel<GV_PARTIAL><<<grid, 128, 0, st>>>((const float*)X, (const float*)W, M, N, K, g); break;
  }
}

}  // namespace he
