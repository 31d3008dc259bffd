// Attention kernels of libhe.
//
// Decode (paper summary, "Inference Mode: Generation Phase Optimizations": attention
// specialised for one new query against a long cached context, and a KV cache to
// which each step appends its keys and values).  One WG per (sequence, head).  The
// WG first finishes the step's q, k, v from the projection's split-K partials
// (fixed-order sum + bias; q scaled by D^-1/2), rounds them to the storage type and
// appends k, v at the current position.  It then streams the cached keys and values
// once: a group of D/8 lanes owns one key at a time (16-byte loads, a wave reads
// whole 256-byte rows), keeps a running max / sum / weighted value sum (online
// softmax), and the groups are merged in a fixed order through LDS.  Every K/V byte
// is used by exactly one lane, so the loads go straight to registers.
//
// Prompt pass: causal attention with MFMA.  One WG per (64-query tile, sequence,
// head); each wave owns 16 queries.  Key tiles of 64 are staged in LDS (values
// transposed for the B operand), scores S = Q K^T and the output O += P V run on
// v_mfma_f32_16x16x32_bf16, softmax is online per row with wave shuffles.  The
// probabilities P enter the second product as a pair of bf16 terms (P rounded,
// plus the rounded remainder), which keeps about 16 significant bits of P.
#include "common.h"
#include "kernels.h"

namespace he {

// ---------------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------------
// Eight storage elements held as loaded (bf16 stays packed: 4 VGPRs, not 8).
template <typename T> struct Raw8;
template <> struct Raw8<bf16> {
  uint4 u;
  __device__ __forceinline__ void load(const bf16* p) { u = ld_once(p); }   // K / V read once
  __device__ __forceinline__ void unpack(float* o) const {
    o[0] = __uint_as_float(u.x << 16); o[1] = __uint_as_float(u.x & 0xffff0000u);
    o[2] = __uint_as_float(u.y << 16); o[3] = __uint_as_float(u.y & 0xffff0000u);
    o[4] = __uint_as_float(u.z << 16); o[5] = __uint_as_float(u.z & 0xffff0000u);
    o[6] = __uint_as_float(u.w << 16); o[7] = __uint_as_float(u.w & 0xffff0000u);
  }
};
template <> struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void unpack(float* o) const {
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
};
// Sum over each aligned group of G lanes (G = 2, 4, 8, 16); every lane of the group
// receives the sum.  DPP lane moves within a row of 16 lanes, no LDS traffic:
// swap neighbours, swap pairs, mirror within 8, mirror within 16.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  auto mv = [](float x, int ctrl) -> float {
    switch (ctrl) {
      case 0xB1: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
      case 0x4E: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
      case 0x141: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
      default: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
    }
  };
  if (G >= 2) v += mv(v, 0xB1);     // quad_perm [1,0,3,2]
  if (G >= 4) v += mv(v, 0x4E);     // quad_perm [2,3,0,1]
  if (G >= 8) v += mv(v, 0x141);    // row_half_mirror
  if (G >= 16) v += mv(v, 0x140);   // row_mirror
  return v;
}

// QIN: q arrives finished ([B, d], scaled, rounded) and the step's k and v are
// already in the cache at `pos` (the QKV projection's epilogue put them there), so
// keys 0..pos all stream from the cache; otherwise q, k and v are finished here from
// the projection's split-K partials and k, v appended.
template <typename T, int D, bool QIN>
__global__ __launch_bounds__(256, (D >= 64 && sizeof(T) == 2 ? 8 : 4)) void attn_decode_kernel(const float* __restrict__ parts,
                                                          int nsplit, const T* __restrict__ bqkv,
                                                          const T* __restrict__ qin,
                                                          T* __restrict__ kc, T* __restrict__ vc,
                                                          const int32_t* __restrict__ pos_dev,
                                                          T* __restrict__ o, int B, int H,
                                                          int S_max, float q_scale, int x_mt) {
  constexpr int LPK = D / 8;            // lanes per key
  constexpr int NG = 256 / LPK;         // key groups per WG
  __shared__ float qs[D], kn[D], vn[D];
  __shared__ float gm[NG], gl[NG];
  __shared__ float gacc[NG][D + 1];

  const int bh = blockIdx.x, b = bh / H, h = bh - b * H;
  const int tid = threadIdx.x;
  const int d = H * D;
  const int pos = *pos_dev;
  const size_t head_base = ((size_t)b * H + h) * S_max * D;
  const int grp = tid / LPK, j = tid - grp * LPK;
  const T* kb = kc + head_base + j * 8;
  const T* vb = vc + head_base + j * 8;
  const int nkeys = QIN ? pos + 1 : pos;   // keys streamed from the cache

  // Keys in blocks of U keys per group, double buffered: block b+1 is in flight
  // while block b is consumed.  Loads are unconditional (keys past the last are
  // clamped to it and not consumed) so every path keeps the same loads in flight.
  constexpr int U = 1;
  const int nblk = (nkeys + U * NG - 1) / (U * NG);
  Raw8<T> kr[2][U], vr[2][U];
  auto load_blk = [&](int blk, Raw8<T> (&kk)[U], Raw8<T> (&vv)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = min(grp + NG * (blk * U + u), nkeys - 1);
      kk[u].load(kb + (size_t)key * D);
      vv[u].load(vb + (size_t)key * D);
    }
  };
  if (QIN) {     // the cache stream starts before q is fetched
    load_blk(0, kr[0], vr[0]);
    for (int i = tid; i < D; i += 256) qs[i] = ld(qin + (size_t)b * d + h * D + i);
  }

  // 1. finish q, k, v of this step and append k, v at `pos`
  for (int i = tid; i < D && !QIN; i += 256) {
    const int c = h * D + i;
    float q = 0.f, k = 0.f, v = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += 8) {     // 8 splits' loads in flight, summed in order
      float tq[8], tk[8], tv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float* pr = parts + ((size_t)min(s0 + u, nsplit - 1) * B + b) * 3 * d;
        tq[u] = pr[c];
        tk[u] = pr[d + c];
        tv[u] = pr[2 * d + c];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (s0 + u < nsplit) { q += tq[u]; k += tk[u]; v += tv[u]; }
    }
    q = (q + ld(bqkv + c)) * q_scale;
    k += ld(bqkv + d + c);
    v += ld(bqkv + 2 * d + c);
    const T qt = to_store<T>(q), kt = to_store<T>(k), vt = to_store<T>(v);
    kc[head_base + (size_t)pos * D + i] = kt;
    vc[head_base + (size_t)pos * D + i] = vt;
    qs[i] = ld(&qt);
    kn[i] = ld(&kt);
    vn[i] = ld(&vt);
  }
  __syncthreads();

  // 2. stream keys from the cache (without QIN the new key, pos, comes from LDS)
  float qv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qv[e] = qs[j * 8 + e];
  float m_run = -INFINITY, l_run = 0.f, acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};

  auto consume = [&](float s, const float* vv) {
    const float mn = fmaxf(m_run, s);
    const float c = __expf(m_run - mn), p = __expf(s - mn);
    l_run = l_run * c + p;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] * c + p * vv[e];
    m_run = mn;
  };
  auto dot = [&](const float* kv) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(qv[e], kv[e], s);
    return group_sum<LPK>(s);
  };

  auto use_blk = [&](int blk, const Raw8<T> (&kk)[U], const Raw8<T> (&vv)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = grp + NG * (blk * U + u);
      float kv[8], vx[8];
      kk[u].unpack(kv);
      vv[u].unpack(vx);
      const float sc = dot(kv);           // all lanes of the group take part
      if (key < nkeys) consume(sc, vx);
    }
  };
  if (nkeys > 0) {
    if (!QIN) load_blk(0, kr[0], vr[0]);
    for (int b = 0; b < nblk; b += 2) {
      load_blk(b + 1, kr[1], vr[1]);
      __builtin_amdgcn_sched_barrier(0);   // issue the next block before using this one
      use_blk(b, kr[0], vr[0]);
      load_blk(b + 2, kr[0], vr[0]);
      __builtin_amdgcn_sched_barrier(0);
      if (b + 1 < nblk) use_blk(b + 1, kr[1], vr[1]);
    }
  }
  if (!QIN && grp == pos % NG) {
    float kv[8], vv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { kv[e] = kn[j * 8 + e]; vv[e] = vn[j * 8 + e]; }
    consume(dot(kv), vv);
  }

  // 3. merge the groups in a fixed order
  if (j == 0) { gm[grp] = m_run; gl[grp] = l_run; }
#pragma unroll
  for (int e = 0; e < 8; ++e) gacc[grp][j * 8 + e] = acc[e];
  __syncthreads();
  for (int i = tid; i < D; i += 256) {
    float M = -INFINITY;
    for (int g = 0; g < NG; ++g) M = fmaxf(M, gm[g]);
    float L = 0.f, O = 0.f;
    for (int g = 0; g < NG; ++g) {
      const float w = gm[g] == -INFINITY ? 0.f : __expf(gm[g] - M);
      L += w * gl[g];
      O += w * gacc[g][i];
    }
    st(o + (x_mt ? xt_off(b, h * D + i, x_mt) : (size_t)b * d + h * D + i), O / L);
  }
}

void launch_attn_decode(int dt, const float* qkv_parts, int splits, const void* b_qkv,
                        void* k_cache, void* v_cache, const int32_t* pos_dev, void* o, int B,
                        int H, int D, int S_max, float q_scale, int x_mt, hipStream_t st) {
#define HE_DEC(T, DD)                                                                         \
  attn_decode_kernel<T, DD, false><<<B * H, 256, 0, st>>>(qkv_parts, splits, (const T*)b_qkv,  \
                                                          nullptr, (T*)k_cache, (T*)v_cache,    \
                                                          pos_dev, (T*)o, B, H, S_max, q_scale, \
                                                          XMT)
  if (dt == DT_BF16) {
    const int XMT = x_mt;
    switch (D) {
      case 16: HE_DEC(bf16, 16); break;
      case 32: HE_DEC(bf16, 32); break;
      case 64: HE_DEC(bf16, 64); break;
      default: HE_DEC(bf16, 128); break;
    }
  } else {
    const int XMT = 0;
    switch (D) {
      case 16: HE_DEC(float, 16); break;
      case 32: HE_DEC(float, 32); break;
      case 64: HE_DEC(float, 64); break;
      default: HE_DEC(float, 128); break;
    }
  }
#undef HE_DEC
}

void launch_attn_decode_q(int dt, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* pos_dev, void* o, int B, int H, int D, int S_max,
                          int x_mt, hipStream_t st) {
#define HE_DECQ(T, DD)                                                                                      \
  do {                                                                                                      \
    if (g_launch_timer.start) {                                                                            \
      hipExtLaunchKernelGGL(attn_decode_kernel<T, DD, true>, dim3(B * H), dim3(256), 0, st,               \
                            g_launch_timer.start, g_launch_timer.stop, 0, (const float*)nullptr, 0,       \
                            (const T*)nullptr, (const T*)q, (T*)k_cache, (T*)v_cache, pos_dev, (T*)o, B, \
                            H, S_max, 1.f, x_mt);                                                         \
      g_launch_timer = LaunchTimer{};                                                                       \
    } else {                                                                                                \
      attn_decode_kernel<T, DD, true><<<B * H, 256, 0, st>>>(nullptr, 0, nullptr, (const T*)q,            \
                                                             (T*)k_cache, (T*)v_cache, pos_dev, (T*)o,   \
                                                             B, H, S_max, 1.f, x_mt);                     \
    }                                                                                                       \
  } while (0)
  if (dt == DT_BF16) {
    switch (D) {
      case 16: HE_DECQ(bf16, 16); break;
      case 32: HE_DECQ(bf16, 32); break;
      case 64: HE_DECQ(bf16, 64); break;
      default: HE_DECQ(bf16, 128); break;
    }
  } else {
    switch (D) {
      case 16: HE_DECQ(float, 16); break;
      case 32: HE_DECQ(float, 32); break;
      case 64: HE_DECQ(float, 64); break;
      default: HE_DECQ(float, 128); break;
    }
  }
#undef HE_DECQ
}

// ---------------------------------------------------------------------------------
// prompt pass, bf16, MFMA
// ---------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_prefill_bf16_kernel(const bf16* __restrict__ q,
                                                                const bf16* __restrict__ kc,
                                                                const bf16* __restrict__ vc,
                                                                bf16* __restrict__ o, int B,
                                                                int S, int H, int S_max, int o_il) {
  constexpr int KT = 64;                 // keys per tile
  constexpr int LDKS = D + 8;            // K tile row stride (bf16)
  constexpr int LDV = KT + 8;            // transposed V row stride
  constexpr int LDP = KT + 8;
  __shared__ __attribute__((aligned(16))) bf16 Ks[KT * LDKS];
  __shared__ __attribute__((aligned(16))) bf16 Vt[D * LDV];
  __shared__ __attribute__((aligned(16))) bf16 Ps[4][16 * LDP];     // P rounded to bf16
  __shared__ __attribute__((aligned(16))) bf16 Pl[4][16 * LDP];     // P - round(P), rounded

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int q0 = blockIdx.x * 64;
  const int bh = blockIdx.y, b = bh / H, h = bh - b * H;
  const int d = H * D;
  const size_t head_base = ((size_t)b * H + h) * S_max * D;
  const int fr = lane & 15, fg = lane >> 4;

  // Q fragments of this wave's 16 queries (A operand): D/32 k-steps
  const int qrow = q0 + wv * 16 + fr;
  bf16x8 qa[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    if (qrow < S)
      qa[c] = *reinterpret_cast<const bf16x8*>(q + ((size_t)b * S + qrow) * d + h * D + c * 32 + fg * 8);
    else
      qa[c] = bf16x8{};
  }
  f32x4 oacc[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_r[4], l_r[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) { m_r[r] = -INFINITY; l_r[r] = 0.f; }

  const int kend = min(q0 + 64, S);
  for (int key0 = 0; key0 < kend; key0 += KT) {
    __syncthreads();
    // stage K (row-major) and V (transposed) of keys key0..key0+63
    for (int c = tid; c < KT * (D / 8); c += 256) {
      const int kk = c / (D / 8), dc = (c - kk * (D / 8)) * 8;
      const int key = key0 + kk;
      uint4 kv4 = make_uint4(0, 0, 0, 0), vv4 = make_uint4(0, 0, 0, 0);
      if (key < S) {
        kv4 = *reinterpret_cast<const uint4*>(kc + head_base + (size_t)key * D + dc);
        vv4 = *reinterpret_cast<const uint4*>(vc + head_base + (size_t)key * D + dc);
      }
      *reinterpret_cast<uint4*>(&Ks[kk * LDKS + dc]) = kv4;
      const bf16* vp = reinterpret_cast<const bf16*>(&vv4);
#pragma unroll
      for (int e = 0; e < 8; ++e) Vt[(dc + e) * LDV + kk] = vp[e];
    }
    __syncthreads();

    // scores: 16 queries x 64 keys = 4 MFMA column tiles
    f32x4 s[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      s[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const bf16x8 kb = *reinterpret_cast<const bf16x8*>(&Ks[(nt * 16 + fr) * LDKS + c * 32 + fg * 8]);
        s[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[c], kb, s[nt], 0, 0, 0);
      }
    }
    // s[nt][r] = score(query q0 + 16*wv + 4*fg + r, key key0 + 16*nt + fr)
    float mx[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int qi = q0 + wv * 16 + fg * 4 + r;
      float m = -INFINITY;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int key = key0 + nt * 16 + fr;
        if (key > qi || key >= S) s[nt][r] = -INFINITY;
        m = fmaxf(m, s[nt][r]);
      }
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
      mx[r] = m;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float mn = fmaxf(m_r[r], mx[r]);
      const float c = (m_r[r] == -INFINITY) ? 0.f : __expf(m_r[r] - mn);
      float sum = 0.f;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const float p = (s[nt][r] == -INFINITY) ? 0.f : __expf(s[nt][r] - mn);
        sum += p;
        const bf16 ph = f2bf(p);
        Ps[wv][(fg * 4 + r) * LDP + nt * 16 + fr] = ph;
        Pl[wv][(fg * 4 + r) * LDP + nt * 16 + fr] = f2bf(p - bf2f(ph));
      }
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
      l_r[r] = l_r[r] * c + sum;
      m_r[r] = mn;
#pragma unroll
      for (int t = 0; t < D / 16; ++t) oacc[t][r] *= c;
    }
    __syncthreads();   // P visible to the wave's lanes
    // O += P V over two 32-key steps
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 pa = *reinterpret_cast<const bf16x8*>(&Ps[wv][fr * LDP + ks * 32 + fg * 8]);
      const bf16x8 pl = *reinterpret_cast<const bf16x8*>(&Pl[wv][fr * LDP + ks * 32 + fg * 8]);
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const bf16x8 vb = *reinterpret_cast<const bf16x8*>(&Vt[(t * 16 + fr) * LDV + ks * 32 + fg * 8]);
        oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, oacc[t], 0, 0, 0);
        oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vb, oacc[t], 0, 0, 0);
      }
    }
  }
  // oacc[t][r] = O(query q0 + 16*wv + 4*fg + r, dim 16*t + fr)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int qi = q0 + wv * 16 + fg * 4 + r;
    if (qi >= S) continue;
    const float inv = 1.f / l_r[r];
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
      o[il_off(b * S + qi, h * D + t * 16 + fr, d, o_il)] = f2bf(oacc[t][r] * inv);
  }
}

// Prompt-pass attention with the keys and values of a head in LDS (below).
typedef short bf16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ short bf_bits(bf16 v) { return (short)v; }
// v combined with the v of lane l ^ 16 (row swap) or l ^ 32 (half swap), gfx950: the
// swap returns each lane's own value and its partner's, and max and + are commutative,
// so both lanes of a pair get the same result.
__device__ __forceinline__ float max16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
constexpr int kPfKV = 32768;           // bf16 elements of each of K and V^T in LDS
// Key window held in LDS at once for head size D and KV elements of each array.
constexpr int pf_window(int D, int KV = kPfKV) { return KV / D; }
// Keys padded for the LDS layout when the head fits in one window (a multiple of 128,
// at least 128); the full window when it takes two; 0 when it does not fit in two.
static int pf_pad(int S, int D, int KV = kPfKV) {
  const int sp = S <= 128 ? 128 : (S + 127) / 128 * 128;
  if (sp * D <= KV) return sp;
  return S <= 2 * pf_window(D, KV) ? pf_window(D, KV) : 0;
}

// Stage keys kw0 .. kw0 + Wp - 1 of one head (zeros past S) into the LDS arrays:
// K row-major, key-local row `key`, chunk c at chunk c ^ ((key / RPB) mod NCH) of the
// row; V transposed, row `dim` of Wp key positions, position chunk j at chunk
// j ^ (dim mod 16), each thread transposing an 8 keys x 8 dims block in registers.  In
// each 32-key block, position chunk g (g = 0..3) holds keys 4 g .. 4 g + 3 and
// 16 + 4 g .. 16 + 4 g + 3: the keys whose scores lane group g holds after S^T (two
// 16-key tiles), so P^T of 32 keys is one 16 x 16 x 32 MFMA operand.
// Every load of a thread (at most KV / 4096 K chunks and one 8 x 8 V block, Wp D <= KV)
// is issued before the first LDS write, so staging costs one memory round trip.
template <int D, int KV>
__device__ __forceinline__ void pf_stage(const bf16* __restrict__ kc, const bf16* __restrict__ vc,
                                         size_t head, int S, int kw0, int Wp, bf16* Ks, bf16* Vt, int tid) {
  constexpr int NCH = D / 8, RPB = 128 / D, NK = (KV / 8 + 511) / 512;
  static_assert(NK + 8 <= 32, "the validity bits of a thread's loads fit one word");
  // loads without branches: a slot past the keys reads the head's first row (always
  // present) and is zeroed where it is written, so the loads issue back to back
  uint4 kv[NK];
  uint32_t okm = 0;                                    // bit j: K chunk j, bit NK + r: V row r
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    const int i = tid + j * 512, key = i / NCH, c = i - key * NCH;
    const bool ok = i < Wp * NCH && kw0 + key < S;
    kv[j] = ld_once(kc + head + (ok ? (size_t)(kw0 + key) * D + c * 8 : 0));
    okm |= (uint32_t)ok << j;
  }
  const int kb = tid / NCH, cv = tid - kb * NCH;       // this thread's 8 keys x 8 dims of V
  const bool vblk = tid < (Wp / 8) * NCH;              // (Wp / 8) NCH <= KV / 64 <= 512
  uint4 vv[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int key = kw0 + (kb >> 2) * 32 + (kb & 3) * 4 + (r & 3) + (r >> 2) * 16;
    const bool ok = vblk && key < S;
    vv[r] = ld_once(vc + head + (ok ? (size_t)key * D + cv * 8 : 0));
    okm |= (uint32_t)ok << (NK + r);
  }
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    const int i = tid + j * 512, key = i / NCH, c = i - key * NCH;
    if (i < Wp * NCH)
      *reinterpret_cast<uint4*>(&Ks[key * D + ((c ^ ((key / RPB) & (NCH - 1))) << 3)]) =
          (okm >> j) & 1 ? kv[j] : make_uint4(0, 0, 0, 0);
  }
  if (vblk) {
    uint32_t e[8][4];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const bool ok = (okm >> (NK + r)) & 1;
      e[r][0] = ok ? vv[r].x : 0u; e[r][1] = ok ? vv[r].y : 0u;
      e[r][2] = ok ? vv[r].z : 0u; e[r][3] = ok ? vv[r].w : 0u;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sh = (j & 1) * 16, wd = j >> 1;
      uint32_t w4[4];
#pragma unroll
      for (int pr = 0; pr < 4; ++pr)
        w4[pr] = ((e[2 * pr][wd] >> sh) & 0xffffu) | (((e[2 * pr + 1][wd] >> sh) & 0xffffu) << 16);
      const int dim = cv * 8 + j;
      *reinterpret_cast<uint4*>(&Vt[dim * Wp + ((kb ^ (dim & 15)) << 3)]) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
  }
}

// Running state of one 16-query block in one wave: O^T accumulators, oacc[t][r] =
// O(query qi, dim 16 t + 4 fg + r) unnormalised, the running max and this lane's
// share of the sum.
template <int D>
struct PfBlock {
  f32x4 oacc[D / 16];
  float m, lsum;
};

template <int D>
__device__ __forceinline__ void pf_init(PfBlock<D>& s) {
#pragma unroll
  for (int t = 0; t < D / 16; ++t) s.oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  s.m = -INFINITY;
  s.lsum = 0.f;
}

// Q^T as the B operand: lane holds query qi, dims 32 c + 8 fg .. + 8.
template <int D>
__device__ __forceinline__ void pf_load_q(const bf16* __restrict__ q, int b, int S, int d, int h, int qi,
                                          int fg, bf16x8 (&qb8)[D / 32]) {
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
    qb8[c] = qi < S ? *reinterpret_cast<const bf16x8*>(q + ((size_t)b * S + qi) * d + h * D + c * 32 + fg * 8)
                    : bf16x8{};
}

// S^T for keys k0 .. k0 + 31 (window-local k0 - kw0): st[t2][r] = score(key k0 + 16 t2 +
// 4 fg + r, query qi).  The K fragments are read before the first MFMA.
template <int D>
__device__ __forceinline__ void pf_scores(f32x4 (&st)[2], const bf16x8 (&qb8)[D / 32], const bf16* Ks,
                                          int kl0, int fr, int fg) {
  constexpr int NCH = D / 8, RPB = 128 / D;
  bf16x8 kf[2][D / 32];
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2) {
    const int key = kl0 + t2 * 16 + fr;            // A-operand row of this lane
    const int sw = (key / RPB) & (NCH - 1);
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
      kf[t2][c] = *reinterpret_cast<const bf16x8*>(&Ks[key * D + (((c * 4 + fg) ^ sw) << 3)]);
  }
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2) {
    st[t2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 32; ++c) st[t2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[t2][c], qb8[c], st[t2], 0, 0, 0);
  }
}

// Keys k_begin .. k_end - 1 (k_begin a multiple of 32, inside the window staged at
// kw0 with Wp padded keys) for this lane's query qi.
template <int D>
__device__ __forceinline__ void pf_keys(PfBlock<D>& s, const bf16x8 (&qb8)[D / 32], const bf16* Ks,
                                        const bf16* Vt, int kw0, int Wp, int k_begin, int k_end, int qi,
                                        int S, int fr, int fg) {
  for (int k0 = k_begin; k0 < k_end; k0 += 32) {
    f32x4 st[2];
    pf_scores<D>(st, qb8, Ks, k0 - kw0, fr, fg);
    float cm = -INFINITY;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + t2 * 16 + fg * 4 + r;
        if (key > qi || key >= S) st[t2][r] = -INFINITY;
        cm = fmaxf(cm, st[t2][r]);
      }
    cm = max32(max16(cm));
    const float mn = fmaxf(s.m, cm);
    const float sc = s.m == -INFINITY ? 0.f : __expf(s.m - mn);
    s.m = mn;
    s.lsum *= sc;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) s.oacc[t] *= sc;
    // P^T of the 32 keys as the B operand of one 16 x 16 x 32 MFMA: this lane's eight
    // keys are 4 fg .. 4 fg + 3 (tile 0) and 16 + 4 fg .. + 3 (tile 1), position chunk fg
    // of the block in V^T
    bf16x8 ph, pl;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = st[t2][r] == -INFINITY ? 0.f : __expf(st[t2][r] - mn);
        s.lsum += p;
        const bf16 hi = f2bf(p);
        ph[t2 * 4 + r] = __builtin_bit_cast(__bf16, hi);
        pl[t2 * 4 + r] = __builtin_bit_cast(__bf16, f2bf(p - bf2f(hi)));
      }
    const int chunk = ((k0 - kw0) >> 3) + fg;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const int dim = t * 16 + fr;
      const bf16x8 va = *reinterpret_cast<const bf16x8*>(&Vt[dim * Wp + ((chunk ^ (dim & 15)) << 3)]);
      s.oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, ph, s.oacc[t], 0, 0, 0);
      s.oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pl, s.oacc[t], 0, 0, 0);
    }
  }
}

// Normalise and store this lane's query (8-byte stores in the output layout).
template <int D>
__device__ __forceinline__ void pf_store(PfBlock<D>& s, bf16* __restrict__ o, int b, int S, int d, int h,
                                         int qi, int fg, int o_il) {
  // the query's sum: the four lane groups' shares (the same value in every lane)
  const float lsum = sum32(sum16(s.lsum));
  if (qi >= S) return;
  const float inv = 1.f / lsum;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    const int dim = t * 16 + fg * 4;
    uint2 u;
    u.x = (uint32_t)f2bf(s.oacc[t][0] * inv) | ((uint32_t)f2bf(s.oacc[t][1] * inv) << 16);
    u.y = (uint32_t)f2bf(s.oacc[t][2] * inv) | ((uint32_t)f2bf(s.oacc[t][3] * inv) << 16);
    *reinterpret_cast<uint2*>(o + il_off(b * S + qi, h * D + dim, d, o_il)) = u;
  }
}

// Prompt pass, bf16, K and V of one (sequence, head) in LDS.  One WG of 8 waves per
// (sequence, head).  The head's keys go to LDS row-major and its values transposed
// (64 KB each at most); then every wave works through 16-query blocks with no
// further block barrier, taking blocks w and 15 - w of each 16 so the causal work is
// even.  Scores are formed transposed, S^T = K Q^T, so each lane holds four
// consecutive keys of one query: exactly the B operand of the 16 x 16 x 16 MFMA, which
// then computes O^T = V^T P^T straight from registers.  Online softmax per 32 keys
// (running max, per-lane partial sums merged at the end); P enters the product as
// bf16 high and low parts (p = hi + lo to ~16 bits).  Both LDS arrays are XOR-swizzled
// by 16-byte chunk so the 16 lanes that read 16 keys (or 16 value rows) at one offset
// hit distinct banks.
// A head longer than one window W = 32768 / D keys (S up to 2 W) is staged in two
// windows: blocks whose queries lie in the first window finish there; the blocks of
// the second window (W / 128 per wave) run over the first window's keys, keep their
// state in registers across the restaging barrier, and finish over the second's.
template <int D, int KV = kPfKV>
__global__ __launch_bounds__(512, KV < kPfKV ? 4 : 2) void attn_prefill_lds_kernel(const bf16* __restrict__ q,
                                                               const bf16* __restrict__ kc,
                                                               const bf16* __restrict__ vc,
                                                               bf16* __restrict__ o, int S, int S_pad,
                                                               int H, int S_max, int o_il) {
  constexpr int W = pf_window(D, KV), ND = W / 128;   // window; second-window blocks per wave
  __shared__ __attribute__((aligned(16))) bf16 Ks[KV];
  __shared__ __attribute__((aligned(16))) bf16 Vt[KV];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = blockIdx.x, b = bh / H, h = bh - b * H, d = H * D;
  const size_t head = ((size_t)b * H + h) * S_max * D;
  const int fr = lane & 15, fg = lane >> 4;
  const bool two = S > W;                       // then S_pad == W
  const int nqb = (S + 15) / 16;
  const int nqb0 = two ? W / 16 : nqb;          // blocks that finish in the first window

  pf_stage<D, KV>(kc, vc, head, S, 0, S_pad, Ks, Vt, tid);
  __syncthreads();

  for (int base = 0; base < nqb0; base += 16) {
    for (int half = 0; half < 2; ++half) {
      const int qb = base + (half ? 15 - wv : wv);
      if (qb >= nqb0) continue;
      const int q0 = qb * 16, qi = q0 + fr;          // this lane's query (all 4 lane groups)
      const int k_end = (min(q0 + 16, S) + 15) / 16 * 16;
      bf16x8 qb8[D / 32];
      pf_load_q<D>(q, b, S, d, h, qi, fg, qb8);
      PfBlock<D> s;
      pf_init(s);
      pf_keys<D>(s, qb8, Ks, Vt, 0, S_pad, 0, k_end, qi, S, fr, fg);
      pf_store<D>(s, o, b, S, d, h, qi, fg, o_il);
    }
  }
  if (!two) return;

  // second-window blocks nqb0 + i, i = 16 j2 + wv and 16 j2 + 15 - wv
  PfBlock<D> def[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j) {
    const int i = 16 * (j >> 1) + ((j & 1) ? 15 - wv : wv);
    const int qi = (nqb0 + i) * 16 + fr;
    pf_init(def[j]);
    if (nqb0 + i < nqb) {
      bf16x8 qb8[D / 32];
      pf_load_q<D>(q, b, S, d, h, qi, fg, qb8);
      pf_keys<D>(def[j], qb8, Ks, Vt, 0, W, 0, W, qi, S, fr, fg);
    }
  }
  __syncthreads();                              // every wave done with the first window
  pf_stage<D, KV>(kc, vc, head, S, W, W, Ks, Vt, tid);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < ND; ++j) {
    const int i = 16 * (j >> 1) + ((j & 1) ? 15 - wv : wv);
    if (nqb0 + i >= nqb) continue;
    const int q0 = (nqb0 + i) * 16, qi = q0 + fr;
    const int k_end = (min(q0 + 16, S) + 15) / 16 * 16;
    bf16x8 qb8[D / 32];
    pf_load_q<D>(q, b, S, d, h, qi, fg, qb8);
    pf_keys<D>(def[j], qb8, Ks, Vt, W, W, W, k_end, qi, S, fr, fg);
    pf_store<D>(def[j], o, b, S, d, h, qi, fg, o_il);
  }
}

// fp32 models (tiny workload): one WG of 64 threads per (query, sequence, head).
__global__ __launch_bounds__(64) void attn_prefill_f32_kernel(const float* __restrict__ q,
                                                              const float* __restrict__ kc,
                                                              const float* __restrict__ vc,
                                                              float* __restrict__ o, int B, int S,
                                                              int H, int D, int S_max) {
  extern __shared__ float sm[];
  float* qs = sm;          // [D]
  float* sc = sm + D;      // [S]
  const int t = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh - b * H;
  const int d = H * D, tid = threadIdx.x;
  const size_t head_base = ((size_t)b * H + h) * S_max * D;
  for (int i = tid; i < D; i += 64) qs[i] = q[((size_t)b * S + t) * d + h * D + i];
  __syncthreads();
  float mx = -INFINITY;
  for (int key = tid; key <= t; key += 64) {
    float s = 0.f;
    for (int i = 0; i < D; ++i) s = fmaf(qs[i], kc[head_base + (size_t)key * D + i], s);
    sc[key] = s;
    mx = fmaxf(mx, s);
  }
  mx = wave_max(mx);
  float sum = 0.f;
  for (int key = tid; key <= t; key += 64) {
    const float p = __expf(sc[key] - mx);
    sc[key] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  __syncthreads();
  for (int i = tid; i < D; i += 64) {
    float acc = 0.f;
    for (int key = 0; key <= t; ++key) acc = fmaf(sc[key], vc[head_base + (size_t)key * D + i], acc);
    o[((size_t)b * S + t) * d + h * D + i] = acc / sum;
  }
}

void launch_attn_prefill(int dt, const void* q, const void* k_cache, const void* v_cache, void* o,
                         int B, int S, int H, int D, int S_max, int o_il, hipStream_t st) {
  if (dt == DT_BF16 && (D == 32 || D == 64 || D == 128) && pf_pad(S, D)) {
    // Heads whose keys fit in two windows of half the LDS take 64 KB per WG, so two WGs
    // share a CU and one stages its head while the other computes.  (At 128 dims that
    // costs register spills; one full window per WG, which needs none, measured slower
    // in the prompt pass all the same: 175.0 against 157.8 us per layer at S 256.)
    const bool half = pf_pad(S, D, kPfKV / 2) != 0;
    const int sp = half ? pf_pad(S, D, kPfKV / 2) : pf_pad(S, D);
#define HE_PF(DD, KV)                                                                                 \
  attn_prefill_lds_kernel<DD, KV><<<B * H, 512, 0, st>>>((const bf16*)q, (const bf16*)k_cache,        \
                                                         (const bf16*)v_cache, (bf16*)o, S, sp, H, S_max, o_il)
    if (D == 128) {
      if (half) HE_PF(128, kPfKV / 2); else HE_PF(128, kPfKV);
    } else if (D == 64) {
      if (half) HE_PF(64, kPfKV / 2); else HE_PF(64, kPfKV);
    } else {
      if (half) HE_PF(32, kPfKV / 2); else HE_PF(32, kPfKV);
    }
#undef HE_PF
  } else if (dt == DT_BF16) {
    dim3 grid((S + 63) / 64, B * H);
    if (D == 64)
      attn_prefill_bf16_kernel<64><<<grid, 256, 0, st>>>((const bf16*)q, (const bf16*)k_cache,
                                                         (const bf16*)v_cache, (bf16*)o, B, S, H, S_max, o_il);
    else if (D == 128)
      attn_prefill_bf16_kernel<128><<<grid, 256, 0, st>>>((const bf16*)q, (const bf16*)k_cache,
                                                          (const bf16*)v_cache, (bf16*)o, B, S, H, S_max, o_il);
    else
      attn_prefill_bf16_kernel<32><<<grid, 256, 0, st>>>((const bf16*)q, (const bf16*)k_cache,
                                                         (const bf16*)v_cache, (bf16*)o, B, S, H, S_max, o_il);
  } else {
    dim3 grid(S, B * H);
    size_t lds = (size_t)(D + S) * sizeof(float);
    attn_prefill_f32_kernel<<<grid, 64, lds, st>>>((const float*)q, (const float*)k_cache,
                                                   (const float*)v_cache, (float*)o, B, S, H, D, S_max);
  }
}

}  // namespace he
