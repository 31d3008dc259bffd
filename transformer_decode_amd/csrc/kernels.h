// Host-side launchers of the libhe HIP kernels (internal interface).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace he {

enum DType { DT_F32 = 0, DT_BF16 = 1 };

// Kernel timing for the runtime's per-class timers: when `start` is set, the next
// launch of a decode GEMM or decode attention kernel is issued with
// hipExtLaunchKernel and these events, which take their timestamps as part of that
// dispatch (no separate event packets around it), and the pair is cleared.
struct LaunchTimer {
  hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local LaunchTimer g_launch_timer;

// ---- weight layout -------------------------------------------------------------
// Inference layout of a bf16 weight with K columns (common.h, il_off): block width
// 2^il_of(K) (the largest power of two <= 512 dividing K).
int il_of(int K);

// ---- LoRA fold ---------------------------------------------------------------
// W[N,K] <- round(W + sign * s * (B[N,r] A[r,K])), fixed-order fp32 accumulation.
// fp32: in place, row-major.  bf16 (N % 16 == 0): sign > 0 reads W row-major and
// writes the inference layout il, sign < 0 the reverse; r == 0 (A, B unused) only
// switches the layout.
void launch_lora(int dt, void* W, const void* A, const void* B, int N, int K, int r,
                 float s, float sign, int il, hipStream_t st);

// ---- embeddings and LayerNorm ----------------------------------------------------
// h[m] = E[id(m)] + P[pos(m) + 2] (fp32); x[m] = LN(h[m]; g, b) in storage type.
//   ids:     token ids, one per row m (row-major [B, S] for prefill)
//   pos_dev: if non-null, every row sits at position *pos_dev (decode step);
//            otherwise row m sits at position m % seq_len (prompt pass)
//   g == nullptr: no LayerNorm, x[m] = round(h[m]) (post-LN models)
//   e_il:    layout of E (0 row-major, else the inference layout)
//   x_lay:   layout of x (act_off): 0 row-major [M, d]; > 0 fragment-tiled with x_lay
//            row tiles (decode); < 0 the inference layout with il = -x_lay (prompt pass)
void launch_embed_norm(int dt, const int32_t* ids, const int32_t* pos_dev, int seq_len,
                       const void* E, const void* P, const void* g, const void* b, float eps,
                       float* h, void* x, int M, int d, int vocab, int e_il, int x_lay,
                       hipStream_t st);

// Word-embedding gather only: xe[m] = E[ids[m]] (width de), storage type.
void launch_embed_gather(int dt, const int32_t* ids, const void* E, void* xe, int M, int de,
                         int vocab, hipStream_t st);

// Residual update and LayerNorm of rows.
//   in row r of the output reads stream row r * row_stride + row_offset
//   if parts != null: h[row] += sum_{s < nsplit} parts[s][r][:] + bias  (fp32, fixed order)
//      (parts are [nsplit][M][d]; r indexes them)
//   post == 0: x[r] = round(LN(h[row]))             (pre-LN: h untouched by the norm)
//   post == 1: h[row] = LN(h[row]); x[r] = round(h[row])  (post-LN)
//   x_lay:   layout of x as for launch_embed_norm (act_off)
//   row_group: output rows come in groups of row_group consecutive stream rows: row r
//      reads stream row (r / row_group) * row_stride + row_offset + r % row_group
void launch_norm(int dt, float* h, const float* parts, int nsplit, const void* bias,
                 const void* g, const void* b, float eps, void* x, int M, int d,
                 int row_stride, int row_offset, int post, int x_lay, hipStream_t st,
                 int row_group = 1);

// ---- GEMM epilogues ------------------------------------------------------------
enum Epi { EPI_QKV = 0, EPI_RESID, EPI_RELU, EPI_POSADD, EPI_F32 };

struct EpiArgs {
  int mode = EPI_F32;
  const void* bias = nullptr;     // [N] storage type (nullable)
  // EPI_QKV: rows m = b * seq_len + t at position pos0 + t
  void* q_out = nullptr;          // [M, d] storage type, scaled by q_scale
  void* k_cache = nullptr;        // this layer's keys   [B_max][H][S_max][D]
  void* v_cache = nullptr;        // this layer's values [B_max][H][S_max][D]
  int d = 0, H = 0, D = 0, S_max = 0, seq_len = 1, pos0 = 0;
  float q_scale = 1.f;
  // EPI_RESID (h += acc + bias) / EPI_POSADD (h = acc + P[pos + 2]; out = round(h))
  float* h = nullptr;             // [M, N] fp32
  const void* pos_emb = nullptr;
  // EPI_RELU (out = round(relu(acc + bias))) / EPI_POSADD
  void* out = nullptr;            // [M, N] storage type
  // EPI_F32
  float* out_f32 = nullptr;       // [M, N], rows ldo apart (ldo 0: N)
  int ldo = 0;
  // layout of the bf16 weight W: 0 row-major, else the inference layout (il_off)
  int w_il = 0;
  // layout of the bf16 activations X (over K) and `out` (over N): 0 row-major, else the
  // inference layout with that il (il_off), whose 16 x 32 fragments are whole cache lines
  int x_il = 0;
  int o_il = 0;
};

// Y[M,N] = X[M,K] W[N,K]^T with the epilogue (prompt-pass shapes, M large).
void launch_gemm(int dt, const void* X, const void* W, int M, int N, int K, const EpiArgs& e,
                 hipStream_t st);

// ---- decode-shaped GEMM (M = batch <= 128) ---------------------------------------
enum GemvOut { GV_PARTIAL = 0, GV_RELU, GV_ARGMAX, GV_QKV };

// Work split of one decode projection.
//   bf16: X fragment-tiled with mt row tiles, W in the inference layout; each wave
//   owns fr 16-row fragments and a K range of kr (a multiple of 128); nwk waves per
//   WG take consecutive K ranges and are reduced in the WG; `splits` = K / (kr nwk)
//   partial groups remain.  fp32: `splits` ways over K.
struct GemvPlan {
  int mt = 0, fr = 0, nwk = 0, kr = 0;
  int splits = 1;
};
// Row tiles of 16 the decode activations use for batch M (a power of two).
int decode_mt(int M);
GemvPlan decode_plan(int dt, int M, int N, int K, bool allow_split, bool whole = false, bool f8 = false);

// Pick rule of the LM head.  inv_temp == 0: greedy (largest logit, lowest index on
// ties).  inv_temp > 0: the Gumbel-max sample of softmax(logit * inv_temp): largest
// logit * inv_temp + G, G from gumbel4 (common.h) with this seed, the batch row and
// the position of the token being generated.  Per (row, column block) the head also
// reports, when blk_max is set, the tempered logit (logit * max(inv_temp, 1 if 0)) of
// the block's pick, the block's largest tempered logit and the sum of
// exp(tempered logit - that maximum), from which the token's log-probability follows.
struct SampleArgs {
  float inv_temp = 0.f;
  uint64_t seed = 0;
  float* best_lg = nullptr;       // [M][n_blocks]
  float* blk_max = nullptr;       // [M][n_blocks]
  float* blk_sum = nullptr;       // [M][n_blocks]
};

struct GemvArgs {
  int out_mode = GV_PARTIAL;
  int w_il = 0;                   // bf16 W: 0 row-major, else the inference layout il_of(K)
  // non-null: W holds E4M3 codes in the f8_off layout and these are its per-row scales
  // (bf16 models, not GV_ARGMAX; the plan's K range a multiple of 256)
  const float* w_scale = nullptr;
  float* parts = nullptr;         // GV_PARTIAL: [splits][M][N] fp32 (no bias)
  const void* bias = nullptr;     // GV_RELU
  void* out = nullptr;            // GV_RELU: bf16 fragment-tiled (plan mt); fp32 [M, N]
  float* logits = nullptr;        // GV_ARGMAX: optional [M, N] fp32
  float* best_val = nullptr;      // GV_ARGMAX: [M][n_blocks] per-block maxima
  int32_t* best_idx = nullptr;    // GV_ARGMAX: [M][n_blocks]
  int n_blocks = 0;               // GV_ARGMAX: gemv_argmax_blocks(dt, plan, N)
  // GV_ARGMAX: the token being picked sits at position *pos_dev + 1 (pos_dev as for
  // GV_QKV, read only); that value is stored to *pos_next (for launch_argmax_finalize)
  int32_t* pos_next = nullptr;
  SampleArgs smp;
  // GV_QKV (bf16, plan.splits == 1): rows n of the packed [q; k; v] projection plus
  // bias; q scaled and rounded into q_out [M][d], k and v rounded and appended to
  // the layer's cache [B_max][H][S_max][D] at position *pos_dev
  void* q_out = nullptr;
  void* k_cache = nullptr;
  void* v_cache = nullptr;
  const int32_t* pos_dev = nullptr;
  int d = 0, H = 0, D = 0, S_max = 0;
  float q_scale = 1.f;
};

// Y = X W^T with the chosen output (GV_RELU, GV_ARGMAX and GV_QKV need plan.splits == 1
// for bf16; GV_QKV is bf16 only).
void launch_gemv(int dt, const void* X, const void* W, int M, int N, int K, const GemvPlan& p,
                 const GemvArgs& g, hipStream_t st);
// Column blocks of the argmax output for N columns under plan p (also the blocking
// of launch_reduce_argmax when p.splits > 1).
int gemv_argmax_blocks(int dt, const GemvPlan& p, int N);

// out[m][n] = round(relu(sum_s parts[s][m][n] + bias[n])) (bf16; N % 4 == 0),
// fragment-tiled with mt row tiles (mt > 0) or row-major.
void launch_reduce_relu(const float* parts, int S, const void* bias, void* out, int M, int N,
                        int mt, hipStream_t st);
// Sum S partial logits, optionally store them, and reduce each row's 128-column
// blocks to (pick value, lowest index) pairs under the rule `smp` for
// launch_argmax_finalize; the token sits at *pos_dev + 1, stored to *pos_next.
void launch_reduce_argmax(const float* parts, int S, int M, int N, float* logits, float* best_val,
                          int32_t* best_idx, int nb, const int32_t* pos_dev, int32_t* pos_next,
                          const SampleArgs& smp, hipStream_t st);

// Reduce per-block partials: pick[m] = lowest index among the block maxima.  p =
// *pos_next is the position of the token being picked.  Writes pick to ids_cur[m],
// tokens[m * tok_stride + p] (if tokens) and d_next[m] (if non-null); with logp (and
// smp's block sums), the pick's log-probability to logp[m * tok_stride + p]: the
// tempered logit minus the logsumexp of the row, blocks combined in a fixed order.
// tok_stride 0 writes tokens[m] and logp[m] instead.  Finally *pos_dev = p (the
// position the next step feeds; skipped when pos_dev is null).
void launch_argmax_finalize(const float* best_val, const int32_t* best_idx, const SampleArgs& smp,
                            int n_blocks, int M, int32_t* ids_cur, int32_t* tokens, float* logp,
                            int tok_stride, const int32_t* pos_next, int32_t* pos_dev, int32_t* d_next,
                            hipStream_t st);

// Teacher-forced log-probabilities from fp32 logits [rows][V] (row-major): chunk row
// r is scored row g = r0 + r, i.e. sequence b = g / n, answer token j = g % n, whose
// target is seq[b * S + S_p + j]; out[g] = logits[r][target] - logsumexp(logits[r]),
// the logsumexp merged over the threads' column slices in a fixed tree.  A target
// outside 0 .. V-1 gives NaN.
void launch_logprob_gather(const float* logits, int rows, int V, const int32_t* seq, int S, int S_p,
                           int n, int r0, float* out, hipStream_t st);

// Top-p pick of each of M rows of fp32 logits [M][V] (V <= topp_max_vocab()): the
// Gumbel-max rule of smp (inv_temp > 0) restricted to the row's nucleus under
// softmax(logit * inv_temp) with mass top_p (0 < top_p < 1), ties at its edge
// included.  Position protocol, outputs and log-probability (of the untruncated
// distribution) as launch_argmax_finalize.
int topp_max_vocab();
void launch_topp_finalize(const float* logits, int M, int V, const SampleArgs& smp, float top_p,
                          int32_t* ids_cur, int32_t* tokens, float* logp, int tok_stride,
                          const int32_t* pos_next, int32_t* pos_dev, hipStream_t st);

// ---- weight-only FP8 decode weights ---------------------------------------------
// Per-output-channel E4M3 codes of bf16 W [N][K] (layout w_il, N % 16 == 0,
// K % 64 == 0) into q (f8_off layout, N K bytes) and scale [N] (amax / 448).
void launch_quantize_fp8(const void* W, int N, int K, int w_il, uint8_t* q, float* scale, hipStream_t st);
// The codes of q back in row-major order [N][K].
void launch_fp8_rowmajor(const uint8_t* q, int N, int K, uint8_t* out, hipStream_t st);

// ---- attention ---------------------------------------------------------------------
// Causal attention of the prompt pass: q [B*S, d] (scaled), keys/values of
// positions 0..S-1 in the layer's cache; o [B*S, d] storage type, in the inference
// layout with o_il (bf16; 0 row-major).
void launch_attn_prefill(int dt, const void* q, const void* k_cache, const void* v_cache,
                         void* o, int B, int S, int H, int D, int S_max, int o_il, hipStream_t st);

// One decode step.  qkv = sum of `splits` partials [splits][B][3d] + b_qkv: q is
// scaled and rounded, k and v are rounded and appended at position *pos_dev;
// attends over positions 0..*pos_dev; o [B, d] storage type, fragment-tiled with
// x_mt row tiles when x_mt > 0.
void launch_attn_decode(int dt, const float* qkv_parts, int splits, const void* b_qkv,
                        void* k_cache, void* v_cache, const int32_t* pos_dev, void* o,
                        int B, int H, int D, int S_max, float q_scale, int x_mt, hipStream_t st);
// The same step when q is finished ([B, d] storage type, scaled) and this step's k
// and v are already in the cache at *pos_dev (GV_QKV): attends over 0..*pos_dev.
void launch_attn_decode_q(int dt, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* pos_dev, void* o, int B, int H, int D, int S_max,
                          int x_mt, hipStream_t st);

// ---- static scratch of the allocation-free entry point ---------------------------
// Capacity: rows x 128-column blocks of the pick rule's per-block partials.
constexpr int kStaticRows = 128, kStaticBlocks = 512;
struct StaticScratch {
  int32_t* pos = nullptr;         // [2] position pair (the LM head's pos_dev, pos_next roles)
  float* best_val = nullptr;      // [kStaticRows * kStaticBlocks] each
  int32_t* best_idx = nullptr;
  float* best_lg = nullptr;
  float* blk_max = nullptr;
  float* blk_sum = nullptr;
};
// The device address of the static scratch on `device` (taken once per device, with
// that device current, and kept until the process ends).
hipError_t static_scratch(int device, StaticScratch* out);
size_t static_scratch_bytes();

// *p = v (a one-thread kernel; safe next to captured work, unlike a memset node)
void launch_set_i32(int32_t* p, int32_t v, hipStream_t st);

// ---- reward head -------------------------------------------------------------------------
// y[b][j] = sum_k x[b*S + S-1][k] Pout[j][k] (the state itself without Pout);
// reward[b] = sum_j y[b][j] w[j]; y (nullable) receives [B][de] float32.
void launch_score(int dt, const void* x, const void* proj_out, const void* w, float* reward, float* y,
                  int B, int S, int d, int de, hipStream_t st);

}  // namespace he
