// Host-side launchers of the libhe HIP kernels (internal interface).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace he {

enum DType { DT_F32 = 0, DT_BF16 = 1 };

// ---- LoRA fold ---------------------------------------------------------------
// W[N,K] <- round(W + sign * s * (B[N,r] A[r,K])), fixed-order fp32 accumulation.
void launch_lora(int dt, void* W, const void* A, const void* B, int N, int K, int r,
                 float s, float sign, hipStream_t st);

// ---- embeddings and LayerNorm ----------------------------------------------------
// h[m] = E[id(m)] + P[pos(m) + 2] (fp32); x[m] = LN(h[m]; g, b) in storage type.
//   ids:     token ids, one per row m (row-major [B, S] for prefill)
//   pos_dev: if non-null, every row sits at position *pos_dev (decode step);
//            otherwise row m sits at position m % seq_len (prompt pass)
//   g == nullptr: no LayerNorm, x[m] = round(h[m]) (post-LN models)
void launch_embed_norm(int dt, const int32_t* ids, const int32_t* pos_dev, int seq_len,
                       const void* E, const void* P, const void* g, const void* b, float eps,
                       float* h, void* x, int M, int d, int vocab, hipStream_t st);

// Word-embedding gather only: xe[m] = E[ids[m]] (width de), storage type.
void launch_embed_gather(int dt, const int32_t* ids, const void* E, void* xe, int M, int de,
                         int vocab, hipStream_t st);

// Residual update and LayerNorm of rows.
//   in row r of the output reads stream row r * row_stride + row_offset
//   if parts != null: h[row] += sum_{s < nsplit} parts[s][r][:] + bias  (fp32, fixed order)
//      (parts are [nsplit][M][d]; r indexes them)
//   post == 0: x[r] = round(LN(h[row]))             (pre-LN: h untouched by the norm)
//   post == 1: h[row] = LN(h[row]); x[r] = round(h[row])  (post-LN)
void launch_norm(int dt, float* h, const float* parts, int nsplit, const void* bias,
                 const void* g, const void* b, float eps, void* x, int M, int d,
                 int row_stride, int row_offset, int post, hipStream_t st);

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
  float* out_f32 = nullptr;       // [M, N]
};

// Y[M,N] = X[M,K] W[N,K]^T with the epilogue (prompt-pass shapes, M large).
void launch_gemm(int dt, const void* X, const void* W, int M, int N, int K, const EpiArgs& e,
                 hipStream_t st);

// ---- decode-shaped GEMM (M = batch <= 128) ---------------------------------------
enum GemvOut { GV_PARTIAL = 0, GV_RELU, GV_ARGMAX };

// Tile/split choice for one decode projection: fr 16-row MFMA fragments per wave
// (64 * fr rows per WG) and `splits` ways over K (partials; 1 when the epilogue
// needs the full sum).
struct GemvPlan {
  int fr = 2;
  int splits = 1;
};
GemvPlan gemv_plan(int M, int N, int K, bool allow_split);

struct GemvArgs {
  int out_mode = GV_PARTIAL;
  int fr = 2;                     // from gemv_plan (GV_ARGMAX always uses 2)
  int splits = 1;                 // split-K count (GV_PARTIAL only)
  float* parts = nullptr;         // GV_PARTIAL: [splits][M][N] fp32 (no bias)
  const void* bias = nullptr;     // GV_RELU
  void* out = nullptr;            // GV_RELU: [M, N] storage type
  float* logits = nullptr;        // GV_ARGMAX: optional [M, N] fp32
  float* best_val = nullptr;      // GV_ARGMAX: [M][n_blocks] per-block maxima
  int32_t* best_idx = nullptr;    // GV_ARGMAX: [M][n_blocks]
  int n_blocks = 0;               // GV_ARGMAX: gemv_argmax_blocks(dt, N)
  int32_t* bump = nullptr;        // GV_ARGMAX: if set, *bump += 1 once (the decode
                                  // position; this kernel never reads it)
};

// Number of column blocks the argmax epilogue produces for N columns.
int gemv_argmax_blocks(int dt, int N);
void launch_gemv(int dt, const void* X, const void* W, int M, int N, int K, const GemvArgs& g,
                 hipStream_t st);

// Reduce per-block argmax partials: pick[m] = lowest index among the maxima.
// Writes pick to ids_cur[m], tokens[m * tok_stride + *pos_dev] (if tokens; the
// LM-head launch has already advanced the position, so this is the slot of the
// token being picked) and d_next[m] (if non-null).
void launch_argmax_finalize(const float* best_val, const int32_t* best_idx, int n_blocks, int M,
                            int32_t* ids_cur, int32_t* tokens, int tok_stride,
                            const int32_t* pos_dev, int32_t* d_next, hipStream_t st);

// ---- attention ---------------------------------------------------------------------
// Causal attention of the prompt pass: q [B*S, d] (scaled), keys/values of
// positions 0..S-1 in the layer's cache; o [B*S, d] storage type.
void launch_attn_prefill(int dt, const void* q, const void* k_cache, const void* v_cache,
                         void* o, int B, int S, int H, int D, int S_max, hipStream_t st);

// One decode step.  qkv = sum of `splits` partials [splits][B][3d] + b_qkv: q is
// scaled and rounded, k and v are rounded and appended at position *pos_dev;
// attends over positions 0..*pos_dev; o [B, d] storage type.
void launch_attn_decode(int dt, const float* qkv_parts, int splits, const void* b_qkv,
                        void* k_cache, void* v_cache, const int32_t* pos_dev, void* o,
                        int B, int H, int D, int S_max, float q_scale, hipStream_t st);

// *p = v (a one-thread kernel; safe next to captured work, unlike a memset node)
void launch_set_i32(int32_t* p, int32_t v, hipStream_t st);

// ---- reward head -------------------------------------------------------------------------
// reward[b] = sum_j (sum_k x[b*S + S-1][k] Pout[j][k]) * w[j]
void launch_score(int dt, const void* x, const void* proj_out, const void* w, float* reward,
                  int B, int S, int d, int de, hipStream_t st);

}  // namespace he
