// libhe runtime: context, state machine, KV workspace, decode-graph cache and the
// C ABI declared in include/he.h.
//
// One context is one model instance (paper summary, "The DeepSpeed Hybrid Engine:
// Architecture and Mode Switching": the engine keeps a single copy of the actor and
// reconfigures it at the eval()/train() boundary).  Inference mode here means: the
// LoRA adapters folded into the weights in place, bf16 weights switched in the same
// pass to the inference layout the decode kernels stream fastest (common.h, il_off),
// and a KV workspace allocated (page 2, section 3: fuse before generate, unfuse
// after; release the workspace after generation, re-take it before the next).
// Generation without a fold runs the base weights in their row-major layout.  The decode step can be replayed
// from a captured hipGraph (page 2, section 4: enable_cuda_graph), with the step's
// position kept in device memory so that one graph serves every step.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <utility>
#include <array>
#include <vector>

#include "../../include/he.h"
#include "kernels.h"

#ifndef HE_BUILD_FLAGS
#define HE_BUILD_FLAGS "unknown"
#endif

using namespace he;

namespace {

constexpr int kMaxDecodeBatch = 128;   // decode GEMM keeps <= 8 MFMA column tiles
constexpr size_t kLogitChunk = 4096;   // vocabulary rows the scoring pass holds at once

struct Timer {
  bool armed = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> live;   // recorded, not yet read
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pool;   // free
  std::vector<double> bytes, flops;
  he_kernel_stat acc{0, 0.0, 0.0, 0.0};
};

size_t esize(int dt) { return dt == DT_BF16 ? 2 : 4; }
int round_up(int x, int m) { return (x + m - 1) / m * m; }

}  // namespace

struct he_ctx {
  he_model_desc desc{};
  he_weight_table wt{};
  std::vector<he_layer_weights> layers;
  hipStream_t stream = nullptr;
  bool own_stream = false;
  int device = 0;                 // the GPU current at he_create
  int dt = DT_BF16, L = 0, d = 0, H = 0, D = 0, F = 0, V = 0, de = 0;
  float q_scale = 1.f;
  bool validate_only = false, use_graph = true;
  bool debug = false;             // HE_DEBUG=1: synchronise and check after every launch
  bool fused = false, failed = false;
  int il_d = 0;                   // inference layout of the K = d weights (bf16)
  std::string err;

  // workspace (library-owned)
  bool cache = false;
  int max_batch = 0, max_seq = 0, bpad = 0, rows = 0;
  void* kv = nullptr;
  size_t kv_layer_elems = 0;     // elements of one [B_max][H][S_max][D] block
  char* scratch = nullptr;
  float* h = nullptr;
  void* x = nullptr;
  void* xe = nullptr;
  void* q = nullptr;
  void* o = nullptr;
  void* a = nullptr;
  float* parts = nullptr;
  float* logits = nullptr;
  float* best_val = nullptr;
  int32_t* best_idx = nullptr;
  int32_t* ids_cur = nullptr;
  int32_t* tokens = nullptr;
  int32_t* pos_dev = nullptr;     // position of the token the next step feeds
  int32_t* pos_next = nullptr;    // position of the token being picked (LM head -> finalize)
  int32_t* spos = nullptr;        // [2] he_sample's own position pair (pos_dev, pos_next roles)
  float* logp = nullptr;          // [B_max][S_max + 1] log-probabilities of the picks
  float* best_lg = nullptr;       // per (row, LM-head column block): pick's tempered logit,
  float* blk_max = nullptr;       // the block's largest tempered logit and its sum of
  float* blk_sum = nullptr;       // exponentials
  int n_argmax_blocks = 0, argmax_cap = 0;
  float* lgc = nullptr;           // [lg_rows][V] fp32 logits of the scoring pass, one chunk
  int lg_rows = 0;
  // pick rule of the LM head: temperature 0 greedy, else Gumbel-max sampling; and
  // whether log-probabilities are formed
  float inv_temp = 0.f;
  uint64_t seed = 0;
  bool want_logp = false;
  float top_p = 1.f;              // nucleus mass; >= 1 off
  // decode GEMM plans and activation row tiles for the current batch (set by the
  // prompt pass)
  GemvPlan p_qkv, p_out, p_fc1, p_fc2, p_lm;
  int xmt = 0;

  // cache epoch
  bool prefilled = false;
  int cur_B = 0, cur_pos = 0;

  // decode graphs: [0] without logits, [1] with logits, for batch graph_B and the
  // weight layout (fused or not) they were captured with
  hipGraphExec_t graph[2] = {nullptr, nullptr};
  int graph_B = -1;
  bool graph_fused = false;
  float graph_itemp = 0.f;        // pick rule the graphs were captured with
  uint64_t graph_seed = 0;
  bool graph_logp = false;
  float graph_topp = 1.f;
  bool capturing = false;

  Timer timers[HE_K_COUNT];
  bool fail_next_alloc = false, fail_next_step = false;

  // weight-only FP8 decode: E4M3 copies (f8_off layout) and per-row scales of the four
  // projections of every layer, in one library-owned allocation kept across
  // workspace release / retake
  bool f8_on = false;
  bool graph_f8 = false;
  char* f8buf = nullptr;
  struct F8Layer { uint8_t* q[4]; float* s[4]; };
  std::vector<F8Layer> f8;
};

// ------------------------------------------------------------------------------------
// helpers
// ------------------------------------------------------------------------------------
static he_status set_err(he_ctx* c, he_status s, const char* fmt, ...) {
  if (c) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    c->err = buf;
  }
  return s;
}

static he_status hip_fail(he_ctx* c, hipError_t e, const char* what) {
  c->failed = true;
  return set_err(c, HE_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(c, call)                                   \
  do {                                                     \
    hipError_t e_ = (call);                                \
    if (e_ != hipSuccess) return hip_fail((c), e_, #call); \
  } while (0)

// After a batch of launches: surface launch errors (and a failure HE_DEBUG found).
static he_status check_launch(he_ctx* c, const char* what) {
  if (c->failed) return HE_E_HIP;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(c, e, what);
  return HE_OK;
}

// HE_DEBUG=1: after a launch, wait for the stream and check for an error, so that a
// fault is reported at the kernel that caused it ("<what>: <error>" in he_last_error).
// Nothing happens during graph capture (debug mode turns graph replay off) or after a
// first failure.
static void dbg_after(he_ctx* c, const char* what) {
  if (!c->debug || c->capturing || c->failed || c->validate_only) return;
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) hip_fail(c, e, what);
}

static const char* const kClassName[HE_K_COUNT] = {"LoRA fold", "embedding / LayerNorm", "prompt-pass GEMM",
                                                   "prompt-pass attention", "decode projection",
                                                   "decode attention", "LM head", "reward head",
                                                   "vocabulary GEMM"};

static void* kcache(he_ctx* c, int l) {
  return (char*)c->kv + (size_t)(2 * l) * c->kv_layer_elems * esize(c->dt);
}
static void* vcache(he_ctx* c, int l) {
  return (char*)c->kv + (size_t)(2 * l + 1) * c->kv_layer_elems * esize(c->dt);
}

// Run one launch, bracketed by events when its kernel class is armed.
template <class Fn>
static void run_k_timed(he_ctx* c, int kclass, double bytes, double flops, Fn&& fn);

// Run one launch of a kernel class (timed when the class is armed; checked right
// after under HE_DEBUG).
template <class Fn>
static void run_k(he_ctx* c, int kclass, double bytes, double flops, Fn&& fn) {
  run_k_timed(c, kclass, bytes, flops, fn);
  dbg_after(c, kClassName[kclass]);
}

template <class Fn>
static void run_k_timed(he_ctx* c, int kclass, double bytes, double flops, Fn&& fn) {
  Timer& t = c->timers[kclass];
  if (!t.armed || c->capturing) {
    fn();
    return;
  }
  std::pair<hipEvent_t, hipEvent_t> ev;
  if (!t.pool.empty()) {
    ev = t.pool.back();
    t.pool.pop_back();
  } else {
    if (hipEventCreate(&ev.first) != hipSuccess || hipEventCreate(&ev.second) != hipSuccess) {
      fn();
      return;
    }
  }
  if (kclass == HE_K_GEMV_DECODE || kclass == HE_K_ATTN_DECODE) {
    // a single kernel whose launch takes the timestamps itself
    g_launch_timer = LaunchTimer{ev.first, ev.second};
    fn();
    const bool consumed = g_launch_timer.start == nullptr;
    g_launch_timer = LaunchTimer{};
    if (!consumed) {   // launched some other way: no sample
      t.pool.push_back(ev);
      return;
    }
  } else {
    hipEventRecord(ev.first, c->stream);
    fn();
    hipEventRecord(ev.second, c->stream);
  }
  t.live.push_back(ev);
  t.bytes.push_back(bytes);
  t.flops.push_back(flops);
}

static bool any_timer_armed(const he_ctx* c) {
  for (const Timer& t : c->timers)
    if (t.armed) return true;
  return false;
}

static void set_plans(he_ctx* c, int B) {
  const bool f8 = c->f8_on;
  c->p_qkv = decode_plan(c->dt, B, 3 * c->d, c->d, true, c->dt == DT_BF16, f8);   // bf16: fused QKV epilogue
  c->p_out = decode_plan(c->dt, B, c->d, c->d, true, false, f8);
  c->p_fc1 = decode_plan(c->dt, B, c->F, c->d, true, false, f8);
  c->p_fc2 = decode_plan(c->dt, B, c->d, c->F, true, false, f8);
  c->p_lm = decode_plan(c->dt, B, c->V, c->d, true, true);
  c->xmt = c->dt == DT_BF16 ? decode_mt(B) : 0;
  c->n_argmax_blocks = gemv_argmax_blocks(c->dt, c->p_lm, c->V);
}

// Largest split-K partial buffer (floats) and argmax block count any batch size up
// to max_batch needs.
static size_t parts_elems(he_ctx* c, int max_batch, int* argmax_cap) {
  size_t need = 0;
  int nb = 0;
  auto room = [&](const GemvPlan& p, int B, int N) { return (size_t)p.splits * (size_t)B * (size_t)N; };
  for (int B = 1; B <= max_batch; ++B)
    for (bool f8 : {false, c->dt == DT_BF16}) {   // plans with and without E4M3 weights
      need = std::max(need, room(decode_plan(c->dt, B, 3 * c->d, c->d, true, c->dt == DT_BF16, f8), B, 3 * c->d));
      need = std::max(need, room(decode_plan(c->dt, B, c->d, c->d, true, false, f8), B, c->d));
      need = std::max(need, room(decode_plan(c->dt, B, c->F, c->d, true, false, f8), B, c->F));
      need = std::max(need, room(decode_plan(c->dt, B, c->d, c->F, true, false, f8), B, c->d));
    }
  for (int B = 1; B <= max_batch; ++B) {
    const GemvPlan lm = decode_plan(c->dt, B, c->V, c->d, true, true);
    need = std::max(need, room(lm, B, c->V));
    nb = std::max(nb, gemv_argmax_blocks(c->dt, lm, c->V));
  }
  *argmax_cap = nb;
  return need;
}

// Layout of a layer weight with K columns as the kernels must read it now.
static int w_il(const he_ctx* c, int K) { return (c->fused && c->dt == DT_BF16) ? il_of(K) : 0; }
// Prompt-pass activations that feed a GEMM ([rows][K], bf16) are held in the inference
// layout too: each 16 x 32 operand fragment is then 1 KB of whole cache lines.
static int a_il(const he_ctx* c, int K) { return c->dt == DT_BF16 ? il_of(K) : 0; }
static int e_il(const he_ctx* c) {
  return (c->fused && c->dt == DT_BF16 && c->desc.head == HE_HEAD_LM) ? c->il_d : 0;
}

static void drop_graphs(he_ctx* c) {
  for (auto& g : c->graph)
    if (g) {
      hipGraphExecDestroy(g);
      g = nullptr;
    }
  c->graph_B = -1;
}

// ------------------------------------------------------------------------------------
// enqueue sequences
// ------------------------------------------------------------------------------------
static const void* ln_g_after(he_ctx* c, int l) {   // norm applied before layer l+1's attention
  return (l + 1 < c->L) ? c->layers[l + 1].ln1_g : c->wt.lnf_g;
}
static const void* ln_b_after(he_ctx* c, int l) {
  return (l + 1 < c->L) ? c->layers[l + 1].ln1_b : c->wt.lnf_b;
}

// One decode projection into split-K partials (plan p).
static void decode_partials(he_ctx* c, const void* X, const void* W, int B, int N, int K,
                            const GemvPlan& p, int il, hipStream_t st, const float* w_scale = nullptr) {
  GemvArgs g;
  g.out_mode = GV_PARTIAL;
  g.w_il = il;
  g.w_scale = w_scale;
  g.parts = c->parts;
  launch_gemv(c->dt, X, W, B, N, K, p, g, st);
}

// Tied LM head over z (x rows 0..B-1) + the pick (greedy or sampled, with its
// log-probability when asked); advances the position counter.
static void enqueue_lm_head(he_ctx* c, int B, bool want_logits) {
  const int d = c->d, dt = c->dt;
  const bool nucleus = c->top_p < 1.f;
  want_logits = want_logits || nucleus;   // the nucleus needs the whole row
  const size_t es = esize(dt);
  hipStream_t st = c->stream;
  SampleArgs smp;
  smp.inv_temp = c->inv_temp;
  smp.seed = c->seed;
  if (c->want_logp) { smp.best_lg = c->best_lg; smp.blk_max = c->blk_max; smp.blk_sum = c->blk_sum; }
  if (c->p_lm.splits > 1) {
    run_k(c, HE_K_LMHEAD, (double)c->V * d * es, 2.0 * B * c->V * d, [&] {
      decode_partials(c, c->x, c->wt.tok_emb, B, c->V, d, c->p_lm, e_il(c), st);
      launch_reduce_argmax(c->parts, c->p_lm.splits, B, c->V, want_logits ? c->logits : nullptr,
                           c->best_val, c->best_idx, c->n_argmax_blocks, c->pos_dev, c->pos_next, smp, st);
    });
  } else {
    GemvArgs g;
    g.out_mode = GV_ARGMAX;
    g.w_il = e_il(c);
    g.logits = want_logits ? c->logits : nullptr;
    g.best_val = c->best_val;
    g.best_idx = c->best_idx;
    g.n_blocks = c->n_argmax_blocks;
    g.pos_dev = c->pos_dev;
    g.pos_next = c->pos_next;
    g.smp = smp;
    run_k(c, HE_K_LMHEAD, (double)c->V * d * es, 2.0 * B * c->V * d,
          [&] { launch_gemv(dt, c->x, c->wt.tok_emb, B, c->V, d, c->p_lm, g, st); });
  }
  if (nucleus)
    launch_topp_finalize(c->logits, B, c->V, smp, c->top_p, c->ids_cur, c->tokens, c->want_logp ? c->logp : nullptr,
                         c->max_seq + 1, c->pos_next, c->pos_dev, st);
  else
    launch_argmax_finalize(c->best_val, c->best_idx, smp, c->n_argmax_blocks, B, c->ids_cur, c->tokens,
                           c->want_logp ? c->logp : nullptr, c->max_seq + 1, c->pos_next, c->pos_dev, nullptr, st);
  dbg_after(c, nucleus ? "top-p pick" : "pick finalisation");
}

// Decoder layers of the prompt pass of a pre-LN LM-head model over ids [B, S]: leaves
// the residual stream in h and every position's K/V in the cache.
static void enqueue_prompt_layers(he_ctx* c, const int32_t* ids, int B, int S) {
  const int M = B * S, d = c->d, F = c->F, dt = c->dt;
  const float eps = c->desc.ln_eps;
  const size_t es = esize(dt);
  hipStream_t st = c->stream;
  const int ild = w_il(c, d), ilf = w_il(c, F), ald = a_il(c, d), alf = a_il(c, F);
  run_k(c, HE_K_EMBED_NORM, (double)M * d * (2 * es + 4 + es), 0, [&] {
    launch_embed_norm(dt, ids, nullptr, S, c->wt.tok_emb, c->wt.pos_emb,
                      c->L ? c->layers[0].ln1_g : c->wt.lnf_g, c->L ? c->layers[0].ln1_b : c->wt.lnf_b,
                      eps, c->h, c->x, M, d, c->V, e_il(c), c->L ? -ald : 0, st);
  });
  for (int l = 0; l < c->L; ++l) {
    const he_layer_weights& w = c->layers[l];
    EpiArgs e;
    e.w_il = ild; e.x_il = ald;
    e.mode = EPI_QKV;
    e.bias = w.b_qkv;
    e.q_out = c->q;
    e.k_cache = kcache(c, l);
    e.v_cache = vcache(c, l);
    e.d = d; e.H = c->H; e.D = c->D; e.S_max = c->max_seq; e.seq_len = S; e.pos0 = 0;
    e.q_scale = c->q_scale;
    run_k(c, HE_K_GEMM_PREFILL, (double)3 * d * d * es, 2.0 * M * 3 * d * d,
          [&] { launch_gemm(dt, c->x, w.w_qkv, M, 3 * d, d, e, st); });
    run_k(c, HE_K_ATTN_PREFILL, (double)M * d * es * 4, 2.0 * B * d * (double)S * (S + 1), [&] {
      launch_attn_prefill(dt, c->q, kcache(c, l), vcache(c, l), c->o, B, S, c->H, c->D, c->max_seq, ald, st);
    });
    EpiArgs r;
    r.mode = EPI_RESID; r.bias = w.b_out; r.h = c->h; r.w_il = ild; r.x_il = ald;
    run_k(c, HE_K_GEMM_PREFILL, (double)d * d * es, 2.0 * M * d * d,
          [&] { launch_gemm(dt, c->o, w.w_out, M, d, d, r, st); });
    run_k(c, HE_K_EMBED_NORM, (double)M * d * (4 + es), 0, [&] {
      launch_norm(dt, c->h, nullptr, 0, nullptr, w.ln2_g, w.ln2_b, eps, c->x, M, d, 1, 0, 0, -ald, st);
    });
    EpiArgs f1;
    f1.mode = EPI_RELU; f1.bias = w.b_fc1; f1.out = c->a; f1.w_il = ild; f1.x_il = ald; f1.o_il = alf;
    run_k(c, HE_K_GEMM_PREFILL, (double)F * d * es, 2.0 * M * F * d,
          [&] { launch_gemm(dt, c->x, w.w_fc1, M, F, d, f1, st); });
    EpiArgs f2;
    f2.mode = EPI_RESID; f2.bias = w.b_fc2; f2.h = c->h; f2.w_il = ilf; f2.x_il = alf;
    run_k(c, HE_K_GEMM_PREFILL, (double)F * d * es, 2.0 * M * F * d,
          [&] { launch_gemm(dt, c->a, w.w_fc2, M, d, F, f2, st); });
    if (l + 1 < c->L)
      run_k(c, HE_K_EMBED_NORM, (double)M * d * (4 + es), 0, [&] {
        launch_norm(dt, c->h, nullptr, 0, nullptr, c->layers[l + 1].ln1_g, c->layers[l + 1].ln1_b,
                    eps, c->x, M, d, 1, 0, 0, -ald, st);
      });
  }
}

// Prompt pass; leaves z (final LN of the last rows) in x and picks the first token.
static void enqueue_prefill_lm(he_ctx* c, const int32_t* ids, int B, int S, bool want_logits) {
  const int d = c->d, dt = c->dt;
  const float eps = c->desc.ln_eps;
  const size_t es = esize(dt);
  hipStream_t st = c->stream;
  enqueue_prompt_layers(c, ids, B, S);
  // final LayerNorm of the last prompt position only, laid out for the LM head
  run_k(c, HE_K_EMBED_NORM, (double)B * d * (4 + es), 0, [&] {
    launch_norm(dt, c->h, nullptr, 0, nullptr, c->wt.lnf_g, c->wt.lnf_b, eps, c->x, B, d, S, S - 1, 0,
                c->xmt, st);
  });
  enqueue_lm_head(c, B, want_logits);
}

// One decode step for batch B: feeds ids_cur at *pos_dev.  Host mirror `pos` is
// only used for the timers' byte counts.
static void enqueue_step(he_ctx* c, int B, bool want_logits, int pos) {
  const int d = c->d, F = c->F, dt = c->dt;
  const float eps = c->desc.ln_eps;
  const size_t es = esize(dt);
  hipStream_t st = c->stream;
  const int xmt = c->xmt;
  run_k(c, HE_K_EMBED_NORM, (double)B * d * (2 * es + 4 + es), 0, [&] {
    launch_embed_norm(dt, c->ids_cur, c->pos_dev, 1, c->wt.tok_emb, c->wt.pos_emb,
                      c->L ? c->layers[0].ln1_g : c->wt.lnf_g, c->L ? c->layers[0].ln1_b : c->wt.lnf_b,
                      eps, c->h, c->x, B, d, c->V, e_il(c), xmt, st);
  });
  for (int l = 0; l < c->L; ++l) {
    const he_layer_weights& w = c->layers[l];
    // the four projections' weights: bf16, or their E4M3 copies with per-row scales
    const bool f8 = c->f8_on;
    const void* Wq = f8 ? (const void*)c->f8[l].q[0] : w.w_qkv;
    const void* Wo = f8 ? (const void*)c->f8[l].q[1] : w.w_out;
    const void* W1 = f8 ? (const void*)c->f8[l].q[2] : w.w_fc1;
    const void* W2 = f8 ? (const void*)c->f8[l].q[3] : w.w_fc2;
    const float* Sq = f8 ? c->f8[l].s[0] : nullptr;
    const float* So = f8 ? c->f8[l].s[1] : nullptr;
    const float* S1 = f8 ? c->f8[l].s[2] : nullptr;
    const float* S2 = f8 ? c->f8[l].s[3] : nullptr;
    const double wb = f8 ? 1.0 : (double)es;   // weight bytes per element
    if (dt == DT_BF16) {   // q, k, v finished in the projection's epilogue
      GemvArgs g;
      g.out_mode = GV_QKV; g.w_il = w_il(c, d); g.bias = w.b_qkv; g.w_scale = Sq;
      g.q_out = c->q; g.k_cache = kcache(c, l); g.v_cache = vcache(c, l); g.pos_dev = c->pos_dev;
      g.d = d; g.H = c->H; g.D = c->D; g.S_max = c->max_seq; g.q_scale = c->q_scale;
      run_k(c, HE_K_GEMV_DECODE, (double)3 * d * d * wb, 2.0 * B * 3 * d * d,
            [&] { launch_gemv(dt, c->x, Wq, B, 3 * d, d, c->p_qkv, g, st); });
      run_k(c, HE_K_ATTN_DECODE, 2.0 * B * d * es * (double)(pos + 1), 4.0 * B * d * (double)(pos + 1), [&] {
        launch_attn_decode_q(dt, c->q, kcache(c, l), vcache(c, l), c->pos_dev, c->o, B, c->H, c->D,
                             c->max_seq, xmt, st);
      });
    } else {
      run_k(c, HE_K_GEMV_DECODE, (double)3 * d * d * es, 2.0 * B * 3 * d * d,
            [&] { decode_partials(c, c->x, w.w_qkv, B, 3 * d, d, c->p_qkv, w_il(c, d), st); });
      run_k(c, HE_K_ATTN_DECODE, 2.0 * B * d * es * (double)(pos + 1), 4.0 * B * d * (double)(pos + 1), [&] {
        launch_attn_decode(dt, c->parts, c->p_qkv.splits, w.b_qkv, kcache(c, l), vcache(c, l), c->pos_dev,
                           c->o, B, c->H, c->D, c->max_seq, c->q_scale, xmt, st);
      });
    }
    run_k(c, HE_K_GEMV_DECODE, (double)d * d * wb, 2.0 * B * d * d,
          [&] { decode_partials(c, c->o, Wo, B, d, d, c->p_out, w_il(c, d), st, So); });
    run_k(c, HE_K_EMBED_NORM, (double)B * d * 8, 0, [&] {
      launch_norm(dt, c->h, c->parts, c->p_out.splits, w.b_out, w.ln2_g, w.ln2_b, eps, c->x, B, d, 1, 0, 0,
                  xmt, st);
    });
    if (dt == DT_BF16 && c->p_fc1.splits > 1) {
      run_k(c, HE_K_GEMV_DECODE, (double)F * d * wb, 2.0 * B * F * d,
            [&] { decode_partials(c, c->x, W1, B, F, d, c->p_fc1, w_il(c, d), st, S1); });
      run_k(c, HE_K_EMBED_NORM, (double)B * F * 4 * c->p_fc1.splits, 0,
            [&] { launch_reduce_relu(c->parts, c->p_fc1.splits, w.b_fc1, c->a, B, F, xmt, st); });
    } else {
      GemvArgs g1;
      g1.out_mode = GV_RELU; g1.w_il = w_il(c, d); g1.bias = w.b_fc1; g1.out = c->a; g1.w_scale = S1;
      run_k(c, HE_K_GEMV_DECODE, (double)F * d * wb, 2.0 * B * F * d,
            [&] { launch_gemv(dt, c->x, W1, B, F, d, c->p_fc1, g1, st); });
    }
    run_k(c, HE_K_GEMV_DECODE, (double)F * d * wb, 2.0 * B * F * d,
          [&] { decode_partials(c, c->a, W2, B, d, F, c->p_fc2, w_il(c, F), st, S2); });
    run_k(c, HE_K_EMBED_NORM, (double)B * d * 8, 0, [&] {
      launch_norm(dt, c->h, c->parts, c->p_fc2.splits, w.b_fc2, ln_g_after(c, l), ln_b_after(c, l), eps,
                  c->x, B, d, 1, 0, 0, xmt, st);
    });
  }
  if (c->L == 0)
    run_k(c, HE_K_EMBED_NORM, (double)B * d * 8, 0, [&] {
      launch_norm(dt, c->h, nullptr, 0, nullptr, c->wt.lnf_g, c->wt.lnf_b, eps, c->x, B, d, 1, 0, 0, xmt, st);
    });
  enqueue_lm_head(c, B, want_logits);
}

// Full causal pass of a scalar-head model, reward at the last position.
static void enqueue_score(he_ctx* c, const int32_t* ids, int B, int S, float* reward, float* y) {
  const int M = B * S, d = c->d, F = c->F, dt = c->dt, de = c->de;
  const float eps = c->desc.ln_eps;
  const size_t es = esize(dt);
  const bool post = c->desc.norm == HE_NORM_POST;
  hipStream_t st = c->stream;
  // x feeds the first layer's QKV projection (inference layout), or with no layers the
  // head (row-major)
  const int ald = a_il(c, d), alf = a_il(c, F), x0 = c->L ? -ald : 0;
  if (de != d) {
    launch_embed_gather(dt, ids, c->wt.tok_emb, c->xe, M, de, c->V, st);
    dbg_after(c, "embedding gather");
    EpiArgs e;
    e.mode = EPI_POSADD; e.pos_emb = c->wt.pos_emb; e.h = c->h; e.out = c->x; e.seq_len = S; e.pos0 = 0;
    e.o_il = (post || !c->L) ? -x0 : 0;   // pre-LN: the norm below writes the GEMM input
    run_k(c, HE_K_GEMM_PREFILL, (double)d * de * es, 2.0 * M * d * de,
          [&] { launch_gemm(dt, c->xe, c->wt.proj_in, M, d, de, e, st); });
    if (!post && c->L)
      launch_norm(dt, c->h, nullptr, 0, nullptr, c->layers[0].ln1_g, c->layers[0].ln1_b, eps, c->x, M, d,
                  1, 0, 0, x0, st);
    dbg_after(c, "LayerNorm");
  } else {
    launch_embed_norm(dt, ids, nullptr, S, c->wt.tok_emb, c->wt.pos_emb,
                      (!post && c->L) ? c->layers[0].ln1_g : nullptr,
                      (!post && c->L) ? c->layers[0].ln1_b : nullptr, eps, c->h, c->x, M, d, c->V,
                      e_il(c), x0, st);
    dbg_after(c, "embedding / LayerNorm");
  }
  const int ild = w_il(c, d), ilf = w_il(c, F);
  for (int l = 0; l < c->L; ++l) {
    const he_layer_weights& w = c->layers[l];
    EpiArgs e;
    e.w_il = ild; e.x_il = ald;
    e.mode = EPI_QKV; e.bias = w.b_qkv; e.q_out = c->q; e.k_cache = kcache(c, l); e.v_cache = vcache(c, l);
    e.d = d; e.H = c->H; e.D = c->D; e.S_max = c->max_seq; e.seq_len = S; e.pos0 = 0; e.q_scale = c->q_scale;
    run_k(c, HE_K_GEMM_PREFILL, (double)3 * d * d * es, 2.0 * M * 3 * d * d,
          [&] { launch_gemm(dt, c->x, w.w_qkv, M, 3 * d, d, e, st); });
    run_k(c, HE_K_ATTN_PREFILL, (double)M * d * es * 4, 2.0 * B * d * (double)S * (S + 1), [&] {
      launch_attn_prefill(dt, c->q, kcache(c, l), vcache(c, l), c->o, B, S, c->H, c->D, c->max_seq, ald, st);
    });
    EpiArgs r;
    r.mode = EPI_RESID; r.bias = w.b_out; r.h = c->h; r.w_il = ild; r.x_il = ald;
    run_k(c, HE_K_GEMM_PREFILL, (double)d * d * es, 2.0 * M * d * d,
          [&] { launch_gemm(dt, c->o, w.w_out, M, d, d, r, st); });
    run_k(c, HE_K_EMBED_NORM, (double)M * d * (4 + es + (post ? 4 : 0)), 0, [&] {
      if (post)
        launch_norm(dt, c->h, nullptr, 0, nullptr, w.ln1_g, w.ln1_b, eps, c->x, M, d, 1, 0, 1, -ald, st);
      else
        launch_norm(dt, c->h, nullptr, 0, nullptr, w.ln2_g, w.ln2_b, eps, c->x, M, d, 1, 0, 0, -ald, st);
    });
    EpiArgs f1;
    f1.mode = EPI_RELU; f1.bias = w.b_fc1; f1.out = c->a; f1.w_il = ild; f1.x_il = ald; f1.o_il = alf;
    run_k(c, HE_K_GEMM_PREFILL, (double)F * d * es, 2.0 * M * F * d,
          [&] { launch_gemm(dt, c->x, w.w_fc1, M, F, d, f1, st); });
    EpiArgs f2;
    f2.mode = EPI_RESID; f2.bias = w.b_fc2; f2.h = c->h; f2.w_il = ilf; f2.x_il = alf;
    run_k(c, HE_K_GEMM_PREFILL, (double)F * d * es, 2.0 * M * F * d,
          [&] { launch_gemm(dt, c->a, w.w_fc2, M, d, F, f2, st); });
    // post-LN: the last layer's output goes to the head, which reads x row-major
    if (post)
      run_k(c, HE_K_EMBED_NORM, (double)M * d * (8 + es), 0, [&] {
        launch_norm(dt, c->h, nullptr, 0, nullptr, w.ln2_g, w.ln2_b, eps, c->x, M, d, 1, 0, 1,
                    l + 1 < c->L ? -ald : 0, st);
      });
    else if (l + 1 < c->L)
      run_k(c, HE_K_EMBED_NORM, (double)M * d * (4 + es), 0, [&] {
        launch_norm(dt, c->h, nullptr, 0, nullptr, c->layers[l + 1].ln1_g, c->layers[l + 1].ln1_b, eps,
                    c->x, M, d, 1, 0, 0, -ald, st);
      });
  }
  int xs = S;
  if (!post) {   // pre-LN: final LayerNorm of the last position
    launch_norm(dt, c->h, nullptr, 0, nullptr, c->wt.lnf_g, c->wt.lnf_b, eps, c->x, B, d, S, S - 1, 0, 0, st);
    dbg_after(c, "final LayerNorm");
    xs = 1;
  }
  run_k(c, HE_K_SCORE, (double)de * d * es, 2.0 * B * de * d,
        [&] { launch_score(dt, c->x, c->wt.proj_out, c->wt.score_w, reward, y, B, xs, d, de, st); });
}

// ------------------------------------------------------------------------------------
// C ABI
// ------------------------------------------------------------------------------------
extern "C" {

const char* he_status_str(he_status s) {
  switch (s) {
    case HE_OK: return "HE_OK";
    case HE_E_ARG: return "HE_E_ARG";
    case HE_E_STATE: return "HE_E_STATE";
    case HE_E_NOCACHE: return "HE_E_NOCACHE";
    case HE_E_RANGE: return "HE_E_RANGE";
    case HE_E_OOM: return "HE_E_OOM";
    case HE_E_HIP: return "HE_E_HIP";
    case HE_E_UNSUPPORTED: return "HE_E_UNSUPPORTED";
    default: return "HE_E_UNKNOWN";
  }
}

const char* he_last_error(const he_ctx* c) { return c ? c->err.c_str() : ""; }

const char* he_build_info(void) { return "libhe gfx950 " HE_BUILD_FLAGS; }

he_status he_create(const he_model_desc* desc, const he_weight_table* w, void* hip_stream,
                    he_ctx** out) {
  if (!desc || !w || !out) return HE_E_ARG;
  *out = nullptr;
  const he_model_desc& D = *desc;
  if (D.tp_size != 1) return HE_E_UNSUPPORTED;
  if (D.n_layers < 0 || D.d_model <= 0 || D.n_heads <= 0 || D.d_ffn <= 0 || D.vocab <= 0 ||
      D.max_pos <= 0 || D.d_model % D.n_heads != 0 || !(D.ln_eps >= 0.f))
    return HE_E_ARG;
  if (D.dtype != HE_DTYPE_F32 && D.dtype != HE_DTYPE_BF16) return HE_E_ARG;
  if (D.norm != HE_NORM_PRE && D.norm != HE_NORM_POST) return HE_E_ARG;
  if (D.head != HE_HEAD_LM && D.head != HE_HEAD_SCALAR) return HE_E_ARG;
  const int de = D.d_embed ? D.d_embed : D.d_model;
  const int hd = D.d_model / D.n_heads;
  const bool bf = D.dtype == HE_DTYPE_BF16;
  if (bf ? !(hd == 32 || hd == 64 || hd == 128) : !(hd == 16 || hd == 32 || hd == 64 || hd == 128))
    return HE_E_UNSUPPORTED;
  if (D.d_model % 32 || D.d_ffn % 32 || de % 32 || D.d_model > 8192) return HE_E_UNSUPPORTED;
  if (D.head == HE_HEAD_LM && (D.norm != HE_NORM_PRE || de != D.d_model)) return HE_E_UNSUPPORTED;
  // bf16 decode kernels: K ranges of 128 and 16-row weight fragments
  if (bf && D.head == HE_HEAD_LM && (D.d_model % 128 || D.d_ffn % 128 || D.vocab % 16))
    return HE_E_UNSUPPORTED;
  if (!w->tok_emb || !w->pos_emb || (D.n_layers > 0 && !w->layers)) return HE_E_ARG;
  if (D.norm == HE_NORM_PRE && (!w->lnf_g || !w->lnf_b)) return HE_E_ARG;
  if (de != D.d_model && (!w->proj_in || (D.head == HE_HEAD_SCALAR && !w->proj_out))) return HE_E_ARG;
  if (D.head == HE_HEAD_SCALAR && !w->score_w) return HE_E_ARG;
  for (int l = 0; l < D.n_layers; ++l) {
    const he_layer_weights& lw = w->layers[l];
    const void* p[] = {lw.ln1_g, lw.ln1_b, lw.w_qkv, lw.b_qkv, lw.w_out, lw.b_out,
                       lw.ln2_g, lw.ln2_b, lw.w_fc1, lw.b_fc1, lw.w_fc2, lw.b_fc2};
    for (const void* q : p)
      if (!q) return HE_E_ARG;
  }

  he_ctx* c = new (std::nothrow) he_ctx();
  if (!c) return HE_E_OOM;
  c->desc = D;
  c->wt = *w;
  c->layers.assign(w->layers, w->layers + D.n_layers);
  c->wt.layers = c->layers.data();
  c->dt = bf ? DT_BF16 : DT_F32;
  c->L = D.n_layers; c->d = D.d_model; c->H = D.n_heads; c->D = hd; c->F = D.d_ffn; c->V = D.vocab;
  c->de = de;
  c->q_scale = (float)(1.0 / std::sqrt((double)hd));
  c->il_d = il_of(c->d);
  c->validate_only = (D.flags & HE_FLAG_VALIDATE_ONLY) != 0;
  const char* ng = std::getenv("HE_NO_GRAPH");
  c->use_graph = D.use_graph && !(ng && ng[0] == '1');
  const char* dbg = std::getenv("HE_DEBUG");
  c->debug = dbg && dbg[0] == '1';
  if (!c->validate_only) {
    if (hipGetDevice(&c->device) != hipSuccess) {
      delete c;
      return HE_E_HIP;
    }
    if (hip_stream) {
      c->stream = (hipStream_t)hip_stream;
    } else {
      hipError_t e = hipStreamCreateWithFlags(&c->stream, hipStreamNonBlocking);
      if (e != hipSuccess) {
        delete c;
        return HE_E_HIP;
      }
      c->own_stream = true;
    }
  }
  *out = c;
  return HE_OK;
}

he_status he_release_cache(he_ctx* c) {
  if (!c) return HE_E_ARG;
  drop_graphs(c);
  if (!c->cache) return HE_OK;
  if (!c->validate_only) {
    hipError_t e1 = hipStreamSynchronize(c->stream);
    hipError_t e2 = c->kv ? hipFree(c->kv) : hipSuccess;
    hipError_t e3 = c->scratch ? hipFree(c->scratch) : hipSuccess;
    c->kv = nullptr;
    c->scratch = nullptr;
    c->cache = false;
    c->prefilled = false;
    if (e1 != hipSuccess) return hip_fail(c, e1, "hipStreamSynchronize");
    if (e2 != hipSuccess) return hip_fail(c, e2, "hipFree(kv)");
    if (e3 != hipSuccess) return hip_fail(c, e3, "hipFree(scratch)");
  }
  c->cache = false;
  c->prefilled = false;
  return HE_OK;
}

he_status he_destroy(he_ctx* c) {
  if (!c) return HE_OK;
  he_status s = he_release_cache(c);
  if (c->f8buf) {
    if (!c->validate_only) (void)hipStreamSynchronize(c->stream);   // no kernel still reads the copy
    hipFree(c->f8buf);
  }
  if (!c->validate_only) {
    for (Timer& t : c->timers) {
      for (auto& p : t.live) { hipEventDestroy(p.first); hipEventDestroy(p.second); }
      for (auto& p : t.pool) { hipEventDestroy(p.first); hipEventDestroy(p.second); }
    }
    if (c->own_stream) hipStreamDestroy(c->stream);
  }
  delete c;
  return s;
}

// E4M3 copies of the current projection weights (in whatever layout they hold now).
static he_status f8_requantize(he_ctx* c) {
  if (!c->f8_on || c->validate_only) return HE_OK;
  const int d = c->d, F = c->F;
  for (int l = 0; l < c->L; ++l) {
    const he_layer_weights& w = c->layers[l];
    launch_quantize_fp8(w.w_qkv, 3 * d, d, w_il(c, d), c->f8[l].q[0], c->f8[l].s[0], c->stream);
    launch_quantize_fp8(w.w_out, d, d, w_il(c, d), c->f8[l].q[1], c->f8[l].s[1], c->stream);
    launch_quantize_fp8(w.w_fc1, F, d, w_il(c, d), c->f8[l].q[2], c->f8[l].s[2], c->stream);
    launch_quantize_fp8(w.w_fc2, d, F, w_il(c, F), c->f8[l].q[3], c->f8[l].s[3], c->stream);
    dbg_after(c, "FP8 quantisation");
  }
  return check_launch(c, "fp8 quantisation launch");
}

he_status he_set_fp8_decode(he_ctx* c, int32_t enable) {
  if (!c) return HE_E_ARG;
  if (c->failed) return set_err(c, HE_E_HIP, "context failed earlier: %s", c->err.c_str());
  if (!enable) {
    c->prefilled = false;   // decode plans depend on the weight format: a new prompt pass
    // captured decode graphs hold the copy's addresses as kernel arguments
    drop_graphs(c);
    if (c->f8buf && !c->validate_only) {
      HIP_TRY(c, hipStreamSynchronize(c->stream));
      hipFree(c->f8buf);
    }
    c->f8buf = nullptr;
    c->f8.clear();
    c->f8_on = false;
    return HE_OK;
  }
  if (c->dt != DT_BF16 || c->desc.head != HE_HEAD_LM)
    return set_err(c, HE_E_UNSUPPORTED, "FP8 decode weights need a bf16 LM-head model");
  if (c->d % 256 || c->F % 256)
    return set_err(c, HE_E_UNSUPPORTED, "FP8 decode weights need d and d_ffn divisible by 256");
  if (c->f8_on) return f8_requantize(c);
  c->prefilled = false;   // decode plans depend on the weight format: a new prompt pass
  const int d = c->d, F = c->F;
  const size_t nq[4] = {(size_t)3 * d * d, (size_t)d * d, (size_t)F * d, (size_t)d * F};
  const size_t ns[4] = {(size_t)3 * d, (size_t)d, (size_t)F, (size_t)d};
  size_t off = 0;
  std::vector<std::array<size_t, 8>> offs(c->L);
  for (int l = 0; l < c->L; ++l)
    for (int j = 0; j < 4; ++j) {
      offs[l][j] = off; off += (nq[j] + 255) / 256 * 256;
      offs[l][4 + j] = off; off += (ns[j] * 4 + 255) / 256 * 256;
    }
  if (c->validate_only) {
    c->f8_on = true;
    return HE_OK;
  }
  drop_graphs(c);   // a new copy at new addresses: no captured graph may point at an old one
  char* buf = nullptr;
  hipError_t e = hipMalloc((void**)&buf, std::max<size_t>(off, 256));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return set_err(c, HE_E_OOM, "FP8 weight allocation of %zu bytes failed: %s", off, hipGetErrorString(e));
  }
  c->f8buf = buf;
  c->f8.resize(c->L);
  for (int l = 0; l < c->L; ++l)
    for (int j = 0; j < 4; ++j) {
      c->f8[l].q[j] = (uint8_t*)(buf + offs[l][j]);
      c->f8[l].s[j] = (float*)(buf + offs[l][4 + j]);
    }
  c->f8_on = true;
  return f8_requantize(c);
}

he_status he_fp8_export(he_ctx* c, int32_t layer, int32_t proj, uint8_t* d_codes, float* d_scales) {
  if (!c) return HE_E_ARG;
  if (!c->f8_on) return set_err(c, HE_E_STATE, "FP8 decode weights are off");
  if (layer < 0 || layer >= c->L || proj < 0 || proj > 3)
    return set_err(c, HE_E_ARG, "layer %d / projection %d out of range", layer, proj);
  if (!d_codes || !d_scales) return set_err(c, HE_E_ARG, "NULL buffer");
  if (c->validate_only) return HE_OK;
  const int d = c->d, F = c->F;
  const int N[4] = {3 * d, d, F, d}, K[4] = {d, d, d, F};
  launch_fp8_rowmajor(c->f8[layer].q[proj], N[proj], K[proj], d_codes, c->stream);
  dbg_after(c, "FP8 export");
  HIP_TRY(c, hipMemcpyAsync(d_scales, c->f8[layer].s[proj], (size_t)N[proj] * 4, hipMemcpyDeviceToDevice,
                            c->stream));
  return check_launch(c, "fp8 export launch");
}

static he_status lora_common(he_ctx* c, const he_lora_table* t, float sign) {
  if (!t || !t->pairs) return set_err(c, HE_E_ARG, "NULL LoRA table");
  if (t->rank < 1 || t->rank > 64) return set_err(c, HE_E_ARG, "LoRA rank %d outside 1..64", t->rank);
  if (!std::isfinite(t->alpha)) return set_err(c, HE_E_ARG, "LoRA alpha not finite");
  for (int i = 0; i < c->L * HE_N_PROJ; ++i)
    if ((t->pairs[i].A == nullptr) != (t->pairs[i].B == nullptr))
      return set_err(c, HE_E_ARG, "LoRA pair %d has only one factor", i);
  if (c->validate_only) return HE_OK;
  const float s = t->alpha / (float)t->rank;
  const int d = c->d, F = c->F;
  const size_t es = esize(c->dt);
  // bf16: every projection changes layout (those without an adapter with r = 0)
  const bool relayout = c->dt == DT_BF16;
  for (int l = 0; l < c->L; ++l) {
    const he_layer_weights& w = c->layers[l];
    for (int p = 0; p < HE_N_PROJ; ++p) {
      const he_lora_pair& pr = t->pairs[l * HE_N_PROJ + p];
      if (!pr.A && !relayout) continue;
      const int r = pr.A ? t->rank : 0;
      void* W;
      int N, K;
      switch (p) {
        case HE_PROJ_Q: W = w.w_qkv; N = d; K = d; break;
        case HE_PROJ_K: W = (char*)w.w_qkv + (size_t)d * d * es; N = d; K = d; break;
        case HE_PROJ_V: W = (char*)w.w_qkv + (size_t)2 * d * d * es; N = d; K = d; break;
        case HE_PROJ_OUT: W = w.w_out; N = d; K = d; break;
        case HE_PROJ_FC1: W = w.w_fc1; N = F; K = d; break;
        default: W = w.w_fc2; N = d; K = F; break;
      }
      run_k(c, HE_K_LORA, 2.0 * N * K * es + (double)(N + K) * r * es, 2.0 * N * K * r, [&] {
        launch_lora(c->dt, W, pr.A, pr.B, N, K, r, s, sign, relayout ? il_of(K) : 0, c->stream);
      });
    }
  }
  if (relayout && c->desc.head == HE_HEAD_LM)   // the tied embedding is the LM head's weight
    run_k(c, HE_K_LORA, 2.0 * c->V * d * es, 0.0, [&] {
      launch_lora(c->dt, (void*)c->wt.tok_emb, nullptr, nullptr, c->V, d, 0, 0.f, sign, c->il_d, c->stream);
    });
  return check_launch(c, "lora kernel launch");
}

he_status he_fuse_lora(he_ctx* c, const he_lora_table* t) {
  if (!c) return HE_E_ARG;
  if (c->failed) return set_err(c, HE_E_HIP, "context failed earlier: %s", c->err.c_str());
  if (c->fused) return set_err(c, HE_E_STATE, "LoRA already fused");
  he_status s = lora_common(c, t, +1.f);
  if (s == HE_OK) c->fused = true;
  if (s == HE_OK) s = f8_requantize(c);
  return s;
}

he_status he_unfuse_lora(he_ctx* c, const he_lora_table* t) {
  if (!c) return HE_E_ARG;
  if (!c->fused) return set_err(c, HE_E_STATE, "LoRA not fused");
  he_status s = lora_common(c, t, -1.f);
  if (s == HE_OK) c->fused = false;
  if (s == HE_OK) s = f8_requantize(c);
  return s;
}

he_status he_retake_cache(he_ctx* c, int32_t max_batch, int32_t max_seq) {
  if (!c) return HE_E_ARG;
  if (c->failed) return set_err(c, HE_E_HIP, "context failed earlier: %s", c->err.c_str());
  if (c->cache) return set_err(c, HE_E_STATE, "workspace already held");
  if (max_batch < 1 || max_seq < 1) return set_err(c, HE_E_ARG, "max_batch and max_seq must be >= 1");
  if (max_seq > c->desc.max_pos)
    return set_err(c, HE_E_RANGE, "max_seq %d exceeds the %d learned positions", max_seq, c->desc.max_pos);
  if (c->desc.head == HE_HEAD_LM && max_batch > kMaxDecodeBatch)
    return set_err(c, HE_E_UNSUPPORTED, "decode batch above %d", kMaxDecodeBatch);
  if (c->fail_next_alloc) {
    c->fail_next_alloc = false;
    return set_err(c, HE_E_OOM, "injected allocation failure");
  }
  const size_t es = esize(c->dt);
  const int bpad = c->dt == DT_BF16 ? 16 * decode_mt(max_batch) : round_up(max_batch, 16);
  // rows rounded to 16: the inference layout of an activation fills whole 16-row blocks
  const size_t rows = (std::max<size_t>((size_t)max_batch * max_seq, (size_t)bpad) + 15) / 16 * 16;
  const size_t kv_layer = (size_t)max_batch * c->H * max_seq * c->D;
  const size_t kv_bytes = kv_layer * 2 * c->L * es;
  // scratch layout (256-byte aligned pieces)
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += (bytes + 255) / 256 * 256; return o; };
  const size_t o_h = take(rows * c->d * 4);
  const size_t o_x = take(rows * std::max(c->d, c->de) * es);
  const size_t o_xe = take(c->de != c->d ? rows * c->de * es : 0);
  const size_t o_q = take(rows * c->d * es);
  const size_t o_o = take(rows * c->d * es);
  const size_t o_a = take(rows * c->F * es);
  int argmax_cap = 0;
  const size_t part_elems = parts_elems(c, max_batch, &argmax_cap);
  argmax_cap = std::max(argmax_cap, (c->V + 127) / 128);   // he_sample's 128-column blocks
  const size_t o_parts = take(part_elems * 4);
  const size_t o_logits = take((size_t)bpad * c->V * 4);
  const size_t o_bv = take((size_t)bpad * argmax_cap * 4);
  const size_t o_bi = take((size_t)bpad * argmax_cap * 4);
  const size_t o_ids = take((size_t)bpad * 4);
  const size_t o_tok = take((size_t)max_batch * (max_seq + 1) * 4);
  const size_t o_logp = take((size_t)max_batch * (max_seq + 1) * 4);
  const size_t o_blg = take((size_t)bpad * argmax_cap * 4);
  const size_t o_bmx = take((size_t)bpad * argmax_cap * 4);
  const size_t o_bsm = take((size_t)bpad * argmax_cap * 4);
  const size_t o_pos = take(256);
  const size_t o_posn = take(256);
  const size_t o_spos = take(256);
  // one chunk of scoring-pass logits: up to kLogitChunk rows of the vocabulary
  const int lg_rows = c->desc.head == HE_HEAD_LM ? (int)std::min<size_t>(rows, kLogitChunk) : 0;
  const size_t o_lgc = take((size_t)lg_rows * c->V * 4);
  c->max_batch = max_batch;
  c->max_seq = max_seq;
  c->bpad = bpad;
  c->argmax_cap = argmax_cap;
  c->rows = (int)rows;
  c->kv_layer_elems = kv_layer;
  if (c->validate_only) {
    c->cache = true;
    c->prefilled = false;
    return HE_OK;
  }
  void* kv = nullptr;
  char* scratch = nullptr;
  hipError_t e = hipMalloc(&kv, std::max<size_t>(kv_bytes, 256));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return set_err(c, HE_E_OOM, "KV cache allocation of %zu bytes failed: %s", kv_bytes, hipGetErrorString(e));
  }
  e = hipMalloc((void**)&scratch, off);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    hipFree(kv);
    return set_err(c, HE_E_OOM, "scratch allocation of %zu bytes failed: %s", off, hipGetErrorString(e));
  }
  c->kv = kv;
  c->scratch = scratch;
  c->h = (float*)(scratch + o_h);
  c->x = scratch + o_x;
  c->xe = scratch + o_xe;
  c->q = scratch + o_q;
  c->o = scratch + o_o;
  c->a = scratch + o_a;
  c->parts = (float*)(scratch + o_parts);
  c->logits = (float*)(scratch + o_logits);
  c->best_val = (float*)(scratch + o_bv);
  c->best_idx = (int32_t*)(scratch + o_bi);
  c->ids_cur = (int32_t*)(scratch + o_ids);
  c->tokens = (int32_t*)(scratch + o_tok);
  c->pos_dev = (int32_t*)(scratch + o_pos);
  c->pos_next = (int32_t*)(scratch + o_posn);
  c->spos = (int32_t*)(scratch + o_spos);
  c->logp = (float*)(scratch + o_logp);
  c->best_lg = (float*)(scratch + o_blg);
  c->blk_max = (float*)(scratch + o_bmx);
  c->blk_sum = (float*)(scratch + o_bsm);
  c->lgc = (float*)(scratch + o_lgc);
  c->lg_rows = lg_rows;
  c->cache = true;
  c->prefilled = false;
  // The decode GEMM reads X rows up to the next multiple of 16: give the padding
  // rows defined contents once (their products are never stored).
  HIP_TRY(c, hipMemsetAsync(c->x, 0, (size_t)bpad * std::max(c->d, c->de) * es, c->stream));
  HIP_TRY(c, hipMemsetAsync(c->o, 0, (size_t)bpad * c->d * es, c->stream));
  HIP_TRY(c, hipMemsetAsync(c->a, 0, (size_t)bpad * c->F * es, c->stream));
  return HE_OK;
}

static he_status check_compute(he_ctx* c) {
  if (c->failed) return set_err(c, HE_E_HIP, "context failed earlier: %s", c->err.c_str());
  if (!c->cache) return set_err(c, HE_E_NOCACHE, "no workspace: call he_retake_cache");
  return HE_OK;
}

static he_status prefill_checks(he_ctx* c, const int32_t* ids, int B, int S, const void* out) {
  he_status s = check_compute(c);
  if (s != HE_OK) return s;
  if (c->desc.head != HE_HEAD_LM) return set_err(c, HE_E_UNSUPPORTED, "generation needs an LM-head model");
  if (!ids || !out) return set_err(c, HE_E_ARG, "NULL buffer");
  if (B < 1 || B > c->max_batch) return set_err(c, HE_E_ARG, "batch %d outside 1..%d", B, c->max_batch);
  if (S < 1) return set_err(c, HE_E_ARG, "prompt length %d < 1", S);
  if (S > c->max_seq) return set_err(c, HE_E_RANGE, "prompt length %d > max_seq %d", S, c->max_seq);
  return HE_OK;
}

static he_status do_prefill(he_ctx* c, const int32_t* ids, int B, int S, bool want_logits) {
  set_plans(c, B);
  launch_set_i32(c->pos_dev, S - 1, c->stream);
  dbg_after(c, "position set");
  enqueue_prefill_lm(c, ids, B, S, want_logits);
  he_status s = check_launch(c, "prefill launch");
  if (s != HE_OK) return s;
  if (c->graph_B != B) drop_graphs(c);
  c->prefilled = true;
  c->cur_B = B;
  c->cur_pos = S;
  return HE_OK;
}

// Greedy picks without log-probabilities: the rule of he_prefill, he_decode_step and
// he_generate.
static void set_greedy(he_ctx* c) {
  c->inv_temp = 0.f;
  c->seed = 0;
  c->want_logp = false;
  c->top_p = 1.f;
}

he_status he_prefill(he_ctx* c, const int32_t* ids, int32_t B, int32_t S, int32_t* d_next, float* d_logits) {
  if (!c) return HE_E_ARG;
  he_status s = prefill_checks(c, ids, B, S, d_next);
  if (s != HE_OK) return s;
  set_greedy(c);
  if (c->validate_only) {
    c->prefilled = true; c->cur_B = B; c->cur_pos = S;
    return HE_OK;
  }
  s = do_prefill(c, ids, B, S, d_logits != nullptr);
  if (s != HE_OK) return s;
  HIP_TRY(c, hipMemcpyAsync(d_next, c->ids_cur, (size_t)B * 4, hipMemcpyDeviceToDevice, c->stream));
  if (d_logits)
    HIP_TRY(c, hipMemcpyAsync(d_logits, c->logits, (size_t)B * c->V * 4, hipMemcpyDeviceToDevice, c->stream));
  return HE_OK;
}

// One step, from the graph or launched directly.
static he_status run_step(he_ctx* c, bool want_logits) {
  if (c->fail_next_step) {
    c->fail_next_step = false;
    c->failed = true;
    return set_err(c, HE_E_HIP, "injected device fault");
  }
  const int B = c->cur_B;
  const bool graph = c->use_graph && !any_timer_armed(c) && !c->debug;
  if (graph) {
    hipGraphExec_t& ge = c->graph[want_logits ? 1 : 0];
    if (c->graph_B != B || c->graph_fused != c->fused || c->graph_itemp != c->inv_temp ||
        c->graph_seed != c->seed || c->graph_logp != c->want_logp || c->graph_topp != c->top_p ||
        c->graph_f8 != c->f8_on)
      drop_graphs(c);
    if (!ge) {
      hipGraph_t g = nullptr;
      HIP_TRY(c, hipStreamBeginCapture(c->stream, hipStreamCaptureModeThreadLocal));
      c->capturing = true;
      enqueue_step(c, B, want_logits, c->cur_pos);
      c->capturing = false;
      hipError_t e = hipStreamEndCapture(c->stream, &g);
      if (e != hipSuccess) return hip_fail(c, e, "hipStreamEndCapture");
      e = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
      hipGraphDestroy(g);
      if (e != hipSuccess) { ge = nullptr; return hip_fail(c, e, "hipGraphInstantiate"); }
      c->graph_B = B;
      c->graph_fused = c->fused;
      c->graph_itemp = c->inv_temp;
      c->graph_seed = c->seed;
      c->graph_logp = c->want_logp;
      c->graph_topp = c->top_p;
      c->graph_f8 = c->f8_on;
    }
    HIP_TRY(c, hipGraphLaunch(ge, c->stream));
  } else {
    enqueue_step(c, B, want_logits, c->cur_pos);
    he_status s = check_launch(c, "decode step launch");
    if (s != HE_OK) return s;
  }
  c->cur_pos += 1;
  return HE_OK;
}

static he_status step_checks(he_ctx* c) {
  he_status s = check_compute(c);
  if (s != HE_OK) return s;
  if (!c->prefilled) return set_err(c, HE_E_STATE, "decode before a prefill in this cache epoch");
  if (c->cur_pos >= c->max_seq)
    return set_err(c, HE_E_RANGE, "position %d reaches max_seq %d", c->cur_pos, c->max_seq);
  return HE_OK;
}

he_status he_decode_step(he_ctx* c, const int32_t* d_in, int32_t* d_next, float* d_logits) {
  if (!c) return HE_E_ARG;
  he_status s = step_checks(c);
  if (s != HE_OK) return s;
  if (!d_in || !d_next) return set_err(c, HE_E_ARG, "NULL buffer");
  set_greedy(c);
  if (c->validate_only) {
    if (c->fail_next_step) { c->fail_next_step = false; c->failed = true; return set_err(c, HE_E_HIP, "injected device fault"); }
    c->cur_pos += 1;
    return HE_OK;
  }
  HIP_TRY(c, hipMemcpyAsync(c->ids_cur, d_in, (size_t)c->cur_B * 4, hipMemcpyDeviceToDevice, c->stream));
  s = run_step(c, d_logits != nullptr);
  if (s != HE_OK) return s;
  HIP_TRY(c, hipMemcpyAsync(d_next, c->ids_cur, (size_t)c->cur_B * 4, hipMemcpyDeviceToDevice, c->stream));
  if (d_logits)
    HIP_TRY(c, hipMemcpyAsync(d_logits, c->logits, (size_t)c->cur_B * c->V * 4, hipMemcpyDeviceToDevice, c->stream));
  return HE_OK;
}

static he_status generate(he_ctx* c, const int32_t* d_prompt, int32_t B, int32_t S, int32_t S_g,
                          int32_t* d_out, float* d_logp) {
  he_status s = prefill_checks(c, d_prompt, B, S, d_out);
  if (s != HE_OK) return s;
  if (S_g < 1) return set_err(c, HE_E_ARG, "S_g %d < 1", S_g);
  if (S + S_g - 1 > c->max_seq)
    return set_err(c, HE_E_RANGE, "S_p + S_g - 1 = %d exceeds max_seq %d", S + S_g - 1, c->max_seq);
  if (c->validate_only) {
    c->prefilled = true; c->cur_B = B; c->cur_pos = S;
    for (int j = 1; j < S_g; ++j) {
      if (c->fail_next_step) { c->fail_next_step = false; c->failed = true; return set_err(c, HE_E_HIP, "injected device fault"); }
      c->cur_pos += 1;
    }
    return HE_OK;
  }
  s = do_prefill(c, d_prompt, B, S, false);
  if (s != HE_OK) return s;
  for (int j = 1; j < S_g; ++j) {
    s = run_step(c, false);
    if (s != HE_OK) return s;
  }
  HIP_TRY(c, hipMemcpy2DAsync(d_out, (size_t)S_g * 4, c->tokens + S, (size_t)(c->max_seq + 1) * 4,
                              (size_t)S_g * 4, B, hipMemcpyDeviceToDevice, c->stream));
  if (d_logp)
    HIP_TRY(c, hipMemcpy2DAsync(d_logp, (size_t)S_g * 4, c->logp + S, (size_t)(c->max_seq + 1) * 4,
                                (size_t)S_g * 4, B, hipMemcpyDeviceToDevice, c->stream));
  return HE_OK;
}

// The pick rule as it stood before a call that may be refused: a refused call
// (argument or state error, nothing enqueued) puts it back.
struct RuleKeep {
  he_ctx* c;
  float it, tp;
  uint64_t seed;
  bool lp;
  explicit RuleKeep(he_ctx* c_) : c(c_), it(c_->inv_temp), tp(c_->top_p), seed(c_->seed), lp(c_->want_logp) {}
  void restore() { c->inv_temp = it; c->top_p = tp; c->seed = seed; c->want_logp = lp; }
  he_status done(he_status s) {
    if (s != HE_OK && s != HE_E_HIP) restore();
    return s;
  }
};

he_status he_generate(he_ctx* c, const int32_t* d_prompt, int32_t B, int32_t S, int32_t S_g, int32_t* d_out) {
  if (!c) return HE_E_ARG;
  RuleKeep keep(c);
  set_greedy(c);
  return keep.done(generate(c, d_prompt, B, S, S_g, d_out, nullptr));
}

// Pick rule from he_sampling (NULL: greedy) into the context; checked before use.
static he_status set_rule(he_ctx* c, const he_sampling* smp, bool want_logp) {
  const float t = smp ? smp->temperature : 0.f;
  if (!(t >= 0.f) || !std::isfinite(t))
    return set_err(c, HE_E_ARG, "temperature %g is not a finite value >= 0", (double)t);
  const float it = t > 0.f ? 1.f / t : 0.f;
  if (t > 0.f && !std::isfinite(it)) return set_err(c, HE_E_ARG, "temperature %g too small", (double)t);
  const float tp = smp ? smp->top_p : 0.f;
  if (!(tp >= 0.f)) return set_err(c, HE_E_ARG, "top_p %g is negative or NaN", (double)tp);
  const bool nucleus = t > 0.f && tp > 0.f && tp < 1.f;
  if (nucleus && c->V > topp_max_vocab())
    return set_err(c, HE_E_UNSUPPORTED, "top-p over a vocabulary of %d (at most %d)", c->V, topp_max_vocab());
  c->inv_temp = it;
  c->seed = smp && t > 0.f ? smp->seed : 0;
  c->want_logp = want_logp;
  c->top_p = nucleus ? tp : 1.f;
  return HE_OK;
}

he_status he_generate_ex(he_ctx* c, const int32_t* d_prompt, int32_t B, int32_t S, int32_t S_g,
                         const he_sampling* smp, int32_t* d_out, float* d_logprobs) {
  if (!c) return HE_E_ARG;
  RuleKeep keep(c);
  he_status s = set_rule(c, smp, d_logprobs != nullptr);
  if (s != HE_OK) return keep.done(s);
  return keep.done(generate(c, d_prompt, B, S, S_g, d_out, d_logprobs));
}

// The pick rule of smp on caller logits [B][V]: per-block partials in (best_val,
// best_idx, and for log-probabilities best_lg / blk_max / blk_sum), the position pair
// in spos.  Checks come first; nothing is enqueued on a refused call.
struct PickScratch {
  int32_t* spos;
  float* best_val;
  int32_t* best_idx;
  float* best_lg;
  float* blk_max;
  float* blk_sum;
};

static he_status sample_checks(he_ctx* c, const float* d_logits, int32_t B, int32_t position,
                               const he_sampling* smp, int32_t* d_tokens, float* d_logprobs, int max_b,
                               float* it, uint64_t* seed, float* tp, bool* want_lp) {
  if (c->failed) return set_err(c, HE_E_HIP, "context failed earlier: %s", c->err.c_str());
  if (c->desc.head != HE_HEAD_LM) return set_err(c, HE_E_UNSUPPORTED, "sampling needs an LM-head model");
  if (!d_logits || !d_tokens) return set_err(c, HE_E_ARG, "NULL buffer");
  if (B < 1 || B > max_b) return set_err(c, HE_E_ARG, "batch %d outside 1..%d", B, max_b);
  if (position < 0) return set_err(c, HE_E_ARG, "position %d < 0", position);
  // the rule of this call only: the context's own (used by he_decode_step) is kept
  RuleKeep keep(c);
  he_status s = set_rule(c, smp, d_logprobs != nullptr);
  *it = c->inv_temp; *tp = c->top_p; *seed = c->seed; *want_lp = c->want_logp;
  keep.restore();
  return s;
}

static he_status enqueue_sample(he_ctx* c, const float* d_logits, int32_t B, int32_t position, float it,
                                uint64_t seed, float tp, bool want_lp, const PickScratch& ps,
                                int32_t* d_tokens, float* d_logprobs) {
  hipStream_t st = c->stream;
  SampleArgs smpa;
  smpa.inv_temp = it;
  smpa.seed = seed;
  if (want_lp) { smpa.best_lg = ps.best_lg; smpa.blk_max = ps.blk_max; smpa.blk_sum = ps.blk_sum; }
  launch_set_i32(ps.spos, position - 1, st);
  if (tp < 1.f) {
    launch_set_i32(ps.spos + 1, position, st);
    launch_topp_finalize(d_logits, B, c->V, smpa, tp, nullptr, d_tokens, d_logprobs, 0, ps.spos + 1,
                         nullptr, st);
  } else {
    const int nb = (c->V + 127) / 128;
    launch_reduce_argmax(d_logits, 1, B, c->V, nullptr, ps.best_val, ps.best_idx, nb, ps.spos, ps.spos + 1,
                         smpa, st);
    launch_argmax_finalize(ps.best_val, ps.best_idx, smpa, nb, B, nullptr, d_tokens,
                           want_lp ? d_logprobs : nullptr, 0, ps.spos + 1, nullptr, nullptr, st);
  }
  dbg_after(c, "sample");
  return check_launch(c, "sample launch");
}

he_status he_sample(he_ctx* c, const float* d_logits, int32_t B, int32_t position, const he_sampling* smp,
                    int32_t* d_tokens, float* d_logprobs) {
  if (!c) return HE_E_ARG;
  he_status s = check_compute(c);
  if (s != HE_OK) return s;
  float it = 0.f, tp = 1.f;
  uint64_t seed = 0;
  bool want_lp = false;
  s = sample_checks(c, d_logits, B, position, smp, d_tokens, d_logprobs, c->max_batch, &it, &seed, &tp, &want_lp);
  if (s != HE_OK || c->validate_only) return s;
  const PickScratch ps{c->spos, c->best_val, c->best_idx, c->best_lg, c->blk_max, c->blk_sum};
  return enqueue_sample(c, d_logits, B, position, it, seed, tp, want_lp, ps, d_tokens, d_logprobs);
}

he_status he_sample_static(he_ctx* c, const float* d_logits, int32_t B, int32_t position,
                           const he_sampling* smp, int32_t* d_tokens, float* d_logprobs) {
  if (!c) return HE_E_ARG;
  const int nb = (c->V + 127) / 128;
  if (nb > kStaticBlocks)
    return set_err(c, HE_E_UNSUPPORTED, "vocabulary %d above the static scratch's %d columns", c->V,
                   kStaticBlocks * 128);
  float it = 0.f, tp = 1.f;
  uint64_t seed = 0;
  bool want_lp = false;
  he_status s = sample_checks(c, d_logits, B, position, smp, d_tokens, d_logprobs,
                              kStaticRows * kStaticBlocks / nb, &it, &seed, &tp, &want_lp);
  if (s != HE_OK || c->validate_only) return s;
  StaticScratch ss;
  const hipError_t e = static_scratch(c->device, &ss);
  if (e != hipSuccess) return hip_fail(c, e, "static scratch address");
  const PickScratch ps{ss.pos, ss.best_val, ss.best_idx, ss.best_lg, ss.blk_max, ss.blk_sum};
  return enqueue_sample(c, d_logits, B, position, it, seed, tp, want_lp, ps, d_tokens, d_logprobs);
}

// Teacher-forced scoring: prompt pass over the whole sequence, final LayerNorm of the
// positions S_p - 1 .. S - 2 of every row (each predicts the next token), then in
// chunks of lg_rows rows the tied-head GEMM into fp32 logits and the log-softmax gather.
static void enqueue_logprobs(he_ctx* c, const int32_t* seq, int B, int S, int S_p, float* out) {
  const int d = c->d, dt = c->dt, n = S - S_p, Mp = B * n;
  const float eps = c->desc.ln_eps;
  const size_t es = esize(dt);
  hipStream_t st = c->stream;
  enqueue_prompt_layers(c, seq, B, S);
  const int ald = a_il(c, d);
  run_k(c, HE_K_EMBED_NORM, (double)Mp * d * (4 + es), 0, [&] {
    launch_norm(dt, c->h, nullptr, 0, nullptr, c->wt.lnf_g, c->wt.lnf_b, eps, c->x, Mp, d, S, S_p - 1, 0,
                -ald, st, n);
  });
  for (int r0 = 0; r0 < Mp; r0 += c->lg_rows) {
    const int mc = std::min(c->lg_rows, Mp - r0);
    EpiArgs e;
    e.mode = EPI_F32;
    e.out_f32 = c->lgc;
    e.w_il = e_il(c);
    e.x_il = ald;
    const char* xr = (const char*)c->x + (size_t)r0 * d * es;   // r0 % 16 == 0: whole row blocks
    // bf16 chunks of whole 256-row tiles: the vocabulary's 256-column tiles on the
    // fast GEMM, the remaining columns (a multiple of 16) on the general one
    const int Nm = (dt == DT_BF16 && mc % 256 == 0 && d % 32 == 0) ? c->V / 256 * 256 : 0;
    run_k(c, HE_K_VOCAB, (double)c->V * d * es + (double)mc * c->V * 8, 2.0 * mc * c->V * d, [&] {
      if (Nm) {
        e.ldo = c->V;
        launch_gemm(dt, xr, c->wt.tok_emb, mc, Nm, d, e, st);
        if (Nm < c->V) {
          EpiArgs t = e;
          t.out_f32 = c->lgc + Nm;
          launch_gemm(dt, xr, (const char*)c->wt.tok_emb + (size_t)Nm * d * es, mc, c->V - Nm, d, t, st);
        }
      } else {
        launch_gemm(dt, xr, c->wt.tok_emb, mc, c->V, d, e, st);
      }
      launch_logprob_gather(c->lgc, mc, c->V, seq, S, S_p, n, r0, out, st);
      dbg_after(c, "log-probability gather");
    });
  }
}

he_status he_logprobs(he_ctx* c, const int32_t* d_seq, int32_t B, int32_t S, int32_t S_p, float* d_logprobs) {
  if (!c) return HE_E_ARG;
  he_status s = prefill_checks(c, d_seq, B, S, d_logprobs);
  if (s != HE_OK) return s;
  if (S_p < 1 || S_p >= S) return set_err(c, HE_E_ARG, "prompt length %d outside 1..%d", S_p, S - 1);
  c->prefilled = false;   // the cache now holds the scored sequences
  if (c->validate_only) return HE_OK;
  enqueue_logprobs(c, d_seq, B, S, S_p, d_logprobs);
  return check_launch(c, "logprobs launch");
}

he_status he_score(he_ctx* c, const int32_t* d_ids, int32_t B, int32_t S, float* d_reward, float* d_y) {
  if (!c) return HE_E_ARG;
  he_status s = check_compute(c);
  if (s != HE_OK) return s;
  if (c->desc.head != HE_HEAD_SCALAR) return set_err(c, HE_E_UNSUPPORTED, "scoring needs a scalar-head model");
  if (!d_ids || !d_reward) return set_err(c, HE_E_ARG, "NULL buffer");
  if (B < 1 || B > c->max_batch) return set_err(c, HE_E_ARG, "batch %d outside 1..%d", B, c->max_batch);
  if (S < 1) return set_err(c, HE_E_ARG, "length %d < 1", S);
  if (S > c->max_seq) return set_err(c, HE_E_RANGE, "length %d > max_seq %d", S, c->max_seq);
  if (c->validate_only) return HE_OK;
  enqueue_score(c, d_ids, B, S, d_reward, d_y);
  c->prefilled = false;   // the cache now holds the scored sequences
  return check_launch(c, "score launch");
}

he_status he_sync(he_ctx* c) {
  if (!c) return HE_E_ARG;
  if (c->validate_only) return HE_OK;
  HIP_TRY(c, hipStreamSynchronize(c->stream));
  HIP_TRY(c, hipGetLastError());
  return c->failed ? HE_E_HIP : HE_OK;
}

he_status he_kernel_timer(he_ctx* c, int32_t k, int32_t enable) {
  if (!c) return HE_E_ARG;
  if (k < 0 || k >= HE_K_COUNT) return set_err(c, HE_E_ARG, "kernel class %d", k);
  if (c->validate_only) return HE_OK;
  Timer& t = c->timers[k];
  if (!t.live.empty()) HIP_TRY(c, hipStreamSynchronize(c->stream));
  for (auto& p : t.live) t.pool.push_back(p);
  t.live.clear();
  t.bytes.clear();
  t.flops.clear();
  t.acc = he_kernel_stat{0, 0.0, 0.0, 0.0};
  t.armed = enable != 0;
  return HE_OK;
}

he_status he_kernel_stats(he_ctx* c, int32_t k, he_kernel_stat* out) {
  if (!c || !out) return HE_E_ARG;
  if (k < 0 || k >= HE_K_COUNT) return set_err(c, HE_E_ARG, "kernel class %d", k);
  if (c->validate_only) { *out = he_kernel_stat{0, 0.0, 0.0, 0.0}; return HE_OK; }
  Timer& t = c->timers[k];
  if (!t.live.empty()) HIP_TRY(c, hipStreamSynchronize(c->stream));
  for (size_t i = 0; i < t.live.size(); ++i) {
    float ms = 0.f;
    HIP_TRY(c, hipEventElapsedTime(&ms, t.live[i].first, t.live[i].second));
    t.acc.launches += 1;
    t.acc.total_ms += ms;
    t.acc.bytes += t.bytes[i];
    t.acc.flops += t.flops[i];
    t.pool.push_back(t.live[i]);
  }
  t.live.clear();
  t.bytes.clear();
  t.flops.clear();
  *out = t.acc;
  return HE_OK;
}

he_status he_debug(he_ctx* c, int32_t what, int64_t value) {
  if (!c) return HE_E_ARG;
  if (what == HE_DBG_FAIL_NEXT_ALLOC) { c->fail_next_alloc = value != 0; return HE_OK; }
  if (what == HE_DBG_FAIL_NEXT_STEP) { c->fail_next_step = value != 0; return HE_OK; }
  return set_err(c, HE_E_ARG, "unknown debug hook %d", what);
}

}  // extern "C"
