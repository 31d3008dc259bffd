/*
 * he.h -- C ABI of the Hybrid-Engine experience-generation library (libhe.so)
 * for AMD MI355X (gfx950).
 *
 * The calls follow the pages' statement of the method:
 *  - "DeepSpeed-Chat: Easy, Fast and Affordable RLHF Training of ChatGPT-like
 *    Models at All Scales" (paper summary, page 1).  Section "The DeepSpeed
 *    Hybrid Engine: Architecture and Mode Switching": one model instance
 *    switches between inference and training layout.  Section "Inference
 *    Mode: Generation Phase Optimizations": inference kernels, a lightweight
 *    KV cache that appends the current step's keys and values.  Section "The
 *    Three-Step RLHF Training Pipeline in Algorithmic Detail": the generation
 *    phase produces 256 tokens for 256-token prompts; the reward model scores
 *    them.  Section "Training Mode: ZeRO and LoRA Optimizations": LoRA update
 *    W + B A.
 *  - "DeepSpeed-Chat selection guide" (page 2), section 3 (engine internals):
 *    generate() fuses the LoRA weights before generating and unfuses them
 *    after; the inference workspace (KV cache and intermediates) is released
 *    after generation and re-taken before the next one; the decode step can
 *    be replayed from a captured graph.  Section 4 (configuration fields):
 *    max_out_tokens, inference_tp_size, release_inference_cache,
 *    enable_cuda_graph.
 *
 * Mode switch in terms of these calls: eval() = he_fuse_lora + he_retake_cache;
 * generate = he_generate (or he_prefill + he_decode_step ...);
 * train() = he_unfuse_lora + he_release_cache.
 *
 * Conventions
 *  - Every pointer named d_* or held in a weight / LoRA table is device memory
 *    on the context's GPU.  Tables themselves (the structs and the arrays they
 *    point to) are host memory, read during the call only.
 *  - Element type of weights, LoRA factors, activations and the KV cache is the
 *    model's storage type (he_model_desc.dtype): IEEE float32 or bfloat16.
 *    Token ids are int32; logits and rewards are float32.
 *  - Matrices are row-major.  A Linear weight is [out, in].
 *  - All device work is enqueued on the stream given to he_create; calls
 *    return once the work is enqueued.  Argument and state errors are
 *    reported before anything is enqueued and leave the context unchanged.
 *  - A HIP failure (launch error, asynchronous fault surfaced by he_sync or
 *    a later call) returns HE_E_HIP and puts the context in a failed state;
 *    after that only he_unfuse_lora, he_release_cache and he_destroy run.
 *  - A context is used by one host thread at a time.  No C++ exception
 *    crosses this interface.  he_last_error() describes the last failure.
 */
#ifndef HE_H_
#define HE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct he_ctx he_ctx;
typedef int32_t he_status;

enum {
  HE_OK = 0,
  HE_E_ARG = -1,          /* bad argument (NULL pointer, size out of range, B > max_batch) */
  HE_E_STATE = -2,        /* call not allowed in the current state */
  HE_E_NOCACHE = -3,      /* needs the KV workspace: call he_retake_cache first */
  HE_E_RANGE = -4,        /* a position would pass max_seq or the position table */
  HE_E_OOM = -5,          /* device allocation failed */
  HE_E_HIP = -6,          /* HIP runtime error or device fault */
  HE_E_UNSUPPORTED = -7   /* shape or option this build does not implement */
};

enum { HE_DTYPE_F32 = 0, HE_DTYPE_BF16 = 1 };
enum { HE_NORM_PRE = 0, HE_NORM_POST = 1 };
enum { HE_HEAD_LM = 0, HE_HEAD_SCALAR = 1 };

/* he_model_desc.flags */
enum {
  HE_FLAG_VALIDATE_ONLY = 1   /* no GPU work at all: argument and state checks only
                                 (host-side tests); compute calls write nothing */
};

/*
 * Model description.  An OPT-style decoder (page 1, pipeline section: OPT
 * actors and an OPT-350M reward model; page 2, section 3: the inference
 * containers replace the layer, Linear, Embedding, LayerNorm and the OPT
 * positional embedding).
 *   n_layers, d_model, n_heads (d_model % n_heads == 0), d_ffn, vocab.
 *   max_pos:   learned positions; the table has max_pos + 2 rows and position
 *              t reads row t + 2.
 *   dtype:     HE_DTYPE_F32 or HE_DTYPE_BF16 (storage type of everything above).
 *   norm:      HE_NORM_PRE (LayerNorm before each block, final LayerNorm, tied
 *              LM head) or HE_NORM_POST (LayerNorm after each residual add, no
 *              final LayerNorm).
 *   head:      HE_HEAD_LM (logits = z E^T, greedy argmax) or HE_HEAD_SCALAR
 *              (reward = (h_last proj_out^T) . score_w).
 *   d_embed:   word-embedding width; equal to d_model, or a smaller width with
 *              proj_in / proj_out (reward model).  0 means d_model.
 *   ln_eps:    LayerNorm epsilon (OPT: 1e-5).
 *   tp_size:   inference tensor-parallel degree (page 2, section 4,
 *              inference_tp_size); only 1 is implemented (HE_E_UNSUPPORTED).
 *   use_graph: replay the decode step from a captured hipGraph (page 2,
 *              section 4, enable_cuda_graph).  The environment variable
 *              HE_NO_GRAPH=1 turns it off.  HE_DEBUG=1 (read at he_create) turns
 *              it off too and makes every call wait for the stream after each
 *              kernel launch and check for an error; the first failure is
 *              returned as HE_E_HIP with the kernel named in he_last_error.
 *   flags:     HE_FLAG_* bits.
 */
typedef struct he_model_desc {
  int32_t n_layers;
  int32_t d_model;
  int32_t n_heads;
  int32_t d_ffn;
  int32_t vocab;
  int32_t max_pos;
  int32_t dtype;
  int32_t norm;
  int32_t head;
  int32_t d_embed;
  float ln_eps;
  int32_t tp_size;
  int32_t use_graph;
  int32_t flags;
} he_model_desc;

/* One decoder layer's parameters (device pointers, storage type).
 *   ln1_g, ln1_b [d]      LayerNorm before attention (pre-LN) / after it (post-LN)
 *   w_qkv [3d, d]         rows 0..d-1 = W_q, d..2d-1 = W_k, 2d..3d-1 = W_v
 *   b_qkv [3d]
 *   w_out [d, d], b_out [d]
 *   ln2_g, ln2_b [d]      LayerNorm of the feed-forward block
 *   w_fc1 [F, d], b_fc1 [F], w_fc2 [d, F], b_fc2 [d]
 * The projection weights are written in place by he_fuse_lora/he_unfuse_lora. */
typedef struct he_layer_weights {
  const void* ln1_g;
  const void* ln1_b;
  void* w_qkv;
  const void* b_qkv;
  void* w_out;
  const void* b_out;
  const void* ln2_g;
  const void* ln2_b;
  void* w_fc1;
  const void* b_fc1;
  void* w_fc2;
  const void* b_fc2;
} he_layer_weights;

/* Whole-model parameters.  The library borrows every device pointer from
 * he_create until he_destroy; the caller keeps the memory alive and does not
 * write it meanwhile (the library itself writes the projections in place
 * during fuse/unfuse, with no second copy: one model instance).
 *   tok_emb [vocab, d_embed]; also the tied LM head
 *   pos_emb [max_pos + 2, d]
 *   lnf_g, lnf_b [d]        final LayerNorm (HE_NORM_PRE only, else NULL)
 *   proj_in [d, d_embed]    when d_embed != d_model, else NULL
 *   proj_out [d_embed, d]   when d_embed != d_model, else NULL
 *   score_w [d_embed]       HE_HEAD_SCALAR only, else NULL
 *   layers                  host array of n_layers entries */
typedef struct he_weight_table {
  const void* tok_emb;
  const void* pos_emb;
  const void* lnf_g;
  const void* lnf_b;
  const void* proj_in;
  const void* proj_out;
  const void* score_w;
  const he_layer_weights* layers;
} he_weight_table;

/* LoRA adapters (page 1, "Training Mode: ZeRO and LoRA Optimizations": W + B A,
 * B [d_out, r], A [r, d_in]).  The update applied is s * B A with
 * s = alpha / rank.  pairs is a host array of n_layers * HE_N_PROJ entries,
 * entry [layer * HE_N_PROJ + proj]; an entry with A == NULL and B == NULL
 * leaves that projection unadapted.  A and B are device memory in the storage
 * type, borrowed for the duration of the call. */
enum { HE_PROJ_Q = 0, HE_PROJ_K, HE_PROJ_V, HE_PROJ_OUT, HE_PROJ_FC1, HE_PROJ_FC2, HE_N_PROJ };

typedef struct he_lora_pair {
  const void* A;
  const void* B;
} he_lora_pair;

typedef struct he_lora_table {
  int32_t rank;             /* 1..64 */
  float alpha;
  const he_lora_pair* pairs;
} he_lora_table;

/* Create a context.  desc and weights are copied (the device memory they name
 * is borrowed).  hip_stream is a hipStream_t (NULL = the null stream).
 * Errors: HE_E_ARG (NULL or inconsistent desc, NULL weight pointers),
 * HE_E_UNSUPPORTED (tp_size != 1, head_dim not in {16, 32, 64, 128}, or a shape
 * the kernels do not tile), HE_E_HIP. */
he_status he_create(const he_model_desc* desc, const he_weight_table* weights,
                    void* hip_stream, he_ctx** out);

/* Destroy: waits for the context's stream, frees the workspace and the
 * context.  Does not touch the weights.  NULL is a no-op. */
he_status he_destroy(he_ctx* ctx);

/* Fold the adapters into the weights in place: W <- round(W + s B A), with s B A
 * accumulated in float32 in a fixed order (page 2, section 3: fuse before
 * generation).  HE_E_STATE if already fused.  HE_E_ARG on a bad table. */
he_status he_fuse_lora(he_ctx* ctx, const he_lora_table* lora);

/* Take the adapters out: W <- round(W - s B A), with the bitwise-same s B A as
 * the fuse.  The round trip returns each element within one bf16 spacing of
 * max(|W|, |W'|).  HE_E_STATE if not fused.  Allowed in the failed state. */
he_status he_unfuse_lora(he_ctx* ctx, const he_lora_table* lora);

/* Allocate the inference workspace: the KV cache [L][2][max_batch][H][max_seq][D]
 * in the storage type plus activation scratch (page 1, Optimization 2: the
 * cache is allocated once and reused by every step; page 2, section 3:
 * retake_inference_cache).  max_seq plays the role of max_out_tokens.
 * HE_E_STATE if a workspace is already held; HE_E_RANGE if max_seq exceeds
 * max_pos; HE_E_OOM if the allocation fails (nothing is kept). */
he_status he_retake_cache(he_ctx* ctx, int32_t max_batch, int32_t max_seq);

/* Free the workspace (page 2, section 3: release_workspace after generation).
 * Also drops the captured decode graph.  No-op if none is held.  Allowed in
 * the failed state. */
he_status he_release_cache(he_ctx* ctx);

/* Prompt pass of the generation phase.  d_ids [B, S_p] int32 (0 <= id < vocab).
 * Writes the KV cache at positions 0..S_p-1, d_next [B] int32 = greedy pick
 * after the last prompt token, and, when d_logits != NULL, d_logits [B, vocab]
 * float32 at that position.  Starts a new cache epoch (position S_p).
 * Errors: HE_E_NOCACHE, HE_E_ARG (B < 1, B > max_batch, S_p < 1, NULL),
 * HE_E_RANGE (S_p > max_seq), HE_E_UNSUPPORTED (scalar-head model). */
he_status he_prefill(he_ctx* ctx, const int32_t* d_ids, int32_t B, int32_t S_p,
                     int32_t* d_next, float* d_logits);

/* One decode step: feeds d_in [B] (the batch of the current epoch) at the
 * current position p, appends its keys and values to the cache, attends over
 * positions 0..p, writes d_next [B] (greedy pick) and optionally d_logits
 * [B, vocab]; the position advances to p + 1.
 * Errors: HE_E_NOCACHE, HE_E_STATE (no prefill in this cache epoch),
 * HE_E_RANGE (p == max_seq), HE_E_ARG (NULL). */
he_status he_decode_step(he_ctx* ctx, const int32_t* d_in, int32_t* d_next, float* d_logits);

/* Greedy generation of S_g tokens per row: the prompt pass gives token 0; steps
 * j = 1..S_g-1 feed token j-1 at position S_p+j-1.  The picks stay on the
 * device between steps.  d_out [B, S_g] int32.  Requires S_p + S_g - 1 <= max_seq.
 * Errors as he_prefill. */
he_status he_generate(he_ctx* ctx, const int32_t* d_prompt, int32_t B, int32_t S_p,
                      int32_t S_g, int32_t* d_out);

/* Pick rule of he_generate_ex.  The paper summary's pipeline section has the actor
 * generate (sample) answers, and the PPO step that follows scores each generated
 * token by its log-probability under the actor; the pages give no sampler.
 * temperature == 0: greedy (largest logit, lowest index on ties).
 * temperature  > 0: the next token is drawn from softmax(logits / temperature) by
 *   the Gumbel-max rule: argmax_n (logit_n / temperature + G_n), G_n = -log(-log U_n),
 *   U_n = (top 23 bits of word n mod 4 of Philox4x64-10 (Salmon et al., SC 2011)
 *   at counter (n div 4, batch row, position of the token, 0), key (seed, 0) + 1/2)
 *   / 2^23, exact in float32 and strictly inside (0, 1).  A pick is a function of (seed, row, position, logits) only: the same
 *   seed reproduces a generation exactly.
 * top_p in (0, 1) with temperature > 0: nucleus sampling (Holtzman et al., ICLR
 *   2020): the same rule restricted to the smallest set of most probable tokens
 *   whose probability under softmax(logits / temperature) reaches top_p, every
 *   token tied with its least probable member included; the threshold is found by
 *   fixed-order sums, so picks stay reproducible.  0 or >= 1 turns it off; it needs
 *   a vocabulary of at most 53248 tokens. */
typedef struct he_sampling {
  float temperature;
  uint64_t seed;
  float top_p;
} he_sampling;

/* he_generate with a pick rule and per-token log-probabilities.  smp == NULL is
 * greedy.  d_out [B, S_g] int32 as he_generate; when d_logprobs != NULL it
 * receives [B, S_g] float32: for each generated token t, log softmax(logits / T')_t
 * with T' = temperature (1 for greedy), the row's logsumexp combined over vocabulary
 * blocks in a fixed order.  Device memory, caller-owned; written by the end of the
 * call's stream work.
 * The log-probability is that of the untruncated distribution, also under top-p.
 * Errors as he_generate, plus HE_E_ARG for a temperature that is negative, not
 * finite, or so small that its reciprocal overflows, or a top_p that is negative
 * or NaN; HE_E_UNSUPPORTED for top-p over a vocabulary above 53248. */
he_status he_generate_ex(he_ctx* ctx, const int32_t* d_prompt, int32_t B, int32_t S_p,
                         int32_t S_g, const he_sampling* smp, int32_t* d_out, float* d_logprobs);

/* The pick rule of he_generate_ex applied to caller logits: d_logits [B, vocab]
 * float32 (device, row-major), row b drawn with batch row index b and token position
 * `position` in the generator's counter, exactly as the generation step draws token
 * `position` of row b.  d_tokens [B] int32 receives the picks; d_logprobs [B]
 * float32 (may be NULL) their log-probabilities.  Uses the workspace's scratch but
 * leaves the generation state alone.  Errors: HE_E_NOCACHE, HE_E_ARG (NULL buffer,
 * batch outside 1..max_batch, negative position, bad rule as he_generate_ex),
 * HE_E_UNSUPPORTED (not an LM-head model; top-p over a vocabulary above 53248). */
he_status he_sample(he_ctx* ctx, const float* d_logits, int32_t B, int32_t position,
                    const he_sampling* smp, int32_t* d_tokens, float* d_logprobs);

/* he_sample for callers that cannot allocate device memory (work under graph capture,
 * tight serving loops, harnesses that forbid allocation): the same rule, arguments,
 * outputs and errors, but it needs no workspace (no he_retake_cache, no HE_E_NOCACHE)
 * and allocates nothing.  Its per-block partials live in a static device array of
 * 1.25 MB (plus 256 bytes) that each GPU the library runs on holds until the process
 * ends; every call on one GPU uses that GPU's array, so calls that overlap on one GPU
 * (other streams, other contexts, other threads) race: order them on one stream.
 * Limits: B * ceil(vocab / 128) <= 65536 (B <= 128 at vocab <= 65536), else HE_E_ARG;
 * vocab <= 65536, else HE_E_UNSUPPORTED. */
he_status he_sample_static(he_ctx* ctx, const float* d_logits, int32_t B, int32_t position,
                           const he_sampling* smp, int32_t* d_tokens, float* d_logprobs);

/* Reward scoring (page 1, pipeline section: the reward model gives each response
 * a scalar score): full causal pass over d_ids [B, S] of a HE_HEAD_SCALAR model,
 * d_reward [B] float32 = y . score_w with y = h[S-1] proj_out^T (h[S-1] itself when
 * the model has no proj_out).  d_y, when not NULL, receives y as [B, d_embed] float32.
 * Both are caller-owned device memory, written by the end of the call's stream work.
 * Uses the workspace.
 * Errors: HE_E_NOCACHE, HE_E_ARG, HE_E_RANGE, HE_E_UNSUPPORTED (LM-head model). */
he_status he_score(he_ctx* ctx, const int32_t* d_ids, int32_t B, int32_t S, float* d_reward, float* d_y);

/* Teacher-forced scoring of finished experience (page 1, pipeline section: the PPO
 * step needs, for every answer token, its log-probability under the actor and under
 * the frozen reference model).  d_seq [B, S] int32 holds each row's prompt
 * (positions 0 .. S_p-1) followed by its answer; d_logprobs [B, S - S_p] float32
 * receives, for j = 0 .. S-S_p-1, log softmax(logits at position S_p-1+j)[seq[S_p+j]]:
 * the log-probability of answer token j given everything before it, at temperature
 * 1, the row's logsumexp merged in a fixed order.  One causal prompt pass over all S
 * positions (the KV cache is overwritten; a following he_decode_step needs a new
 * prefill), the final LayerNorm of the S - S_p scored positions, and the tied head in
 * chunks of at most 4096 rows of fp32 logits held in the workspace.  Device memory,
 * caller-owned, written by the end of the call's stream work; a target id outside
 * 0 .. vocab-1 yields NaN for that position.
 * Errors: HE_E_NOCACHE, HE_E_ARG (NULL buffer, batch outside 1..max_batch, S_p
 * outside 1..S-1), HE_E_RANGE (S > max_seq), HE_E_UNSUPPORTED (not an LM-head model). */
he_status he_logprobs(he_ctx* ctx, const int32_t* d_seq, int32_t B, int32_t S, int32_t S_p,
                      float* d_logprobs);

/* Weight-only FP8 decode (Chapter 11 "System Architecture & Infrastructure at
 * Scale", section "The Generation Bottleneck: Quantitative Analysis": 8-bit weights
 * halve the bytes a bandwidth-bound generation step streams).  enable != 0 makes an
 * OCP E4M3 copy of the q/k/v, out, fc1 and fc2 weights of every layer, per output
 * channel: scale_n = max_k |W[n,k]| / 448 (float32), code = E4M3(W[n,k] / scale_n)
 * rounded to nearest even, saturating at 448.  Decode steps then read those copies
 * (half the weight bytes), multiplying each output row by its scale; the prompt
 * pass, the LM head and reward scoring keep bf16.  The copy is library-owned
 * (about 1 byte per projection weight, kept across workspace release / retake)
 * and is remade after every he_fuse_lora / he_unfuse_lora; call again with
 * enable != 0 after changing the weights in place.  enable == 0 frees it.  Either
 * way a new prompt pass must precede the next decode step.
 * Errors: HE_E_UNSUPPORTED (fp32 or scalar-head model, d or d_ffn not a multiple of
 * 256), HE_E_OOM. */
he_status he_set_fp8_decode(he_ctx* ctx, int32_t enable);

/* The E4M3 codes of one FP8 projection copy in row-major order: proj 0 q/k/v
 * ([3d, d]), 1 out ([d, d]), 2 fc1 ([d_ffn, d]), 3 fc2 ([d, d_ffn]); d_codes receives
 * N x K bytes, d_scales N float32 (device, caller-owned, written by the end of the
 * call's stream work).  Errors: HE_E_STATE (FP8 decode off), HE_E_ARG. */
he_status he_fp8_export(he_ctx* ctx, int32_t layer, int32_t proj, uint8_t* d_codes, float* d_scales);

/* Wait for the context's stream; reports deferred device faults as HE_E_HIP. */
he_status he_sync(he_ctx* ctx);

/* Text of the last failure on this context ("" if none); valid until the next
 * call on the context.  he_status_str names a status code. */
const char* he_last_error(const he_ctx* ctx);
const char* he_status_str(he_status s);

/* ---- measurement ---------------------------------------------------------
 * Kernel classes for the per-kernel timer.  While a class is armed, every
 * launch of it made outside graph replay is bracketed by hipEvents on the
 * context's stream; he_kernel_stats synchronises and returns the launch count,
 * the summed device time and the summed algorithmic HBM bytes and flops of
 * those launches (the minimum the operation must move / compute, not counter
 * readings). */
enum {
  HE_K_LORA = 0,
  HE_K_EMBED_NORM,
  HE_K_GEMM_PREFILL,
  HE_K_ATTN_PREFILL,
  HE_K_GEMV_DECODE,
  HE_K_ATTN_DECODE,
  HE_K_LMHEAD,
  HE_K_SCORE,
  HE_K_VOCAB,
  HE_K_COUNT
};

typedef struct he_kernel_stat {
  int64_t launches;
  double total_ms;
  double bytes;
  double flops;
} he_kernel_stat;

/* Arm (enable != 0) or disarm the timer of one kernel class; arming clears its
 * statistics.  Armed timing forces the non-graph decode path. */
he_status he_kernel_timer(he_ctx* ctx, int32_t kernel_class, int32_t enable);
he_status he_kernel_stats(he_ctx* ctx, int32_t kernel_class, he_kernel_stat* out);

/* Build information: offload architecture and compile flags. */
const char* he_build_info(void);

/* Test hooks.  HE_DBG_FAIL_NEXT_ALLOC: the next he_retake_cache fails with
 * HE_E_OOM before allocating.  HE_DBG_FAIL_NEXT_STEP: the next he_decode_step
 * (or a step inside he_generate) fails with HE_E_HIP and the context enters
 * the failed state, as after a device fault. */
enum { HE_DBG_FAIL_NEXT_ALLOC = 1, HE_DBG_FAIL_NEXT_STEP = 2 };
he_status he_debug(he_ctx* ctx, int32_t what, int64_t value);

#ifdef __cplusplus
}
#endif

#endif /* HE_H_ */
