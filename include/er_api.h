/*
 * er_api.h -- C ABI of the self-speculative rollout step (MI355X / gfx950).
 *
 * One rollout step for the active batch: a drafter made by quantizing the
 * target's own weights (W4 group-128 asymmetric or W8 per-channel symmetric)
 * proposes gamma tokens per sequence while sharing the target's paged KV
 * cache; the target verifies all gamma+1 positions in one forward; a lossless
 * rejection sampler keeps a prefix, resamples the first rejection or adds a
 * bonus token, and the rejected KV tail is rolled back.  A roofline model of
 * the live batch turns speculation on or off and picks gamma from an EMA of
 * the acceptance rate.
 *
 * Sources (titles of the pages this follows; sections in quotes):
 *  - "EfficientRollout: system-aware self-speculative decoding for RL
 *    rollouts" (ai-feeds summary of arXiv 2606.18967): "关键模块" items 1-3
 *    (quantized self-drafter sharing the KV cache; roofline SD toggle;
 *    acceptance-aware draft length), "与现有工作流的接口" (inputs: the policy
 *    model and its quantized copy; W4A16), "局限" (per-GPU calibration).
 *  - "Accelerating RL Post-Training Rollouts via System-Integrated
 *    Speculative Decoding" (abstract): speculation must be lossless.
 *  - "TLT" reading notes, section 1 (parallel verification discards drafts
 *    after the first failure) and section 2 (elastic enable, per-batch-size
 *    parameters).
 *  - "History Tree Dynamic RL" (cann-recipes-train PR), section 2.2 (draft
 *    token count default 4; EMA coefficient 0.3; switch margin 1.02) and
 *    section 4 (speculative-decoding metrics).
 *
 * Conventions for every call:
 *  - Return 0 (ER_OK) or a negative ER_* code.  No C++ exception crosses the
 *    ABI.  er_last_error() holds a message owned by the context, valid until
 *    the next call on that context.
 *  - A context is single-threaded and bound to the HIP stream given at init.
 *    Every call that launches work is synchronous: it returns after the
 *    results it reports have been copied to host memory.
 *  - A failing step changes no sequence state (results are committed on the
 *    host after the device work succeeded).  ER_ENOMEM from er_kv_alloc or
 *    from a step's KV reservation is recoverable by freeing sequences.
 *  - Host pointers are caller-owned and only read/written during the call.
 *    Device pointers passed to er_rollout_init (weights, arena) are borrowed
 *    for the life of the context.
 */
#ifndef ER_API_H
#define ER_API_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define ER_OK        0
#define ER_EINVAL   -1   /* bad argument: null pointer, bad size, unknown sequence id */
#define ER_ENOMEM   -2   /* device arena or KV block pool exhausted */
#define ER_EDEVICE  -3   /* a HIP call failed (message in er_last_error) */
#define ER_ESTATE   -4   /* sequence finished / not prefilled / wrong order of calls */

/* ---- enums ---------------------------------------------------------------- */
#define ER_F32  0        /* target weights, KV and linear inputs in fp32 */
#define ER_BF16 1        /* target weights, KV and linear inputs in bf16 */

#define ER_W8_PERCH_SYM  0   /* int8 codes, one fp32 scale per output row */
#define ER_W4_G128_ASYM  1   /* 4-bit codes, bf16 scale + u8 zero per row and 128 inputs */

#define ER_POLICY_AUTO      0   /* roofline toggle + adaptive gamma; while it stays
                                   autoregressive where alpha_init would make speculation
                                   pay, a speculative probe step refreshes the EMA (after
                                   32 steps, the gap doubling to at most 1024; see
                                   er_controller_plan) */
#define ER_POLICY_FORCE_SD  1   /* always speculate (gamma adaptive unless pinned) */
#define ER_POLICY_FORCE_AR  2   /* never speculate */
#define ER_POLICY_TIMING    3   /* measured-timing guard (er_guard_* below) chooses
                                   between AR and speculation per batch bucket;
                                   gamma as under ER_POLICY_AUTO when it speculates */
#define ER_POLICY_HISTORY   4   /* drafts copied from earlier rollouts (er_set_history):
                                   a history step while the attached cache holds a
                                   record and the batch is at most its max_batch,
                                   else AR */

#define ER_MODE_AR 0
#define ER_MODE_SD 1
#define ER_MODE_HISTORY 3  /* a step with drafts copied from earlier rollouts */

typedef struct er_ctx er_ctx;

/* Decoder shape.  Pre-norm layers: RMSNorm, RoPE (rotate-half), GQA with
 * n_q_heads % n_kv_heads == 0, SwiGLU FFN; untied lm_head; no biases. */
typedef struct er_model_desc {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  int32_t dtype;            /* ER_F32 or ER_BF16 */
  float rms_eps;
  float rope_theta;
} er_model_desc;

/* Self-drafter: the target's linears (q/k/v/o, gate/up/down, lm_head)
 * quantized; embedding and norm gains shared unquantized.  W4 needs every
 * input dimension K to be a multiple of 128 and a bf16 model. */
typedef struct er_draft_desc {
  int32_t quant;            /* ER_W8_PERCH_SYM or ER_W4_G128_ASYM */
  int32_t group_size;       /* 128 (W4 only) */
  int32_t quant_lm_head;    /* 1: lm_head quantized too (default); 0: drafter uses the bf16 lm_head */
} er_draft_desc;

typedef struct er_rollout_desc {
  uint64_t seed;            /* Philox key */
  float temperature;        /* 0 = greedy */
  float top_p;              /* >= 1 disables nucleus filtering */
  int32_t gamma_init;       /* initial draft length (4) */
  int32_t gamma_min;        /* adaptive range, 1..gamma_max */
  int32_t gamma_max;        /* <= 16 */
  float ema_beta;           /* weight of the newest acceptance sample (0.3) */
  float switch_margin;      /* a new (mode, gamma) must score this factor better (1.02) */
  float alpha_init;         /* acceptance prior before the first speculative step */
  int32_t policy;           /* ER_POLICY_* */
  int32_t kv_block;         /* tokens per KV block; must be 16 */
  int32_t max_seqs;         /* sequences alive at once */
  int32_t max_batch;        /* sequences per step (<= max_seqs); (n_q_heads/n_kv_heads)*(gamma_max+1) <= 64 */
  int32_t max_ctx;          /* max tokens per sequence (prompt + generated + gamma_max + 1) */
  int32_t prefill_chunk;    /* max prompt tokens per prefill forward */
  int64_t kv_pool_blocks;   /* 0: every block the arena can hold after the other buffers */
  double hbm_bytes_per_s;   /* roofline constants; <= 0: measured at init */
  double flops_per_s;       /* <= 0: the rate a target forward over 512 rows reaches, measured at
                               init (2.5e15 if that forward stays bound by the weight stream) */
  double t_fwd_s;           /* fixed time per forward (launch overhead); < 0: measured at init */
} er_rollout_desc;

/* Device pointers to the target's weights, row-major, element type
 * model.dtype.  Borrowed: they must stay valid and unchanged until
 * er_update_weights or er_destroy.  Per-layer entries are host arrays of
 * n_layers device pointers. */
typedef struct er_weights {
  const void *embed;        /* [vocab, d_model] */
  const void *final_norm;   /* [d_model] */
  const void *lm_head;      /* [vocab, d_model] */
  const void *const *attn_norm;  /* [d_model] */
  const void *const *wqkv;       /* [(n_q_heads + 2 n_kv_heads) head_dim, d_model]: q rows, k rows, v rows */
  const void *const *wo;         /* [d_model, n_q_heads head_dim] */
  const void *const *mlp_norm;   /* [d_model] */
  const void *const *wgate_up;   /* [2 ffn, d_model]: gate rows, then up rows */
  const void *const *wdown;      /* [d_model, ffn] */
} er_weights;

typedef struct er_step_info {
  int32_t mode;             /* ER_MODE_SD or ER_MODE_AR */
  int32_t gamma;            /* draft length used (0 for AR) */
  int32_t batch;            /* sequences in the step */
  int32_t accepted;         /* drafts accepted, summed over the batch */
  int32_t emitted;          /* tokens emitted before stop truncation */
  int32_t kept;             /* tokens kept after stop truncation */
  int32_t finished;         /* sequences that reached their stop length in this step */
  float alpha_step;         /* trials-based acceptance of this step */
  float alpha_ema;          /* after the update */
  float ms_draft, ms_verify, ms_sample, ms_total;   /* device time per phase (timed steps only) */
} er_step_info;

/* Counters named after the speculative-decoding metrics of the History Tree
 * Dynamic RL page (section 4), plus the controller state. */
typedef struct er_stats {
  int64_t predict_times;      /* speculative attempts: SD steps x sequences */
  int64_t effective_times;    /* attempts that accepted >= 1 draft */
  int64_t total_right_length; /* accepted drafts, summed */
  double effective_length;    /* total_right_length / effective_times */
  double effective_percent;   /* effective_times / predict_times */
  int64_t sd_steps, ar_steps;
  int64_t drafted, accepted, emitted, bonus;
  int64_t tokens_kept;        /* generated tokens after stop truncation (prefill's first tokens included) */
  double alpha_ema;
  int32_t gamma;              /* current choice: 0 = AR */
  int32_t mode;
  double ms_draft, ms_verify, ms_sample, ms_ar, ms_prefill;   /* accumulated, timed steps only */
  int64_t history_steps;      /* steps with drafts copied from earlier rollouts */
  int64_t history_drafted, history_accepted;
} er_stats;

/* Create a context.  Carves dev_arena (device memory the caller owns, e.g. a
 * torch uint8 tensor) into the drafter pack, the KV block pool and step
 * workspaces, then quantizes the target into the drafter (EfficientRollout
 * "关键模块" item 1).  hip_stream: a hipStream_t, or NULL for the null stream.
 * Returns ER_ENOMEM if the arena is too small (the message states the bytes
 * needed), ER_EINVAL for an inconsistent description. */
int er_rollout_init(const er_model_desc *model, const er_weights *w, const er_draft_desc *draft,
                    const er_rollout_desc *rollout, void *dev_arena, size_t arena_bytes,
                    void *hip_stream, er_ctx **out);

/* Bytes of arena er_rollout_init needs for these descriptions (kv_pool_blocks
 * blocks of KV; 0 counts none).  Pure host computation. */
int er_arena_bytes(const er_model_desc *model, const er_draft_desc *draft,
                   const er_rollout_desc *rollout, int64_t kv_pool_blocks, size_t *bytes_out);

/* Re-point the context at (possibly new) target weights and re-quantize the
 * drafter; call after every policy update so the drafter tracks the policy
 * (EfficientRollout "关键模块" item 1). */
int er_update_weights(er_ctx *ctx, const er_weights *w);

/* Register n new sequences.  prompt_lens[i] >= 1 prompt tokens;
 * max_new[i] >= 1 generated tokens after which sequence i stops (the token
 * drawn by er_prefill counts); share_group[i] >= 0 makes sequences with equal
 * groups share their prompt's full KV blocks (their prompts must be equal),
 * -1 = private; share_group may be NULL.  Writes the new sequence ids, which
 * are also the Philox sequence words: ids are assigned 0, 1, 2, ... in call
 * order over the context's life.  ER_ENOMEM if max_seqs would be exceeded or
 * the prompt blocks do not fit. */
int er_kv_alloc(er_ctx *ctx, int n, const int32_t *prompt_lens, const int32_t *max_new,
                const int32_t *share_group, int32_t *seq_ids_out);

/* Fork a running sequence into n children that continue from its state (the
 * SRT review, section "三、技术架构": rollouts of one prompt form a tree whose
 * nodes share the KV of their common prefix, with copy-on-write at the fork
 * point).  Each child shares the parent's full committed KV blocks
 * (reference-counted; committed positions are never rewritten) and gets a
 * private copy of the parent's partial last block; it inherits the pending
 * token, the position and the generated count, and gets a new sequence id,
 * which is also its Philox sequence word, so its draws are its own.
 * max_new[i] is child i's total generated-token cap (it must exceed the
 * parent's generated count).  The parent must be prefilled and not finished.
 * ER_ENOMEM if max_seqs would be exceeded or no block is free for a copy; on
 * any error nothing changes.  Writes child_ids_out[n]. */
int er_kv_fork(er_ctx *ctx, int32_t parent, int n, const int32_t *max_new, int32_t *child_ids_out);

/* Run the target over each sequence's prompt (tokens of sequence i are
 * tokens[offsets[i] .. offsets[i+1])) and draw its first generated token as
 * an autoregressive sample at position prompt_len.  first_tok_out[n]. */
int er_prefill(er_ctx *ctx, int n, const int32_t *seq_ids, const int32_t *tokens,
               const int64_t *offsets, int32_t *first_tok_out);

/* One speculative step for the given active sequences with the current gamma
 * (pinned by er_set_gamma, else the controller's).  tokens_out[n * (gamma_max+1)]
 * receives sequence i's emitted tokens at [i*(gamma_max+1), ...), n_emitted_out[i]
 * of them (after stop truncation).  info_out may be NULL. */
int er_spec_step(er_ctx *ctx, int n, const int32_t *seq_ids, int32_t *tokens_out,
                 int32_t *n_emitted_out, er_step_info *info_out);

/* One autoregressive step (target forward at M = n, one sample each). */
int er_ar_step(er_ctx *ctx, int n, const int32_t *seq_ids, int32_t *tokens_out,
               er_step_info *info_out);

/* Controller-driven step: the roofline toggle and the gamma rule choose
 * between er_ar_step and er_spec_step for this batch.  Output layout as
 * er_spec_step. */
int er_step(er_ctx *ctx, int n, const int32_t *seq_ids, int32_t *tokens_out,
            int32_t *n_emitted_out, er_step_info *info_out);

/* Run every given sequence to its stop length with er_step, dropping
 * finished sequences from the batch as they finish (the shrinking batch).
 * out_tokens[i * max_new_cap ...] receives the tokens this call generates for
 * sequence i (the first token, returned by er_prefill, is not repeated),
 * out_len[i] their count.  Sequences must be prefilled; n <= max_batch;
 * max_new_cap >= every max_new.  stats_out (nullable) gets er_get_stats. */
int er_rollout(er_ctx *ctx, int n, const int32_t *seq_ids, int32_t max_new_cap,
               int32_t *out_tokens, int32_t *out_len, er_stats *stats_out);

/* Pin gamma to 1..gamma_max, or 0 to let the controller adapt it; anything
 * else is ER_EINVAL. */
int er_set_gamma(er_ctx *ctx, int gamma);

/* Change the policy (ER_POLICY_*). */
int er_set_policy(er_ctx *ctx, int policy);

/* Release sequences and their KV blocks (shared blocks when their last user goes). */
int er_kv_free(er_ctx *ctx, int n, const int32_t *seq_ids);

/* Sequence state: generated count, committed context length, finished flag. */
int er_seq_info(er_ctx *ctx, int32_t seq_id, int32_t *generated, int32_t *context_len, int32_t *finished);

int er_get_stats(er_ctx *ctx, er_stats *out);
/* Clear the counters and restart the controller: acceptance EMA back to
 * alpha_init, no current choice, the timing guard's state cleared (its
 * parameters kept). */
int er_reset_stats(er_ctx *ctx);

/* Record device time per phase for every `period`-th step and the first
 * `first_n` steps (0, 0 = never, the default). */
int er_set_timing(er_ctx *ctx, int period, int first_n);

/* bf16 models run a fused forward by default: RMSNorm formed on the input
 * load of the following projection, RoPE and the KV append in the QKV
 * projection's epilogue, SwiGLU in the gate/up projection's epilogue, the
 * residual add in the output projections' epilogues.  on = 0 selects the
 * unfused sequence of kernels (same arithmetic, separate passes); fp32 models
 * always run unfused.  Takes effect at the next forward. */
int er_set_fused(er_ctx *ctx, int on);

/* Persistent decode forward (bf16 models): a forward of at most 16 rows
 * (decode and drafting at batch <= 16, verify at batch * (gamma + 1) <= 16)
 * runs the embedding and every decoder layer as one cooperative launch with
 * grid barriers between the projection and attention phases, instead of ~6
 * launches per layer; the final norm, lm_head and sampler are unchanged.  Same
 * arithmetic per element (fp32 accumulation, bf16 stores at the same points);
 * K-split sums are added in a fixed order.  Off by default (on MI355X the
 * kernel sequence is faster at every measured batch); available where the
 * device can keep one work-group per compute unit resident.  ER_ESTATE when
 * asked to switch it on where it cannot run.  A grid-barrier wait that times out fails
 * the step with ER_EDEVICE and switches the path off. */
int er_set_persistent(er_ctx *ctx, int on);
int er_get_persistent(const er_ctx *ctx, int *on);
/* Polls a grid-barrier wait of the persistent decode forward makes before it
 * gives up (default 2^21, a few seconds).  A tiny value forces the time-out
 * path (every work-group still leaves the kernel), for testing the recovery:
 * the step fails with ER_EDEVICE, no sequence state changes, and later steps
 * run the kernel sequence.  ER_EINVAL for polls < 1. */
int er_set_decode_spin_limit(er_ctx *ctx, int64_t polls);
/* Phase timing of the persistent decode forward, for profiling: while on,
 * each launch records the 100 MHz clock at every grid barrier (one device
 * buffer, allocated here, freed by on = 0 or er_destroy).
 * er_get_decode_trace reports the last traced forward: for phase k (the
 * embedding, then per layer QKV, attention, [merge], output, gate/up, down)
 * work_us[k] = time from the first release of the previous barrier to the
 * last arrival at this one, release_us[k] = time from that arrival to the last
 * release; n_out = phases (min(max, phases) written).  ER_ESTATE if nothing
 * was traced. */
int er_set_decode_trace(er_ctx *ctx, int on);
int er_get_decode_trace(er_ctx *ctx, double *work_us, double *release_us, int max, int *n_out);

/* Library GEMMs (bf16 models): the target's projections run as hipBLASLt
 * bf16 GEMMs with fp32 accumulation, their fused work around them as small
 * kernels of this library (x' = RMSNorm(h) g formed once, RoPE and the KV
 * append, SwiGLU, the residual added by the GEMM itself and the next norm's
 * sums of squares), from a row count that depends on the shape.  min_rows =
 * -1 (the default): each shape from the rows where the library's GEMM was
 * measured faster on MI355X (output width >= 16384: 16 rows; >= 65536: 48;
 * >= 4096: 80; narrower: 17; K >= 8192: 1024); > 0: every shape from that
 * many rows (K >= 8192 still from 1024); 0: never.  Steps recorded into
 * graphs use this library's kernels only.  The first step with a new shape
 * of up to 512 rows times a few of the library's algorithms for it and keeps
 * the fastest (that step waits for the stream once per shape and projection),
 * so runs may pick different algorithms.  Same arithmetic per element up to
 * the order of the fp32 sums.  ER_EINVAL for min_rows < -1; ER_ESTATE for
 * min_rows != 0 where no library GEMM is available (fp32 models). */
int er_set_library_gemm(er_ctx *ctx, int min_rows);

/* ---- bucketed graph capture ------------------------------------------------
 * TLT notes, section 3, Design A, A3: a range of batch sizes shares one set
 * of recorded graphs, and the drafter's graphs are recorded apart from the
 * target's.  With max_batch > 0, a step over n <= max_batch sequences runs as
 * nb sequences, nb = n for n <= 16, else the next power of two >= n, and
 * replays up to two graphs: AR steps one (target forward and draw);
 * speculative steps the drafter's (gamma forwards and draws) and the
 * target's (verify forward and lossless decision); history steps only that
 * verify graph, shared with the self-drafted steps.  Conditions: gamma + 1 <=
 * 16, nb <= max_batch of er_rollout_init, nb * (gamma + 1) rows within the
 * activation buffers, the attention partials within their area; other steps
 * run eagerly, as do steps with the kernel profile or the persistent forward
 * on.  A graph is recorded at the first step of its key (kind, nb, gamma,
 * capacity) and replayed after; capacity = the smallest power-of-two number
 * of 16-token blocks >= 16 that holds every sequence's context plus this
 * step's positions, so a key is recorded again only when the longest context
 * crosses a power of two.  The padding sequences n .. nb-1 decode token 0 at
 * positions 0 .. gamma of one reserved KV block (taken from the pool while
 * graphs are on) and are dropped; attention gives every sequence the same
 * number of work units (units past a sequence's end read nothing).  Tokens,
 * acceptances and sequence state follow the same kernels and per-row
 * arithmetic as the eager step; the attention split may differ, which changes
 * rounding only.  Timed steps time each graph as a whole (the split between
 * forward and sampling is folded into ms_verify, ms_sample = 0).  At most 64
 * graphs are kept (least recently replayed evicted); er_update_weights,
 * er_set_fused and max_batch = 0 drop them (0 also returns the reserved
 * block).  Default 0 (off).  ER_ENOMEM when no KV block is free for the
 * padding rows. */
int er_set_graphs(er_ctx *ctx, int max_batch);
typedef struct er_graph_stats {
  int32_t max_batch;  /* er_set_graphs value (0: off) */
  int32_t cached;     /* graphs held */
  int64_t captures;   /* graphs recorded */
  int64_t replays;    /* graph launches */
  int64_t evictions;  /* graphs dropped to stay within 64 */
} er_graph_stats;
int er_get_graph_stats(const er_ctx *ctx, er_graph_stats *out);

/* ---- model-free history drafter --------------------------------------------
 * History Tree Dynamic RL page, section 1 (drafts taken from the responses of
 * earlier rollouts, high-reward pieces first, for later rollouts of the same
 * prompt) and section 3.3 (a fixed-prefix history cache per prompt plus a
 * global fallback; candidates at a fixed prefix length; reward-first
 * updates); section 2.2 (4 draft tokens, at most 64 requests by default).
 * The cache is a host object independent of any context.  A record is one
 * earlier rollout (prompt, response, reward); position i of its response is
 * keyed by the prefix_len tokens before it in prompt + response and offers the
 * record's tokens from i on.  Each prompt has its own map and one global map
 * holds every prompt's keys; a key keeps the candidate of the highest reward,
 * among equal rewards the one recorded last.  A sequence's draft: the key of
 * its last prefix_len tokens (prompt + generated) in its prompt's map, else in
 * the global map, and the first gamma tokens of that candidate. */
typedef struct er_history er_history;
/* prefix_len >= 1, else ER_EINVAL. */
int er_history_create(int prefix_len, er_history **out);
int er_history_destroy(er_history *h);
/* Record one rollout (tokens copied).  ER_EINVAL for negative lengths, null
 * arrays with positive lengths, or a NaN reward. */
int er_history_add(er_history *h, int prompt_len, const int32_t *prompt, int resp_len, const int32_t *resp,
                   float reward);
/* The draft for a sequence with this prompt and these tokens so far (ctx =
 * prompt + generated): up to gamma tokens into out, their count into *n_out
 * (0 when the cache has no candidate).  Pure host computation. */
int er_history_propose(const er_history *h, int prompt_len, const int32_t *prompt, int ctx_len,
                       const int32_t *ctx, int gamma, int32_t *out, int32_t *n_out);
int er_history_records(const er_history *h, int64_t *n);
/* Attach a cache to a context (borrowed: it must outlive its use; NULL
 * detaches): history steps draft gamma (1..gamma_max) tokens per sequence,
 * and ER_POLICY_HISTORY takes them for batches of at most max_batch. */
int er_set_history(er_ctx *ctx, er_history *h, int gamma, int max_batch);
/* One step with drafts from the attached cache: each sequence's gamma drafts
 * (where the cache offers fewer, the rest are the sequence's pending token;
 * any fixed token is a valid proposal), one target forward over the gamma + 1
 * positions, and the lossless decision with the point mass on each draft as
 * the proposal: draft i is accepted with probability p_i(draft), a rejection
 * is redrawn from p_i without the draft, and full acceptance adds a bonus
 * token.  Outputs as er_spec_step; info->mode = ER_MODE_HISTORY.  ER_ESTATE
 * without an attached cache. */
int er_history_step(er_ctx *ctx, int n, const int32_t *seq_ids, int32_t *tokens_out, int32_t *n_emitted_out,
                    er_step_info *info);

/* Free KV blocks in the pool. */
int er_kv_free_blocks(er_ctx *ctx, int64_t *free_blocks, int64_t *total_blocks);

/* ---- per-kernel timing ---------------------------------------------------
 * When on, every linear-layer and attention launch of the steps is bracketed
 * with HIP events on the context's stream; totals are kept per kernel name
 * (the name the profiler shows, e.g. "er::k_linear_mfma<3, 16, 2>") with the
 * algorithmic bytes (weights incl. scales/zeros + activations in + results
 * out; attention: K/V of every key read + q + out, a shared prompt block that
 * several members of a group read in one launch counted once) and flops of
 * each launch (every member's keys). */
typedef struct er_kernel_stat {
  char name[64];
  int64_t launches;
  double ms;        /* summed device time */
  double bytes;     /* summed algorithmic bytes */
  double flops;     /* summed algorithmic flops */
} er_kernel_stat;
/* on: ER_KPROF_OFF, ER_KPROF_ALL (every linear-layer and attention launch) or
 * ER_KPROF_ATTENTION (the attention launches only: two event records per
 * layer instead of per launch, for timing that kernel inside a timed run);
 * other values give ER_EINVAL. */
#define ER_KPROF_OFF 0
#define ER_KPROF_ALL 1
#define ER_KPROF_ATTENTION 2
int er_set_kernel_profile(er_ctx *ctx, int on);
/* Copies min(max, count) entries; *n_out = count. */
int er_get_kernel_profile(er_ctx *ctx, er_kernel_stat *out, int max, int *n_out);
int er_reset_kernel_profile(er_ctx *ctx);

/* ---- diagnostics: the last step's logits and drafts, for checking ------- */
/* which = 0: drafter logits of batch slot `slot` ([gamma, vocab] fp32);
 * which = 1: target logits ([gamma+1, vocab] after a speculative step,
 * [1, vocab] after an autoregressive step or prefill).  rows_out gets the row
 * count; host_out must hold rows * vocab floats (pass NULL to query rows). */
int er_debug_logits(er_ctx *ctx, int which, int slot, float *host_out, int32_t *rows_out);
/* Drafts of the last speculative step, [batch, gamma] int32. */
int er_debug_drafts(er_ctx *ctx, int32_t *host_out);

/* Pure host functions of the controller (no device work), exposed so that a
 * caller running its own loop gets the same decisions:
 * er_controller_choose returns in *gamma_out the argmax over {0 (AR)} U
 * [gamma_min, gamma_max] of B * E[n](alpha, gamma) / T(B, C, gamma), keeping
 * `current` unless the best beats it by `margin`. */
typedef struct er_cost_model {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  double w_bytes, q_bytes, kv_bytes_el;
  double hbm_bytes_per_s, flops_per_s, t_fwd_s;
  /* time per row beyond the first that drafter / target forwards take beyond
   * the roofline (0 unless measured at init, see er_controller_times) */
  double t_row_draft_s, t_row_target_s;
} er_cost_model;
int er_controller_choose(const er_cost_model *m, int batch, double mean_ctx, double alpha,
                         int gamma_min, int gamma_max, int current, double margin, int *gamma_out);
double er_expected_tokens(double alpha, int gamma);
/* The cost model a context's controller uses (roofline constants as given or
 * as calibrated at init). */
int er_get_cost_model(const er_ctx *ctx, er_cost_model *out);

/* Modelled step times of the controller (EfficientRollout "关键模块" item 2:
 * decode latency from a roofline, per-GPU constants): *t_ar = T(AR step),
 * *t_sd = gamma T(draft forward) + T(verify forward), each forward
 * T = t_fwd + (rows - 1) t_row + max(bytes / hbm_bytes_per_s, flops / flops_per_s)
 * (rows = B for AR and a draft forward, B (g+1) for the verify; t_row =
 * t_row_draft_s for drafter forwards, t_row_target_s for the target's) with
 *   AR:     bytes = wb P + B C kvb + B kvb + 4 B V,   flops = 2 P B + 4 B C hq hd L
 *   draft:  bytes = bq P + B C kvb + B kvb + 4 B V,   flops = 2 P B + 4 B C hq hd L
 *   verify: bytes = wb P + B C kvb + B (g+1) kvb + 4 B (g+1) V,
 *           flops = 2 P B (g+1) + 4 B (g+1) C hq hd L
 * (P = streamed linear parameters incl. lm_head, wb / bq = target / drafter
 * bytes per parameter, kvb = KV bytes per token over all layers, C = mean
 * committed context).  Either output may be NULL.  ER_EINVAL on batch < 1,
 * gamma < 1 or non-positive rates. */
int er_controller_times(const er_cost_model *m, int batch, double mean_ctx, int gamma, double *t_ar,
                        double *t_sd);

/* State of the roofline policy between steps: the last recorded choice
 * (0 = AR, -1 = none yet), consecutive AR choices since the last probe or
 * speculative choice, and the current probe gap (0 = not started). */
typedef struct er_plan_state {
  int32_t choice, ar_streak, probe_every;
} er_plan_state;
/* One step of the policy a context runs under ER_POLICY_AUTO / FORCE_SD /
 * FORCE_AR, as a pure host function over caller-held state (EfficientRollout
 * "关键模块" items 2-3; History Tree Dynamic RL section 2.2 margin).
 * FORCE_AR: 0.  FORCE_SD: the argmax over [gamma_lo, gamma_hi] with the
 * current choice kept unless beaten by `margin`.  AUTO: the same over
 * {0 (AR)} U [gamma_lo, gamma_hi]; while the choice stays AR where alpha_init
 * would make speculation pay, every probe_every-th consecutive AR choice
 * returns the speculative argmax at alpha_ema instead (a probe that refreshes
 * the acceptance estimate; the recorded choice stays AR), the gap starting at
 * 32 and doubling up to 1024 after each probe, reset by a speculative choice.
 * The pages leave the refresh of the estimate while speculation is off
 * unstated; this schedule is the library's reading.  ER_EINVAL on a null
 * pointer, batch < 1, a bad range or another policy. */
int er_controller_plan(const er_cost_model *m, er_plan_state *st, int policy, int batch, double mean_ctx,
                       double alpha_ema, double alpha_init, int gamma_lo, int gamma_hi, double margin,
                       int *gamma_out);
/* The policy state of a context (as er_controller_plan would receive it for
 * the next step). */
int er_get_plan_state(const er_ctx *ctx, er_plan_state *out);

/* Measured-timing guard of the SD toggle (the timing_guard policy of the
 * History Tree Dynamic RL page, section 2.2 parameters and section 3.3 logic,
 * with autoregressive decoding as the default branch and speculation as the
 * alternative).  Per batch bucket (bucket = ceil(log2(batch)): 1, 2, 3-4, 5-8,
 * ...) it keeps an EMA of measured tokens/ms for each branch.
 *   choose: batch > max_sd_batch -> AR.  A probe in progress -> SD.  Fewer
 *   than compare_after AR steps observed in the bucket, or the bucket cooling
 *   down -> AR.  With a speculative score: SD iff it exceeds margin x the AR
 *   score.  Without one: start a probe of probe_steps SD steps if batch <=
 *   probe_max_batch, else AR.  Every call advances the step counter.
 *   observe: a step's tokens / ms updates its branch's EMA (weight ema_alpha
 *   on the new sample; the first sample sets it).  A speculative step below
 *   bad_ratio x the AR score is bad: it ends the probe, clears the speculative
 *   score and cools the bucket down for cooldown steps, a length that grows by
 *   cooldown_growth (up to cooldown_max) with each consecutive bad probe and
 *   is reset by a probe that completes.
 * The state is caller-allocated plain data; a context with ER_POLICY_TIMING
 * holds its own, fed with the wall time of each step (plan to synchronized
 * end). */
#define ER_GUARD_BUCKETS 16
typedef struct er_guard_params {
  int32_t max_sd_batch;      /* 8 */
  int32_t probe_max_batch;   /* 2 */
  int32_t compare_after;     /* 64 */
  int32_t probe_steps;       /* 8 */
  double ema_alpha;          /* 0.3 */
  double margin;             /* 1.02 */
  int64_t cooldown;          /* 8192 */
  int64_t cooldown_max;      /* 65536 */
  double cooldown_growth;    /* 4.0 */
  double bad_ratio;          /* 0.98 */
} er_guard_params;
typedef struct er_guard_state {
  er_guard_params p;
  int64_t step;                                   /* choose calls so far */
  double ema_ar[ER_GUARD_BUCKETS], ema_sd[ER_GUARD_BUCKETS];   /* tokens/ms, < 0: none */
  int64_t n_ar[ER_GUARD_BUCKETS];                 /* AR steps observed */
  int32_t probe_left[ER_GUARD_BUCKETS];
  int64_t cool_until[ER_GUARD_BUCKETS];           /* AR while step < cool_until */
  int64_t cool_len[ER_GUARD_BUCKETS];             /* next cooldown length */
} er_guard_state;
/* Defaults above. */
void er_guard_default_params(er_guard_params *p);
/* ER_EINVAL on bad parameters (max_sd_batch outside [1, 2^15], negative
 * counts, ema_alpha outside (0, 1], margin or ratios <= 0). */
int er_guard_init(er_guard_state *g, const er_guard_params *p);
/* 1: speculate, 0: autoregressive; -1 on a null state or batch < 1. */
int er_guard_choose(er_guard_state *g, int batch);
/* branch: 1 speculative, 0 autoregressive; ER_EINVAL on ms <= 0, tokens < 0. */
int er_guard_observe(er_guard_state *g, int batch, int branch, double tokens, double ms);
/* The guard state of a context (ER_ESTATE unless its policy is ER_POLICY_TIMING). */
int er_get_guard(const er_ctx *ctx, er_guard_state *out);

const char *er_last_error(const er_ctx *ctx);
void er_destroy(er_ctx *ctx);

#ifdef __cplusplus
}
#endif
#endif /* ER_API_H */
