/*
 * er_ops.h -- operation-level C ABI: the individual gfx950 kernels of the
 * self-speculative step, on caller-provided device buffers.  The rollout
 * API (er_api.h) composes the same kernels; these entry points let a caller
 * (and the parity tests) run one operation on inputs of its choice.
 *
 * Conventions: every pointer named d_* is device memory the caller owns;
 * `stream` is a hipStream_t (NULL = null stream).  Calls enqueue work and
 * return without synchronizing, except where stated.  Return 0 or a negative
 * ER_* code (er_api.h); a shape the kernel does not support is ER_EINVAL.
 * Workspace the kernels need (split-K partials) is allocated once per
 * process on first use and kept.
 */
#ifndef ER_OPS_H
#define ER_OPS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight formats of er_op_linear. */
#define ER_FMT_F32  0   /* fp32 [N, K] */
#define ER_FMT_BF16 1   /* bf16 [N, K] */
#define ER_FMT_W8   2   /* int8 codes [N, K] + fp32 scale [N] */
#define ER_FMT_W4   3   /* 4-bit codes [N, K/2] in kernel nibble order + bf16 scale [N, K/128] + u8 zero [N, K/128] */

/* Drafter quantization of one weight matrix W [N, K] (EfficientRollout,
 * "关键模块" item 1; W4A16 in "与现有工作流的接口").
 * W8: d_codes int8 [N, K], d_scale fp32 [N]: s = max|w|/127 rounded up to
 *     fp32, q = clamp(rint(w/s), -127, 127); d_zero unused.  w_dtype ER_F32 or ER_BF16.
 * W4: d_codes uint8 [N, K/2], canonical order (low nibble = even k),
 *     d_scale bf16 [N, K/128], d_zero u8 [N, K/128]: per 128-group lo =
 *     min(min w, 0), hi = max(max w, 0), s = (hi-lo)/15 rounded up to bf16,
 *     z = clamp(rint(-lo/s), 0, 15), q = clamp(rint(w/s) + z, 0, 15).  bf16 W only, K % 128 == 0. */
int er_op_quantize(int quant, int w_dtype, const void *d_w, int N, int K, void *d_codes, void *d_scale,
                   void *d_zero, void *stream);

/* Canonical W4 (row-major [N][K/2] bytes, code k at bits 4k of its word) ->
 * the layout er_op_linear's ER_FMT_W4 reads: within each 32-bit word covering
 * k..k+7, k+2i at bits 4i and k+2i+1 at bits 16+4i; the rows in groups of 8,
 * each group's 64-byte pieces (128 codes of one row) stored chunk after chunk
 * with the group's rows adjacent within a chunk (the last group may have fewer
 * rows).  Same size, N * K / 2 bytes; K % 128 == 0 (else ER_EINVAL). */
int er_op_w4_kernel_order(const void *d_canon, int N, int K, void *d_out, void *stream);

/* y[m, n] = sum_k x[m, k] W[n, k] for m < M, n < N; y fp32 [M, ldy].
 * x: [M, ldx] of x_dtype (ER_BF16 or ER_F32).  The verify pass runs the
 * target's linears at M = B (gamma + 1); the drafter runs its quantized copies
 * at M = B.  path (ER_EINVAL where a kernel does not take the shape):
 *   0      automatic (what the rollout uses)
 *   1      VALU (fp32 activations or weights)
 *   2      register-fed skinny MFMA kernel, 32-row m-tiles (bf16 x, K % 128 == 0)
 *   3      LDS-tiled 128x128 GEMM (bf16 W)
 *   1000 + 100*NR + 10*KS + MT/16   that register-fed variant (16*NR rows per
 *          wave, K split over KS of the 8 waves, m-tile MT in {16, 32})
 *   2000 + 100*NR + 10*KS + D       streaming kernel, M <= 16: x staged in LDS,
 *          weights through a D-deep register ring
 *   30000 + 1000*NR + 100*KS + 10*D + i   weight-streaming GEMM over m-tiles of 16 * {2,4,8,16}[i]
 *          rows (bf16 weights: M at most one m-tile; W8/W4: any M, one m-tile per work-group)
 *   40000 + 100*i + 10*D + w        deep-pipelined GEMM, BM = {_,64,128,256}[i] with 64-wide
 *          k steps (i = 1..3) or BM = 128 with 32-wide k steps (i = 5), register
 *          ring depth D, split-K until 256*w work-groups */
int er_op_linear(int x_dtype, const void *d_x, int ldx, int M, int fmt, const void *d_w, const void *d_scale,
                 const void *d_zero, int N, int K, float *d_y, int ldy, int path, void *stream);

/* Fused linear with bf16 activations (MFMA paths; the bf16 model's forward
 * runs its projections through this).  Input: xnorm = 0 reads x' = d_x as
 * bf16 [M, ldx]; xnorm = 1 forms x'[m] = bf16(h[r] * rstd(r) * g) on load, h =
 * d_x fp32 [rows, ldx], r = d_xrow ? d_xrow[m] : m, rstd(r) = 1/sqrt(S[r]/K +
 * eps) with S[r] = d_ssq_in[r] * 2^-24 (fixed-point sum of squares of h's row)
 * and g = d_gnorm bf16 [K] (RMSNorm, EfficientRollout's Qwen2.5 family;
 * standard pre-norm decoder).  acc = x' W^T (fmt as er_op_linear).
 * Epilogue epi:
 *   ER_EPI_F32    d_y fp32 [M, ldy] = acc
 *   ER_EPI_RESID  d_y fp32 [M, ldy] += acc; if d_ssq_acc, d_ssq_acc[m] +=
 *                 the updated row's sum of squares in 2^-24 fixed point
 *                 (each work-group adds its rounded partial)
 *   ER_EPI_SWIGLU W = [gate (F rows); up (F rows)], d_y bf16 [M, ldy]:
 *                 y[m, f] = silu(acc[m, f]) * acc[m, F + f]
 *   ER_EPI_QKV    W = [q; k; v] heads of hd rows; rotate-half RoPE on q and k
 *                 at position pos[m] (cos/sin table [max_pos, hd/2] of
 *                 (cos, sin) fp32 pairs); q -> d_q_out bf16 [M, hq, hd]; k, v ->
 *                 the paged KV pool (er_op_attention's layout) at slot[m].
 * If d_ssq_zero, rows [0, M) of it are set to 0 (it may not alias d_ssq_in or
 * d_ssq_acc).  path as er_op_linear (0, 2, 3 or a skinny variant). */
#define ER_EPI_F32    0
#define ER_EPI_RESID  2
#define ER_EPI_SWIGLU 3
#define ER_EPI_QKV    4
typedef struct {
  int hq, hkv, hd;
  const int32_t *d_pos;       /* [M] */
  const int64_t *d_slot;      /* [M] block * 16 + offset */
  const float *d_cos_sin;     /* [max_pos, hd/2, 2] */
  void *d_q_out;              /* bf16 [M, hq, hd] */
  void *d_kv_pool;            /* bf16 pool */
  int layer, n_layers;
} er_qkv_args;
int er_op_linear_fused(int epi, const void *d_x, int ldx, int M, int xnorm, const int32_t *d_xrow,
                       const uint64_t *d_ssq_in, const void *d_gnorm, float eps, int fmt, const void *d_w,
                       const void *d_scale, const void *d_zero, int N, int K, void *d_y, int ldy,
                       uint64_t *d_ssq_acc, uint64_t *d_ssq_zero, const er_qkv_args *qkv, int path, void *stream);

/* Paged GQA attention (TLT reading notes, section 1: the target scores all
 * drafted positions in one pass).  q: [Mq, hq, hd] of act_dtype; out same
 * shape.  KV pool of blocks of 16 positions: block b, layer l, kv head h holds
 * K as [16][hd] starting at ((((b*L + l)*2 + 0)*hkv + h)*16)*hd and V
 * transposed, [hd][16], starting at ((((b*L + l)*2 + 1)*hkv + h)*16)*hd.
 * Item i: q rows q_row0[i] .. + q_count[i]-1 at positions q_pos0[i] .. of the
 * sequence whose block table row is bt_row[i] (block_table [rows, bt_stride]);
 * a query at position t sees keys 0..t.  (n_q_heads/n_kv_heads)*max_q_count <= 64,
 * hd in {64, 128}. */
int er_op_attention(int act_dtype, const void *d_q, void *d_out, const void *d_kv_pool, int n_layers, int layer,
                    int hq, int hkv, int hd, const int32_t *d_block_table, int bt_stride, const int32_t *d_bt_row,
                    const int32_t *d_q_row0, const int32_t *d_q_pos0, const int32_t *d_q_count, int n_items,
                    int max_q_count, int max_ctx, void *stream);

/* er_op_attention for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * same arguments, layout and result, bit for bit; it allocates nothing.  The
 * partial results of a key range split over work-groups go to a 16 MiB
 * device array of the library (one copy per GPU, held until the process
 * ends) instead of the lazily allocated workspace of er_op_attention.
 * Returns ER_ENOMEM, launching nothing, when the call's partials would need
 * more than those 16 MiB (floats: work units x hkv x (hq/hkv) x max_q_count x
 * (hd + 2), the units set by max_ctx and n_items); use er_op_attention then.
 * ER_EDEVICE if the array's address cannot be obtained.  Every call on one
 * GPU shares that GPU's array: calls that overlap on one GPU (other streams,
 * other threads) race. */
int er_op_attention_noalloc(int act_dtype, const void *d_q, void *d_out, const void *d_kv_pool, int n_layers,
                            int layer, int hq, int hkv, int hd, const int32_t *d_block_table, int bt_stride,
                            const int32_t *d_bt_row, const int32_t *d_q_row0, const int32_t *d_q_pos0,
                            const int32_t *d_q_count, int n_items, int max_q_count, int max_ctx, void *stream);

/* Per-row sampling statistics of fp32 logits rows [rows, ld]: per vocabulary
 * chunk of 2048 tokens the max, its first index and the softmax mass relative
 * to it (fp64), plus the top-p threshold.  d_stats: er_op_stats_bytes(V) per row. */
size_t er_op_stats_bytes(int V);
int er_op_row_stats(const float *d_logits, int rows, int V, long ld, float temperature, float top_p, void *d_stats,
                    void *stream);

/* One draw per row from pi(row; T, top_p): the smallest index whose running
 * sum in vocabulary order reaches u * total, u = Philox4x32-10 uniform of
 * (seed; seq_id[r], pos[r], draft_idx, purpose).  d_out[r * out_stride]. */
int er_op_sample_rows(const float *d_logits, const void *d_stats, int rows, int V, long ld, float temperature,
                      float top_p, uint64_t seed, const int32_t *d_seq_id, const int32_t *d_pos, int draft_idx,
                      int purpose, int32_t *d_out, int out_stride, void *stream);

/* Speculative decision for B sequences (standard speculative sampling, the
 * lossless rule): target rows [B*(gamma+1), V] b-major, drafter rows
 * [gamma*B, V] draft-index-major, with their stats; d_tokens [B, gamma+1]
 * holds (pending, d_1..d_gamma); accept d_j iff u*q_j(d_j) <= p_j(d_j), else
 * resample normalize(max(0, p_j - q_j)) and stop; bonus from p_{gamma+1}
 * after a full acceptance.  d_out_tok [B, gamma+1], d_n_acc [B]. */
int er_op_spec_decide(const float *d_p_logits, const void *d_p_stats, const float *d_q_logits, const void *d_q_stats,
                      const int32_t *d_tokens, int B, int gamma, int V, float temperature, float top_p, uint64_t seed,
                      const int32_t *d_seq_id, const int32_t *d_pos0, int32_t *d_out_tok, int32_t *d_n_acc,
                      void *stream);

/* u[i] = Philox4x32-10 uniform of counter d_ctr[4i..4i+3] under key seed:
 * ((out0 >> 8) + 1) * 2^-24, as fp64. */
int er_op_philox_uniform(uint64_t seed, const uint32_t *d_ctr, int n, double *d_u, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* ER_OPS_H */
