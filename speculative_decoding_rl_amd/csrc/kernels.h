// Host-side launch API of the gfx950 kernels (one translation unit per family).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace er {

// Weight formats of a linear layer y[m, n] = sum_k x[m, k] W[n, k].
enum WFmt { FMT_F32 = 0, FMT_BF16 = 1, FMT_W8 = 2, FMT_W4 = 3 };

// W row-major [N, K].  FMT_W8: int8 codes + fp32 scale[N].  FMT_W4: packed
// nibbles [N, K/2] in the kernel order (within each 32-bit word covering
// k..k+7: k+2i at bits 4i, k+2i+1 at bits 16+4i), bf16 scale[N, K/128] and
// u8 zero[N, K/128].
struct LinearW {
  int fmt;
  const void* w;
  const void* scale;
  const void* zero;
  int N, K;
};

// Epilogues of the linear kernels.
enum Epi {
  EPI_F32 = 0,    // y (fp32) [m*ldy + n] = acc
  EPI_ACT = 1,    // y (bf16 if act_bf16 else fp32) = acc
  EPI_RESID = 2,  // y (fp32 residual stream) += acc
};

struct LinearWs {
  float* partial;     // split-K partial tiles
  size_t partial_floats;
  int* counters;      // zero-initialised tile counters
  int n_counters;
};

// Path choice: 0 = automatic, 1 = force VALU, 2 = force MFMA (when legal).
int launch_linear(const void* x, bool act_bf16, int ldx, int M, const LinearW& W, void* y, int ldy,
                  int epi, const LinearWs& ws, int path, hipStream_t st);

// Small fused ops.
int launch_embed(const int32_t* tokens, int tok_stride, int M, const void* embed, bool bf16, int d,
                 float* h, hipStream_t st);
int launch_rmsnorm(const float* h, int M, int d, const void* g, bool bf16, float eps, void* x,
                   const int32_t* row_index, hipStream_t st);
// q/k/v from the fused projection qkv [M, (hq+2hkv)hd] (fp32): rotate q, k
// (rotate-half RoPE with the cos/sin table [max_pos, hd/2] x 2), store q into
// qout [M, hq, hd] (act type) and k, v into the paged KV pool at slot[m].
int launch_rope_kv(const float* qkv, int M, int hq, int hkv, int hd, const int32_t* pos,
                   const int64_t* slot, const float2* cs, void* qout, void* kv_pool, int layer,
                   int n_layers, bool bf16, hipStream_t st);
int launch_swiglu(const float* gu, int M, int F, void* act, bool bf16, hipStream_t st);

// Paged GQA attention.  Query rows are grouped per "item": item i covers
// q_count[i] consecutive positions starting at q_pos0[i] of the sequence whose
// block table row is bt_row[i]; query row r of item i is q row
// q_row0[i] + r.  A query at position t sees keys 0..t.
struct AttnArgs {
  const void* q;            // [Mq, hq, hd] act type
  void* out;                // [Mq, hq*hd] act type
  const void* kv_pool;
  const int32_t* block_table;  // [n_bt_rows, bt_stride]
  int bt_stride;
  const int32_t* item_bt_row;
  const int32_t* item_q_row0;
  const int32_t* item_q_pos0;
  const int32_t* item_q_count;
  int n_items;
  int max_q_count;
  int max_ctx;               // upper bound on keys any item sees (for split sizing)
  int hq, hkv, hd, n_layers, layer;
  bool bf16;
  float* ws;                 // split partials
  size_t ws_floats;
};
int launch_attention(const AttnArgs& a, hipStream_t st);

// Quantizers (drafter build) and layout conversion.
int launch_quantize_w8(const void* W, bool bf16, int N, int K, int8_t* q, float* scale, hipStream_t st);
int launch_quantize_w4(const void* W, int N, int K, uint8_t* packed_canon, uint16_t* scale,
                       uint8_t* zero, hipStream_t st);
int launch_w4_to_kernel_order(const uint8_t* canon, int N, int K, uint8_t* out, hipStream_t st);

// Philox counter word 3: which draw of a position this is.
enum Purpose { PURPOSE_DRAFT = 0, PURPOSE_ACCEPT = 1, PURPOSE_RESIDUAL = 2, PURPOSE_AR = 3 };

// Sampler.
struct RowStats {            // per logits row
  float zmax;
  int32_t argmax;
  double total;              // sum exp((z - zmax)/T) over all tokens
  double kept;               // mass kept by top-p (== total when top_p >= 1)
  uint32_t thr_key;          // tokens with key > thr_key are kept ...
  int32_t thr_idx;           // ... and those with key == thr_key and index <= thr_idx
};
int launch_row_stats(const float* logits, int rows, int V, long ld, float T, float top_p,
                     RowStats* stats, hipStream_t st);
// Draw one token per row r from pi(logits row row_map[r] (or r)) with
// u(seed, seq_id[r], pos[r], didx, purpose); writes out[r * out_stride].
int launch_sample_rows(const float* logits, const RowStats* stats, int rows, int V, long ld,
                       float T, uint64_t seed, const int32_t* seq_id, const int32_t* pos,
                       int didx, int purpose, int32_t* out, int out_stride, const int32_t* row_map,
                       hipStream_t st);
// Speculative decision for each sequence b of a batch: target rows
// [B*(g+1)] (b-major), drafter rows [g*B] (draft-index-major), drafts =
// tokens[b*(g+1) + 1 .. g]; writes out_tok[b*(g+1) ...], n_acc[b].
int launch_spec_decide(const float* p_logits, const RowStats* p_stats, const float* q_logits,
                       const RowStats* q_stats, const int32_t* tokens, int B, int gamma, int V,
                       float T, uint64_t seed, const int32_t* seq_id, const int32_t* pos0,
                       int32_t* out_tok, int32_t* n_acc, hipStream_t st);

int launch_philox_uniform(uint64_t seed, const uint32_t* ctr4, int n, double* u, hipStream_t st);

// Device micro-benchmarks for the roofline constants.
int launch_stream_read(const void* p, size_t bytes, uint32_t* sink, hipStream_t st);

}  // namespace er
