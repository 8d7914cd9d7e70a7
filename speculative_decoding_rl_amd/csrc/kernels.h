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
  EPI_F32 = 0,     // y (fp32) [m*ldy + n] = acc
  EPI_ACT = 1,     // y (bf16 if act_bf16 else fp32) = acc
  EPI_RESID = 2,   // y (fp32 residual stream) += acc; optional per-row sum-of-squares partials
  EPI_SWIGLU = 3,  // W = [gate; up] (2F rows): y (act) [m*ldy + f] = silu(gate_f) * up_f
  EPI_QKV = 4,     // W = [q; k; v]: rotate-half RoPE on q, k; q -> qout, k, v -> paged KV pool
};

// Fused linear: y = epilogue(x' W^T) where x' is x (act type) or, with
// xnorm, RMSNorm(h) * g formed on load from the fp32 residual stream h.
// Row sums of squares of h travel between kernels as 64-bit fixed point
// (units of 2^-24) so that the accumulation is exact and order-free:
// residual epilogues add into ssq_acc, and the next residual producer clears
// the buffer the previous consumer read (ssq_zero).
constexpr double SSQ_SCALE = 16777216.0;  // 2^24
struct LinArgs {
  const void* x;            // act [M, ldx], or fp32 h [*, ldx] when xnorm
  int ldx, M;
  int xnorm;
  const int32_t* xrow;      // xnorm: row m of x' is row xrow[m] of h (nullable = identity)
  const unsigned long long* ssq_in;  // xnorm: [rows of h] fixed-point sums of squares
  const void* gnorm;        // xnorm: gain [K], model dtype
  float eps;
  LinearW W;
  int epi;
  void* y;
  int ldy;
  int act_bf16;
  unsigned long long* ssq_acc;   // EPI_RESID: add the updated rows' sums of squares (nullable)
  unsigned long long* ssq_zero;  // cleared for rows [0, M) by work-group 0 (nullable)
  // The three sum-of-squares buffers may be split into ssq_slots slots (slot s
  // of row r at s * ssq_stride + r; a row's value is the sum over its slots):
  // producers add into slot blockIdx.x % ssq_slots, so that the work-groups
  // of one row do not all update one cache line.  ssq_slots <= 1: one slot.
  int ssq_slots;
  long ssq_stride;
  // EPI_QKV
  int hq, hkv, hd;
  const int32_t* pos;       // [M]
  const int64_t* slot;      // [M] KV slot (block * 16 + offset)
  const float2* cs;         // cos/sin [max_pos][hd/2]
  void* qout;               // [M, hq, hd] act
  void* kv_pool;
  int layer, n_layers;
  // EPI_SWIGLU
  int F;
};

// Plain bf16 GEMMs through hipBLASLt (blas.hip): y = beta * y + x W^T, x
// [M][ldx] bf16, W [N][K] bf16, y [M][ldy] fp32 (out32) or bf16.  Returns 0,
// 1 when the library has no algorithm for the shape (nothing launched), or a
// negative error.  The first call of a shape with up to 512 rows times
// candidate algorithms and waits for the stream (never under stream capture);
// scratch (scratch_floats fp32) receives the timing runs of accumulating
// calls (beta = 1).
struct Blas;
Blas* blas_create(void* workspace, size_t ws_bytes, float* scratch, size_t scratch_floats);
void blas_destroy(Blas* b);
int blas_gemm(Blas* b, const void* x, int ldx, int M, const void* W, int N, int K, void* y, int ldy, bool out32,
              float beta, hipStream_t st);

struct LinearWs {
  float* partial;     // split-K partial tiles
  size_t partial_floats;
  int* counters;      // zero-initialised tile counters
  int n_counters;
  uint16_t* xn;       // bf16 x' for kernels that do not normalize on load (nullable)
  size_t xn_elems;
  // Library GEMMs for bf16 weights (nullable = never): blas_min_m < 0 from
  // each shape's measured row threshold, > 0 from that many rows for every
  // shape, 0 never.  The fp32 result of the QKV and gate/up projections goes
  // to blas_out before its epilogue kernel.
  Blas* blas;
  int blas_min_m;
  float* blas_out;
  size_t blas_out_floats;
};

// What a launch_linear call ran (for per-kernel timing): kernel name as the
// profiler demangles it, split count.
struct LinearInfo {
  char name[64];
  int nsplit;
};

// Path choice: 0 = automatic, 1 = VALU, 2 = MFMA (when legal), 3 = tiled GEMM (bf16),
// 1000 + 100*NR + 10*KS + MT/16 = that skinny MFMA variant.
int launch_linear(const void* x, bool act_bf16, int ldx, int M, const LinearW& W, void* y, int ldy,
                  int epi, const LinearWs& ws, int path, hipStream_t st, LinearInfo* info = nullptr);
// bf16 activations only (MFMA paths).
int launch_linear_fused(const LinArgs& a, const LinearWs& ws, int path, hipStream_t st, LinearInfo* info = nullptr);

// Small fused ops.
// h[m] = embed[token]; optional ssq[m] = fixed-point sum h^2 (plain store,
// other slots 0), ssq_zero[m] = 0 in every slot.
int launch_embed(const int32_t* tokens, int tok_stride, int M, const void* embed, bool bf16, int d,
                 float* h, unsigned long long* ssq, unsigned long long* ssq_zero, hipStream_t st,
                 int ssq_slots = 1, long ssq_stride = 0);
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
  // Work units (optional): item i owns units unit_start[i] .. unit_start[i+1]-1
  // (exclusive prefix sum, n_items + 1 entries, n_units in total), each of
  // unit_start[n_items + 1 + i] blocks (the last one shorter).  Null: every
  // item gets the same split count.
  const int32_t* unit_start;
  // One record of eight int32 per unit (with unit_start; null: looked up from
  // unit_start and the item arrays): item, split index | units of the item
  // << 16, first block, blocks per unit, query count, first query position,
  // first query row, block-table row.
  const int32_t* unit_rec;
  int n_units;
  int max_units;             // most units of one item (0: unknown, bounded from max_ctx)
  // Items that have more than one unit (they alone need the combine); with a
  // unit table, null means none.
  const int32_t* split_items;
  int n_split;
};
// phase 0: scores + combine; 1: the scoring kernel only; 2: the combine only
// (same arguments).  *combined (nullable) tells whether a combine is needed.
// Waves per work-group of the bf16 attention kernel (k_attn_mfma<hd, waves>).
constexpr int kAttnWaves = 4;
int launch_attention(const AttnArgs& a, hipStream_t st, int phase = 0, int* combined = nullptr);
// Ring depth (1 or 2) launch_attention picks for the bf16 scoring kernel.
int attn_ring(const AttnArgs& a);

// Persistent decode forward (bf16 models, 1..16 rows): embedding, every
// decoder layer and the final residual stream in one cooperative launch (see
// k_decode.hip).  The weights of one forward share one format (the bf16
// target, or the W4/W8 drafter).
struct DecLayerW {
  LinearW qkv, o, gu, down;
  const void* attn_norm;
  const void* mlp_norm;
};
struct DecodeArgs {
  int M, L, d, hq, hkv, hd, F;
  float eps;
  const DecLayerW* layers;        // device array [L]
  const void* embed;
  const int32_t* tokens;
  int tok_stride;
  const int32_t* pos;             // [M]
  const int64_t* slot;            // [M] KV slot (block * 16 + offset)
  const float2* cs;               // RoPE cos/sin [max_pos][hd/2]
  void* kv_pool;
  // attention work units (push_units layout)
  const int32_t* block_table;
  int bt_stride;
  const int32_t* unit_rec;        // 8 int32 per unit
  const int32_t* unit_start;      // [n_items + 1] exclusive prefix sums of units
  const int32_t* split_items;     // items with more than one unit
  const int32_t* item_q_row0;
  const int32_t* item_q_count;
  int n_items, n_units, n_split, max_q;
  // workspaces (device).  Every activation a phase writes lives in its own
  // buffer, written once per forward (so other work-groups can read it through
  // their L2 without a stale copy); rows are allocated for 16.
  float* hbuf;                    // [2L][16][d] residual stream entering each layer / after its attention block
  float* h_final;                 // [M, d] the residual stream after the last layer (the result)
  uint16_t* qbuf;                 // [L][16][hq * hd] rotated queries
  uint16_t* abuf;                 // [L][16][hq * hd] attention output
  uint16_t* act;                  // [L][16][F] SwiGLU output
  float* apart;                   // attention partials [units][hkv][grp * max_q][hd + 2] (reused per layer)
  unsigned long long* ssq;        // [2L][slots][16] fixed-point sums of squares of each h buffer
  unsigned long long* ssq_out;    // the final sums of squares, slot layout of LinArgs::ssq_in
  int ssq_slots;
  long ssq_stride;                // of ssq_out
  unsigned* bar;                  // barrier words (zeroed once before the first launch)
  unsigned* err;                  // nonzero after a barrier time-out
  int ks[4];                      // waves splitting K in the qkv and gate/up phases ([0], [2]: 8, 4 or 2)
  int n_wg;                       // grid size (decode_grid)
  long spin_limit;                // polls before a barrier wait gives up
  // optional phase trace (nullable): per grid barrier k and work-group b, the
  // 100 MHz clock when b arrived ([k][b][0]) and when it was released ([k][b][1])
  unsigned long long* trace;
  int trace_max;                  // barriers the trace holds
};
// Work-groups of the grid (one per compute unit), 0 if the kernel cannot run.
int decode_grid(int fmt, int hd);
// K slices of an [N, K] projection in weight format fmt for a grid of nwg work-groups.
int decode_ksplit(int N, int K, int nwg, int fmt);
// Dynamic LDS of a launch (n_max: the widest projection's output rows).
size_t decode_lds_bytes(int hd, int M, int d, int n_max, int nwg);
// Device bytes of the write-once activation buffers for a model (16 rows).
inline size_t decode_ws_bytes(int L, int d, int hq, int hd, int F, int slots) {
  return (size_t)2 * L * 16 * d * 4 + (size_t)2 * L * 16 * hq * hd * 2 + (size_t)L * 16 * F * 2 +
         (size_t)2 * L * slots * 16 * 8 + 4 * 256;
}
// 0, -1 for arguments it does not take, -3 on a launch error.
int launch_decode(const DecodeArgs& a, int fmt, hipStream_t st);
constexpr int kDecodeMaxRows = 16;

constexpr int kDecodeBarWords = 10 * 32;

// Quantizers (drafter build) and layout conversion.
int launch_quantize_w8(const void* W, bool bf16, int N, int K, int8_t* q, float* scale, hipStream_t st);
int launch_quantize_w4(const void* W, int N, int K, uint8_t* packed_canon, uint16_t* scale,
                       uint8_t* zero, hipStream_t st);
int launch_w4_to_kernel_order(const uint8_t* canon, int N, int K, uint8_t* out, hipStream_t st);

// Philox counter word 3: which draw of a position this is.
enum Purpose { PURPOSE_DRAFT = 0, PURPOSE_ACCEPT = 1, PURPOSE_RESIDUAL = 2, PURPOSE_AR = 3 };

// Sampler.  Statistics of a logits row live in one record of
// stats_row_bytes(nch) bytes: the top-p threshold, then one ChunkStat per
// vocabulary chunk of 2048 tokens.
struct RowStats {            // tokens with key > thr_key are kept, and those with key == thr_key and index <= thr_idx
  uint32_t thr_key;
  int32_t thr_idx;
  uint32_t pad[2];
};
struct ChunkStat {           // per vocabulary chunk: max logit, its first index, sum exp((z - m)/T) of kept tokens
  float m;
  int32_t arg;
  double s;
};
__host__ __device__ inline int sampler_chunks(int V) { return (V + 2047) / 2048; }
__host__ __device__ inline long stats_row_bytes(int nch) { return (long)sizeof(RowStats) + (long)nch * sizeof(ChunkStat); }

// Point-mass logit rows for drafts that are not sampled (k_sample.hip).
int launch_point_mass(float* q, int g, int n, int V, const int32_t* tok, int G1, hipStream_t st);
int launch_row_stats(const float* logits, int rows, int V, long ld, float T, float top_p, void* stats,
                     hipStream_t st);
// Draw one token per row r from pi(logits row row_map[r] (or r)) with
// u(seed, seq_id[r], pos[r], didx, purpose); writes out[r * out_stride].
int launch_sample_rows(const float* logits, const void* stats, int rows, int V, long ld, float T, float top_p,
                       uint64_t seed, const int32_t* seq_id, const int32_t* pos, int didx, int purpose,
                       int32_t* out, int out_stride, const int32_t* row_map, hipStream_t st);
// Speculative decision for each sequence b of a batch: target rows
// [B*(g+1)] (b-major), drafter rows [g*B] (draft-index-major), drafts =
// tokens[b*(g+1) + 1 .. g]; writes out_tok[b*(g+1) ...], n_acc[b].
// resid: workspace of B * sampler_chunks(V) doubles.
int launch_spec_decide(const float* p_logits, const void* p_stats, const float* q_logits, const void* q_stats,
                       const int32_t* tokens, int B, int gamma, int V, float T, float top_p, uint64_t seed,
                       const int32_t* seq_id, const int32_t* pos0, int32_t* out_tok, int32_t* n_acc,
                       double* resid, hipStream_t st);

int launch_philox_uniform(uint64_t seed, const uint32_t* ctr4, int n, double* u, hipStream_t st);

// Device micro-benchmarks for the roofline constants.
int launch_stream_read(const void* p, size_t bytes, uint32_t* sink, hipStream_t st);

}  // namespace er
