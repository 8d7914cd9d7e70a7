// C ABI of the self-speculative rollout step: context, arena, drafter build,
// paged KV bookkeeping, the step drivers (speculative / autoregressive /
// controller-chosen), prefill, the full shrinking-batch rollout loop,
// statistics and diagnostics.  See include/er_api.h for the contract.
//
// The step follows the EfficientRollout page ("关键模块" items 1-3): the
// drafter is the target with quantized linears and shares the target's KV
// cache; the target verifies gamma+1 positions in one forward; a lossless
// rejection sampler (standard speculative sampling, the "lossless primitive"
// of the System-Integrated Speculative Decoding abstract) decides; the KV
// tail past the accepted prefix is released (TLT notes, section 1); a
// roofline toggle and an EMA of the acceptance rate pick AR vs SD and gamma.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/er_api.h"
#include "controller.h"
#include "kernels.h"
#include "history.h"
#include "kvpool.h"
#include "work_units.h"

using namespace er;

namespace {

struct Lin4 {
  LinearW qkv, o, gu, down;
};

struct Seq {
  bool alive = false, prefilled = false, finished = false;
  int32_t prompt_len = 0, max_new = 0, generated = 0;
  int32_t n = 0;        // position of the pending token == committed KV entries
  int32_t pending = 0;
  int32_t group = -1;
  bool leader = true;   // computes the shared prompt for its group
  int32_t leader_id = -1;
  // sequences whose leading KV blocks are the same physical blocks (a share
  // group, or a sequence and its forks): family id (-1 = none) and how many
  // leading positions this sequence shares with the family
  int32_t family = -1;
  int32_t shared_len = 0;
  std::vector<int32_t> toks;  // prompt + generated tokens (the last one is the pending token)
  BlockTable bt;
};

// Slots of the fixed-point sums of squares (see LinArgs): the residual
// producers of one row spread their atomic adds over this many cache lines.
constexpr int kSsqSlots = 16;

}  // namespace

struct er_history {
  er::HistoryCache cache;
  explicit er_history(int prefix_len) : cache(prefix_len) {}
};

struct er_ctx {
  er_model_desc md{};
  er_draft_desc dd{};
  er_rollout_desc rd{};
  bool bf16 = true;
  int act_bytes = 2;
  hipStream_t st = nullptr;

  // weights
  const void* embed = nullptr;
  const void* final_norm = nullptr;
  std::vector<const void*> attn_norm, mlp_norm;
  std::vector<Lin4> tgt, drf;
  LinearW lm_t{}, lm_d{};

  // arena
  char* arena = nullptr;
  size_t arena_bytes = 0, arena_used = 0;

  // device buffers
  float2* cs = nullptr;
  float* h = nullptr;
  void* xbuf = nullptr;
  float* qkv = nullptr;
  void* qb = nullptr;
  float* gu = nullptr;
  float* logits_p = nullptr;
  float* logits_q = nullptr;
  void* stats_p = nullptr;     // sampler statistics, stats_row_bytes(nch) per logits row
  void* stats_q = nullptr;
  double* resid = nullptr;     // residual chunk masses [max_batch, nch]
  // fixed-point row sums of squares of h (ping-pong between the residual
  // producers and the normalizing consumers of the fused bf16 forward)
  unsigned long long* ssq[2] = {nullptr, nullptr};
  bool fuse = false;
  int nch = 1;
  int32_t* out_d = nullptr;     // [rows] tokens + [max_batch] accepted counts
  int32_t* out_h = nullptr;     // pinned
  LinearWs lws{};
  float* attn_ws = nullptr;
  size_t attn_ws_floats = 0;
  uint8_t* w4_tmp = nullptr;
  size_t w4_tmp_bytes = 0;
  uint32_t* sink = nullptr;
  void* kv_pool = nullptr;
  size_t block_bytes = 0;
  Meta meta;

  // Uploads of `meta.h` (pinned) are DMA reads done when the stream reaches
  // them: the host must not rewrite the region before the last one has run.
  hipEvent_t meta_ev = nullptr;
  bool meta_pending = false;

  int max_rows = 0;       // rows of the activation buffers
  int logit_rows = 0;     // rows of logits_p
  int lin_path = 0;

  BlockPool pool;
  std::vector<Seq> seqs;
  int32_t alive = 0;

  // controller
  CostModel cost{};
  double alpha_ema = 0.8;
  double alpha_init = 0.8;
  int gamma_pinned = 0;
  PlanState plan;         // roofline policy state: last choice (0 = AR, -1 none), probe schedule
  int policy = ER_POLICY_AUTO;
  er_guard_state guard{};  // measured-timing guard (ER_POLICY_TIMING)

  er_stats stats{};
  std::string err;

  // diagnostics
  int last_mode = -1, last_gamma = 0, last_B = 0;
  int last_rows = 0;      // sequences the last step ran (last_B plus graph padding): the drafter logits' stride
  size_t last_tok_off = 0;  // verify tokens [B, gamma+1] of the last speculative step, in the metadata region
  std::vector<int32_t> last_prefill_row;

  // per-kernel timing (events around each linear / attention launch)
  int kprof = 0;  // launches bracketed: KPROF_LINEAR | KPROF_ATTENTION bits
  er_history* hist = nullptr;  // borrowed: drafts copied from earlier rollouts (er_set_history)
  int hist_gamma = 4, hist_max_batch = 64;
  std::vector<hipEvent_t> kev;
  size_t kev_used = 0;
  struct KRec { std::string name; double bytes, flops; int e0, e1; };
  std::vector<KRec> krec;
  struct KStat { long n = 0; double ms = 0, bytes = 0, flops = 0; };
  std::map<std::string, KStat> kstat;

  // persistent decode forward (k_decode): bf16 forwards of at most
  // kDecodeMaxRows rows run as one cooperative launch
  bool dec_on = false;               // enabled (er_set_persistent) and available on this device
  int dec_nwg[4] = {0, 0, 0, 0};     // its grid per weight format (0: cannot run)
  int dec_ks[2][4] = {{8, 8, 8, 8}, {8, 8, 8, 8}};  // waves splitting K per projection: target, drafter
  bool dec_avail = false;            // the kernel can run on this device for both weight formats
  DecLayerW* dec_layers[2] = {nullptr, nullptr};  // device descriptors: target, drafter
  char* dec_ws = nullptr;            // write-once activation buffers (decode_ws_bytes)
  unsigned* dec_bar = nullptr;
  unsigned* dec_err = nullptr;
  int dec_err_slot = 0;              // out_h index the error word is copied to
  bool dec_ran = false;              // the current step launched it
  long dec_spin_limit = 1L << 21;    // polls before a grid-barrier wait gives up
  unsigned long long* dec_trace = nullptr;  // phase trace buffer (er_set_decode_trace), device
  int dec_trace_max = 0;
  int dec_trace_nwg = 0;             // grid of the last traced launch

  // bucketed graph capture (er_set_graphs): steps of at most graph_max rows
  // per phase run padded to a power-of-two batch bucket and replay graphs
  // recorded per (kind, bucket, gamma, context capacity in blocks)
  struct GKey {
    int kind, nb, g, cap;
    bool operator<(const GKey& o) const { return std::tie(kind, nb, g, cap) < std::tie(o.kind, o.nb, o.g, o.cap); }
  };
  struct GEnt {
    hipGraphExec_t x = nullptr;
    size_t meta_used = 0;   // metadata layout size the graph was recorded with
    long used = 0;          // last replay (least recently used is evicted)
  };
  int graph_max = 0;                 // largest batch run through graphs (0: off)
  int graph_keep = 64;               // graphs kept
  hipStream_t cap_st = nullptr;      // private stream the graphs are recorded on
  int32_t pad_block = -1;            // KV block the padding rows write and read
  std::map<GKey, GEnt> graphs;
  long graph_tick = 0;
  int64_t graph_captures = 0, graph_replays = 0, graph_evictions = 0;

  // timing
  int timing_period = 0, timing_first = 0;
  long step_count = 0;
  hipEvent_t ev[6] = {};
  bool have_ev = false;
};

namespace {

int fail(er_ctx* c, int code, const char* fmt, ...) {
  if (c) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    c->err = buf;
  }
  return code;
}

#define HIPC(c, x)                                                                      \
  do {                                                                                  \
    hipError_t e_ = (x);                                                                \
    if (e_ != hipSuccess) return fail((c), ER_EDEVICE, "%s: %s", #x, hipGetErrorString(e_)); \
  } while (0)

#define KC(c, x)                                                                        \
  do {                                                                                  \
    int r_ = (x);                                                                       \
    if (r_ != 0) {                                                                      \
      hipError_t e_ = hipGetLastError();                                                \
      return fail((c), r_ == -2 ? ER_ENOMEM : (r_ == -1 ? ER_EINVAL : ER_EDEVICE),      \
                  "%s failed (%d): %s", #x, r_, hipGetErrorString(e_));                 \
    }                                                                                   \
  } while (0)

// Propagate an error code already recorded by fail().
#define HIPC_OK(x)              \
  do {                          \
    const int r_ = (x);         \
    if (r_ != ER_OK) return r_; \
  } while (0)

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Start filling the metadata region: waits until the last queued upload of
// it has been read (a multi-chunk prefill queues one per chunk without
// waiting for the GPU otherwise).
int meta_begin(er_ctx* c) {
  if (c->meta_pending) {
    HIPC(c, hipEventSynchronize(c->meta_ev));
    c->meta_pending = false;
  }
  c->meta.reset();
  return ER_OK;
}

// Queue the upload of the filled part of the metadata region on the stream.
int meta_upload(er_ctx* c) {
  HIPC(c, hipMemcpyAsync(c->meta.d, c->meta.h, c->meta.used, hipMemcpyHostToDevice, c->st));
  HIPC(c, hipEventRecord(c->meta_ev, c->st));
  c->meta_pending = true;
  return ER_OK;
}

// ---- bucketed graph capture --------------------------------------------------
// TLT notes, section 3, Design A, A3: a batch range shares one set of
// recorded graphs (here: every batch up to 16 alone, then 17-32, 33-64, ...
// padded to the range's top), and the
// drafter's and the target's graphs are recorded apart, so that the verify
// graph serves both self-drafted and history-drafted steps.  Everything a
// replayed kernel reads that changes from step to step sits in the metadata
// region at offsets fixed by the key: the block table (stride = the
// context-capacity class), the work-unit table (a fixed number of units per
// item), positions, slots and tokens.
constexpr int GRAPH_AR = 0, GRAPH_DRAFT = 1, GRAPH_VERIFY = 2;

int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Batch bucket: batches of 1 .. 16 run as they are, larger ones padded to
// the next power of two.  On MI355X at the 7B shape padding costs more than
// a replay saves (3 to 4: 2-6 %; 6 to 8: 2-4 %; 11 to 16: 3-8 % slower than
// the eager step, where exact buckets gain 1-4 %), while a recorded graph
// holds only kernel nodes, so graphs per exact batch cost little memory.
int graph_bucket(int n) { return n <= 16 ? n : pow2_at_least(n); }

void graph_drop(er_ctx* c) {
  for (auto& kv : c->graphs) (void)hipGraphExecDestroy(kv.second.x);
  c->graphs.clear();
}

// How a step over n sequences of rows_per_seq query rows each runs through
// graphs: nb padded rows (0: eagerly), capacity cap blocks per sequence, U
// attention units per item.
struct GraphPlan {
  int nb = 0, cap = 0, U = 0;
};
GraphPlan graph_plan(const er_ctx* c, int n, const int32_t* ids, int rows_per_seq) {
  GraphPlan p;
  // (the padding rows' positions 0 .. rows_per_seq - 1 must stay inside the one padding block)
  if (c->graph_max <= 0 || c->kprof || c->dec_on || n > c->graph_max || c->pad_block < 0 ||
      rows_per_seq > KV_BLOCK)
    return p;
  const int nb = graph_bucket(n);
  if (nb > c->rd.max_batch || nb * rows_per_seq > c->max_rows || nb * rows_per_seq > c->logit_rows) return p;
  int most = 1;
  for (int i = 0; i < n; ++i) most = std::max(most, (c->seqs[ids[i]].n + rows_per_seq + KV_BLOCK - 1) / KV_BLOCK);
  const int cap = std::max(16, pow2_at_least(most));
  const int hkv = c->md.n_kv_heads, grp = c->md.n_q_heads / hkv;
  const int U = graph_units_per_item(nb, hkv, cap);
  if ((size_t)nb * U * hkv * grp * rows_per_seq * (size_t)(c->md.head_dim + 2) > c->attn_ws_floats) return p;
  p.nb = nb;
  p.cap = cap;
  p.U = U;
  return p;
}

// Replay the graph of key (kind, nb, g, cap) on the context's stream,
// recording it from `body` (kernel launches only) when the cache has none:
// the launches are captured on the private capture stream (torch's default
// stream cannot be captured).  A cached graph recorded with a different
// metadata layout size is recorded again.
template <class F>
int graph_run(er_ctx* c, int kind, int nb, int g, int cap, F&& body) {
  const er_ctx::GKey k{kind, nb, g, cap};
  auto it = c->graphs.find(k);
  if (it != c->graphs.end() && it->second.meta_used != c->meta.used) {
    (void)hipGraphExecDestroy(it->second.x);
    c->graphs.erase(it);
    it = c->graphs.end();
  }
  if (it == c->graphs.end()) {
    while (!c->graphs.empty() && (int)c->graphs.size() >= c->graph_keep) {
      auto lru = c->graphs.begin();
      for (auto j = c->graphs.begin(); j != c->graphs.end(); ++j)
        if (j->second.used < lru->second.used) lru = j;
      (void)hipGraphExecDestroy(lru->second.x);
      c->graphs.erase(lru);
      ++c->graph_evictions;
    }
    HIPC(c, hipStreamBeginCapture(c->cap_st, hipStreamCaptureModeThreadLocal));
    hipStream_t user = c->st;
    c->st = c->cap_st;
    const int r = body();
    c->st = user;
    hipGraph_t gr = nullptr;
    const hipError_t e = hipStreamEndCapture(c->cap_st, &gr);
    if (r) {
      if (gr) (void)hipGraphDestroy(gr);
      return r;
    }
    if (e != hipSuccess || !gr) return fail(c, ER_EDEVICE, "graph capture: %s", hipGetErrorString(e));
    hipGraphExec_t x = nullptr;
    const hipError_t e2 = hipGraphInstantiate(&x, gr, nullptr, nullptr, 0);
    (void)hipGraphDestroy(gr);
    if (e2 != hipSuccess) return fail(c, ER_EDEVICE, "graph instantiate: %s", hipGetErrorString(e2));
    er_ctx::GEnt ent;
    ent.x = x;
    ent.meta_used = c->meta.used;
    it = c->graphs.emplace(k, ent).first;
    ++c->graph_captures;
  }
  it->second.used = ++c->graph_tick;
  HIPC(c, hipGraphLaunch(it->second.x, c->st));
  ++c->graph_replays;
  return ER_OK;
}

constexpr int KPROF_LINEAR = 1, KPROF_ATTENTION = 2;
int kp_begin(er_ctx* c, int kind) {
  if (!(c->kprof & kind) || c->kev_used + 2 > c->kev.size()) return -1;
  const int i = (int)c->kev_used;
  c->kev_used += 2;
  if (hipEventRecord(c->kev[(size_t)i], c->st) != hipSuccess) return -1;
  return i;
}
void kp_end(er_ctx* c, int i, const char* name, double bytes, double flops) {
  if (i < 0) return;
  if (hipEventRecord(c->kev[(size_t)i + 1], c->st) != hipSuccess) return;
  c->krec.push_back(er_ctx::KRec{name, bytes, flops, i, i + 1});
}
// After the stream is synchronized: fold the recorded launches into the totals.
void kp_flush(er_ctx* c) {
  for (const auto& r : c->krec) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, c->kev[(size_t)r.e0], c->kev[(size_t)r.e1]) != hipSuccess) continue;
    auto& k = c->kstat[r.name];
    k.n += 1;
    k.ms += ms;
    k.bytes += r.bytes;
    k.flops += r.flops;
  }
  c->krec.clear();
  c->kev_used = 0;
}

double weight_bytes(const LinearW& W) {
  const double nk = (double)W.N * W.K;
  switch (W.fmt) {
    case FMT_F32: return 4 * nk;
    case FMT_BF16: return 2 * nk;
    case FMT_W8: return nk + 4.0 * W.N;
    default: return nk / 2 + 3.0 * W.N * (W.K / 128);
  }
}

// Layout of everything but the KV pool, shared by er_arena_bytes and init.
struct Layout {
  size_t drafter = 0, cs = 0, h = 0, xbuf = 0, qkv = 0, qb = 0, gu = 0, lp = 0, lq = 0, sp = 0, sq = 0;
  size_t out = 0, partial = 0, counters = 0, attn = 0, w4tmp = 0, sink = 0, meta = 0, resid = 0, ssq = 0, xn = 0;
  size_t dec = 0;  // persistent decode forward: layer descriptors, sums of squares, counters, barrier
  size_t blas = 0; // library GEMM workspace (bf16 models)
  size_t block_bytes = 0;
  int max_rows = 0, logit_rows = 0;
  size_t total_fixed() const {
    return drafter + cs + h + xbuf + qkv + qb + gu + lp + lq + sp + sq + out + partial + counters + attn + w4tmp +
           sink + meta + resid + ssq + xn + dec + blas;
  }
};

size_t quant_bytes(const er_draft_desc& dd, long N, long K) {
  if (dd.quant == ER_W8_PERCH_SYM) return align256((size_t)N * K) + align256((size_t)N * 4);
  const long G = K / 128;
  return align256((size_t)N * K / 2) + align256((size_t)N * G * 2) + align256((size_t)N * G);
}

int make_layout(const er_model_desc& m, const er_draft_desc& dd, const er_rollout_desc& r, Layout* L,
                std::string* why) {
  const long d = m.d_model, hq = m.n_q_heads, hkv = m.n_kv_heads, hd = m.head_dim, F = m.ffn, V = m.vocab;
  const int ab = m.dtype == ER_BF16 ? 2 : 4;
  const int G1 = r.gamma_max + 1;
  L->max_rows = std::max(r.max_batch * G1, r.prefill_chunk);
  L->logit_rows = std::max(r.max_batch * G1, r.max_batch);
  const long qkvN = (hq + 2 * hkv) * hd;
  size_t dr = 0;
  for (int l = 0; l < m.n_layers; ++l) {
    dr += quant_bytes(dd, qkvN, d) + quant_bytes(dd, d, hq * hd) + quant_bytes(dd, 2 * F, d) + quant_bytes(dd, d, F);
  }
  if (dd.quant_lm_head) dr += quant_bytes(dd, V, d);
  L->drafter = dr;
  L->cs = align256((size_t)r.max_ctx * (hd / 2) * sizeof(float2));
  const long R = L->max_rows;
  L->h = align256((size_t)R * d * 4);
  L->xbuf = align256((size_t)R * std::max(std::max(d, hq * hd), F) * ab);
  L->qkv = align256((size_t)R * qkvN * 4);
  L->qb = align256((size_t)R * hq * hd * ab);
  L->gu = align256((size_t)R * 2 * F * 4);
  L->lp = align256((size_t)L->logit_rows * V * 4);
  L->lq = align256((size_t)r.max_batch * r.gamma_max * V * 4);
  const long srb = stats_row_bytes(sampler_chunks((int)V));
  L->sp = align256((size_t)L->logit_rows * srb);
  L->sq = align256((size_t)r.max_batch * r.gamma_max * srb);
  L->resid = align256((size_t)r.max_batch * sampler_chunks((int)V) * 8);
  L->ssq = 2 * align256((size_t)kSsqSlots * R * 8);
  L->xn = align256((size_t)R * d * 2);
  L->out = align256((size_t)(L->max_rows + r.max_batch + 64) * 4);  // + the decode kernel's error word
  L->partial = align256((size_t)16 << 20) * 4;  // 16M floats
  L->counters = align256((size_t)65536 * 4);
  {
    // attention partials: one record of (hd + 2) floats per (work unit, kv head, query row); the worst case
    // is every sequence of the largest batch at max_ctx with gamma_max + 1 query rows
    const size_t units = (size_t)r.max_batch * ((r.max_ctx + 16 * 8 - 1) / (16 * 8));  // units are >= 8 blocks
    const size_t recs = units * hkv * (size_t)(hq / hkv) * G1;
    L->attn = align256(std::max((size_t)8 << 20, recs * (size_t)(hd + 2)) * 4);
  }
  size_t w4 = 0;
  if (dd.quant == ER_W4_G128_ASYM) {
    w4 = std::max({(size_t)qkvN * d / 2, (size_t)d * hq * hd / 2, (size_t)2 * F * d / 2, (size_t)d * F / 2});
    if (dd.quant_lm_head) w4 = std::max(w4, (size_t)V * d / 2);
  }
  L->w4tmp = align256(w4);
  L->sink = 256;
  if (m.dtype == ER_BF16) {
    L->dec = align256((size_t)2 * m.n_layers * sizeof(DecLayerW)) +
             align256(decode_ws_bytes(m.n_layers, (int)d, (int)hq, (int)hd, (int)F, kSsqSlots)) +
             align256((size_t)kDecodeBarWords * 4) + 256;
  }
  L->meta = align256((size_t)64 << 20);
  if (m.dtype == ER_BF16) L->blas = (size_t)64 << 20;  // the library's largest 7B-shaped prefill GEMMs want 64 MiB
  L->block_bytes = (size_t)m.n_layers * 2 * hkv * KV_BLOCK * hd * ab;
  (void)why;
  return 0;
}

int validate(const er_model_desc* m, const er_draft_desc* dd, const er_rollout_desc* r, std::string* why) {
  auto bad = [&](const char* s) { *why = s; return ER_EINVAL; };
  if (!m || !dd || !r) return bad("null description");
  if (m->n_layers <= 0 || m->d_model <= 0 || m->n_q_heads <= 0 || m->n_kv_heads <= 0 || m->ffn <= 0 || m->vocab <= 0)
    return bad("model sizes must be positive");
  if (m->n_q_heads % m->n_kv_heads) return bad("n_q_heads must be a multiple of n_kv_heads");
  if (m->head_dim != 64 && m->head_dim != 128) return bad("head_dim must be 64 or 128");
  if (m->dtype != ER_F32 && m->dtype != ER_BF16) return bad("dtype must be ER_F32 or ER_BF16");
  if (m->d_model % 8 || m->ffn % 8) return bad("d_model and ffn must be multiples of 8");
  if (dd->quant != ER_W8_PERCH_SYM && dd->quant != ER_W4_G128_ASYM) return bad("unknown drafter format");
  if (dd->quant == ER_W4_G128_ASYM) {
    if (m->dtype != ER_BF16) return bad("W4 drafter needs a bf16 model");
    if (dd->group_size != 128) return bad("W4 group_size must be 128");
    if (m->d_model % 128 || m->ffn % 128 || (m->n_q_heads * m->head_dim) % 128)
      return bad("W4 needs every input dimension to be a multiple of 128");
  }
  if (r->kv_block != KV_BLOCK) return bad("kv_block must be 16");
  if (r->gamma_max < 1 || r->gamma_max > 16) return bad("gamma_max must be in 1..16");
  if (r->gamma_min < 1 || r->gamma_min > r->gamma_max) return bad("gamma_min must be in 1..gamma_max");
  if (r->gamma_init < 1 || r->gamma_init > r->gamma_max) return bad("gamma_init must be in 1..gamma_max");
  if (r->max_seqs <= 0 || r->max_batch <= 0 || r->max_batch > r->max_seqs) return bad("bad max_seqs / max_batch");
  if (r->max_ctx <= 0 || r->prefill_chunk <= 0) return bad("bad max_ctx / prefill_chunk");
  if (!(r->temperature >= 0.f)) return bad("temperature must be >= 0");
  if (!(r->top_p > 0.f)) return bad("top_p must be > 0");
  if (r->policy < ER_POLICY_AUTO || r->policy > ER_POLICY_HISTORY) return bad("unknown policy");
  const int grp = m->n_q_heads / m->n_kv_heads;
  if (grp * (r->gamma_max + 1) > 64) return bad("(n_q_heads/n_kv_heads) * (gamma_max+1) must be <= 64");
  return ER_OK;
}

// ---- forward ---------------------------------------------------------------
struct Fwd {
  bool draft = false;
  int M = 0;
  const int32_t* tokens = nullptr;
  int tok_stride = 1;
  const int32_t* pos = nullptr;
  const int64_t* slot = nullptr;
  const int32_t* bt = nullptr;
  int bt_stride = 0;
  const int32_t *it_bt = nullptr, *it_row0 = nullptr, *it_pos0 = nullptr, *it_cnt = nullptr;
  int n_items = 0, max_q = 0, max_ctx = 0;
  const int32_t* unit_start = nullptr;   // attention work units (see push_units); null = uniform splits
  const int32_t* unit_rec = nullptr;     // per-unit records (see push_units), with unit_start
  int n_units = 0, n_split = 0, max_units = 0;
  double kv_keys = 0;                    // sum over items of keys read (for per-kernel flop counts)
  double kv_shared = 0;                  // of those, keys of shared prompt blocks read again by other
                                         // members of a group in the same forward (bytes count them once)
  const int32_t* logit_rows = nullptr;  // rows whose logits are computed (with n_logit > 0)
  int n_logit = -1;                      // -1: every row; 0: none (prefill chunk with no last token)
  float* logits = nullptr;
  long ldl = 0;
  bool dec_ok = false;                   // a decode / draft / verify forward (the persistent kernel may run it)
};

int lin(er_ctx* c, const void* x, int M, const LinearW& W, void* y, int ldy, int epi) {
  const int ldx = W.K;
  LinearInfo li{};
  const int e = kp_begin(c, KPROF_LINEAR);
  KC(c, launch_linear(x, c->bf16, ldx, M, W, y, ldy, epi, c->lws, c->lin_path, c->st, &li));
  if (e >= 0) {
    // algorithmic bytes: weights (with scales/zeros) + activations in + result out (read+write for +=)
    const double by = weight_bytes(W) + (double)M * W.K * c->act_bytes + (double)M * W.N * (epi == EPI_RESID ? 8 : 4);
    kp_end(c, e, li.name, by, 2.0 * M * (double)W.N * W.K);
  }
  return ER_OK;
}

// Fused linear (bf16 models): x' = RMSNorm(h) on load when `xn` (sums of
// squares from ssq_in), epilogue `epi`; residual epilogues accumulate the new
// sums of squares into ssq_acc and clear ssq_zero.
struct FLin {
  const void* x = nullptr;
  int ldx = 0;
  const void* gnorm = nullptr;
  const int32_t* xrow = nullptr;
  const unsigned long long* ssq_in = nullptr;
  unsigned long long* ssq_acc = nullptr;
  unsigned long long* ssq_zero = nullptr;
};

int flin(er_ctx* c, const Fwd& f, const FLin& fl, int M, const LinearW& W, void* y, int ldy, int epi, int layer) {
  const er_model_desc& m = c->md;
  LinArgs a{};
  a.x = fl.x;
  a.ldx = fl.ldx;
  a.M = M;
  a.xnorm = fl.gnorm != nullptr;
  a.xrow = fl.xrow;
  a.ssq_in = fl.ssq_in;
  a.gnorm = fl.gnorm;
  a.eps = m.rms_eps;
  a.W = W;
  a.epi = epi;
  a.y = y;
  a.ldy = ldy;
  a.act_bf16 = 1;
  a.ssq_acc = fl.ssq_acc;
  a.ssq_zero = fl.ssq_zero;
  a.ssq_slots = kSsqSlots;
  a.ssq_stride = c->max_rows;
  a.hq = m.n_q_heads;
  a.hkv = m.n_kv_heads;
  a.hd = m.head_dim;
  a.pos = f.pos;
  a.slot = f.slot;
  a.cs = c->cs;
  a.qout = c->qb;
  a.kv_pool = c->kv_pool;
  a.layer = layer;
  a.n_layers = m.n_layers;
  a.F = m.ffn;
  LinearInfo li{};
  const int e = kp_begin(c, KPROF_LINEAR);
  KC(c, launch_linear_fused(a, c->lws, c->lin_path, c->st, &li));
  if (e >= 0) {
    // algorithmic bytes: weights (with scales/zeros) + x' in (fp32 h when normalized on load) + outputs
    double out_b;
    if (epi == EPI_RESID) out_b = (double)M * W.N * 8;
    else if (epi == EPI_SWIGLU) out_b = (double)M * (W.N / 2) * 2;
    else if (epi == EPI_QKV) out_b = (double)M * W.N * 2;
    else out_b = (double)M * W.N * 4;
    const double by = weight_bytes(W) + (double)M * W.K * (a.xnorm ? 4 : 2) + out_b;
    kp_end(c, e, li.name, by, 2.0 * M * (double)W.N * W.K);
  }
  return ER_OK;
}

// Final norm + lm_head over the rows that need logits.
int logits_tail(er_ctx* c, const Fwd& f) {
  const er_model_desc& m = c->md;
  const int d = m.d_model;
  const int nl = f.n_logit < 0 ? f.M : f.n_logit;
  if (nl == 0) return ER_OK;
  const LinearW& lm = f.draft ? c->lm_d : c->lm_t;
  if (c->fuse) {
    FLin h;
    h.x = c->h;
    h.ldx = d;
    h.gnorm = c->final_norm;
    h.xrow = f.logit_rows;
    h.ssq_in = c->ssq[0];
    return flin(c, f, h, nl, lm, f.logits, (int)f.ldl, EPI_F32, 0);
  }
  KC(c, launch_rmsnorm(c->h, nl, d, c->final_norm, c->bf16, m.rms_eps, c->xbuf, f.logit_rows, c->st));
  return lin(c, c->xbuf, nl, lm, f.logits, (int)f.ldl, EPI_F32);
}

double layers_weight_bytes(const er_ctx* c, bool draft) {
  const std::vector<Lin4>& W = draft ? c->drf : c->tgt;
  double b = 0;
  for (const Lin4& l : W) b += weight_bytes(l.qkv) + weight_bytes(l.o) + weight_bytes(l.gu) + weight_bytes(l.down);
  return b;
}

// The embedding and every decoder layer as one persistent launch (k_decode).
// Returns ER_OK when it ran, 1 when this forward does not fit it (the caller
// runs the kernel sequence), or an error.
int forward_decode(er_ctx* c, const Fwd& f) {
  const er_model_desc& m = c->md;
  const int hq = m.n_q_heads, hkv = m.n_kv_heads, hd = m.head_dim;
  const int fmt = f.draft ? c->drf[0].qkv.fmt : FMT_BF16;
  if (!c->dec_on || !f.dec_ok || !c->fuse || f.M > kDecodeMaxRows || !f.unit_start || !f.unit_rec) return 1;
  if (c->dec_nwg[fmt] <= 0 || !c->dec_layers[f.draft ? 1 : 0]) return 1;
  if ((size_t)f.n_units * hkv * (size_t)(hq / hkv) * f.max_q * (size_t)(hd + 2) > c->attn_ws_floats) return 1;
  if ((hq / hkv) * f.max_q > 64 ||
      decode_lds_bytes(hd, f.M, m.d_model, std::max({(hq + 2 * hkv) * hd, m.d_model, 2 * m.ffn}), c->dec_nwg[fmt]) >
          (size_t)150 * 1024)
    return 1;
  DecodeArgs a{};
  a.M = f.M;
  a.L = m.n_layers;
  a.d = m.d_model;
  a.hq = hq;
  a.hkv = hkv;
  a.hd = hd;
  a.F = m.ffn;
  a.eps = m.rms_eps;
  a.layers = c->dec_layers[f.draft ? 1 : 0];
  a.embed = c->embed;
  a.tokens = f.tokens;
  a.tok_stride = f.tok_stride;
  a.pos = f.pos;
  a.slot = f.slot;
  a.cs = c->cs;
  a.kv_pool = c->kv_pool;
  a.block_table = f.bt;
  a.bt_stride = f.bt_stride;
  a.unit_rec = f.unit_rec;
  a.unit_start = f.unit_start;
  a.split_items = f.unit_start + 2 * f.n_items + 1;
  a.item_q_row0 = f.it_row0;
  a.item_q_count = f.it_cnt;
  a.n_items = f.n_items;
  a.n_units = f.n_units;
  a.n_split = f.n_split;
  a.max_q = f.max_q;
  {
    // write-once buffers: h per layer boundary, q / attention output / SwiGLU output per layer, sums of squares
    const long L = m.n_layers, d = m.d_model, qn = (long)hq * hd, F = m.ffn;
    char* p = c->dec_ws;
    a.hbuf = (float*)p;
    p += align256((size_t)2 * L * 16 * d * 4);
    a.qbuf = (uint16_t*)p;
    p += align256((size_t)L * 16 * qn * 2);
    a.abuf = (uint16_t*)p;
    p += align256((size_t)L * 16 * qn * 2);
    a.act = (uint16_t*)p;
    p += align256((size_t)L * 16 * F * 2);
    a.ssq = (unsigned long long*)p;
  }
  a.h_final = c->h;
  a.apart = c->attn_ws;
  a.ssq_out = c->ssq[0];
  a.ssq_slots = kSsqSlots;
  a.ssq_stride = c->max_rows;
  a.bar = c->dec_bar;
  a.err = c->dec_err;
  for (int i = 0; i < 4; ++i) a.ks[i] = c->dec_ks[f.draft ? 1 : 0][i];
  a.n_wg = c->dec_nwg[fmt];
  a.spin_limit = c->dec_spin_limit;
  a.trace = c->dec_trace;
  a.trace_max = c->dec_trace_max;
  if (c->dec_trace) c->dec_trace_nwg = a.n_wg;
  const int e = kp_begin(c, KPROF_LINEAR | KPROF_ATTENTION);
  KC(c, launch_decode(a, fmt, c->st));
  c->dec_ran = true;
  if (e >= 0) {
    // algorithmic bytes: every layer's weights (with scales / zeros), the K/V
    // read and written, the embedding rows; flops of the projections and attention
    const double kvb = 2.0 * hkv * hd * c->act_bytes;
    const double by = layers_weight_bytes(c, f.draft) + (f.kv_keys - f.kv_shared + f.M) * kvb * m.n_layers +
                      (double)f.M * m.d_model * c->act_bytes;
    const double P = c->cost.p_lin() - (double)m.vocab * m.d_model;
    char nm[64];
    snprintf(nm, sizeof nm, "er::k_decode<%d, %d>", fmt, hd);
    kp_end(c, e, nm, by, 2.0 * P * f.M + 4.0 * f.kv_keys * f.max_q * (double)hq * hd * m.n_layers);
  }
  return ER_OK;
}

int forward(er_ctx* c, const Fwd& f) {
  const er_model_desc& m = c->md;
  const int d = m.d_model, hq = m.n_q_heads, hkv = m.n_kv_heads, hd = m.head_dim, F = m.ffn;
  {
    const int r = forward_decode(c, f);
    if (r == ER_OK) return logits_tail(c, f);
    if (r < 0) return r;
  }
  const std::vector<Lin4>& W = f.draft ? c->drf : c->tgt;
  unsigned long long* S0 = c->ssq[0];
  unsigned long long* S1 = c->ssq[1];
  KC(c, launch_embed(f.tokens, f.tok_stride, f.M, c->embed, c->bf16, d, c->h, c->fuse ? S0 : nullptr,
                     c->fuse ? S1 : nullptr, c->st, kSsqSlots, c->max_rows));
  AttnArgs a{};
  a.q = c->qb;
  a.out = c->xbuf;
  a.kv_pool = c->kv_pool;
  a.block_table = f.bt;
  a.bt_stride = f.bt_stride;
  a.item_bt_row = f.it_bt;
  a.item_q_row0 = f.it_row0;
  a.item_q_pos0 = f.it_pos0;
  a.item_q_count = f.it_cnt;
  a.n_items = f.n_items;
  a.max_q_count = f.max_q;
  a.max_ctx = f.max_ctx;
  a.unit_start = f.unit_start;
  a.unit_rec = f.unit_start ? f.unit_rec : nullptr;
  a.n_units = f.n_units;
  a.split_items = f.unit_start ? f.unit_start + 2 * f.n_items + 1 : nullptr;
  a.n_split = f.n_split;
  a.max_units = f.max_units;
  if (a.unit_start &&
      (size_t)a.n_units * hkv * (size_t)(hq / hkv) * f.max_q * (size_t)(hd + 2) > c->attn_ws_floats)
    a.unit_start = a.unit_rec = nullptr;  // more units than the partials area holds: uniform splits instead
  a.hq = hq;
  a.hkv = hkv;
  a.hd = hd;
  a.n_layers = m.n_layers;
  a.bf16 = c->bf16;
  a.ws = c->attn_ws;
  a.ws_floats = c->attn_ws_floats;
  for (int l = 0; l < m.n_layers; ++l) {
    int r;
    if (c->fuse) {
      // h (sums of squares in S0) -> norm -> qkv with RoPE and the KV append
      FLin q;
      q.x = c->h;
      q.ldx = d;
      q.gnorm = c->attn_norm[l];
      q.ssq_in = S0;
      r = flin(c, f, q, f.M, W[l].qkv, nullptr, 0, EPI_QKV, l);
    } else {
      KC(c, launch_rmsnorm(c->h, f.M, d, c->attn_norm[l], c->bf16, m.rms_eps, c->xbuf, nullptr, c->st));
      r = lin(c, c->xbuf, f.M, W[l].qkv, c->qkv, (hq + 2 * hkv) * hd, EPI_F32);
      if (r) return r;
      KC(c, launch_rope_kv(c->qkv, f.M, hq, hkv, hd, f.pos, f.slot, c->cs, c->qb, c->kv_pool, l, m.n_layers, c->bf16,
                           c->st));
    }
    if (r) return r;
    a.layer = l;
    {
      // scoring kernel and (when keys were split) the combine, timed apart
      int e = kp_begin(c, KPROF_ATTENTION);
      int combined = 0;
      KC(c, launch_attention(a, c->st, 1, &combined));
      if (e >= 0) {
        const double kvb = 2.0 * hkv * hd * c->act_bytes;  // K and V of one position, one layer
        const double by = (f.kv_keys - f.kv_shared) * kvb + 2.0 * f.M * hq * hd * c->act_bytes;
        const char* nm = !c->bf16 ? "er::k_attn_valu" : (hd == 128 ? "er::k_attn_mfma<128, 4>" : "er::k_attn_mfma<64, 4>");
        static_assert(kAttnWaves == 4, "kernel-profile names carry the wave count");
        kp_end(c, e, nm, by, 4.0 * f.kv_keys * f.max_q * (double)hq * hd);
      }
      if (combined) {
        e = kp_begin(c, KPROF_ATTENTION);
        KC(c, launch_attention(a, c->st, 2));
        if (e >= 0) {
          const double units = a.unit_start ? (double)a.n_units : (double)f.n_items;
          const double by = units * hkv * (double)(hq / hkv) * f.max_q * (hd + 2) * 4.0 + 2.0 * f.M * hq * hd * c->act_bytes;
          kp_end(c, e, c->bf16 ? "er::k_attn_combine<true>" : "er::k_attn_combine<false>", by, 0.0);
        }
      }
    }
    if (c->fuse) {
      FLin o;  // h += attn W_o^T; new sums of squares -> S1; S0 (read above) cleared
      o.x = c->xbuf;
      o.ldx = hq * hd;
      o.ssq_acc = S1;
      o.ssq_zero = S0;
      r = flin(c, f, o, f.M, W[l].o, c->h, d, EPI_RESID, l);
      if (r) return r;
      FLin g;  // norm(h) -> gate/up -> SwiGLU
      g.x = c->h;
      g.ldx = d;
      g.gnorm = c->mlp_norm[l];
      g.ssq_in = S1;
      r = flin(c, f, g, f.M, W[l].gu, c->xbuf, F, EPI_SWIGLU, l);
      if (r) return r;
      FLin dn;  // h += act W_down^T; sums of squares -> S0; S1 cleared
      dn.x = c->xbuf;
      dn.ldx = F;
      dn.ssq_acc = S0;
      dn.ssq_zero = S1;
      r = flin(c, f, dn, f.M, W[l].down, c->h, d, EPI_RESID, l);
      if (r) return r;
      continue;
    }
    r = lin(c, c->xbuf, f.M, W[l].o, c->h, d, EPI_RESID);
    if (r) return r;
    KC(c, launch_rmsnorm(c->h, f.M, d, c->mlp_norm[l], c->bf16, m.rms_eps, c->xbuf, nullptr, c->st));
    r = lin(c, c->xbuf, f.M, W[l].gu, c->gu, 2 * F, EPI_F32);
    if (r) return r;
    KC(c, launch_swiglu(c->gu, f.M, F, c->xbuf, c->bf16, c->st));
    r = lin(c, c->xbuf, f.M, W[l].down, c->h, d, EPI_RESID);
    if (r) return r;
  }
  return logits_tail(c, f);
}

// ---- drafter build (A0) -----------------------------------------------------
int quantize_into(er_ctx* c, const void* W, long N, long K, LinearW* out, char** cursor) {
  out->N = (int)N;
  out->K = (int)K;
  if (c->dd.quant == ER_W8_PERCH_SYM) {
    out->fmt = FMT_W8;
    int8_t* q = (int8_t*)*cursor;
    *cursor += align256((size_t)N * K);
    float* s = (float*)*cursor;
    *cursor += align256((size_t)N * 4);
    KC(c, launch_quantize_w8(W, c->bf16, (int)N, (int)K, q, s, c->st));
    out->w = q;
    out->scale = s;
    out->zero = nullptr;
  } else {
    out->fmt = FMT_W4;
    const long G = K / 128;
    uint8_t* p = (uint8_t*)*cursor;
    *cursor += align256((size_t)N * K / 2);
    uint16_t* s = (uint16_t*)*cursor;
    *cursor += align256((size_t)N * G * 2);
    uint8_t* z = (uint8_t*)*cursor;
    *cursor += align256((size_t)N * G);
    KC(c, launch_quantize_w4(W, (int)N, (int)K, c->w4_tmp, s, z, c->st));
    KC(c, launch_w4_to_kernel_order(c->w4_tmp, (int)N, (int)K, p, c->st));
    out->w = p;
    out->scale = s;
    out->zero = z;
  }
  return ER_OK;
}

int set_weights(er_ctx* c, const er_weights* w) {
  const er_model_desc& m = c->md;
  graph_drop(c);  // recorded graphs hold the old weight pointers
  if (!w || !w->embed || !w->final_norm || !w->lm_head || !w->attn_norm || !w->wqkv || !w->wo || !w->mlp_norm ||
      !w->wgate_up || !w->wdown)
    return fail(c, ER_EINVAL, "null weight pointer");
  const long d = m.d_model, hq = m.n_q_heads, hkv = m.n_kv_heads, hd = m.head_dim, F = m.ffn, V = m.vocab;
  const int tf = c->bf16 ? FMT_BF16 : FMT_F32;
  c->embed = w->embed;
  c->final_norm = w->final_norm;
  c->attn_norm.assign(w->attn_norm, w->attn_norm + m.n_layers);
  c->mlp_norm.assign(w->mlp_norm, w->mlp_norm + m.n_layers);
  c->tgt.resize(m.n_layers);
  c->drf.resize(m.n_layers);
  for (int l = 0; l < m.n_layers; ++l) {
    if (!w->attn_norm[l] || !w->wqkv[l] || !w->wo[l] || !w->mlp_norm[l] || !w->wgate_up[l] || !w->wdown[l])
      return fail(c, ER_EINVAL, "null weight pointer in layer %d", l);
    c->tgt[l].qkv = LinearW{tf, w->wqkv[l], nullptr, nullptr, (int)((hq + 2 * hkv) * hd), (int)d};
    c->tgt[l].o = LinearW{tf, w->wo[l], nullptr, nullptr, (int)d, (int)(hq * hd)};
    c->tgt[l].gu = LinearW{tf, w->wgate_up[l], nullptr, nullptr, (int)(2 * F), (int)d};
    c->tgt[l].down = LinearW{tf, w->wdown[l], nullptr, nullptr, (int)d, (int)F};
  }
  c->lm_t = LinearW{tf, w->lm_head, nullptr, nullptr, (int)V, (int)d};
  char* cur = c->arena;  // the drafter pack sits at the start of the arena
  for (int l = 0; l < m.n_layers; ++l) {
    int r;
    if ((r = quantize_into(c, c->tgt[l].qkv.w, c->tgt[l].qkv.N, d, &c->drf[l].qkv, &cur))) return r;
    if ((r = quantize_into(c, c->tgt[l].o.w, d, hq * hd, &c->drf[l].o, &cur))) return r;
    if ((r = quantize_into(c, c->tgt[l].gu.w, 2 * F, d, &c->drf[l].gu, &cur))) return r;
    if ((r = quantize_into(c, c->tgt[l].down.w, d, F, &c->drf[l].down, &cur))) return r;
  }
  if (c->dd.quant_lm_head) {
    int r;
    if ((r = quantize_into(c, w->lm_head, V, d, &c->lm_d, &cur))) return r;
  } else {
    c->lm_d = c->lm_t;
  }
  if (c->dec_layers[0]) {
    // layer descriptors of the persistent decode forward (target, drafter)
    for (int which = 0; which < 2; ++which) {
      std::vector<DecLayerW> v((size_t)m.n_layers);
      const std::vector<Lin4>& W = which ? c->drf : c->tgt;
      for (int l = 0; l < m.n_layers; ++l)
        v[(size_t)l] = DecLayerW{W[l].qkv, W[l].o, W[l].gu, W[l].down, c->attn_norm[l], c->mlp_norm[l]};
      HIPC(c, hipMemcpyAsync(c->dec_layers[which], v.data(), v.size() * sizeof(DecLayerW), hipMemcpyHostToDevice,
                             c->st));
      HIPC(c, hipStreamSynchronize(c->st));
    }
  }
  HIPC(c, hipStreamSynchronize(c->st));
  return ER_OK;
}

// ---- sequences --------------------------------------------------------------
int check_batch(er_ctx* c, int n, const int32_t* ids, bool need_prefilled) {
  if (n <= 0 || !ids) return fail(c, ER_EINVAL, "empty batch");
  if (n > c->rd.max_batch) return fail(c, ER_EINVAL, "batch %d exceeds max_batch %d", n, c->rd.max_batch);
  for (int i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || id >= (int32_t)c->seqs.size() || !c->seqs[id].alive)
      return fail(c, ER_EINVAL, "unknown sequence id %d", id);
    const Seq& s = c->seqs[id];
    if (need_prefilled && !s.prefilled) return fail(c, ER_ESTATE, "sequence %d not prefilled", id);
    if (need_prefilled && s.finished) return fail(c, ER_ESTATE, "sequence %d already finished", id);
    for (int j = 0; j < i; ++j)
      if (ids[j] == id) return fail(c, ER_EINVAL, "sequence %d listed twice", id);
  }
  return ER_OK;
}

bool timed_step(er_ctx* c) {
  if (!c->have_ev) return false;
  if (c->step_count < c->timing_first) return true;
  return c->timing_period > 0 && (c->step_count % c->timing_period) == 0;
}

float ev_ms(er_ctx* c, int a, int b) {
  float ms = 0.f;
  if (hipEventElapsedTime(&ms, c->ev[a], c->ev[b]) != hipSuccess) return 0.f;
  return ms;
}

// Build the block table of a batch into the metadata region.
int32_t* put_block_table(er_ctx* c, int n, const int32_t* ids, int* stride, size_t* off) {
  size_t mx = 1;
  for (int i = 0; i < n; ++i) mx = std::max(mx, c->seqs[ids[i]].bt.blocks.size());
  *stride = (int)mx;
  int32_t* bt = c->meta.push<int32_t>((size_t)n * mx, off);
  if (!bt) return nullptr;
  for (int i = 0; i < n; ++i) {
    const auto& b = c->seqs[ids[i]].bt.blocks;
    for (size_t j = 0; j < mx; ++j) bt[(size_t)i * mx + j] = j < b.size() ? b[j] : 0;
  }
  return bt;
}

// The block table of a graph step: nb rows of stride cap; rows n .. nb-1
// (padding) name only the padding block.
int32_t* put_block_table_padded(er_ctx* c, int n, int nb, const int32_t* ids, int cap, size_t* off) {
  int32_t* bt = c->meta.push<int32_t>((size_t)nb * cap, off);
  if (!bt) return nullptr;
  for (int i = 0; i < nb; ++i) {
    int32_t* row = bt + (size_t)i * cap;
    if (i >= n) {
      row[0] = c->pad_block;
      for (int j = 1; j < cap; ++j) row[j] = 0;
      continue;
    }
    const auto& b = c->seqs[ids[i]].bt.blocks;
    for (int j = 0; j < cap; ++j) row[j] = (size_t)j < b.size() ? b[(size_t)j] : 0;
  }
  return bt;
}

int64_t slot_of(const Seq& s, int32_t pos) {
  return (int64_t)s.bt.blocks[(size_t)(pos / KV_BLOCK)] * KV_BLOCK + (pos % KV_BLOCK);
}

void finish_seq(er_ctx* c, Seq& s) {
  s.finished = true;
  s.bt.release(c->pool);
}

// Queue the copy of the persistent decode kernel's error word (if it ran).
int dec_queue_err(er_ctx* c) {
  if (c->dec_ran) HIPC(c, hipMemcpyAsync(c->out_h + c->dec_err_slot, c->dec_err, 4, hipMemcpyDeviceToHost, c->st));
  return ER_OK;
}

// After the stream is synchronized: did a grid-barrier wait of the persistent
// decode kernel time out?  Then that path is switched off for the context and
// its barrier words are cleared.
int dec_check(er_ctx* c) {
  if (!c->dec_ran) return ER_OK;
  c->dec_ran = false;
  if (c->out_h[c->dec_err_slot] == 0) return ER_OK;
  c->out_h[c->dec_err_slot] = 0;
  c->dec_on = false;
  HIPC(c, hipMemsetAsync(c->dec_bar, 0, (size_t)kDecodeBarWords * 4, c->st));
  HIPC(c, hipMemsetAsync(c->dec_err, 0, 4, c->st));
  HIPC(c, hipStreamSynchronize(c->st));
  return fail(c, ER_EDEVICE, "persistent decode forward: a grid-barrier wait timed out (path switched off)");
}

// Keys of shared blocks that more than one of the n sequences read: a family
// (share group, or a sequence and its forks) shares its leading full blocks,
// so every member after the first one in the batch reads
// floor(shared_len / 16) * 16 keys another member reads too.
double shared_keys(const er_ctx* c, int n, const int32_t* ids) {
  double dup = 0;
  std::vector<int32_t> seen;
  for (int i = 0; i < n; ++i) {
    const Seq& s = c->seqs[ids[i]];
    if (s.family == -1) continue;
    if (std::find(seen.begin(), seen.end(), s.family) != seen.end())
      dup += (double)(s.shared_len / KV_BLOCK) * KV_BLOCK;
    else
      seen.push_back(s.family);
  }
  return dup;
}

int do_ar(er_ctx* c, int n, const int32_t* ids, int32_t* tokens_out, int out_stride, int32_t* n_emitted,
          er_step_info* info) {
  const bool timed = timed_step(c);
  std::vector<size_t> had(n);
  for (int i = 0; i < n; ++i) {
    Seq& s = c->seqs[ids[i]];
    had[i] = s.bt.blocks.size();
    if (!s.bt.reserve(c->pool, (int64_t)s.n + 1)) {
      for (int j = 0; j < i; ++j) c->seqs[ids[j]].bt.truncate(c->pool, (int64_t)had[j] * KV_BLOCK);
      return fail(c, ER_ENOMEM, "KV pool exhausted (%lld free blocks)", (long long)c->pool.free_count());
    }
  }
  auto rollback = [&]() {
    for (int j = 0; j < n; ++j) c->seqs[ids[j]].bt.truncate(c->pool, (int64_t)c->seqs[ids[j]].n);
  };
  // graph steps run nr = nb rows; padding rows n .. nr-1 decode token 0 at
  // position 0 of the padding block and are dropped
  const GraphPlan gp = graph_plan(c, n, ids, 1);
  const int nr = gp.nb ? gp.nb : n;
  Meta& M = c->meta;
  if (int r_ = meta_begin(c)) { rollback(); return r_; }
  size_t o_ids, o_tok, o_pos, o_spos, o_slot, o_bt, o_ib, o_ir, o_ip, o_ic;
  int32_t* h_ids = M.push<int32_t>(nr, &o_ids);
  int32_t* h_tok = M.push<int32_t>(nr, &o_tok);
  int32_t* h_pos = M.push<int32_t>(nr, &o_pos);
  int32_t* h_spos = M.push<int32_t>(nr, &o_spos);
  int64_t* h_slot = M.push<int64_t>(nr, &o_slot);
  int stride = gp.cap;
  int32_t* h_bt =
      gp.nb ? put_block_table_padded(c, n, nr, ids, gp.cap, &o_bt) : put_block_table(c, n, ids, &stride, &o_bt);
  int32_t* h_ib = M.push<int32_t>(nr, &o_ib);
  int32_t* h_ir = M.push<int32_t>(nr, &o_ir);
  int32_t* h_ip = M.push<int32_t>(nr, &o_ip);
  int32_t* h_ic = M.push<int32_t>(nr, &o_ic);
  if (!M.ok || !h_bt) { rollback(); return fail(c, ER_ENOMEM, "metadata region too small"); }
  int max_ctx = 1;
  double kv_keys = 0;
  for (int i = 0; i < nr; ++i) {
    h_ib[i] = i;
    h_ir[i] = i;
    h_ic[i] = 1;
    if (i >= n) {
      h_ids[i] = -1;
      h_tok[i] = 0;
      h_pos[i] = 0;
      h_spos[i] = 1;
      h_slot[i] = (int64_t)c->pad_block * KV_BLOCK;
      h_ip[i] = 0;
      continue;
    }
    const Seq& s = c->seqs[ids[i]];
    kv_keys += s.n + 1;
    h_ids[i] = ids[i];
    h_tok[i] = s.pending;
    h_pos[i] = s.n;
    h_spos[i] = s.n + 1;
    h_slot[i] = slot_of(s, s.n);
    h_ip[i] = s.n;
    max_ctx = std::max(max_ctx, s.n + 1);
  }
  int n_units = 0;
  int n_split = 0;
  int max_units = 0;
  size_t o_rec = 0;
  size_t o_us;
  if (gp.nb) {
    o_us = push_units_fixed(M, nr, gp.U, h_ip, h_ic, h_ir, h_ib, &o_rec);
    n_units = nr * gp.U;
    n_split = gp.U > 1 ? nr : 0;
    max_units = gp.U;
    max_ctx = gp.cap * KV_BLOCK;
  } else {
    o_us = push_units(M, n, (int)c->md.n_kv_heads, h_ip, h_ic, h_ir, h_ib, &n_units, &n_split, &max_units, &o_rec);
  }
  if (!M.ok) { rollback(); return fail(c, ER_ENOMEM, "metadata region too small"); }
  // the step's kernels: target forward over nr rows, then the AR draw (mid:
  // record the event between the two, on eager timed steps)
  auto ar_body = [&](bool mid) -> int {
    Fwd f;
    f.draft = false;
    f.dec_ok = true;
    f.M = nr;
    f.tokens = M.dev<int32_t>(o_tok);
    f.pos = M.dev<int32_t>(o_pos);
    f.slot = M.dev<int64_t>(o_slot);
    f.bt = M.dev<int32_t>(o_bt);
    f.bt_stride = stride;
    f.it_bt = M.dev<int32_t>(o_ib);
    f.it_row0 = M.dev<int32_t>(o_ir);
    f.it_pos0 = M.dev<int32_t>(o_ip);
    f.it_cnt = M.dev<int32_t>(o_ic);
    f.n_items = nr;
    f.max_q = 1;
    f.max_ctx = max_ctx;
    f.unit_start = M.dev<int32_t>(o_us);
    f.unit_rec = M.dev<int32_t>(o_rec);
    f.n_units = n_units;
    f.n_split = n_split;
    f.max_units = max_units;
    f.kv_keys = kv_keys;
    f.kv_shared = shared_keys(c, n, ids);
    f.logits = c->logits_p;
    f.ldl = c->md.vocab;
    int r = forward(c, f);
    if (r) return r;
    if (mid) HIPC(c, hipEventRecord(c->ev[1], c->st));
    KC(c, launch_row_stats(c->logits_p, nr, c->md.vocab, c->md.vocab, c->rd.temperature, c->rd.top_p, c->stats_p,
                           c->st));
    KC(c, launch_sample_rows(c->logits_p, c->stats_p, nr, c->md.vocab, c->md.vocab, c->rd.temperature, c->rd.top_p,
                             c->rd.seed, M.dev<int32_t>(o_ids), M.dev<int32_t>(o_spos), 0, PURPOSE_AR, c->out_d, 1,
                             nullptr, c->st));
    return ER_OK;
  };
  auto run = [&]() -> int {
    if (int r_ = meta_upload(c)) return r_;
    if (timed) HIPC(c, hipEventRecord(c->ev[0], c->st));
    if (gp.nb) {
      // one graph: forward and draw (the split between them is not timed)
      HIPC_OK(graph_run(c, GRAPH_AR, nr, 0, gp.cap, [&]() { return ar_body(false); }));
      if (timed) HIPC(c, hipEventRecord(c->ev[1], c->st));
    } else {
      HIPC_OK(ar_body(timed));
    }
    if (timed) HIPC(c, hipEventRecord(c->ev[2], c->st));
    HIPC(c, hipMemcpyAsync(c->out_h, c->out_d, (size_t)n * 4, hipMemcpyDeviceToHost, c->st));
    if (int r_ = dec_queue_err(c)) return r_;
    HIPC(c, hipStreamSynchronize(c->st));
    return dec_check(c);
  };
  c->dec_ran = false;
  const int r = run();
  kp_flush(c);
  if (r) { rollback(); return r; }
  // commit
  int kept_tot = 0, fin = 0;
  for (int i = 0; i < n; ++i) {
    Seq& s = c->seqs[ids[i]];
    const int32_t t = c->out_h[i];
    s.n += 1;
    s.pending = t;
    s.generated += 1;
    s.toks.push_back(t);
    tokens_out[(size_t)i * out_stride] = t;
    if (n_emitted) n_emitted[i] = 1;
    ++kept_tot;
    if (s.generated >= s.max_new) { finish_seq(c, s); ++fin; }
  }
  c->stats.ar_steps += 1;
  c->stats.emitted += n;
  c->stats.tokens_kept += kept_tot;
  float ms_f = 0.f, ms_s = 0.f;
  if (timed) {
    ms_f = ev_ms(c, 0, 1);
    ms_s = ev_ms(c, 1, 2);
    c->stats.ms_ar += ms_f + ms_s;
  }
  c->last_mode = ER_MODE_AR;
  c->last_gamma = 0;
  c->last_B = n;
  c->last_rows = nr;
  if (info) {
    *info = er_step_info{};
    info->mode = ER_MODE_AR;
    info->gamma = 0;
    info->batch = n;
    info->emitted = n;
    info->kept = kept_tot;
    info->finished = fin;
    info->alpha_ema = (float)c->alpha_ema;
    info->ms_verify = ms_f;
    info->ms_sample = ms_s;
    info->ms_total = ms_f + ms_s;
  }
  ++c->step_count;
  return ER_OK;
}

// One speculative step.  hdraft (host, [n][g]) null: the self-drafter proposes g
// tokens per sequence; else those tokens are the drafts (copied from earlier
// rollouts, not sampled) and their proposal is the point mass on each.
int do_spec(er_ctx* c, int n, const int32_t* ids, int g, int32_t* tokens_out, int out_stride, int32_t* n_emitted,
            er_step_info* info, const int32_t* hdraft = nullptr) {
  const bool timed = timed_step(c);
  const int G1 = g + 1;
  const int V = c->md.vocab;
  std::vector<size_t> had(n);
  for (int i = 0; i < n; ++i) {
    Seq& s = c->seqs[ids[i]];
    had[i] = s.bt.blocks.size();
    if (!s.bt.reserve(c->pool, (int64_t)s.n + G1)) {
      for (int j = 0; j < i; ++j) c->seqs[ids[j]].bt.truncate(c->pool, (int64_t)had[j] * KV_BLOCK);
      return fail(c, ER_ENOMEM, "KV pool exhausted (%lld free blocks)", (long long)c->pool.free_count());
    }
  }
  auto rollback = [&]() {
    for (int j = 0; j < n; ++j) c->seqs[ids[j]].bt.truncate(c->pool, (int64_t)c->seqs[ids[j]].n);
  };
  // graph steps run nr = nb padded sequences; padding sequences draft and
  // verify from token 0 at position 0 of the padding block and are dropped
  const GraphPlan gp = graph_plan(c, n, ids, G1);
  const int nr = gp.nb ? gp.nb : n;
  Meta& M = c->meta;
  if (int r_ = meta_begin(c)) { rollback(); return r_; }
  size_t o_ids, o_pos0, o_tok, o_bt;
  int32_t* h_ids = M.push<int32_t>(nr, &o_ids);
  int32_t* h_pos0 = M.push<int32_t>(nr, &o_pos0);
  int32_t* h_tok = M.push<int32_t>((size_t)nr * G1, &o_tok);
  int stride = gp.cap;
  int32_t* h_bt =
      gp.nb ? put_block_table_padded(c, n, nr, ids, gp.cap, &o_bt) : put_block_table(c, n, ids, &stride, &o_bt);
  // per draft step j (1..g): positions, slots, items (bt row, q row0, pos0, count), sample positions
  std::vector<size_t> o_dp(g), o_ds(g), o_dsp(g);
  size_t o_ib, o_ir, o_ic, o_vp, o_vs, o_vir, o_vic;
  std::vector<int32_t*> h_dp(g), h_dsp(g);
  std::vector<int64_t*> h_ds(g);
  for (int j = 0; j < g; ++j) {
    h_dp[j] = M.push<int32_t>(nr, &o_dp[j]);
    h_ds[j] = M.push<int64_t>(nr, &o_ds[j]);
    h_dsp[j] = M.push<int32_t>(nr, &o_dsp[j]);
  }
  int32_t* h_ib = M.push<int32_t>(nr, &o_ib);   // item b -> block-table row b (draft and verify)
  int32_t* h_ir = M.push<int32_t>(nr, &o_ir);   // draft: q row b
  int32_t* h_ic = M.push<int32_t>(nr, &o_ic);   // draft: 1 query
  int32_t* h_vp = M.push<int32_t>((size_t)nr * G1, &o_vp);
  int64_t* h_vs = M.push<int64_t>((size_t)nr * G1, &o_vs);
  int32_t* h_vir = M.push<int32_t>(nr, &o_vir);  // verify: q row b*G1
  int32_t* h_vic = M.push<int32_t>(nr, &o_vic);  // verify: G1 queries
  if (!M.ok || !h_bt) { rollback(); return fail(c, ER_ENOMEM, "metadata region too small"); }
  int max_ctx = 1;
  double kv_sum = 0;
  for (int b = 0; b < nr; ++b) {
    const bool pad = b >= n;
    const Seq* s = pad ? nullptr : &c->seqs[ids[b]];
    const int32_t n0 = pad ? 0 : s->n;
    const int64_t pslot = (int64_t)c->pad_block * KV_BLOCK;
    if (!pad) kv_sum += n0;
    h_ids[b] = pad ? -1 : ids[b];
    h_pos0[b] = n0;
    h_tok[(size_t)b * G1] = pad ? 0 : s->pending;
    for (int i = 1; i < G1; ++i) h_tok[(size_t)b * G1 + i] = (hdraft && !pad) ? hdraft[(size_t)b * g + i - 1] : 0;
    for (int j = 0; j < g; ++j) {
      h_dp[j][b] = n0 + j;
      h_ds[j][b] = pad ? pslot + j : slot_of(*s, n0 + j);
      h_dsp[j][b] = n0 + j + 1;
    }
    h_ib[b] = b;
    h_ir[b] = b;
    h_ic[b] = 1;
    for (int i = 0; i < G1; ++i) {
      h_vp[(size_t)b * G1 + i] = n0 + i;
      h_vs[(size_t)b * G1 + i] = pad ? pslot + i : slot_of(*s, n0 + i);
    }
    h_vir[b] = b * G1;
    h_vic[b] = G1;
    if (!pad) max_ctx = std::max(max_ctx, n0 + G1);
  }
  std::vector<size_t> o_dus(g);
  std::vector<int> n_dus(g);
  std::vector<int> s_dus(g);
  std::vector<int> m_dus(g);
  std::vector<size_t> o_drec(g);
  int n_vus = 0;
  int s_vus = 0;
  int m_vus = 0;
  size_t o_vrec = 0;
  size_t o_vus;
  if (gp.nb) {
    for (int j = 0; j < g; ++j) {
      o_dus[j] = push_units_fixed(M, nr, gp.U, h_dp[j], h_ic, h_ir, h_ib, &o_drec[j]);
      n_dus[j] = nr * gp.U;
      s_dus[j] = gp.U > 1 ? nr : 0;
      m_dus[j] = gp.U;
    }
    o_vus = push_units_fixed(M, nr, gp.U, h_pos0, h_vic, h_vir, h_ib, &o_vrec);
    n_vus = nr * gp.U;
    s_vus = gp.U > 1 ? nr : 0;
    m_vus = gp.U;
    max_ctx = gp.cap * KV_BLOCK;
  } else {
    for (int j = 0; j < g; ++j)
      o_dus[j] = push_units(M, n, (int)c->md.n_kv_heads, h_dp[j], h_ic, h_ir, h_ib, &n_dus[j], &s_dus[j], &m_dus[j],
                            &o_drec[j]);
    o_vus = push_units(M, n, (int)c->md.n_kv_heads, h_pos0, h_vic, h_vir, h_ib, &n_vus, &s_vus, &m_vus, &o_vrec);
  }
  if (!M.ok) { rollback(); return fail(c, ER_ENOMEM, "metadata region too small"); }
  const double kv_dup = shared_keys(c, n, ids);
  int32_t* d_tok = M.dev<int32_t>(o_tok);
  // the drafter's g forwards over nr rows, each followed by its draw
  auto draft_body = [&]() -> int {
    for (int j = 0; j < g; ++j) {
      Fwd f;
      f.draft = true;
      f.dec_ok = true;
      f.M = nr;
      f.tokens = d_tok + j;
      f.tok_stride = G1;
      f.pos = M.dev<int32_t>(o_dp[j]);
      f.slot = M.dev<int64_t>(o_ds[j]);
      f.bt = M.dev<int32_t>(o_bt);
      f.bt_stride = stride;
      f.it_bt = M.dev<int32_t>(o_ib);
      f.it_row0 = M.dev<int32_t>(o_ir);
      f.it_pos0 = M.dev<int32_t>(o_dp[j]);
      f.it_cnt = M.dev<int32_t>(o_ic);
      f.n_items = nr;
      f.max_q = 1;
      f.max_ctx = max_ctx;
      f.unit_start = M.dev<int32_t>(o_dus[j]);
      f.unit_rec = M.dev<int32_t>(o_drec[j]);
      f.n_units = n_dus[j];
      f.n_split = s_dus[j];
      f.max_units = m_dus[j];
      f.kv_keys = kv_sum + (double)n * (j + 1);
      f.kv_shared = kv_dup;
      f.logits = c->logits_q + (size_t)j * nr * V;
      f.ldl = V;
      int r = forward(c, f);
      if (r) return r;
      void* sq = (char*)c->stats_q + (size_t)j * nr * stats_row_bytes(c->nch);
      KC(c, launch_row_stats(f.logits, nr, V, V, c->rd.temperature, c->rd.top_p, sq, c->st));
      KC(c, launch_sample_rows(f.logits, sq, nr, V, V, c->rd.temperature, c->rd.top_p, c->rd.seed,
                               M.dev<int32_t>(o_ids), M.dev<int32_t>(o_dsp[j]), j + 1, PURPOSE_DRAFT, d_tok + j + 1,
                               G1, nullptr, c->st));
    }
    return ER_OK;
  };
  // the target's verify forward over nr * (g + 1) rows, then the lossless
  // decision (mid: record the event between the two, on eager timed steps)
  auto verify_body = [&](bool mid) -> int {
    Fwd f;
    f.draft = false;
    f.dec_ok = true;
    f.M = nr * G1;
    f.tokens = d_tok;
    f.tok_stride = 1;
    f.pos = M.dev<int32_t>(o_vp);
    f.slot = M.dev<int64_t>(o_vs);
    f.bt = M.dev<int32_t>(o_bt);
    f.bt_stride = stride;
    f.it_bt = M.dev<int32_t>(o_ib);
    f.it_row0 = M.dev<int32_t>(o_vir);
    f.it_pos0 = M.dev<int32_t>(o_pos0);
    f.it_cnt = M.dev<int32_t>(o_vic);
    f.n_items = nr;
    f.max_q = G1;
    f.max_ctx = max_ctx;
    f.unit_start = M.dev<int32_t>(o_vus);
    f.unit_rec = M.dev<int32_t>(o_vrec);
    f.n_units = n_vus;
    f.n_split = s_vus;
    f.max_units = m_vus;
    f.kv_keys = kv_sum + (double)n * G1;
    f.kv_shared = kv_dup;
    f.logits = c->logits_p;
    f.ldl = V;
    int r = forward(c, f);
    if (r) return r;
    if (mid) HIPC(c, hipEventRecord(c->ev[2], c->st));
    KC(c, launch_row_stats(c->logits_p, nr * G1, V, V, c->rd.temperature, c->rd.top_p, c->stats_p, c->st));
    KC(c, launch_spec_decide(c->logits_p, c->stats_p, c->logits_q, c->stats_q, d_tok, nr, g, V, c->rd.temperature,
                             c->rd.top_p, c->rd.seed, M.dev<int32_t>(o_ids), M.dev<int32_t>(o_pos0), c->out_d,
                             c->out_d + nr * G1, c->resid, c->st));
    return ER_OK;
  };
  auto run = [&]() -> int {
    if (int r_ = meta_upload(c)) return r_;
    if (timed) HIPC(c, hipEventRecord(c->ev[0], c->st));
    if (hdraft) {
      // point-mass proposals of the copied drafts (not recorded: a few small launches)
      KC(c, launch_point_mass(c->logits_q, g, nr, V, d_tok, G1, c->st));
      for (int j = 0; j < g; ++j)
        KC(c, launch_row_stats(c->logits_q + (size_t)j * nr * V, nr, V, V, c->rd.temperature, c->rd.top_p,
                               (char*)c->stats_q + (size_t)j * nr * stats_row_bytes(c->nch), c->st));
    } else if (gp.nb) {
      HIPC_OK(graph_run(c, GRAPH_DRAFT, nr, g, gp.cap, draft_body));
    } else {
      HIPC_OK(draft_body());
    }
    if (timed) HIPC(c, hipEventRecord(c->ev[1], c->st));
    if (gp.nb) {
      // one graph: verify forward and decision (the split between them is not timed)
      HIPC_OK(graph_run(c, GRAPH_VERIFY, nr, g, gp.cap, [&]() { return verify_body(false); }));
      if (timed) HIPC(c, hipEventRecord(c->ev[2], c->st));
    } else {
      HIPC_OK(verify_body(timed));
    }
    if (timed) HIPC(c, hipEventRecord(c->ev[3], c->st));
    HIPC(c, hipMemcpyAsync(c->out_h, c->out_d, (size_t)(nr * G1 + nr) * 4, hipMemcpyDeviceToHost, c->st));
    if (int r_ = dec_queue_err(c)) return r_;
    HIPC(c, hipStreamSynchronize(c->st));
    return dec_check(c);
  };
  c->dec_ran = false;
  const int r = run();
  kp_flush(c);
  if (r) { rollback(); return r; }
  c->last_tok_off = o_tok;
  // commit
  AlphaAcc acc;
  int acc_tot = 0, emit_tot = 0, kept_tot = 0, fin = 0;
  const int32_t* out_tok = c->out_h;
  const int32_t* nacc = c->out_h + nr * G1;
  for (int b = 0; b < n; ++b) {
    Seq& s = c->seqs[ids[b]];
    const int a = nacc[b];
    const int em = a + 1;
    const int room = s.max_new - s.generated;
    const int kept = std::min(em, room);
    for (int i = 0; i < kept; ++i) tokens_out[(size_t)b * out_stride + i] = out_tok[(size_t)b * G1 + i];
    s.toks.insert(s.toks.end(), out_tok + (size_t)b * G1, out_tok + (size_t)b * G1 + em);
    if (n_emitted) n_emitted[b] = kept;
    s.generated += kept;
    s.n += a + 1;
    s.pending = out_tok[(size_t)b * G1 + a];
    s.bt.truncate(c->pool, (int64_t)s.n);
    acc.add(a, g);
    acc_tot += a;
    emit_tot += em;
    kept_tot += kept;
    c->stats.predict_times += 1;
    if (a > 0) c->stats.effective_times += 1;
    c->stats.total_right_length += a;
    if (a == g) c->stats.bonus += 1;
    if (s.generated >= s.max_new) { finish_seq(c, s); ++fin; }
  }
  const double a_step = acc.value();
  if (hdraft) {
    // the self-drafter's acceptance EMA tracks the self-drafter only
    c->stats.history_steps += 1;
    c->stats.history_drafted += (int64_t)n * g;
    c->stats.history_accepted += acc_tot;
  } else {
    c->alpha_ema = ema(c->alpha_ema, a_step, c->rd.ema_beta);
    c->stats.sd_steps += 1;
    c->stats.drafted += (int64_t)n * g;
    c->stats.accepted += acc_tot;
  }
  c->stats.emitted += emit_tot;
  c->stats.tokens_kept += kept_tot;
  float md = 0.f, mv = 0.f, ms = 0.f;
  if (timed) {
    md = ev_ms(c, 0, 1);
    mv = ev_ms(c, 1, 2);
    ms = ev_ms(c, 2, 3);
    c->stats.ms_draft += md;
    c->stats.ms_verify += mv;
    c->stats.ms_sample += ms;
  }
  c->last_mode = ER_MODE_SD;
  c->last_gamma = g;
  c->last_B = n;
  c->last_rows = nr;
  if (info) {
    *info = er_step_info{};
    info->mode = hdraft ? ER_MODE_HISTORY : ER_MODE_SD;
    info->gamma = g;
    info->batch = n;
    info->accepted = acc_tot;
    info->emitted = emit_tot;
    info->kept = kept_tot;
    info->finished = fin;
    info->alpha_step = (float)a_step;
    info->alpha_ema = (float)c->alpha_ema;
    info->ms_draft = md;
    info->ms_verify = mv;
    info->ms_sample = ms;
    info->ms_total = md + mv + ms;
  }
  ++c->step_count;
  return ER_OK;
}

// One step with drafts copied from earlier rollouts: each sequence's g drafts
// from the history cache (padded with its pending token where the cache has
// fewer or none: any fixed token is a valid proposal), then the target's
// verify pass and the lossless decision with point-mass proposals.
int do_history(er_ctx* c, int n, const int32_t* ids, int32_t* tokens_out, int out_stride, int32_t* n_emitted,
               er_step_info* info) {
  const int g = c->hist_gamma;
  const int V = c->md.vocab;
  std::vector<int32_t> d((size_t)n * g);
  for (int b = 0; b < n; ++b) {
    const Seq& s = c->seqs[ids[b]];
    int32_t* db = d.data() + (size_t)b * g;
    int k = c->hist->cache.propose(s.toks.data(), s.prompt_len, s.toks.data(), (int)s.toks.size(), g, db);
    for (int i = 0; i < k; ++i)
      if (db[i] < 0 || db[i] >= V) { k = i; break; }
    for (int i = k; i < g; ++i) db[i] = s.pending;
  }
  return do_spec(c, n, ids, g, tokens_out, out_stride, n_emitted, info, d.data());
}

// Controller choice for this batch (0 = AR).
int plan(er_ctx* c, int n, const int32_t* ids) {
  if (c->policy == ER_POLICY_FORCE_AR) return 0;
  double C = 0;
  for (int i = 0; i < n; ++i) C += c->seqs[ids[i]].n;
  C /= n;
  const int lo = c->gamma_pinned ? c->gamma_pinned : c->rd.gamma_min;
  const int hi = c->gamma_pinned ? c->gamma_pinned : c->rd.gamma_max;
  if (c->policy == ER_POLICY_TIMING) {
    // the guard picks the branch from measured tokens/ms; the draft length
    // when it speculates is the acceptance-aware argmax over gamma >= 1
    if (er_guard_choose(&c->guard, n) != 1) return c->plan.choice = 0;
    return c->plan.choice = choose(c->cost, n, C, c->alpha_ema, lo, hi, false, -1, 1.0);
  }
  return plan_step(c->cost, c->plan, c->policy == ER_POLICY_AUTO, n, C, c->alpha_ema, c->alpha_init, lo, hi,
                   c->rd.switch_margin);
}

int current_gamma(er_ctx* c) {
  if (c->gamma_pinned) return c->gamma_pinned;
  if (c->plan.choice > 0) return c->plan.choice;
  return c->rd.gamma_init;
}

// Roofline constants: streaming-read bandwidth over part of the KV pool, and
// the per-forward overhead fitted from a target and a drafter forward at M = 1
// (EfficientRollout "局限": the compute/memory boundary is calibrated per GPU).
int calibrate(er_ctx* c) {
  const er_model_desc& m = c->md;
  c->cost.n_layers = m.n_layers;
  c->cost.d_model = m.d_model;
  c->cost.n_q_heads = m.n_q_heads;
  c->cost.n_kv_heads = m.n_kv_heads;
  c->cost.head_dim = m.head_dim;
  c->cost.ffn = m.ffn;
  c->cost.vocab = m.vocab;
  c->cost.w_bytes = c->bf16 ? 2.0 : 4.0;
  c->cost.q_bytes = c->dd.quant == ER_W8_PERCH_SYM ? 1.0 : 0.5 + 3.0 / 128.0;
  c->cost.kv_bytes_el = c->bf16 ? 2.0 : 4.0;
  c->cost.bw = c->rd.hbm_bytes_per_s > 0 ? c->rd.hbm_bytes_per_s : 0.0;
  c->cost.flops = c->rd.flops_per_s > 0 ? c->rd.flops_per_s : 2.5e15;  // replaced by the measurement below
  c->cost.t_fwd = c->rd.t_fwd_s >= 0 ? c->rd.t_fwd_s : 0.0;
  if (c->cost.bw <= 0) {
    const size_t bytes = std::min((size_t)1 << 30, (size_t)c->pool.total() * c->block_bytes) & ~(size_t)4095;
    if (bytes < ((size_t)64 << 20)) {
      c->cost.bw = 8.0e12;
    } else {
      hipEvent_t a, b;
      HIPC(c, hipEventCreate(&a));
      HIPC(c, hipEventCreate(&b));
      KC(c, launch_stream_read(c->kv_pool, bytes, c->sink, c->st));
      HIPC(c, hipEventRecord(a, c->st));
      for (int i = 0; i < 4; ++i) KC(c, launch_stream_read(c->kv_pool, bytes, c->sink, c->st));
      HIPC(c, hipEventRecord(b, c->st));
      HIPC(c, hipEventSynchronize(b));
      float ms = 0.f;
      HIPC(c, hipEventElapsedTime(&ms, a, b));
      (void)hipEventDestroy(a);
      (void)hipEventDestroy(b);
      c->cost.bw = ms > 0 ? 4.0 * bytes / (ms * 1e-3) : 8.0e12;
    }
  }
  if (c->rd.t_fwd_s < 0 && c->pool.free_count() >= 1) {
    // One scratch block: forwards of `rows` rows, every row at position 0 of
    // the block (each writes and reads that one key), timed after a warm one.
    // The target's and the drafter's forwards at 1 row give the fixed time
    // per forward beyond the roofline, at Mr rows the time per further row
    // (the kernels read the same bytes more slowly as rows are added:
    // dequantizing linears past 8 rows, more attention items).
    BlockTable bt;
    if (!bt.reserve(c->pool, 1)) return ER_OK;
    auto time_fwd = [&](int rows, bool draft, double* sec) -> int {
      Meta& M = c->meta;
      if (int r_ = meta_begin(c)) return r_;
      size_t o_tok, o_pos, o_slot, o_bt, o_ib, o_ir, o_ic;
      int32_t* t = M.push<int32_t>(rows, &o_tok);
      int32_t* p = M.push<int32_t>(rows, &o_pos);
      int64_t* s = M.push<int64_t>(rows, &o_slot);
      int32_t* btp = M.push<int32_t>(1, &o_bt);
      int32_t* ib = M.push<int32_t>(rows, &o_ib);
      int32_t* ir = M.push<int32_t>(rows, &o_ir);
      int32_t* ic = M.push<int32_t>(rows, &o_ic);
      if (!M.ok) return fail(c, ER_ENOMEM, "metadata region too small");
      for (int i = 0; i < rows; ++i) {
        t[i] = 0;
        p[i] = 0;
        s[i] = (int64_t)bt.blocks[0] * KV_BLOCK;
        ib[i] = 0;
        ir[i] = i;
        ic[i] = 1;
      }
      *btp = bt.blocks[0];
      int nu = 0, ns = 0, mu = 0;
      size_t o_rec = 0;
      const size_t o_us = push_units(M, rows, (int)m.n_kv_heads, p, ic, ir, ib, &nu, &ns, &mu, &o_rec);
      if (!M.ok) return fail(c, ER_ENOMEM, "metadata region too small");
      if (int r_ = meta_upload(c)) return r_;
      Fwd f;
      f.draft = draft;
      f.M = rows;
      f.tokens = M.dev<int32_t>(o_tok);
      f.pos = M.dev<int32_t>(o_pos);
      f.slot = M.dev<int64_t>(o_slot);
      f.bt = M.dev<int32_t>(o_bt);
      f.bt_stride = 1;
      f.it_bt = M.dev<int32_t>(o_ib);
      f.it_row0 = M.dev<int32_t>(o_ir);
      f.it_pos0 = M.dev<int32_t>(o_pos);
      f.it_cnt = M.dev<int32_t>(o_ic);
      f.n_items = rows;
      f.max_q = 1;
      f.max_ctx = 1;
      f.unit_start = M.dev<int32_t>(o_us);
      f.unit_rec = M.dev<int32_t>(o_rec);
      f.n_units = nu;
      f.n_split = ns;
      f.max_units = mu;
      f.kv_keys = rows;
      f.dec_ok = true;  // time the forward the decode steps run
      f.logits = c->logits_p;
      f.ldl = m.vocab;
      int r = forward(c, f);  // warm
      if (r) return r;
      hipEvent_t a, b;
      HIPC(c, hipEventCreate(&a));
      HIPC(c, hipEventCreate(&b));
      HIPC(c, hipEventRecord(a, c->st));
      for (int i = 0; i < 3 && r == ER_OK; ++i) r = forward(c, f);
      if (r == ER_OK) {
        HIPC(c, hipEventRecord(b, c->st));
        HIPC(c, hipEventSynchronize(b));
      }
      float ms = 0.f;
      if (r == ER_OK) HIPC(c, hipEventElapsedTime(&ms, a, b));
      (void)hipEventDestroy(a);
      (void)hipEventDestroy(b);
      *sec = ms / 3.0 * 1e-3;
      return r;
    };
    const int Mr = std::min({16, c->rd.max_batch, c->max_rows, c->logit_rows});
    double t1[2] = {0, 0}, tr[2] = {0, 0};
    int r = ER_OK;
    for (int which = 0; which < 2 && r == ER_OK; ++which) r = time_fwd(1, which == 1, &t1[which]);
    for (int which = 0; which < 2 && r == ER_OK && Mr >= 2; ++which) r = time_fwd(Mr, which == 1, &tr[which]);
    bt.release(c->pool);
    if (r) return r;
    if (c->dec_ran) {
      HIPC(c, hipMemcpy(c->out_h + c->dec_err_slot, c->dec_err, 4, hipMemcpyDeviceToHost));
      if (int r_ = dec_check(c)) return r_;
    }
    const double P = c->cost.p_lin(), kvb = c->cost.kvb(), V = m.vocab;
    auto roof = [&](double wb, int rows) {
      return std::max((wb * P + rows * kvb + 4.0 * rows * V) / c->cost.bw, 2.0 * P * rows / c->cost.flops);
    };
    const double rt = t1[0] - roof(c->cost.w_bytes, 1), rd = t1[1] - roof(c->cost.q_bytes, 1);
    c->cost.t_fwd = std::max(0.0, 0.5 * (rt + rd));
    if (Mr >= 2) {
      c->cost.t_row_target = std::max(0.0, (tr[0] - roof(c->cost.w_bytes, Mr) - rt) / (Mr - 1));
      c->cost.t_row_draft = std::max(0.0, (tr[1] - roof(c->cost.q_bytes, Mr) - rd) / (Mr - 1));
    }
  }
  if (c->rd.flops_per_s <= 0) {
    // Dense-contraction rate the kernels reach: a target forward over Mc
    // prompt-like rows of one throwaway sequence (positions 0..Mc-1), logits
    // for every row, timed beyond the fixed time and the weight stream.
    const int grp = (int)(m.n_q_heads / m.n_kv_heads);
    const int qmax = std::max(1, 64 / grp);
    const int Mc = std::min(512, std::min(c->max_rows, c->logit_rows));
    BlockTable bt;
    if (Mc >= 64 && c->pool.free_count() >= (Mc + KV_BLOCK - 1) / KV_BLOCK &&
        bt.reserve(c->pool, Mc)) {
      const int nb = (int)bt.blocks.size();
      const int n_items = (Mc + qmax - 1) / qmax;
      Meta& M = c->meta;
      if (int r_ = meta_begin(c)) { bt.release(c->pool); return r_; }
      size_t o_tok, o_pos, o_slot, o_bt, o_ib, o_ir, o_ip, o_ic;
      int32_t* t = M.push<int32_t>(Mc, &o_tok);
      int32_t* p = M.push<int32_t>(Mc, &o_pos);
      int64_t* sl = M.push<int64_t>(Mc, &o_slot);
      int32_t* btp = M.push<int32_t>(nb, &o_bt);
      int32_t* ib = M.push<int32_t>(n_items, &o_ib);
      int32_t* ir = M.push<int32_t>(n_items, &o_ir);
      int32_t* ip = M.push<int32_t>(n_items, &o_ip);
      int32_t* ic = M.push<int32_t>(n_items, &o_ic);
      if (M.ok) {
        for (int i = 0; i < Mc; ++i) {
          t[i] = i % m.vocab;
          p[i] = i;
          sl[i] = (int64_t)bt.blocks[i / KV_BLOCK] * KV_BLOCK + i % KV_BLOCK;
        }
        for (int b = 0; b < nb; ++b) btp[b] = bt.blocks[b];
        for (int k = 0; k < n_items; ++k) {
          ib[k] = 0;
          ir[k] = k * qmax;
          ip[k] = k * qmax;
          ic[k] = std::min(qmax, Mc - k * qmax);
        }
        int n_units = 0, n_split = 0, max_units = 0;
        size_t o_rec = 0;
        const size_t o_us =
            push_units(M, n_items, (int)m.n_kv_heads, ip, ic, ir, ib, &n_units, &n_split, &max_units, &o_rec);
        if (M.ok) {
          if (int r_ = meta_upload(c)) return r_;
          Fwd f;
          f.M = Mc;
          f.tokens = M.dev<int32_t>(o_tok);
          f.pos = M.dev<int32_t>(o_pos);
          f.slot = M.dev<int64_t>(o_slot);
          f.bt = M.dev<int32_t>(o_bt);
          f.bt_stride = nb;
          f.it_bt = M.dev<int32_t>(o_ib);
          f.it_row0 = M.dev<int32_t>(o_ir);
          f.it_pos0 = M.dev<int32_t>(o_ip);
          f.it_cnt = M.dev<int32_t>(o_ic);
          f.n_items = n_items;
          f.max_q = qmax;
          f.max_ctx = Mc;
          f.unit_start = M.dev<int32_t>(o_us);
          f.unit_rec = M.dev<int32_t>(o_rec);
          f.n_units = n_units;
          f.n_split = n_split;
          f.max_units = max_units;
          f.logits = c->logits_p;
          f.ldl = m.vocab;
          hipEvent_t a, b;
          HIPC(c, hipEventCreate(&a));
          HIPC(c, hipEventCreate(&b));
          int r = forward(c, f);  // warm
          if (!r) {
            HIPC(c, hipEventRecord(a, c->st));
            for (int i = 0; i < 2 && !r; ++i) r = forward(c, f);
            HIPC(c, hipEventRecord(b, c->st));
            HIPC(c, hipEventSynchronize(b));
          }
          float ms = 0.f;
          if (!r) HIPC(c, hipEventElapsedTime(&ms, a, b));
          (void)hipEventDestroy(a);
          (void)hipEventDestroy(b);
          if (r) { bt.release(c->pool); return r; }
          const double T = ms / 2.0 * 1e-3;
          const double P = c->cost.p_lin();
          const double busy = T - c->cost.t_fwd;
          // above the weight stream: compute-bound at Mc rows, take the rate
          if (busy > c->cost.w_bytes * P / c->cost.bw) c->cost.flops = 2.0 * P * Mc / busy;
        }
      }
      bt.release(c->pool);
    }
  }
  return ER_OK;
}

}  // namespace

// =============================================================================
// C ABI
// =============================================================================
extern "C" {

int er_arena_bytes(const er_model_desc* model, const er_draft_desc* draft, const er_rollout_desc* rollout,
                   int64_t kv_pool_blocks, size_t* bytes_out) {
  try {
    std::string why;
    if (!bytes_out) return ER_EINVAL;
    int r = validate(model, draft, rollout, &why);
    if (r) return r;
    Layout L;
    make_layout(*model, *draft, *rollout, &L, &why);
    *bytes_out = L.total_fixed() + (size_t)std::max<int64_t>(0, kv_pool_blocks) * L.block_bytes + 4096;
    return ER_OK;
  } catch (...) {
    return ER_EINVAL;
  }
}

int er_rollout_init(const er_model_desc* model, const er_weights* w, const er_draft_desc* draft,
                    const er_rollout_desc* rollout, void* dev_arena, size_t arena_bytes, void* hip_stream,
                    er_ctx** out) {
  if (!out) return ER_EINVAL;
  *out = nullptr;
  er_ctx* c = nullptr;
  try {
    c = new er_ctx();
    std::string why;
    int r = validate(model, draft, rollout, &why);
    if (r) { c->err = why; *out = c; return r; }
    if (!dev_arena) { *out = c; return fail(c, ER_EINVAL, "null arena"); }
    c->md = *model;
    c->dd = *draft;
    c->rd = *rollout;
    c->bf16 = model->dtype == ER_BF16;
    c->act_bytes = c->bf16 ? 2 : 4;
    c->st = (hipStream_t)hip_stream;
    c->arena = (char*)dev_arena;
    c->arena_bytes = arena_bytes;
    c->policy = rollout->policy;
    {
      er_guard_params gp;
      er_guard_default_params(&gp);
      er_guard_init(&c->guard, &gp);
    }
    c->alpha_ema = rollout->alpha_init > 0 ? rollout->alpha_init : 0.8;
    c->alpha_init = c->alpha_ema;
    Layout L;
    make_layout(*model, *draft, *rollout, &L, &why);
    const size_t fixed = L.total_fixed() + 4096;
    if (fixed > arena_bytes) {
      *out = c;
      return fail(c, ER_ENOMEM, "arena of %zu bytes is smaller than the %zu fixed bytes needed", arena_bytes, fixed);
    }
    // carve
    char* cur = c->arena + L.drafter;  // drafter pack first (filled by set_weights)
    auto take = [&](size_t n) { char* p = cur; cur += n; return p; };
    c->cs = (float2*)take(L.cs);
    c->h = (float*)take(L.h);
    c->xbuf = take(L.xbuf);
    c->qkv = (float*)take(L.qkv);
    c->qb = take(L.qb);
    c->gu = (float*)take(L.gu);
    c->logits_p = (float*)take(L.lp);
    c->logits_q = (float*)take(L.lq);
    c->stats_p = take(L.sp);
    c->stats_q = take(L.sq);
    c->resid = (double*)take(L.resid);
    c->ssq[0] = (unsigned long long*)take(L.ssq / 2);
    c->ssq[1] = (unsigned long long*)take(L.ssq / 2);
    c->fuse = c->bf16;
    c->nch = sampler_chunks(model->vocab);
    c->out_d = (int32_t*)take(L.out);
    c->lws.partial = (float*)take(L.partial);
    c->lws.partial_floats = L.partial / 4;
    c->lws.counters = (int*)take(L.counters);
    c->lws.n_counters = (int)(L.counters / 4);
    c->lws.xn = (uint16_t*)take(L.xn);
    c->lws.xn_elems = L.xn / 2;
    c->attn_ws = (float*)take(L.attn);
    c->attn_ws_floats = L.attn / 4;
    c->w4_tmp = (uint8_t*)take(L.w4tmp);
    c->w4_tmp_bytes = L.w4tmp;
    c->sink = (uint32_t*)take(L.sink);
    c->meta.d = take(L.meta);
    c->meta.cap = L.meta;
    if (L.blas) {
      // library GEMMs for the target's projections from each shape's row threshold (er_set_library_gemm)
      char* bw = take(L.blas);
      c->lws.blas = blas_create(bw, L.blas, c->gu, L.gu / 4);
      c->lws.blas_min_m = -1;
      c->lws.blas_out = c->gu;
      c->lws.blas_out_floats = L.gu / 4;
    }
    if (L.dec) {
      char* d0 = take(L.dec);
      char* dc = d0;
      const size_t nl = (size_t)model->n_layers;
      c->dec_layers[0] = (DecLayerW*)dc;
      c->dec_layers[1] = c->dec_layers[0] + nl;
      dc += align256(2 * nl * sizeof(DecLayerW));
      c->dec_ws = dc;
      dc += align256(decode_ws_bytes(model->n_layers, model->d_model, model->n_q_heads, model->head_dim,
                                     model->ffn, kSsqSlots));
      c->dec_bar = (unsigned*)dc;
      dc += align256((size_t)kDecodeBarWords * 4);
      c->dec_err = (unsigned*)dc;
      if (hipMemsetAsync(d0, 0, L.dec, c->st) != hipSuccess) { *out = c; return fail(c, ER_EDEVICE, "memset"); }
      c->dec_err_slot = L.max_rows + rollout->max_batch;
    }
    c->max_rows = L.max_rows;
    c->logit_rows = L.logit_rows;
    c->block_bytes = L.block_bytes;
    // KV pool: the rest of the arena (block aligned to 256 bytes)
    char* kv0 = (char*)(((uintptr_t)cur + 255) & ~(uintptr_t)255);
    const size_t left = (size_t)(c->arena + arena_bytes - kv0);
    int64_t nblk = (int64_t)(left / L.block_bytes);
    if (rollout->kv_pool_blocks > 0) {
      if (rollout->kv_pool_blocks > nblk) {
        *out = c;
        return fail(c, ER_ENOMEM, "arena holds %lld KV blocks, %lld requested", (long long)nblk,
                    (long long)rollout->kv_pool_blocks);
      }
      nblk = rollout->kv_pool_blocks;
    }
    if (nblk < 1) { *out = c; return fail(c, ER_ENOMEM, "no room for KV blocks"); }
    c->kv_pool = kv0;
    c->pool.init(nblk);
    c->seqs.clear();
    // host buffers
    if (hipHostMalloc((void**)&c->meta.h, L.meta) != hipSuccess) { *out = c; return fail(c, ER_EDEVICE, "hipHostMalloc"); }
    if (hipHostMalloc((void**)&c->out_h, L.out) != hipSuccess) { *out = c; return fail(c, ER_EDEVICE, "hipHostMalloc"); }
    for (auto& e : c->ev) {
      if (hipEventCreate(&e) != hipSuccess) { *out = c; return fail(c, ER_EDEVICE, "hipEventCreate"); }
    }
    if (hipEventCreateWithFlags(&c->meta_ev, hipEventDisableTiming) != hipSuccess) {
      *out = c;
      return fail(c, ER_EDEVICE, "hipEventCreate");
    }
    c->have_ev = true;
    // counters start at zero
    if (hipMemsetAsync(c->lws.counters, 0, L.counters, c->st) != hipSuccess) { *out = c; return fail(c, ER_EDEVICE, "memset"); }
    if (hipMemsetAsync(c->ssq[0], 0, L.ssq, c->st) != hipSuccess) { *out = c; return fail(c, ER_EDEVICE, "memset"); }
    // RoPE table: cos/sin of pos * theta^(-2i/hd), fp64 on the host
    {
      const int half = model->head_dim / 2;
      std::vector<float2> tab((size_t)rollout->max_ctx * half);
      for (int p = 0; p < rollout->max_ctx; ++p)
        for (int i = 0; i < half; ++i) {
          const double inv = std::pow((double)model->rope_theta, -2.0 * i / model->head_dim);
          const double ang = (double)p * inv;
          tab[(size_t)p * half + i] = make_float2((float)std::cos(ang), (float)std::sin(ang));
        }
      if (hipMemcpy(c->cs, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice) != hipSuccess) {
        *out = c;
        return fail(c, ER_EDEVICE, "upload RoPE table");
      }
    }
    r = set_weights(c, w);
    if (r) { *out = c; return r; }
    if (c->dec_layers[0]) {
      // the persistent decode forward: grid per weight format, K slices per projection
      const int fmts[2] = {FMT_BF16, c->drf[0].qkv.fmt};
      for (int f : fmts) c->dec_nwg[f] = decode_grid(f, model->head_dim);
      const int G = std::max(c->dec_nwg[FMT_BF16], c->dec_nwg[fmts[1]]);
      if (c->dec_nwg[FMT_BF16] > 0 && c->dec_nwg[fmts[1]] > 0 && c->dec_nwg[FMT_BF16] == c->dec_nwg[fmts[1]] &&
          model->head_dim == 128) {
        const int d = model->d_model, F = model->ffn, qn = model->n_q_heads * model->head_dim;
        const int qkvN = (model->n_q_heads + 2 * model->n_kv_heads) * model->head_dim;
        const int NK[4][2] = {{qkvN, d}, {d, qn}, {2 * F, d}, {d, F}};
        bool ok = true;
        for (int which = 0; which < 2; ++which)
          for (int i = 0; i < 4; ++i) {
            c->dec_ks[which][i] = decode_ksplit(NK[i][0], NK[i][1], G, fmts[which]);
            ok = ok && c->dec_ks[which][i] > 0;
          }
        c->dec_avail = ok;
        c->dec_on = false;  // off until er_set_persistent: the kernel sequence is faster on MI355X today
      }
    }
    r = calibrate(c);
    if (r) { *out = c; return r; }
    c->stats.alpha_ema = c->alpha_ema;
    c->stats.gamma = rollout->gamma_init;
    *out = c;
    return ER_OK;
  } catch (...) {
    if (c) { *out = c; c->err = "internal error"; }
    return ER_EINVAL;
  }
}

int er_update_weights(er_ctx* c, const er_weights* w) {
  if (!c) return ER_EINVAL;
  try {
    return set_weights(c, w);
  } catch (...) {
    return fail(c, ER_EINVAL, "internal error");
  }
}

int er_kv_alloc(er_ctx* c, int n, const int32_t* prompt_lens, const int32_t* max_new, const int32_t* share_group,
                int32_t* seq_ids_out) {
  if (!c) return ER_EINVAL;
  try {
    if (n <= 0 || !prompt_lens || !max_new || !seq_ids_out) return fail(c, ER_EINVAL, "bad arguments");
    if (c->alive + n > c->rd.max_seqs) return fail(c, ER_ENOMEM, "max_seqs %d exceeded", c->rd.max_seqs);
    for (int i = 0; i < n; ++i) {
      if (prompt_lens[i] < 1 || max_new[i] < 1) return fail(c, ER_EINVAL, "prompt_lens and max_new must be >= 1");
      if ((int64_t)prompt_lens[i] + max_new[i] + c->rd.gamma_max + 1 > c->rd.max_ctx)
        return fail(c, ER_EINVAL, "sequence of %d + %d tokens exceeds max_ctx %d", prompt_lens[i], max_new[i],
                    c->rd.max_ctx);
    }
    // groups: the first member of a group in this call leads
    const size_t base = c->seqs.size();
    std::vector<Seq> add((size_t)n);
    std::vector<int32_t> leader_of(n, -1);
    for (int i = 0; i < n; ++i) {
      Seq& s = add[(size_t)i];
      s.alive = true;
      s.prompt_len = prompt_lens[i];
      s.max_new = max_new[i];
      s.group = share_group ? share_group[i] : -1;
      s.family = s.group >= 0 ? s.group : -1;
      s.shared_len = s.group >= 0 ? s.prompt_len : 0;
      s.leader = true;
      s.leader_id = (int32_t)(base + i);
      if (s.group >= 0) {
        for (int j = 0; j < i; ++j)
          if (add[(size_t)j].group == s.group && add[(size_t)j].leader) {
            if (prompt_lens[j] != prompt_lens[i]) return fail(c, ER_EINVAL, "group %d has unequal prompt lengths", s.group);
            s.leader = false;
            s.leader_id = (int32_t)(base + j);
            leader_of[i] = j;
            break;
          }
      }
    }
    // blocks: leaders/private reserve their prompt; members share full blocks
    int i_ok = 0;
    bool oom = false;
    for (int i = 0; i < n && !oom; ++i) {
      Seq& s = add[(size_t)i];
      if (s.leader) {
        if (!s.bt.reserve(c->pool, s.prompt_len)) oom = true;
      } else {
        const Seq& L = add[(size_t)leader_of[i]];
        const int full = s.prompt_len / KV_BLOCK;
        for (int b = 0; b < full; ++b) {
          s.bt.blocks.push_back(L.bt.blocks[(size_t)b]);
          c->pool.incref(L.bt.blocks[(size_t)b]);
        }
        if (!s.bt.reserve(c->pool, s.prompt_len)) oom = true;
      }
      if (!oom) i_ok = i + 1;
    }
    if (oom) {
      for (int i = 0; i <= std::min(i_ok, n - 1); ++i) add[(size_t)i].bt.release(c->pool);
      return fail(c, ER_ENOMEM, "KV pool exhausted while allocating prompts");
    }
    for (int i = 0; i < n; ++i) {
      c->seqs.push_back(std::move(add[(size_t)i]));
      seq_ids_out[i] = (int32_t)(base + i);
    }
    c->alive += n;
    return ER_OK;
  } catch (...) {
    return fail(c, ER_EINVAL, "internal error");
  }
}

int er_kv_fork(er_ctx* c, int32_t parent, int n, const int32_t* max_new, int32_t* child_ids_out) {
  if (!c) return ER_EINVAL;
  try {
    if (n <= 0 || !max_new || !child_ids_out) return fail(c, ER_EINVAL, "bad arguments");
    if (parent < 0 || parent >= (int32_t)c->seqs.size() || !c->seqs[parent].alive)
      return fail(c, ER_EINVAL, "unknown sequence %d", parent);
    if (!c->seqs[parent].prefilled || c->seqs[parent].finished)
      return fail(c, ER_ESTATE, "sequence %d must be prefilled and not finished to fork", parent);
    if (c->alive + n > c->rd.max_seqs) return fail(c, ER_ENOMEM, "max_seqs %d exceeded", c->rd.max_seqs);
    const Seq P = c->seqs[parent];
    for (int i = 0; i < n; ++i) {
      if (max_new[i] <= P.generated) return fail(c, ER_EINVAL, "max_new must exceed the %d tokens already generated", P.generated);
      if ((int64_t)P.prompt_len + max_new[i] + c->rd.gamma_max + 1 > c->rd.max_ctx)
        return fail(c, ER_EINVAL, "fork of %d + %d tokens exceeds max_ctx %d", P.prompt_len, max_new[i], c->rd.max_ctx);
    }
    // the parent's committed positions [0, n): full blocks shared, the partial one copied
    const int full = P.n / KV_BLOCK;
    const bool partial = P.n % KV_BLOCK != 0;
    if (partial && c->pool.free_count() < n) return fail(c, ER_ENOMEM, "KV pool exhausted while forking");
    const int32_t fam = P.family != -1 ? P.family : -2 - parent;
    // the children's copies of the partial block first, so that a failed copy changes nothing
    std::vector<int32_t> tail;
    if (partial) {
      for (int i = 0; i < n; ++i) tail.push_back(c->pool.alloc());  // available: checked above
      for (int i = 0; i < n; ++i) {
        const hipError_t e = hipMemcpyAsync((char*)c->kv_pool + (size_t)tail[(size_t)i] * c->block_bytes,
                                            (char*)c->kv_pool + (size_t)P.bt.blocks[(size_t)full] * c->block_bytes,
                                            c->block_bytes, hipMemcpyDeviceToDevice, c->st);
        if (e != hipSuccess) {
          for (int32_t b : tail) c->pool.decref(b);
          return fail(c, ER_EDEVICE, "copy of the partial block: %s", hipGetErrorString(e));
        }
      }
    }
    const size_t base = c->seqs.size();
    for (int i = 0; i < n; ++i) {
      Seq s = P;
      s.bt.blocks.clear();
      for (int b = 0; b < full; ++b) {
        s.bt.blocks.push_back(P.bt.blocks[(size_t)b]);
        c->pool.incref(P.bt.blocks[(size_t)b]);
      }
      if (partial) s.bt.blocks.push_back(tail[(size_t)i]);
      s.max_new = max_new[i];
      s.group = -1;
      s.leader = true;
      s.leader_id = (int32_t)(base + i);
      s.family = fam;
      s.shared_len = full * KV_BLOCK;
      c->seqs.push_back(std::move(s));
      child_ids_out[i] = (int32_t)(base + i);
    }
    Seq& Pm = c->seqs[parent];
    if (Pm.family == -1) {
      Pm.family = fam;
      Pm.shared_len = full * KV_BLOCK;
    }
    c->alive += n;
    return ER_OK;
  } catch (...) {
    return fail(c, ER_EINVAL, "internal error");
  }
}

int er_prefill(er_ctx* c, int n, const int32_t* ids, const int32_t* tokens, const int64_t* offsets,
               int32_t* first_tok_out) {
  if (!c) return ER_EINVAL;
  try {
    if (n <= 0 || !ids || !tokens || !offsets || !first_tok_out) return fail(c, ER_EINVAL, "bad arguments");
    if (n > c->logit_rows) return fail(c, ER_EINVAL, "at most %d sequences per prefill call", c->logit_rows);
    for (int i = 0; i < n; ++i) {
      const int32_t id = ids[i];
      if (id < 0 || id >= (int32_t)c->seqs.size() || !c->seqs[id].alive) return fail(c, ER_EINVAL, "unknown sequence %d", id);
      const Seq& s = c->seqs[id];
      if (s.prefilled) return fail(c, ER_ESTATE, "sequence %d already prefilled", id);
      if (offsets[i + 1] - offsets[i] != s.prompt_len)
        return fail(c, ER_EINVAL, "sequence %d: %lld tokens given, prompt_len %d", id,
                    (long long)(offsets[i + 1] - offsets[i]), s.prompt_len);
      for (int64_t k = offsets[i]; k < offsets[i + 1]; ++k)
        if (tokens[k] < 0 || tokens[k] >= c->md.vocab) return fail(c, ER_EINVAL, "token out of range");
      for (int j = 0; j < i; ++j)
        if (ids[j] == id) return fail(c, ER_EINVAL, "sequence %d listed twice", id);
      if (!s.leader) {
        bool found = false;
        for (int j = 0; j < n; ++j) found |= ids[j] == s.leader_id;
        if (!found && !c->seqs[s.leader_id].prefilled)
          return fail(c, ER_ESTATE, "sequence %d shares the prompt of %d, which is not prefilled", id, s.leader_id);
      }
    }
    const int grp = c->md.n_q_heads / c->md.n_kv_heads;
    const int qmax = std::max(1, 64 / grp);
    const int V = c->md.vocab;
    // computing sequences: leaders and private ones in this call
    std::vector<int> comp;
    for (int i = 0; i < n; ++i)
      if (c->seqs[ids[i]].leader) comp.push_back(i);
    // logits row of each computing sequence once its last token is processed
    std::vector<int32_t> row_of_call(n, -1);
    int next_row = 0;
    size_t ci = 0;
    int64_t done_in_seq = 0;
    while (ci < comp.size()) {
      // pack one chunk
      struct Seg { int call_i; int32_t p0; int32_t cnt; };
      std::vector<Seg> segs;
      int rows = 0;
      while (ci < comp.size() && rows < c->rd.prefill_chunk) {
        const int i = comp[ci];
        const Seq& s = c->seqs[ids[i]];
        const int32_t take = (int32_t)std::min<int64_t>(s.prompt_len - done_in_seq, c->rd.prefill_chunk - rows);
        segs.push_back(Seg{i, (int32_t)done_in_seq, take});
        rows += take;
        done_in_seq += take;
        if (done_in_seq == s.prompt_len) { ++ci; done_in_seq = 0; }
      }
      Meta& M = c->meta;
      if (int r_ = meta_begin(c)) return r_;
      std::vector<int32_t> cids;
      for (auto& sg : segs) cids.push_back(ids[sg.call_i]);
      size_t o_tok, o_pos, o_slot, o_bt, o_ib, o_ir, o_ip, o_ic, o_lr;
      int32_t* h_tok = M.push<int32_t>(rows, &o_tok);
      int32_t* h_pos = M.push<int32_t>(rows, &o_pos);
      int64_t* h_slot = M.push<int64_t>(rows, &o_slot);
      int stride = 0;
      int32_t* h_bt = put_block_table(c, (int)cids.size(), cids.data(), &stride, &o_bt);
      int n_items = 0;
      for (auto& sg : segs) n_items += (sg.cnt + qmax - 1) / qmax;
      int32_t* h_ib = M.push<int32_t>(n_items, &o_ib);
      int32_t* h_ir = M.push<int32_t>(n_items, &o_ir);
      int32_t* h_ip = M.push<int32_t>(n_items, &o_ip);
      int32_t* h_ic = M.push<int32_t>(n_items, &o_ic);
      int32_t* h_lr = M.push<int32_t>(segs.size(), &o_lr);
      if (!M.ok || !h_bt) return fail(c, ER_ENOMEM, "metadata region too small for a prefill chunk");
      int row = 0, it = 0, nl = 0, max_ctx = 1;
      std::vector<int> finishing;
      for (size_t k = 0; k < segs.size(); ++k) {
        const Seg& sg = segs[k];
        const Seq& s = c->seqs[ids[sg.call_i]];
        const int32_t* tk = tokens + offsets[sg.call_i];
        for (int32_t q = 0; q < sg.cnt; ++q) {
          const int32_t p = sg.p0 + q;
          h_tok[row + q] = tk[p];
          h_pos[row + q] = p;
          h_slot[row + q] = slot_of(s, p);
        }
        for (int32_t q = 0; q < sg.cnt; q += qmax) {
          h_ib[it] = (int32_t)k;
          h_ir[it] = row + q;
          h_ip[it] = sg.p0 + q;
          h_ic[it] = std::min(qmax, sg.cnt - q);
          ++it;
        }
        max_ctx = std::max(max_ctx, sg.p0 + sg.cnt);
        if (sg.p0 + sg.cnt == s.prompt_len) {
          h_lr[nl++] = row + sg.cnt - 1;
          finishing.push_back(sg.call_i);
        }
        row += sg.cnt;
      }
      int n_units = 0;
      int n_split = 0;
      int max_units = 0;
      size_t o_rec = 0;
      const size_t o_us =
          push_units(M, n_items, (int)c->md.n_kv_heads, h_ip, h_ic, h_ir, h_ib, &n_units, &n_split, &max_units, &o_rec);
      if (!M.ok) return fail(c, ER_ENOMEM, "metadata region too small for a prefill chunk");
      if (int r_ = meta_upload(c)) return r_;
      Fwd f;
      f.M = rows;
      f.tokens = M.dev<int32_t>(o_tok);
      f.pos = M.dev<int32_t>(o_pos);
      f.slot = M.dev<int64_t>(o_slot);
      f.bt = M.dev<int32_t>(o_bt);
      f.bt_stride = stride;
      f.it_bt = M.dev<int32_t>(o_ib);
      f.it_row0 = M.dev<int32_t>(o_ir);
      f.it_pos0 = M.dev<int32_t>(o_ip);
      f.it_cnt = M.dev<int32_t>(o_ic);
      f.n_items = n_items;
      f.max_q = qmax;
      f.max_ctx = max_ctx;
      f.unit_start = M.dev<int32_t>(o_us);
      f.unit_rec = M.dev<int32_t>(o_rec);
      f.n_units = n_units;
      f.n_split = n_split;
      f.max_units = max_units;
      f.logit_rows = M.dev<int32_t>(o_lr);
      f.n_logit = nl;
      f.logits = c->logits_p + (size_t)next_row * V;
      f.ldl = V;
      {
        int r = forward(c, f);  // nl == 0: the layers still run (they write the KV)
        if (r) return r;
      }
      for (size_t k = 0; k < finishing.size(); ++k) row_of_call[finishing[k]] = next_row + (int)k;
      next_row += nl;
    }
    // shared members: copy the leader's partial tail block, reuse its logits row
    for (int i = 0; i < n; ++i) {
      Seq& s = c->seqs[ids[i]];
      if (s.leader) continue;
      int li = -1;
      for (int j = 0; j < n; ++j)
        if (ids[j] == s.leader_id) li = j;
      if (li < 0) return fail(c, ER_ESTATE, "leader of sequence %d must be prefilled in the same call", ids[i]);
      row_of_call[i] = row_of_call[li];
      if (s.prompt_len % KV_BLOCK) {
        const Seq& L = c->seqs[s.leader_id];
        const size_t b = (size_t)(s.prompt_len / KV_BLOCK);
        HIPC(c, hipMemcpyAsync((char*)c->kv_pool + (size_t)s.bt.blocks[b] * c->block_bytes,
                               (char*)c->kv_pool + (size_t)L.bt.blocks[b] * c->block_bytes, c->block_bytes,
                               hipMemcpyDeviceToDevice, c->st));
      }
    }
    // first tokens: AR draws at position prompt_len
    Meta& M = c->meta;
    if (int r_ = meta_begin(c)) return r_;
    size_t o_ids, o_pos, o_map;
    int32_t* h_ids = M.push<int32_t>(n, &o_ids);
    int32_t* h_pos = M.push<int32_t>(n, &o_pos);
    int32_t* h_map = M.push<int32_t>(n, &o_map);
    for (int i = 0; i < n; ++i) {
      h_ids[i] = ids[i];
      h_pos[i] = c->seqs[ids[i]].prompt_len;
      h_map[i] = row_of_call[i];
    }
    if (int r_ = meta_upload(c)) return r_;
    KC(c, launch_row_stats(c->logits_p, next_row, V, V, c->rd.temperature, c->rd.top_p, c->stats_p, c->st));
    KC(c, launch_sample_rows(c->logits_p, c->stats_p, n, V, V, c->rd.temperature, c->rd.top_p, c->rd.seed,
                             M.dev<int32_t>(o_ids), M.dev<int32_t>(o_pos), 0, PURPOSE_AR, c->out_d, 1,
                             M.dev<int32_t>(o_map), c->st));
    HIPC(c, hipMemcpyAsync(c->out_h, c->out_d, (size_t)n * 4, hipMemcpyDeviceToHost, c->st));
    HIPC(c, hipStreamSynchronize(c->st));
    c->last_prefill_row.assign(row_of_call.begin(), row_of_call.end());
    c->last_mode = 2;
    c->last_B = n;
    for (int i = 0; i < n; ++i) {
      Seq& s = c->seqs[ids[i]];
      s.prefilled = true;
      s.n = s.prompt_len;
      s.pending = c->out_h[i];
      s.generated = 1;
      s.toks.assign(tokens + offsets[i], tokens + offsets[i + 1]);
      s.toks.push_back(s.pending);
      first_tok_out[i] = c->out_h[i];
      c->stats.tokens_kept += 1;
      if (s.generated >= s.max_new) finish_seq(c, s);
    }
    return ER_OK;
  } catch (...) {
    return fail(c, ER_EINVAL, "internal error");
  }
}

int er_spec_step(er_ctx* c, int n, const int32_t* ids, int32_t* tokens_out, int32_t* n_emitted_out,
                 er_step_info* info) {
  if (!c) return ER_EINVAL;
  try {
    int r = check_batch(c, n, ids, true);
    if (r) return r;
    if (!tokens_out || !n_emitted_out) return fail(c, ER_EINVAL, "null output");
    return do_spec(c, n, ids, current_gamma(c), tokens_out, c->rd.gamma_max + 1, n_emitted_out, info);
  } catch (...) {
    return fail(c, ER_EINVAL, "internal error");
  }
}

int er_ar_step(er_ctx* c, int n, const int32_t* ids, int32_t* tokens_out, er_step_info* info) {
  if (!c) return ER_EINVAL;
  try {
    int r = check_batch(c, n, ids, true);
    if (r) return r;
    if (!tokens_out) return fail(c, ER_EINVAL, "null output");
    return do_ar(c, n, ids, tokens_out, 1, nullptr, info);
  } catch (...) {
    return fail(c, ER_EINVAL, "internal error");
  }
}

int er_step(er_ctx* c, int n, const int32_t* ids, int32_t* tokens_out, int32_t* n_emitted_out, er_step_info* info) {
  if (!c) return ER_EINVAL;
  try {
    int r = check_batch(c, n, ids, true);
    if (r) return r;
    if (!tokens_out || !n_emitted_out) return fail(c, ER_EINVAL, "null output");
    const auto t0 = std::chrono::steady_clock::now();
    const int stride = c->rd.gamma_max + 1;
    if (c->policy == ER_POLICY_HISTORY) {
      // history drafts once the cache holds a record and the batch is small enough, else AR
      const bool hist = c->hist && c->hist->cache.records() >= 1 && n <= c->hist_max_batch;
      return hist ? do_history(c, n, ids, tokens_out, stride, n_emitted_out, info)
                  : do_ar(c, n, ids, tokens_out, stride, n_emitted_out, info);
    }
    const int g = plan(c, n, ids);
    r = g == 0 ? do_ar(c, n, ids, tokens_out, stride, n_emitted_out, info)
               : do_spec(c, n, ids, g, tokens_out, stride, n_emitted_out, info);
    if (r == ER_OK && c->policy == ER_POLICY_TIMING) {
      // wall time of the step, plan to the synchronized end, as the guard's sample
      const double ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
      double tok = 0;
      for (int i = 0; i < n; ++i) tok += n_emitted_out[i];
      if (ms > 0) er_guard_observe(&c->guard, n, g > 0 ? 1 : 0, tok, ms);
    }
    return r;
  } catch (...) {
    return fail(c, ER_EINVAL, "internal error");
  }
}

int er_rollout(er_ctx* c, int n, const int32_t* ids, int32_t cap, int32_t* out_tokens, int32_t* out_len,
               er_stats* stats_out) {
  if (!c) return ER_EINVAL;
  try {
    if (n <= 0 || !ids || !out_tokens || !out_len || cap <= 0) return fail(c, ER_EINVAL, "bad arguments");
    if (n > c->rd.max_batch) return fail(c, ER_EINVAL, "batch %d exceeds max_batch %d", n, c->rd.max_batch);
    for (int i = 0; i < n; ++i) {
      const int32_t id = ids[i];
      if (id < 0 || id >= (int32_t)c->seqs.size() || !c->seqs[id].alive) return fail(c, ER_EINVAL, "unknown sequence %d", id);
      const Seq& s = c->seqs[id];
      if (!s.prefilled) return fail(c, ER_ESTATE, "sequence %d not prefilled", id);
      if (s.max_new > cap) return fail(c, ER_EINVAL, "max_new of %d exceeds cap", id);
      out_len[i] = 0;
    }
    // the prefill token (and any generated since) is not retrievable here;
    // the loop records what it generates after the current state.
    std::vector<int32_t> act, slot;
    for (int i = 0; i < n; ++i)
      if (!c->seqs[ids[i]].finished) { act.push_back(ids[i]); slot.push_back(i); }
    const int stride = c->rd.gamma_max + 1;
    std::vector<int32_t> tok((size_t)n * stride), ne(n);
    while (!act.empty()) {
      const int B = (int)act.size();
      int r = er_step(c, B, act.data(), tok.data(), ne.data(), nullptr);
      if (r) return r;
      std::vector<int32_t> act2, slot2;
      for (int b = 0; b < B; ++b) {
        const int i = slot[b];
        for (int k = 0; k < ne[b]; ++k) out_tokens[(size_t)i * cap + out_len[i] + k] = tok[(size_t)b * stride + k];
        out_len[i] += ne[b];
        if (!c->seqs[act[b]].finished) { act2.push_back(act[b]); slot2.push_back(i); }
      }
      act.swap(act2);
      slot.swap(slot2);
    }
    if (stats_out) return er_get_stats(c, stats_out);
    return ER_OK;
  } catch (...) {
    return fail(c, ER_EINVAL, "internal error");
  }
}

int er_set_gamma(er_ctx* c, int gamma) {
  if (!c) return ER_EINVAL;
  if (gamma < 0 || gamma > c->rd.gamma_max) return fail(c, ER_EINVAL, "gamma %d outside 0..%d", gamma, c->rd.gamma_max);
  c->gamma_pinned = gamma;
  if (gamma > 0 && c->plan.choice > 0) c->plan.choice = gamma;
  return ER_OK;
}

int er_set_policy(er_ctx* c, int policy) {
  if (!c) return ER_EINVAL;
  if (policy < ER_POLICY_AUTO || policy > ER_POLICY_HISTORY) return fail(c, ER_EINVAL, "unknown policy %d", policy);
  if (policy == ER_POLICY_TIMING && c->policy != ER_POLICY_TIMING) {
    er_guard_params gp = c->guard.p;
    if (er_guard_init(&c->guard, &gp) != ER_OK) {
      er_guard_default_params(&gp);
      er_guard_init(&c->guard, &gp);
    }
  }
  c->policy = policy;
  c->plan.choice = -1;
  return ER_OK;
}

int er_kv_free(er_ctx* c, int n, const int32_t* ids) {
  if (!c) return ER_EINVAL;
  if (n < 0 || (n > 0 && !ids)) return fail(c, ER_EINVAL, "bad arguments");
  for (int i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || id >= (int32_t)c->seqs.size() || !c->seqs[id].alive) return fail(c, ER_EINVAL, "unknown sequence %d", id);
  }
  for (int i = 0; i < n; ++i) {
    Seq& s = c->seqs[ids[i]];
    s.bt.release(c->pool);
    s.alive = false;
    --c->alive;
  }
  return ER_OK;
}

int er_seq_info(er_ctx* c, int32_t id, int32_t* generated, int32_t* context_len, int32_t* finished) {
  if (!c) return ER_EINVAL;
  if (id < 0 || id >= (int32_t)c->seqs.size() || !c->seqs[id].alive) return fail(c, ER_EINVAL, "unknown sequence %d", id);
  const Seq& s = c->seqs[id];
  if (generated) *generated = s.generated;
  if (context_len) *context_len = s.n;
  if (finished) *finished = s.finished ? 1 : 0;
  return ER_OK;
}

int er_get_stats(er_ctx* c, er_stats* out) {
  if (!c || !out) return ER_EINVAL;
  er_stats s = c->stats;
  s.effective_length = s.effective_times ? (double)s.total_right_length / (double)s.effective_times : 0.0;
  s.effective_percent = s.predict_times ? (double)s.effective_times / (double)s.predict_times : 0.0;
  s.alpha_ema = c->alpha_ema;
  s.gamma = c->plan.choice < 0 ? current_gamma(c) : c->plan.choice;
  s.mode = c->plan.choice == 0 ? ER_MODE_AR : ER_MODE_SD;
  *out = s;
  return ER_OK;
}

int er_reset_stats(er_ctx* c) {
  if (!c) return ER_EINVAL;
  c->stats = er_stats{};
  c->alpha_ema = c->alpha_init;
  c->plan = PlanState{};
  {
    er_guard_params gp = c->guard.p;
    er_guard_init(&c->guard, &gp);
  }
  return ER_OK;
}

int er_set_timing(er_ctx* c, int period, int first_n) {
  if (!c || period < 0 || first_n < 0) return ER_EINVAL;
  c->timing_period = period;
  c->timing_first = first_n;
  c->step_count = 0;
  return ER_OK;
}

int er_set_persistent(er_ctx* c, int on) {
  if (!c) return ER_EINVAL;
  if (on && !c->dec_avail) return fail(c, ER_ESTATE, "the persistent decode forward cannot run here");
  c->dec_on = on != 0 && c->dec_avail;
  return ER_OK;
}

int er_set_graphs(er_ctx* c, int max_batch) {
  if (!c) return ER_EINVAL;
  if (max_batch < 0) return fail(c, ER_EINVAL, "max_batch must be >= 0");
  try {
    HIPC(c, hipStreamSynchronize(c->st));
    graph_drop(c);
    if (max_batch == 0) {
      c->graph_max = 0;
      if (c->pad_block >= 0) c->pool.decref(c->pad_block);
      c->pad_block = -1;
      if (c->cap_st) (void)hipStreamDestroy(c->cap_st);
      c->cap_st = nullptr;
      return ER_OK;
    }
    if (!c->cap_st) HIPC(c, hipStreamCreateWithFlags(&c->cap_st, hipStreamNonBlocking));
    if (c->pad_block < 0) {
      c->pad_block = c->pool.alloc();
      if (c->pad_block < 0) return fail(c, ER_ENOMEM, "no free KV block for the padding rows");
      HIPC(c, hipMemsetAsync((char*)c->kv_pool + (size_t)c->pad_block * c->block_bytes, 0, c->block_bytes, c->st));
      HIPC(c, hipStreamSynchronize(c->st));
    }
    c->graph_max = max_batch;
    return ER_OK;
  } catch (...) {
    return fail(c, ER_EINVAL, "internal error");
  }
}

int er_set_library_gemm(er_ctx* c, int min_rows) {
  if (!c || min_rows < -1) return ER_EINVAL;
  if (min_rows != 0 && !c->lws.blas) return fail(c, ER_ESTATE, "no library GEMM here (fp32 model or hipBLASLt unavailable)");
  c->lws.blas_min_m = min_rows;
  return ER_OK;
}

int er_get_graph_stats(const er_ctx* c, er_graph_stats* out) {
  if (!c || !out) return ER_EINVAL;
  out->max_batch = c->graph_max;
  out->cached = (int32_t)c->graphs.size();
  out->captures = c->graph_captures;
  out->replays = c->graph_replays;
  out->evictions = c->graph_evictions;
  return ER_OK;
}

int er_set_decode_spin_limit(er_ctx* c, int64_t polls) {
  if (!c || polls < 1) return ER_EINVAL;
  c->dec_spin_limit = (long)polls;
  return ER_OK;
}

int er_set_decode_trace(er_ctx* c, int on) {
  if (!c) return ER_EINVAL;
  if (!on) {
    if (c->dec_trace) (void)hipFree(c->dec_trace);
    c->dec_trace = nullptr;
    c->dec_trace_max = 0;
    return ER_OK;
  }
  if (c->dec_trace) return ER_OK;
  const int nb = 8 * c->md.n_layers + 8;  // barriers of one forward, with room
  const int G = std::max(c->dec_nwg[FMT_BF16], 1024);
  HIPC(c, hipMalloc((void**)&c->dec_trace, ((size_t)nb * G * 2 + G) * 8));
  c->dec_trace_max = nb;
  return ER_OK;
}

int er_get_decode_trace(er_ctx* c, double* work_us, double* release_us, int max, int* n_out) {
  if (!c || !n_out) return ER_EINVAL;
  *n_out = 0;
  if (!c->dec_trace || c->dec_trace_nwg <= 0) return fail(c, ER_ESTATE, "no traced persistent forward");
  const int G = c->dec_trace_nwg, nb = c->dec_trace_max;
  std::vector<unsigned long long> t((size_t)nb * G * 2 + G);
  HIPC(c, hipStreamSynchronize(c->st));
  HIPC(c, hipMemcpy(t.data(), c->dec_trace, t.size() * 8, hipMemcpyDeviceToHost));
  // phase k runs from the first release of barrier k-1 (kernel start for k = 0) to the last
  // arrival at barrier k; the release is the time from that arrival to the last group's release
  int n = 0;
  unsigned long long prev_start = ~0ull;
  for (int b = 0; b < G; ++b) prev_start = std::min(prev_start, t[(size_t)nb * G * 2 + b]);
  for (int k = 0; k < nb; ++k) {
    unsigned long long arr = 0, rel = 0, first_rel = ~0ull;
    bool any = false;
    for (int b = 0; b < G; ++b) {
      const unsigned long long a0 = t[((size_t)k * G + b) * 2], a1 = t[((size_t)k * G + b) * 2 + 1];
      if (a0 == 0 || a1 == 0) continue;
      any = true;
      arr = std::max(arr, a0);
      rel = std::max(rel, a1);
      first_rel = std::min(first_rel, a1);
    }
    if (!any || arr < prev_start) break;
    if (n < max && work_us) work_us[n] = (double)(arr - prev_start) * 0.01;
    if (n < max && release_us) release_us[n] = (double)(rel - arr) * 0.01;
    ++n;
    prev_start = first_rel;
  }
  *n_out = n;
  HIPC(c, hipMemset(c->dec_trace, 0, t.size() * 8));
  return ER_OK;
}

int er_get_persistent(const er_ctx* c, int* on) {
  if (!c || !on) return ER_EINVAL;
  *on = c->dec_on ? 1 : 0;
  return ER_OK;
}

int er_set_fused(er_ctx* c, int on) {
  if (!c) return ER_EINVAL;
  graph_drop(c);
  c->fuse = c->bf16 && on != 0;
  return ER_OK;
}

int er_history_create(int prefix_len, er_history** out) {
  if (!out || prefix_len < 1) return ER_EINVAL;
  try {
    *out = new er_history(prefix_len);
    return ER_OK;
  } catch (...) {
    return ER_ENOMEM;
  }
}

int er_history_destroy(er_history* h) {
  delete h;
  return ER_OK;
}

int er_history_add(er_history* h, int prompt_len, const int32_t* prompt, int resp_len, const int32_t* resp,
                   float reward) {
  if (!h || prompt_len < 0 || resp_len < 0 || (prompt_len > 0 && !prompt) || (resp_len > 0 && !resp) ||
      !(reward == reward))
    return ER_EINVAL;
  try {
    h->cache.add(prompt, prompt_len, resp, resp_len, reward);
    return ER_OK;
  } catch (...) {
    return ER_ENOMEM;
  }
}

int er_history_propose(const er_history* h, int prompt_len, const int32_t* prompt, int ctx_len, const int32_t* ctx,
                       int gamma, int32_t* out, int32_t* n_out) {
  if (!h || !n_out || prompt_len < 0 || ctx_len < 0 || gamma < 0 || (prompt_len > 0 && !prompt) ||
      (ctx_len > 0 && !ctx) || (gamma > 0 && !out))
    return ER_EINVAL;
  *n_out = h->cache.propose(prompt, prompt_len, ctx, ctx_len, gamma, out);
  return ER_OK;
}

int er_history_records(const er_history* h, int64_t* n) {
  if (!h || !n) return ER_EINVAL;
  *n = h->cache.records();
  return ER_OK;
}

int er_set_history(er_ctx* c, er_history* h, int gamma, int max_batch) {
  if (!c) return ER_EINVAL;
  if (gamma < 1 || gamma > c->rd.gamma_max || max_batch < 1)
    return fail(c, ER_EINVAL, "history gamma must be in 1..%d and max_batch >= 1", c->rd.gamma_max);
  c->hist = h;
  c->hist_gamma = gamma;
  c->hist_max_batch = max_batch;
  return ER_OK;
}

int er_history_step(er_ctx* c, int n, const int32_t* ids, int32_t* tokens_out, int32_t* n_emitted_out,
                    er_step_info* info) {
  if (!c) return ER_EINVAL;
  try {
    int r = check_batch(c, n, ids, true);
    if (r) return r;
    if (!tokens_out || !n_emitted_out) return fail(c, ER_EINVAL, "null output");
    if (!c->hist) return fail(c, ER_ESTATE, "no history cache attached (er_set_history)");
    return do_history(c, n, ids, tokens_out, c->rd.gamma_max + 1, n_emitted_out, info);
  } catch (...) {
    return fail(c, ER_EINVAL, "internal error");
  }
}

int er_kv_free_blocks(er_ctx* c, int64_t* free_blocks, int64_t* total_blocks) {
  if (!c) return ER_EINVAL;
  if (free_blocks) *free_blocks = c->pool.free_count();
  if (total_blocks) *total_blocks = c->pool.total();
  return ER_OK;
}

int er_debug_logits(er_ctx* c, int which, int slot, float* host_out, int32_t* rows_out) {
  if (!c) return ER_EINVAL;
  const int V = c->md.vocab;
  if (slot < 0 || slot >= c->last_B) return fail(c, ER_EINVAL, "slot %d outside the last batch", slot);
  std::vector<const float*> rows;
  if (which == 0) {
    if (c->last_mode != ER_MODE_SD) return fail(c, ER_ESTATE, "last step was not speculative");
    for (int j = 0; j < c->last_gamma; ++j) rows.push_back(c->logits_q + ((size_t)j * c->last_rows + slot) * V);
  } else if (which == 1) {
    if (c->last_mode == ER_MODE_SD) {
      for (int i = 0; i <= c->last_gamma; ++i) rows.push_back(c->logits_p + ((size_t)slot * (c->last_gamma + 1) + i) * V);
    } else if (c->last_mode == ER_MODE_AR) {
      rows.push_back(c->logits_p + (size_t)slot * V);
    } else if (c->last_mode == 2) {
      rows.push_back(c->logits_p + (size_t)c->last_prefill_row[(size_t)slot] * V);
    } else {
      return fail(c, ER_ESTATE, "no step yet");
    }
  } else {
    return fail(c, ER_EINVAL, "which must be 0 or 1");
  }
  if (rows_out) *rows_out = (int32_t)rows.size();
  if (!host_out) return ER_OK;
  for (size_t i = 0; i < rows.size(); ++i)
    HIPC(c, hipMemcpy(host_out + i * V, rows[i], (size_t)V * 4, hipMemcpyDeviceToHost));
  return ER_OK;
}

int er_debug_drafts(er_ctx* c, int32_t* host_out) {
  if (!c || !host_out) return ER_EINVAL;
  if (c->last_mode != ER_MODE_SD) return fail(c, ER_ESTATE, "last step was not speculative");
  const int G1 = c->last_gamma + 1;
  std::vector<int32_t> tok((size_t)c->last_B * G1);
  HIPC(c, hipMemcpy(tok.data(), c->meta.d + c->last_tok_off, tok.size() * 4, hipMemcpyDeviceToHost));
  for (int b = 0; b < c->last_B; ++b)
    for (int j = 0; j < c->last_gamma; ++j) host_out[(size_t)b * c->last_gamma + j] = tok[(size_t)b * G1 + 1 + j];
  return ER_OK;
}

int er_set_kernel_profile(er_ctx* c, int on) {
  if (!c) return ER_EINVAL;
  if (on && c->kev.empty()) {
    c->kev.resize(16384);
    for (auto& e : c->kev)
      if (hipEventCreate(&e) != hipSuccess) return fail(c, ER_EDEVICE, "hipEventCreate");
  }
  if (on < 0 || on > ER_KPROF_ATTENTION) return fail(c, ER_EINVAL, "kernel profile mode %d", on);
  c->kprof = on == ER_KPROF_ALL ? (KPROF_LINEAR | KPROF_ATTENTION) : (on == ER_KPROF_ATTENTION ? KPROF_ATTENTION : 0);
  c->krec.clear();
  c->kev_used = 0;
  return ER_OK;
}

int er_get_kernel_profile(er_ctx* c, er_kernel_stat* out, int max, int* n_out) {
  if (!c || !n_out || max < 0 || (max > 0 && !out)) return ER_EINVAL;
  int i = 0;
  for (const auto& kv : c->kstat) {
    if (i < max) {
      er_kernel_stat& o = out[i];
      memset(&o, 0, sizeof o);
      snprintf(o.name, sizeof o.name, "%s", kv.first.c_str());
      o.launches = kv.second.n;
      o.ms = kv.second.ms;
      o.bytes = kv.second.bytes;
      o.flops = kv.second.flops;
    }
    ++i;
  }
  *n_out = i;
  return ER_OK;
}

int er_reset_kernel_profile(er_ctx* c) {
  if (!c) return ER_EINVAL;
  c->kstat.clear();
  return ER_OK;
}

void er_guard_default_params(er_guard_params* p) {
  if (!p) return;
  p->max_sd_batch = 8;
  p->probe_max_batch = 2;
  p->compare_after = 64;
  p->probe_steps = 8;
  p->ema_alpha = 0.3;
  p->margin = 1.02;
  p->cooldown = 8192;
  p->cooldown_max = 65536;
  p->cooldown_growth = 4.0;
  p->bad_ratio = 0.98;
}

int er_guard_init(er_guard_state* g, const er_guard_params* p) {
  if (!g || !p) return ER_EINVAL;
  if (p->max_sd_batch < 1 || p->max_sd_batch > (1 << 15) || p->probe_max_batch < 0 || p->compare_after < 1 ||
      p->probe_steps < 0 || !(p->ema_alpha > 0 && p->ema_alpha <= 1) || !(p->margin > 0) || p->cooldown < 0 ||
      p->cooldown_max < 0 || !(p->cooldown_growth > 0) || !(p->bad_ratio > 0))
    return ER_EINVAL;
  std::memset(g, 0, sizeof *g);
  g->p = *p;
  for (int b = 0; b < ER_GUARD_BUCKETS; ++b) {
    g->ema_ar[b] = -1.0;
    g->ema_sd[b] = -1.0;
    g->cool_len[b] = p->cooldown;
  }
  return ER_OK;
}

namespace {
int guard_bucket(int batch) {  // smallest b with 2^b >= batch
  int b = 0;
  while ((1 << b) < batch) ++b;
  return b;
}
}  // namespace

int er_guard_choose(er_guard_state* g, int batch) {
  if (!g || batch < 1) return -1;
  const int64_t now = g->step++;
  if (batch > g->p.max_sd_batch) return 0;
  const int b = guard_bucket(batch);
  if (g->probe_left[b] > 0) return 1;
  if (g->n_ar[b] < g->p.compare_after || now < g->cool_until[b]) return 0;
  if (g->ema_sd[b] >= 0) return g->ema_sd[b] > g->p.margin * g->ema_ar[b] ? 1 : 0;
  if (batch <= g->p.probe_max_batch) {
    g->probe_left[b] = g->p.probe_steps;
    return 1;
  }
  return 0;
}

int er_guard_observe(er_guard_state* g, int batch, int branch, double tokens, double ms) {
  if (!g || batch < 1 || (branch != 0 && branch != 1) || !(ms > 0) || !(tokens >= 0)) return ER_EINVAL;
  if (batch > g->p.max_sd_batch) return ER_OK;
  const int b = guard_bucket(batch);
  const double rate = tokens / ms;
  if (branch == 0) {
    ++g->n_ar[b];
  } else {
    if (g->ema_ar[b] >= 0 && rate < g->p.bad_ratio * g->ema_ar[b]) {
      // bad speculative step: back to autoregressive, drop the score, cool down
      const int64_t len = g->cool_len[b];
      g->cool_until[b] = g->step + len;
      g->cool_len[b] = std::min((int64_t)((double)len * g->p.cooldown_growth), (int64_t)g->p.cooldown_max);
      g->probe_left[b] = 0;
      g->ema_sd[b] = -1.0;
      return ER_OK;
    }
    if (g->probe_left[b] > 0 && --g->probe_left[b] == 0) g->cool_len[b] = g->p.cooldown;
  }
  double& e = branch ? g->ema_sd[b] : g->ema_ar[b];
  e = e < 0 ? rate : (1.0 - g->p.ema_alpha) * e + g->p.ema_alpha * rate;
  return ER_OK;
}

int er_get_guard(const er_ctx* c, er_guard_state* out) {
  if (!c || !out) return ER_EINVAL;
  if (c->policy != ER_POLICY_TIMING) return ER_ESTATE;
  *out = c->guard;
  return ER_OK;
}

static CostModel cost_of(const er_cost_model* m) {
  return CostModel{m->n_layers, m->d_model, m->n_q_heads, m->n_kv_heads, m->head_dim, m->ffn, m->vocab,
                   m->w_bytes, m->q_bytes, m->kv_bytes_el, m->hbm_bytes_per_s, m->flops_per_s, m->t_fwd_s,
                   m->t_row_draft_s, m->t_row_target_s};
}

int er_controller_choose(const er_cost_model* m, int batch, double mean_ctx, double alpha, int gamma_min,
                         int gamma_max, int current, double margin, int* gamma_out) {
  if (!m || !gamma_out || batch <= 0 || gamma_min < 1 || gamma_max < gamma_min) return ER_EINVAL;
  *gamma_out = choose(cost_of(m), batch, mean_ctx, alpha, gamma_min, gamma_max, true, current, margin);
  return ER_OK;
}

double er_expected_tokens(double alpha, int gamma) { return expected_tokens(alpha, gamma); }

int er_controller_times(const er_cost_model* m, int batch, double mean_ctx, int gamma, double* t_ar, double* t_sd) {
  if (!m || batch <= 0 || gamma < 1 || !(m->hbm_bytes_per_s > 0) || !(m->flops_per_s > 0)) return ER_EINVAL;
  const CostModel cm = cost_of(m);
  if (t_ar) *t_ar = ar_time(cm, batch, mean_ctx);
  if (t_sd) *t_sd = sd_time(cm, batch, mean_ctx, gamma);
  return ER_OK;
}

int er_controller_plan(const er_cost_model* m, er_plan_state* st, int policy, int batch, double mean_ctx,
                       double alpha_ema, double alpha_init, int gamma_lo, int gamma_hi, double margin,
                       int* gamma_out) {
  if (!m || !st || !gamma_out || batch <= 0 || gamma_lo < 1 || gamma_hi < gamma_lo) return ER_EINVAL;
  if (policy != ER_POLICY_AUTO && policy != ER_POLICY_FORCE_SD && policy != ER_POLICY_FORCE_AR) return ER_EINVAL;
  if (policy == ER_POLICY_FORCE_AR) { *gamma_out = 0; return ER_OK; }
  PlanState ps;
  ps.choice = st->choice;
  ps.ar_streak = st->ar_streak;
  ps.probe_every = st->probe_every;
  *gamma_out = plan_step(cost_of(m), ps, policy == ER_POLICY_AUTO, batch, mean_ctx, alpha_ema, alpha_init, gamma_lo,
                         gamma_hi, margin);
  st->choice = ps.choice;
  st->ar_streak = ps.ar_streak;
  st->probe_every = ps.probe_every;
  return ER_OK;
}

int er_get_plan_state(const er_ctx* c, er_plan_state* out) {
  if (!c || !out) return ER_EINVAL;
  out->choice = c->plan.choice;
  out->ar_streak = c->plan.ar_streak;
  out->probe_every = c->plan.probe_every;
  return ER_OK;
}

int er_get_cost_model(const er_ctx* c, er_cost_model* out) {
  if (!c || !out) return ER_EINVAL;
  const CostModel& m = c->cost;
  *out = er_cost_model{m.n_layers, m.d_model, m.n_q_heads, m.n_kv_heads, m.head_dim, m.ffn, m.vocab,
                       m.w_bytes, m.q_bytes, m.kv_bytes_el, m.bw, m.flops, m.t_fwd, m.t_row_draft, m.t_row_target};
  return ER_OK;
}

const char* er_last_error(const er_ctx* c) { return c ? c->err.c_str() : "null context"; }

void er_destroy(er_ctx* c) {
  if (!c) return;
  if (c->st) (void)hipStreamSynchronize(c->st);
  else (void)hipDeviceSynchronize();
  graph_drop(c);
  if (c->cap_st) (void)hipStreamDestroy(c->cap_st);
  blas_destroy(c->lws.blas);
  if (c->meta.h) (void)hipHostFree(c->meta.h);
  if (c->out_h) (void)hipHostFree(c->out_h);
  if (c->dec_trace) (void)hipFree(c->dec_trace);
  if (c->have_ev)
    for (auto& e : c->ev) (void)hipEventDestroy(e);
  for (auto& e : c->kev) (void)hipEventDestroy(e);
  if (c->meta_ev) (void)hipEventDestroy(c->meta_ev);
  delete c;
}

}  // extern "C"
