// Operation-level C ABI (include/er_ops.h): thin argument checks around the
// kernel launchers.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/er_api.h"
#include "../../include/er_ops.h"
#include "kernels.h"

using namespace er;

namespace {

struct OpWs {
  float* partial = nullptr;
  int* counters = nullptr;
  float* attn = nullptr;
  double* resid = nullptr;
  uint16_t* xn = nullptr;
  int device = -1;
};
OpWs g_ws;
std::mutex g_mu;

constexpr size_t kPartialFloats = (size_t)16 << 20;
constexpr int kCounters = 65536;
constexpr size_t kAttnFloats = (size_t)8 << 20;
constexpr size_t kResidDoubles = (size_t)1 << 20;
constexpr size_t kXnElems = (size_t)8 << 20;

int ensure_ws() {
  std::lock_guard<std::mutex> lk(g_mu);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ER_EDEVICE;
  if (g_ws.partial && g_ws.device == dev) return ER_OK;
  if (hipMalloc(&g_ws.partial, kPartialFloats * 4) != hipSuccess) return ER_ENOMEM;
  if (hipMalloc(&g_ws.counters, kCounters * 4) != hipSuccess) return ER_ENOMEM;
  if (hipMemset(g_ws.counters, 0, kCounters * 4) != hipSuccess) return ER_EDEVICE;
  if (hipMalloc(&g_ws.attn, kAttnFloats * 4) != hipSuccess) return ER_ENOMEM;
  if (hipMalloc(&g_ws.resid, kResidDoubles * 8) != hipSuccess) return ER_ENOMEM;
  if (hipMalloc(&g_ws.xn, kXnElems * 2) != hipSuccess) return ER_ENOMEM;
  g_ws.device = dev;
  return ER_OK;
}

int code(int r) { return r == 0 ? ER_OK : (r == -1 ? ER_EINVAL : (r == -2 ? ER_ENOMEM : ER_EDEVICE)); }

}  // namespace

// Scratch of er_op_attention_noalloc: the split partials of one call, in a
// fixed device array (each GPU holds its own copy for the life of the
// process).  Host code never passes the array's name to a kernel: its device
// address comes from hipGetSymbolAddress, once per device, with that device
// current.
constexpr size_t kNoAllocScratchFloats = (size_t)4 << 20;   // 16 MiB
static __device__ __align__(256) float scratch[kNoAllocScratchFloats];

namespace {

constexpr int kMaxDevices = 64;
float* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

// The calling thread's device's copy of the scratch array, or null on failure.
float* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int er_op_quantize(int quant, int w_dtype, const void* d_w, int N, int K, void* d_codes, void* d_scale, void* d_zero,
                   void* stream) {
  if (!d_w || !d_codes || !d_scale || N <= 0 || K <= 0) return ER_EINVAL;
  if (w_dtype != ER_F32 && w_dtype != ER_BF16) return ER_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  if (quant == ER_W8_PERCH_SYM)
    return code(launch_quantize_w8(d_w, w_dtype == ER_BF16, N, K, (int8_t*)d_codes, (float*)d_scale, st));
  if (quant == ER_W4_G128_ASYM) {
    if (w_dtype != ER_BF16 || K % 128 || !d_zero) return ER_EINVAL;
    return code(launch_quantize_w4(d_w, N, K, (uint8_t*)d_codes, (uint16_t*)d_scale, (uint8_t*)d_zero, st));
  }
  return ER_EINVAL;
}

int er_op_w4_kernel_order(const void* d_canon, int N, int K, void* d_out, void* stream) {
  if (!d_canon || !d_out || N <= 0 || K <= 0 || K % 8) return ER_EINVAL;
  return code(launch_w4_to_kernel_order((const uint8_t*)d_canon, N, K, (uint8_t*)d_out, (hipStream_t)stream));
}

int er_op_linear(int x_dtype, const void* d_x, int ldx, int M, int fmt, const void* d_w, const void* d_scale,
                 const void* d_zero, int N, int K, float* d_y, int ldy, int path, void* stream) {
  if (!d_x || !d_w || !d_y || M < 0 || N <= 0 || K <= 0 || ldx < K || ldy < N) return ER_EINVAL;
  if (x_dtype != ER_F32 && x_dtype != ER_BF16) return ER_EINVAL;
  if (fmt < ER_FMT_F32 || fmt > ER_FMT_W4 || path < 0 || (path > 3 && path < 1000)) return ER_EINVAL;
  if ((fmt == ER_FMT_W8 || fmt == ER_FMT_W4) && !d_scale) return ER_EINVAL;
  if (fmt == ER_FMT_W4 && !d_zero) return ER_EINVAL;
  int r = ensure_ws();
  if (r) return r;
  LinearW W{fmt, d_w, d_scale, d_zero, N, K};
  LinearWs ws{g_ws.partial, kPartialFloats, g_ws.counters, kCounters, g_ws.xn, kXnElems};
  return code(launch_linear(d_x, x_dtype == ER_BF16, ldx, M, W, d_y, ldy, EPI_F32, ws, path, (hipStream_t)stream));
}

int er_op_linear_fused(int epi, const void* d_x, int ldx, int M, int xnorm, const int32_t* d_xrow,
                       const uint64_t* d_ssq_in, const void* d_gnorm, float eps, int fmt, const void* d_w,
                       const void* d_scale, const void* d_zero, int N, int K, void* d_y, int ldy,
                       uint64_t* d_ssq_acc, uint64_t* d_ssq_zero, const er_qkv_args* qkv, int path, void* stream) {
  if (!d_x || !d_w || M < 0 || N <= 0 || K <= 0 || ldx < K) return ER_EINVAL;
  if (fmt < ER_FMT_BF16 || fmt > ER_FMT_W4 || path < 0 || path == 1 || (path > 3 && path < 1000)) return ER_EINVAL;
  if ((fmt == ER_FMT_W8 || fmt == ER_FMT_W4) && !d_scale) return ER_EINVAL;
  if (fmt == ER_FMT_W4 && !d_zero) return ER_EINVAL;
  if (xnorm && (!d_ssq_in || !d_gnorm)) return ER_EINVAL;
  if (epi != ER_EPI_F32 && epi != ER_EPI_RESID && epi != ER_EPI_SWIGLU && epi != ER_EPI_QKV) return ER_EINVAL;
  if (epi == ER_EPI_QKV) {
    if (!qkv || !qkv->d_pos || !qkv->d_slot || !qkv->d_cos_sin || !qkv->d_q_out || !qkv->d_kv_pool) return ER_EINVAL;
    if (qkv->hq <= 0 || qkv->hkv <= 0 || qkv->n_layers <= 0 || qkv->layer < 0 || qkv->layer >= qkv->n_layers)
      return ER_EINVAL;
  } else if (!d_y || ldy < (epi == ER_EPI_SWIGLU ? N / 2 : N)) {
    return ER_EINVAL;
  }
  if (d_ssq_zero && (d_ssq_zero == d_ssq_in || d_ssq_zero == d_ssq_acc)) return ER_EINVAL;
  int r = ensure_ws();
  if (r) return r;
  LinArgs a{};
  a.x = d_x;
  a.ldx = ldx;
  a.M = M;
  a.xnorm = xnorm != 0;
  a.xrow = d_xrow;
  a.ssq_in = (const unsigned long long*)d_ssq_in;
  a.gnorm = d_gnorm;
  a.eps = eps;
  a.W = LinearW{fmt, d_w, d_scale, d_zero, N, K};
  a.epi = epi;
  a.y = d_y;
  a.ldy = ldy;
  a.act_bf16 = 1;
  a.ssq_acc = (unsigned long long*)d_ssq_acc;
  a.ssq_zero = (unsigned long long*)d_ssq_zero;
  if (epi == ER_EPI_QKV) {
    a.hq = qkv->hq;
    a.hkv = qkv->hkv;
    a.hd = qkv->hd;
    a.pos = qkv->d_pos;
    a.slot = qkv->d_slot;
    a.cs = (const float2*)qkv->d_cos_sin;
    a.qout = qkv->d_q_out;
    a.kv_pool = qkv->d_kv_pool;
    a.layer = qkv->layer;
    a.n_layers = qkv->n_layers;
  }
  if (epi == ER_EPI_SWIGLU) a.F = N / 2;
  LinearWs ws{g_ws.partial, kPartialFloats, g_ws.counters, kCounters, g_ws.xn, kXnElems};
  return code(launch_linear_fused(a, ws, path, (hipStream_t)stream));
}

int er_op_attention(int act_dtype, const void* d_q, void* d_out, const void* d_kv_pool, int n_layers, int layer,
                    int hq, int hkv, int hd, const int32_t* d_block_table, int bt_stride, const int32_t* d_bt_row,
                    const int32_t* d_q_row0, const int32_t* d_q_pos0, const int32_t* d_q_count, int n_items,
                    int max_q_count, int max_ctx, void* stream) {
  if (!d_q || !d_out || !d_kv_pool || !d_block_table || !d_bt_row || !d_q_row0 || !d_q_pos0 || !d_q_count)
    return ER_EINVAL;
  if (act_dtype != ER_F32 && act_dtype != ER_BF16) return ER_EINVAL;
  if (n_layers <= 0 || layer < 0 || layer >= n_layers || hq <= 0 || hkv <= 0 || n_items < 0 || max_q_count <= 0)
    return ER_EINVAL;
  int r = ensure_ws();
  if (r) return r;
  AttnArgs a{};
  a.q = d_q;
  a.out = d_out;
  a.kv_pool = d_kv_pool;
  a.block_table = d_block_table;
  a.bt_stride = bt_stride;
  a.item_bt_row = d_bt_row;
  a.item_q_row0 = d_q_row0;
  a.item_q_pos0 = d_q_pos0;
  a.item_q_count = d_q_count;
  a.n_items = n_items;
  a.max_q_count = max_q_count;
  a.max_ctx = max_ctx;
  a.hq = hq;
  a.hkv = hkv;
  a.hd = hd;
  a.n_layers = n_layers;
  a.layer = layer;
  a.bf16 = act_dtype == ER_BF16;
  a.ws = g_ws.attn;
  a.ws_floats = kAttnFloats;
  return code(launch_attention(a, (hipStream_t)stream));
}

int er_op_attention_noalloc(int act_dtype, const void* d_q, void* d_out, const void* d_kv_pool, int n_layers,
                            int layer, int hq, int hkv, int hd, const int32_t* d_block_table, int bt_stride,
                            const int32_t* d_bt_row, const int32_t* d_q_row0, const int32_t* d_q_pos0,
                            const int32_t* d_q_count, int n_items, int max_q_count, int max_ctx, void* stream) {
  if (!d_q || !d_out || !d_kv_pool || !d_block_table || !d_bt_row || !d_q_row0 || !d_q_pos0 || !d_q_count)
    return ER_EINVAL;
  if (act_dtype != ER_F32 && act_dtype != ER_BF16) return ER_EINVAL;
  if (n_layers <= 0 || layer < 0 || layer >= n_layers || hq <= 0 || hkv <= 0 || n_items < 0 || max_q_count <= 0)
    return ER_EINVAL;
  float* ws = scratch_ptr();
  if (!ws) return ER_EDEVICE;
  AttnArgs a{};
  a.q = d_q;
  a.out = d_out;
  a.kv_pool = d_kv_pool;
  a.block_table = d_block_table;
  a.bt_stride = bt_stride;
  a.item_bt_row = d_bt_row;
  a.item_q_row0 = d_q_row0;
  a.item_q_pos0 = d_q_pos0;
  a.item_q_count = d_q_count;
  a.n_items = n_items;
  a.max_q_count = max_q_count;
  a.max_ctx = max_ctx;
  a.hq = hq;
  a.hkv = hkv;
  a.hd = hd;
  a.n_layers = n_layers;
  a.layer = layer;
  a.bf16 = act_dtype == ER_BF16;
  // the launcher checks the partials' size against ws_floats before launching
  // anything (-2 -> ER_ENOMEM); nothing in the scratch needs clearing, every
  // partial row the merge reads is written by its unit in the same call
  a.ws = ws;
  a.ws_floats = kNoAllocScratchFloats;
  return code(launch_attention(a, (hipStream_t)stream));
}

size_t er_op_stats_bytes(int V) { return V > 0 ? (size_t)stats_row_bytes(sampler_chunks(V)) : 0; }

int er_op_row_stats(const float* d_logits, int rows, int V, long ld, float temperature, float top_p, void* d_stats,
                    void* stream) {
  if (!d_logits || !d_stats || rows < 0 || V <= 0 || ld < V || !(temperature >= 0.f) || !(top_p > 0.f))
    return ER_EINVAL;
  return code(launch_row_stats(d_logits, rows, V, ld, temperature, top_p, d_stats, (hipStream_t)stream));
}

int er_op_sample_rows(const float* d_logits, const void* d_stats, int rows, int V, long ld, float temperature,
                      float top_p, uint64_t seed, const int32_t* d_seq_id, const int32_t* d_pos, int draft_idx,
                      int purpose, int32_t* d_out, int out_stride, void* stream) {
  if (!d_logits || !d_stats || !d_seq_id || !d_pos || !d_out || rows < 0 || V <= 0 || ld < V || out_stride < 1)
    return ER_EINVAL;
  return code(launch_sample_rows(d_logits, d_stats, rows, V, ld, temperature, top_p, seed, d_seq_id, d_pos, draft_idx,
                                 purpose, d_out, out_stride, nullptr, (hipStream_t)stream));
}

int er_op_spec_decide(const float* d_p_logits, const void* d_p_stats, const float* d_q_logits, const void* d_q_stats,
                      const int32_t* d_tokens, int B, int gamma, int V, float temperature, float top_p, uint64_t seed,
                      const int32_t* d_seq_id, const int32_t* d_pos0, int32_t* d_out_tok, int32_t* d_n_acc,
                      void* stream) {
  if (!d_p_logits || !d_p_stats || !d_tokens || !d_seq_id || !d_pos0 || !d_out_tok || !d_n_acc) return ER_EINVAL;
  if (gamma > 0 && (!d_q_logits || !d_q_stats)) return ER_EINVAL;
  if (B < 0 || gamma < 0 || V <= 0) return ER_EINVAL;
  if ((size_t)B * sampler_chunks(V) > kResidDoubles) return ER_EINVAL;
  int r = ensure_ws();
  if (r) return r;
  return code(launch_spec_decide(d_p_logits, d_p_stats, d_q_logits, d_q_stats, d_tokens, B, gamma, V, temperature,
                                 top_p, seed, d_seq_id, d_pos0, d_out_tok, d_n_acc, g_ws.resid, (hipStream_t)stream));
}

int er_op_philox_uniform(uint64_t seed, const uint32_t* d_ctr, int n, double* d_u, void* stream) {
  if (!d_ctr || !d_u || n < 0) return ER_EINVAL;
  return code(launch_philox_uniform(seed, d_ctr, n, d_u, (hipStream_t)stream));
}

}  // extern "C"
