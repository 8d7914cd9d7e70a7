// Fused sampler of the speculative step: softmax / temperature / top-p
// statistics of logits rows, categorical draws by inverse CDF in vocabulary
// order, and the speculative decision (accept with probability
// min(1, p/q), resample the first rejection from normalize(max(0, p - q)),
// bonus draw from p_{gamma+1} after a full acceptance).
//
// Losslessness is the requirement of the "Accelerating RL Post-Training
// Rollouts via System-Integrated Speculative Decoding" abstract (the target's
// output distribution is preserved); discarding everything after the first
// rejected draft follows the TLT reading notes, section 1.  The accept /
// residual / bonus rule is standard speculative sampling.
//
// Layout of the work: the vocabulary is cut into chunks of 2048 tokens, each
// owned by one wavefront that walks it in 32 tiles of 64.  Per (row, chunk) a
// single pass keeps the chunk max m_c, its first argmax and
// s_c = sum exp((z - m_c)/T) over the chunk (fp64, tiles summed in order).  A
// row's softmax mass is S = sum_c s_c exp((m_c - M)/T).  A draw with uniform u
// picks the first chunk whose running mass reaches u*S, then rescans that
// chunk with the same additions in the same order (so the crossing is always
// inside it) and finds the lane by an inclusive shuffle scan.  Everything is
// deterministic; uniforms come from Philox4x32-10 keyed by the seed with
// counter (sequence, position, draft index, purpose).
//
// Top-p (< 1): the nucleus threshold is found per row by a radix select over
// the order-preserving key of the logit (ties in index order), then the chunk
// masses are recomputed over the kept tokens only.  The radix histograms add
// each token's weight as a 64-bit fixed-point integer (units of 2^-44; a
// weight is at most 1, so a row of up to 2^20 tokens cannot overflow), so the
// bins are exact sums whatever order the threads add in and the threshold is
// the same on every run; a bin sum differs from the exact real sum by at most
// half a unit per token (V * 2^-45, 4.3e-9 at V = 152064, against a row mass
// of at least 1).

#include "common.h"
#include "kernels.h"

namespace er {

constexpr int SCH = 2048;   // tokens per chunk
constexpr int SB = 256;

ER_DEV bool kept(const RowStats& t, float z, int i) {
  const uint32_t k = float_key(z);
  return !(k < t.thr_key || (k == t.thr_key && i > t.thr_idx));
}

ER_DEV const RowStats& row_thr(const void* stats, long r, int nch) {
  return *(const RowStats*)((const char*)stats + r * stats_row_bytes(nch));
}
ER_DEV RowStats& row_thr_w(void* stats, long r, int nch) {
  return *(RowStats*)((char*)stats + r * stats_row_bytes(nch));
}
ER_DEV const ChunkStat* row_chunks(const void* stats, long r, int nch) {
  return (const ChunkStat*)((const char*)stats + r * stats_row_bytes(nch) + sizeof(RowStats));
}
ER_DEV ChunkStat* row_chunks_w(void* stats, long r, int nch) {
  return (ChunkStat*)((char*)stats + r * stats_row_bytes(nch) + sizeof(RowStats));
}

// Row combination: global max (first chunk attaining it gives the lowest-index argmax).
struct RowView {
  float M;
  int arg;
  double S;
};
ER_DEV RowView row_view_mem(const ChunkStat* ch, int nch, float T) {
  RowView v{-INFINITY, 0, 0.0};
  for (int c = 0; c < nch; ++c)
    if (ch[c].m > v.M) { v.M = ch[c].m; v.arg = ch[c].arg; }
  if (T == 0.0f) { v.S = 1.0; return v; }
  for (int c = 0; c < nch; ++c)
    if (ch[c].s > 0.0) v.S += ch[c].s * exp(((double)ch[c].m - (double)v.M) / (double)T);
  return v;
}

// A row's chunk statistics held by one wavefront (every lane active): lane l
// keeps chunks l, l + 64, l + 128 and l + 192, loaded once, unpredicated;
// chunk c is read back by any lane through a shuffle from lane c % 64.  The
// chunk-order loops then cost register shuffles instead of one dependent
// memory round trip per chunk.
constexpr int kRegChunks = 4 * 64;
struct ChunkRegs {
  // four named slots per field; chunk c lives in slot c / 64 of lane c % 64
  float m0, m1, m2, m3;
  int a0, a1, a2, a3;
  double s0, s1, s2, s3;
  double f0, f1, f2, f3;  // exp((m - M) / T) once the row max M is known (row_view_regs)
  ER_DEV void load(const ChunkStat* ch, int nch) {
    const int lane = threadIdx.x & 63;
    const ChunkStat& c0 = ch[min(lane, nch - 1)];
    const ChunkStat& c1 = ch[min(lane + 64, nch - 1)];
    const ChunkStat& c2 = ch[min(lane + 128, nch - 1)];
    const ChunkStat& c3 = ch[min(lane + 192, nch - 1)];
    m0 = c0.m; m1 = c1.m; m2 = c2.m; m3 = c3.m;
    a0 = c0.arg; a1 = c1.arg; a2 = c2.arg; a3 = c3.arg;
    s0 = c0.s; s1 = c1.s; s2 = c2.s; s3 = c3.s;
  }
  // One chunk's fields by a run-time index: every slot is shuffled and the
  // value selected (selecting a slot first made the compiler address the
  // struct in scratch memory).  For single reads, not for loops.
  ER_DEV float mget(int c) const {
    const int k = c >> 6, l = c & 63;
    const float v0 = __shfl(m0, l, 64), v1 = __shfl(m1, l, 64), v2 = __shfl(m2, l, 64), v3 = __shfl(m3, l, 64);
    return k == 0 ? v0 : k == 1 ? v1 : k == 2 ? v2 : v3;
  }
};

// The same loops as row_view_mem over the registers (same operations, same
// order): the four slots in turn, lanes 0..63 within each.  Each lane forms
// its own chunks' factors exp((m - M) / T) once M is known (kept in r for
// the draw), so the in-order sum reads them instead of evaluating them in turn.
ER_DEV RowView row_view_regs(ChunkRegs& r, int nch, float T) {
  RowView v{-INFINITY, 0, 0.0};
  auto scan_m = [&](float mv, int av, int k) {
    const int n = min(64, nch - 64 * k);
    for (int j = 0; j < n; ++j) {
      const float mc = __shfl(mv, j, 64);
      const int ac = __shfl(av, j, 64);
      if (mc > v.M) { v.M = mc; v.arg = ac; }
    }
  };
  scan_m(r.m0, r.a0, 0);
  scan_m(r.m1, r.a1, 1);
  scan_m(r.m2, r.a2, 2);
  scan_m(r.m3, r.a3, 3);
  if (T == 0.0f) { v.S = 1.0; return v; }
  const double M = (double)v.M, dT = (double)T;
  r.f0 = exp(((double)r.m0 - M) / dT);
  r.f1 = exp(((double)r.m1 - M) / dT);
  r.f2 = exp(((double)r.m2 - M) / dT);
  r.f3 = exp(((double)r.m3 - M) / dT);
  auto scan_s = [&](double sv, double fv, int k) {
    const int n = min(64, nch - 64 * k);
    for (int j = 0; j < n; ++j) {
      const double sc = __shfl(sv, j, 64);
      const double fc = __shfl(fv, j, 64);
      if (sc > 0.0) v.S += sc * fc;
    }
  };
  scan_s(r.s0, r.f0, 0);
  scan_s(r.s1, r.f1, 1);
  scan_s(r.s2, r.f2, 2);
  scan_s(r.s3, r.f3, 3);
  return v;
}

// Row combination: global max (first chunk attaining it gives the lowest-index
// argmax) and the mass relative to it, summed in chunk order.  Called by whole
// wavefronts.
ER_DEV RowView row_view(const ChunkStat* ch, int nch, float T) {
  if (nch > kRegChunks) return row_view_mem(ch, nch, T);
  ChunkRegs r;
  r.load(ch, nch);
  return row_view_regs(r, nch, T);
}

// Weight of token i relative to reference m: exp((z - m)/T) if kept, else 0.
ER_DEV double w_rel(float z, int i, double m, float T, const RowStats& t, bool topp) {
  if (topp && !kept(t, z, i)) return 0.0;
  return exp(((double)z - m) / (double)T);
}

// ---------------------------------------------------------------------------
// Per-chunk statistics: one wave per (row, chunk).
// ---------------------------------------------------------------------------
template <bool KEPT>
__global__ __launch_bounds__(SB) void k_chunk_stats(const float* __restrict__ logits, int V, long ld, float T,
                                                    void* __restrict__ stats, int nch) {
  const int r = blockIdx.x;
  const int c = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (c >= nch) return;
  const float* z = logits + (long)r * ld;
  const int base = c * SCH;
  // The chunk's 32 values per lane are loaded once, unpredicated (indices
  // clamped into the row; lanes past V are masked by value below), and both
  // passes run on the registers: a load under the `i < V` predicate made the
  // compiler wait for each one in turn.
  float zv[SCH / 64];
#pragma unroll
  for (int t = 0; t < SCH / 64; ++t) zv[t] = z[min(base + t * 64 + lane, V - 1)];
  float m = -INFINITY;
  int arg = 0x7FFFFFFF;
#pragma unroll
  for (int t = 0; t < SCH / 64; ++t) {
    const int i = base + t * 64 + lane;
    if (i < V) {
      const float v = zv[t];
      if (v > m) { m = v; arg = i; }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(m, o, 64);
    const int oa = __shfl_xor(arg, o, 64);
    if (om > m || (om == m && oa < arg)) { m = om; arg = oa; }
  }
  double s = 0.0;
  if (T != 0.0f) {
    RowStats thr{0u, 0x7FFFFFFF};
    if (KEPT) thr = row_thr(stats, r, nch);
#pragma unroll
    for (int t = 0; t < SCH / 64; ++t) {
      const int i = base + t * 64 + lane;
      const double w = (i < V) ? w_rel(zv[t], i, (double)m, T, thr, KEPT) : 0.0;
      s += wave_sum_d(w);
    }
  }
  if (lane == 0) {
    ChunkStat& o = row_chunks_w(stats, r, nch)[c];
    o.m = m;
    o.arg = arg;
    o.s = s;
  }
}

// Nucleus threshold (top_p < 1), one work-group per row: the kept set is the
// shortest probability-descending prefix (equal probabilities by index)
// whose mass reaches top_p * S.
__global__ __launch_bounds__(SB) void k_topp(const float* __restrict__ logits, int V, long ld, float T, float top_p,
                                             void* __restrict__ stats, int nch) {
  const int r = blockIdx.x;
  const float* z = logits + (long)r * ld;
  const int tid = threadIdx.x;
  __shared__ unsigned long long hist[256];
  __shared__ uint32_t s_prefix;
  __shared__ unsigned long long s_above;
  __shared__ int s_cnt[SB];
  __shared__ int s_any;
  constexpr double FX = 17592186044416.0;  // 2^44: fixed-point units per unit of weight
  const RowView rv = row_view(row_chunks(stats, r, nch), nch, T);
  const double M = rv.M;
  const double target = (double)top_p * rv.S;
  const double target_fx = target * FX;
  uint32_t prefix = 0, mask = 0;
  unsigned long long above = 0;
  for (int d = 3; d >= 0; --d) {
    for (int b = tid; b < 256; b += SB) hist[b] = 0ull;
    __syncthreads();
    for (int i = tid; i < V; i += SB) {
      const uint32_t k = float_key(z[i]);
      if ((k & mask) == prefix)
        atomicAdd(&hist[(k >> (8 * d)) & 255u], (unsigned long long)rint(exp(((double)z[i] - M) / (double)T) * FX));
    }
    __syncthreads();
    if (tid == 0) {
      // highest bin whose cumulative mass reaches the target; if rounding
      // leaves none, the lowest non-empty bin (so the bin always holds tokens)
      unsigned long long cum = above, cum_last = above;
      int chosen = -1, last_nz = -1;
      for (int b = 255; b >= 0; --b) {
        if (hist[b] > 0ull) {
          if ((double)(cum + hist[b]) >= target_fx) { chosen = b; break; }
          last_nz = b;
          cum_last = cum;
        }
        cum += hist[b];
      }
      if (chosen < 0) { chosen = last_nz < 0 ? 0 : last_nz; cum = cum_last; }
      s_prefix = prefix | ((uint32_t)chosen << (8 * d));
      s_above = cum;
    }
    __syncthreads();
    prefix = s_prefix;
    above = s_above;
    mask |= 255u << (8 * d);
  }
  // tokens with key == prefix share one weight; keep the first c in index order
  if (tid == 0) s_any = 0x7FFFFFFF;
  __syncthreads();
  for (int i = tid; i < V; i += SB)
    if (float_key(z[i]) == prefix) { atomicMin(&s_any, i); break; }
  __syncthreads();
  if (s_any == 0x7FFFFFFF) {  // cannot happen (the chosen bin holds mass); keep everything
    if (tid == 0) row_thr_w(stats, r, nch) = RowStats{0u, 0x7FFFFFFF};
    return;
  }
  const double wt = exp(((double)z[s_any] - M) / (double)T);
  int c = (int)ceil((target - (double)above / FX) / wt);
  if (c < 1) c = 1;
  const int chunk = (V + SB - 1) / SB;
  const int lo = tid * chunk, hi = min(V, lo + chunk);
  int cnt = 0;
  for (int i = lo; i < hi; ++i) cnt += (float_key(z[i]) == prefix);
  s_cnt[tid] = cnt;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int t = 0; t < SB; ++t) { const int v = s_cnt[t]; s_cnt[t] = run; run += v; }
    if (c > run) c = run;
    s_any = c;
  }
  __syncthreads();
  c = s_any;
  int idx = -1;
  {
    int run = s_cnt[tid];
    if (run < c)
      for (int i = lo; i < hi; ++i)
        if (float_key(z[i]) == prefix && ++run == c) { idx = i; break; }
  }
  __syncthreads();
  if (idx >= 0) s_any = idx;
  __syncthreads();
  if (tid == 0) row_thr_w(stats, r, nch) = RowStats{prefix, s_any};
}

// Logit rows whose distribution is the point mass on one token (a draft that
// is not sampled, e.g. copied from an earlier rollout): row j * n + b of a
// [g][n][V] block gets 0 at tok[b * G1 + j + 1] and -1e30 elsewhere.  exp of
// -1e30 / T underflows to exactly 0, so the row's softmax, its top-p nucleus
// and its argmax are the point mass, and the lossless rule accepts the draft
// with probability p(draft).
__global__ __launch_bounds__(256) void k_point_mass(float* __restrict__ q, int n, int V, const int32_t* __restrict__ tok,
                                                    int G1) {
  const int row = blockIdx.y;
  const int j = row / n, b = row - j * n;
  const int d = tok[(long)b * G1 + j + 1];
  float* r = q + (long)row * V;
  for (int k = blockIdx.x * blockDim.x + threadIdx.x; k < V; k += gridDim.x * blockDim.x) r[k] = (k == d) ? 0.0f : -1e30f;
}

int launch_point_mass(float* q, int g, int n, int V, const int32_t* tok, int G1, hipStream_t st) {
  if (g <= 0 || n <= 0) return 0;
  if ((long)g * n > 65535) return -1;
  hipLaunchKernelGGL(k_point_mass, dim3(64, g * n), dim3(256), 0, st, q, n, V, tok, G1);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int launch_row_stats(const float* logits, int rows, int V, long ld, float T, float top_p, void* stats,
                     hipStream_t st) {
  if (rows <= 0) return 0;
  const int nch = sampler_chunks(V);
  // The row headers (top-p thresholds) are written by k_topp, the only case
  // that reads them (top_p < 1 and T > 0); other readers check that flag
  // first, so no initializing launch is needed.
  hipLaunchKernelGGL(k_chunk_stats<false>, dim3(rows, (nch + 3) / 4), dim3(SB), 0, st, logits, V, ld, T, stats, nch);
  if (T != 0.0f && top_p < 1.0f) {
    if (V > (1 << 20)) return -1;  // the fixed-point radix histogram holds rows of up to 2^20 tokens
    hipLaunchKernelGGL(k_topp, dim3(rows), dim3(SB), 0, st, logits, V, ld, T, top_p, stats, nch);
    hipLaunchKernelGGL(k_chunk_stats<true>, dim3(rows, (nch + 3) / 4), dim3(SB), 0, st, logits, V, ld, T, stats, nch);
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// ---------------------------------------------------------------------------
// Inverse-CDF draw by one wavefront: first chunk whose running mass reaches
// target, then the same tile sums in the same order inside that chunk.
// WF(i, mref) gives token i's weight relative to mref; chunk c's sum was
// formed relative to ref(c) and enters the row total scaled by f(c).
// ---------------------------------------------------------------------------
template <class WF, class CS>
ER_DEV int wave_draw(const WF& wf, const CS& cs, int nch, int V, double u, double total) {
  const int lane = threadIdx.x & 63;
  const double target = u * total;
  double pre = 0.0;
  const int cc = cs.find(nch, target, &pre);
  if (cc < 0) return 0;
  const double f = cs.f(cc);
  const double ref = cs.ref(cc);
  const int base = cc * SCH;
  // With WF::kPreload the chunk's inputs are loaded once, unpredicated
  // (indices clamped into the row, lanes past V masked below), before the
  // in-order rescan; otherwise each tile loads its own (the two-row residual
  // did not stay in registers that way).
  typename WF::Val vals[WF::kPreload ? SCH / 64 : 1];
  if constexpr (WF::kPreload) {
#pragma unroll
    for (int t = 0; t < SCH / 64; ++t) vals[t] = wf.load(min(base + t * 64 + lane, V - 1));
  }
  double r = 0.0;
  int found = -1, last_nz = -1;
#pragma unroll
  for (int t = 0; t < SCH / 64 && found == -1; ++t) {
    const int i = base + t * 64 + lane;
    double w = 0.0;
    if constexpr (WF::kPreload) {
      w = (i < V) ? wf.weight(vals[t], i, ref) : 0.0;
    } else {
      w = (i < V) ? wf.weight(wf.load(i), i, ref) : 0.0;
    }
    const double ts = wave_sum_d(w);
    if (w > 0.0) last_nz = i;
    if (pre + (r + ts) * f >= target) {
      double sc = w;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const double v = __shfl_up(sc, o, 64);
        if (lane >= o) sc += v;
      }
      const bool hit = (pre + (r + sc) * f >= target) && (w > 0.0);
      const unsigned long long msk = __ballot(hit);
      found = msk ? base + t * 64 + __ffsll(msk) - 1 : -2;  // -2: rounding left no lane; fall back below
    }
    r += ts;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) last_nz = max(last_nz, __shfl_xor(last_nz, o, 64));
  return found >= 0 ? found : (last_nz >= 0 ? last_nz : base);
}

// First chunk whose running mass (chunk sums times their factors, in chunk
// order) reaches target, with the mass before it in *pre; when rounding
// leaves none, the last chunk with mass.  -1 when no chunk has mass.
template <class CS>
ER_DEV int find_chunk_mem(const CS& cs, int nch, double target, double* pre_out) {
  double pre = 0.0, pre_last = 0.0;
  int cc = -1, last_c = -1;
  for (int c = 0; c < nch; ++c) {
    const double sc = cs.sum(c);
    if (sc > 0.0) {
      if (pre + sc * cs.f(c) >= target) { cc = c; break; }
      last_c = c;
      pre_last = pre;
    }
    pre += sc * cs.f(c);
  }
  if (cc < 0) { cc = last_c; pre = pre_last; }
  *pre_out = pre;
  return cc;
}

struct ChunkView {
  const ChunkStat* ch;
  float M;
  float T;
  ER_DEV double sum(int c) const { return ch[c].s; }
  ER_DEV double f(int c) const { return exp(((double)ch[c].m - (double)M) / (double)T); }
  ER_DEV double ref(int c) const { return (double)ch[c].m; }
  ER_DEV int find(int nch, double target, double* pre) const { return find_chunk_mem(*this, nch, target, pre); }
};
// The same view over a wavefront's registers (rows of at most kRegChunks
// chunks): the scan walks the slots in turn with the same operations.
struct ChunkViewRegs {
  ChunkRegs r;
  float M;
  float T;
  // the factors were formed by row_view_regs with this M
  ER_DEV double f(int c) const {
    const int k = c >> 6, l = c & 63;
    const double v0 = __shfl(r.f0, l, 64), v1 = __shfl(r.f1, l, 64), v2 = __shfl(r.f2, l, 64),
                 v3 = __shfl(r.f3, l, 64);
    return k == 0 ? v0 : k == 1 ? v1 : k == 2 ? v2 : v3;
  }
  ER_DEV double ref(int c) const { return (double)r.mget(c); }
  ER_DEV int find(int nch, double target, double* pre_out) const {
    double pre = 0.0, pre_last = 0.0;
    int cc = -1, last_c = -1;
    auto scan = [&](double sv, double fv, int k) {
      const int n = min(64, nch - 64 * k);
      for (int j = 0; j < n && cc < 0; ++j) {
        const double sc = __shfl(sv, j, 64);
        const double fc = __shfl(fv, j, 64);
        if (sc > 0.0) {
          if (pre + sc * fc >= target) { cc = 64 * k + j; break; }
          last_c = 64 * k + j;
          pre_last = pre;
        }
        pre += sc * fc;
      }
    };
    scan(r.s0, r.f0, 0);
    if (cc < 0) scan(r.s1, r.f1, 1);
    if (cc < 0) scan(r.s2, r.f2, 2);
    if (cc < 0) scan(r.s3, r.f3, 3);
    if (cc < 0) { cc = last_c; pre = pre_last; }
    *pre_out = pre;
    return cc;
  }
};

struct RowW {
  const float* z;
  RowStats thr;
  float T;
  bool topp;
  typedef float Val;
  static constexpr bool kPreload = true;
  ER_DEV Val load(int i) const { return z[i]; }
  ER_DEV double weight(Val v, int i, double ref) const { return w_rel(v, i, ref, T, thr, topp); }
};

__global__ __launch_bounds__(64) void k_sample_rows(const float* __restrict__ logits, const void* __restrict__ stats,
                                                   int V, long ld, float T, float top_p, uint64_t seed,
                                                   const int32_t* __restrict__ seq_id, const int32_t* __restrict__ pos,
                                                   int didx, int purpose, int32_t* __restrict__ out, int out_stride,
                                                   const int32_t* __restrict__ row_map, int nch) {
  const int r = blockIdx.x;
  const long lr = row_map ? row_map[r] : r;
  const ChunkStat* ch = row_chunks(stats, lr, nch);
  int t;
  if (nch <= kRegChunks) {
    ChunkRegs cr;
    cr.load(ch, nch);
    const RowView rv = row_view_regs(cr, nch, T);
    if (T == 0.0f) {
      t = rv.arg;
    } else {
      const double u = philox_uniform(seed, (uint32_t)seq_id[r], (uint32_t)pos[r], (uint32_t)didx, (uint32_t)purpose);
      RowW wf{logits + lr * ld, row_thr(stats, lr, nch), T, top_p < 1.0f};
      t = wave_draw(wf, ChunkViewRegs{cr, rv.M, T}, nch, V, u, rv.S);
    }
  } else {
    const RowView rv = row_view_mem(ch, nch, T);
    if (T == 0.0f) {
      t = rv.arg;
    } else {
      const double u = philox_uniform(seed, (uint32_t)seq_id[r], (uint32_t)pos[r], (uint32_t)didx, (uint32_t)purpose);
      RowW wf{logits + lr * ld, row_thr(stats, lr, nch), T, top_p < 1.0f};
      t = wave_draw(wf, ChunkView{ch, rv.M, T}, nch, V, u, rv.S);
    }
  }
  if (threadIdx.x == 0) out[(long)r * out_stride] = t;
}

int launch_sample_rows(const float* logits, const void* stats, int rows, int V, long ld, float T, float top_p,
                       uint64_t seed, const int32_t* seq_id, const int32_t* pos, int didx, int purpose, int32_t* out,
                       int out_stride, const int32_t* row_map, hipStream_t st) {
  if (rows <= 0) return 0;
  hipLaunchKernelGGL(k_sample_rows, dim3(rows), dim3(64), 0, st, logits, stats, V, ld, T, top_p, seed, seq_id, pos,
                     didx, purpose, out, out_stride, row_map, sampler_chunks(V));
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// ---------------------------------------------------------------------------
// Speculative decision.
//  1. k_decide_accept (one wave per sequence): accept tests in order; records
//     the accepted count and writes the accepted drafts.
//  2. k_resid_chunks (one wave per (sequence, chunk)): mass of
//     max(0, p_j - q_j) per chunk at the first rejected position j (skipped
//     after a full acceptance).
//  3. k_decide_draw (one wave per sequence): the residual or bonus draw.
// ---------------------------------------------------------------------------
ER_DEV double prob(const float* z, int i, const RowStats& thr, float T, bool topp, const RowView& rv) {
  if (T == 0.0f) return i == rv.arg ? 1.0 : 0.0;
  return w_rel(z[i], i, (double)rv.M, T, thr, topp) / rv.S;
}

__global__ __launch_bounds__(64) void k_decide_accept(const float* __restrict__ p_logits, const void* __restrict__ p_stats,
                                                     const float* __restrict__ q_logits, const void* __restrict__ q_stats,
                                                     const int32_t* __restrict__ tokens, int B, int gamma, int V,
                                                     float T, int topp, uint64_t seed,
                                                     const int32_t* __restrict__ seq_id,
                                                     const int32_t* __restrict__ pos0, int32_t* __restrict__ out_tok,
                                                     int32_t* __restrict__ n_acc, int nch) {
  const int b = blockIdx.x;
  const int G1 = gamma + 1;
  const uint32_t sid = (uint32_t)seq_id[b];
  const uint32_t n = (uint32_t)pos0[b];
  const int32_t* drafts = tokens + (long)b * G1 + 1;
  int a = gamma;
  for (int j = 1; j <= gamma; ++j) {
    const long pr = (long)b * G1 + (j - 1);
    const long qr = (long)(j - 1) * B + b;
    const RowView pv = row_view(row_chunks(p_stats, pr, nch), nch, T);
    const RowView qv = row_view(row_chunks(q_stats, qr, nch), nch, T);
    const int d = drafts[j - 1];
    const double pd = prob(p_logits + pr * V, d, row_thr(p_stats, pr, nch), T, topp, pv);
    const double qd = prob(q_logits + qr * V, d, row_thr(q_stats, qr, nch), T, topp, qv);
    const double u = philox_uniform(seed, sid, n + j, (uint32_t)j, PURPOSE_ACCEPT);
    if (!(u * qd <= pd)) { a = j - 1; break; }
  }
  if (threadIdx.x == 0) {
    for (int i = 0; i < a; ++i) out_tok[(long)b * G1 + i] = drafts[i];
    n_acc[b] = a;
  }
}

struct ResidW {
  const float* zp;
  const float* zq;
  RowStats tp, tq;
  RowView pv, qv;
  float T;
  bool topp;
  // token i's residual weight from its two logits (a from p, b from q)
  ER_DEV double from(float a, float b, int i) const {
    double p, q;
    if (T == 0.0f) {
      p = i == pv.arg ? 1.0 : 0.0;
      q = i == qv.arg ? 1.0 : 0.0;
    } else {
      p = w_rel(a, i, (double)pv.M, T, tp, topp) / pv.S;
      q = w_rel(b, i, (double)qv.M, T, tq, topp) / qv.S;
    }
    return p > q ? p - q : 0.0;
  }
  struct Val {
    float p, q;
  };
  static constexpr bool kPreload = false;
  ER_DEV Val load(int i) const { return Val{zp[i], zq[i]}; }
  ER_DEV double weight(Val v, int i, double) const { return from(v.p, v.q, i); }
};

__global__ __launch_bounds__(SB) void k_resid_chunks(const float* __restrict__ p_logits, const void* __restrict__ p_stats,
                                                     const float* __restrict__ q_logits, const void* __restrict__ q_stats,
                                                     const int32_t* __restrict__ n_acc, int B, int gamma, int V, float T,
                                                     int topp, double* __restrict__ resid, int nch) {
  const int b = blockIdx.x;
  const int c = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (c >= nch) return;
  const int a = n_acc[b];
  if (a >= gamma) return;  // full acceptance: the bonus draw uses p_{gamma+1}'s own chunks
  const int j = a + 1;
  const int G1 = gamma + 1;
  const long pr = (long)b * G1 + (j - 1);
  const long qr = (long)(j - 1) * B + b;
  ResidW rw{p_logits + pr * V, q_logits + qr * V, row_thr(p_stats, pr, nch), row_thr(q_stats, qr, nch),
            row_view(row_chunks(p_stats, pr, nch), nch, T), row_view(row_chunks(q_stats, qr, nch), nch, T), T,
            topp != 0};
  double s = 0.0;
  const int base = c * SCH;
  // both rows' chunk values loaded once, unpredicated (indices clamped into
  // the row, lanes past V masked by value), then the same sums as the draw
  float ap[SCH / 64], aq[SCH / 64];
#pragma unroll
  for (int t = 0; t < SCH / 64; ++t) {
    const int ic = min(base + t * 64 + lane, V - 1);
    ap[t] = rw.zp[ic];
    aq[t] = rw.zq[ic];
  }
#pragma unroll
  for (int t = 0; t < SCH / 64; ++t) {
    const int i = base + t * 64 + lane;
    s += wave_sum_d(i < V ? rw.from(ap[t], aq[t], i) : 0.0);
  }
  if (lane == 0) resid[(long)b * nch + c] = s;
}

struct ResidChunks {
  const double* s;
  ER_DEV double sum(int c) const { return s[c]; }
  ER_DEV double f(int) const { return 1.0; }
  ER_DEV double ref(int) const { return 0.0; }
  ER_DEV int find(int nch, double target, double* pre) const { return find_chunk_mem(*this, nch, target, pre); }
};

__global__ __launch_bounds__(64) void k_decide_draw(const float* __restrict__ p_logits, const void* __restrict__ p_stats,
                                                   const float* __restrict__ q_logits, const void* __restrict__ q_stats,
                                                   const int32_t* __restrict__ n_acc, int B, int gamma, int V, float T,
                                                   int topp, uint64_t seed, const int32_t* __restrict__ seq_id,
                                                   const int32_t* __restrict__ pos0, const double* __restrict__ resid,
                                                   int32_t* __restrict__ out_tok, int nch) {
  const int b = blockIdx.x;
  const int G1 = gamma + 1;
  const uint32_t sid = (uint32_t)seq_id[b];
  const uint32_t n = (uint32_t)pos0[b];
  const int a = n_acc[b];
  const int j = a + 1;  // position index of the draw (gamma+1 = bonus)
  const double u = philox_uniform(seed, sid, n + j, (uint32_t)j, PURPOSE_RESIDUAL);
  const long pr = (long)b * G1 + (j - 1);
  const ChunkStat* pc = row_chunks(p_stats, pr, nch);
  const RowView pv = row_view(pc, nch, T);
  const RowW pw{p_logits + pr * V, row_thr(p_stats, pr, nch), T, topp != 0};
  int t;
  if (a < gamma) {
    const long qr = (long)(j - 1) * B + b;
    const double* rs = resid + (long)b * nch;
    double tot = 0.0;
    for (int c = 0; c < nch; ++c) tot += rs[c];
    if (tot > 0.0) {
      ResidW rw{p_logits + pr * V, q_logits + qr * V, row_thr(p_stats, pr, nch), row_thr(q_stats, qr, nch), pv,
                row_view(row_chunks(q_stats, qr, nch), nch, T), T, topp != 0};
      t = wave_draw(rw, ResidChunks{rs}, nch, V, u, tot);
    } else {  // residual without mass: fall back to p
      t = T == 0.0f ? pv.arg : wave_draw(pw, ChunkView{pc, pv.M, T}, nch, V, u, pv.S);
    }
  } else {
    t = T == 0.0f ? pv.arg : wave_draw(pw, ChunkView{pc, pv.M, T}, nch, V, u, pv.S);
  }
  if (threadIdx.x == 0) out_tok[(long)b * G1 + a] = t;
}

int launch_spec_decide(const float* p_logits, const void* p_stats, const float* q_logits, const void* q_stats,
                       const int32_t* tokens, int B, int gamma, int V, float T, float top_p, uint64_t seed,
                       const int32_t* seq_id, const int32_t* pos0, int32_t* out_tok, int32_t* n_acc, double* resid,
                       hipStream_t st) {
  if (B <= 0) return 0;
  const int nch = sampler_chunks(V);
  const int topp = (T != 0.0f && top_p < 1.0f) ? 1 : 0;
  hipLaunchKernelGGL(k_decide_accept, dim3(B), dim3(64), 0, st, p_logits, p_stats, q_logits, q_stats, tokens, B,
                     gamma, V, T, topp, seed, seq_id, pos0, out_tok, n_acc, nch);
  if (gamma > 0)
    hipLaunchKernelGGL(k_resid_chunks, dim3(B, (nch + 3) / 4), dim3(SB), 0, st, p_logits, p_stats, q_logits, q_stats,
                       n_acc, B, gamma, V, T, topp, resid, nch);
  hipLaunchKernelGGL(k_decide_draw, dim3(B), dim3(64), 0, st, p_logits, p_stats, q_logits, q_stats, n_acc, B, gamma, V,
                     T, topp, seed, seq_id, pos0, resid, out_tok, nch);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace er
