// Fused sampler of the speculative step: softmax / temperature / top-p
// statistics per logits row, categorical draws by inverse CDF in vocabulary
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
// All probability arithmetic is fp64 (exp of (z - zmax)/T formed from the
// fp32 logits in fp64), prefix sums are wavefront scans in a fixed order, and
// every draw takes its uniform from Philox4x32-10 keyed by (seed) with counter
// (sequence, position, draft index, purpose), so a step is a deterministic
// function of its logits.

#include "common.h"
#include "kernels.h"

namespace er {

constexpr int SB = 256;  // threads per sampler block (4 waves)

// Un-normalised weight of token i in row r: exp((z - zmax)/T) if kept by
// top-p, else 0; greedy (T == 0) rows are one-hot at the argmax.
ER_DEV double tok_weight(const float* __restrict__ z, int i, const RowStats& s, float T) {
  if (T == 0.0f) return i == s.argmax ? 1.0 : 0.0;
  const float zi = z[i];
  const uint32_t k = float_key(zi);
  if (k < s.thr_key || (k == s.thr_key && i > s.thr_idx)) return 0.0;
  return exp(((double)zi - (double)s.zmax) / (double)T);
}

// Block-wide fixed-order sum of one double per thread.
ER_DEV double block_sum_d(double v, double* red) {
  v = wave_sum_d(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(SB) void k_row_stats(const float* __restrict__ logits, int V, long ld, float T,
                                                  float top_p, RowStats* __restrict__ stats) {
  const int r = blockIdx.x;
  const float* z = logits + (long)r * ld;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ double red[4];
  __shared__ float redm[4];
  __shared__ int redi[4];
  __shared__ double hist[256];
  __shared__ uint32_t s_prefix;
  __shared__ double s_above;
  __shared__ int s_cnt[SB];

  // argmax (lowest index among equal maxima)
  float bm = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int i = tid; i < V; i += SB) {
    const float v = z[i];
    if (v > bm) { bm = v; bi = i; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(bm, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (om > bm || (om == bm && oi < bi)) { bm = om; bi = oi; }
  }
  if (lane == 0) { redm[wave] = bm; redi[wave] = bi; }
  __syncthreads();
  float zmax = redm[0];
  int amax = redi[0];
  for (int w = 1; w < 4; ++w)
    if (redm[w] > zmax || (redm[w] == zmax && redi[w] < amax)) { zmax = redm[w]; amax = redi[w]; }

  RowStats s;
  s.zmax = zmax;
  s.argmax = amax;
  if (T == 0.0f) {
    s.total = 1.0;
    s.kept = 1.0;
    s.thr_key = 0;
    s.thr_idx = 0x7FFFFFFF;
    if (tid == 0) stats[r] = s;
    return;
  }
  double tot = 0.0;
  for (int i = tid; i < V; i += SB) tot += exp(((double)z[i] - (double)zmax) / (double)T);
  tot = block_sum_d(tot, red);
  s.total = tot;
  s.kept = tot;
  s.thr_key = 0;
  s.thr_idx = 0x7FFFFFFF;
  if (top_p < 1.0f) {
    // Nucleus threshold: the kept set is the longest-probability prefix (ties
    // by index) whose mass first reaches top_p * total.  Radix select over
    // the order-preserving key of the logit, 8 bits per pass, masses in fp64.
    const double target = (double)top_p * tot;
    uint32_t prefix = 0, mask = 0;
    double above = 0.0;
    for (int d = 3; d >= 0; --d) {
      for (int b = tid; b < 256; b += SB) hist[b] = 0.0;
      __syncthreads();
      for (int i = tid; i < V; i += SB) {
        const uint32_t k = float_key(z[i]);
        if ((k & mask) == prefix) {
          const double w = exp(((double)z[i] - (double)zmax) / (double)T);
          atomicAdd(&hist[(k >> (8 * d)) & 255u], w);
        }
      }
      __syncthreads();
      if (tid == 0) {
        // highest bin whose cumulative mass reaches the target; if rounding
        // leaves none, the lowest non-empty bin (so the bin always holds tokens)
        double cum = above, cum_last = above;
        int chosen = -1, last_nz = -1;
        for (int b = 255; b >= 0; --b) {
          if (hist[b] > 0.0) {
            if (cum + hist[b] >= target) { chosen = b; break; }
            last_nz = b;
            cum_last = cum;
          }
          cum += hist[b];
        }
        if (chosen < 0) { chosen = last_nz; cum = cum_last; }
        s_prefix = prefix | ((uint32_t)chosen << (8 * d));
        s_above = cum;
      }
      __syncthreads();
      prefix = s_prefix;
      above = s_above;
      mask |= 255u << (8 * d);
    }
    // Tokens with key == prefix all carry the same weight; keep the first c in
    // index order, c the smallest count that reaches the target.
    int tie_i = -1;
    for (int i = tid; i < V && tie_i < 0; i += SB)
      if (float_key(z[i]) == prefix) tie_i = i;
    // weight of a tied token
    __shared__ int s_anyi;
    if (tid == 0) s_anyi = 0x7FFFFFFF;
    __syncthreads();
    if (tie_i >= 0) atomicMin(&s_anyi, tie_i);
    __syncthreads();
    if (s_anyi == 0x7FFFFFFF) {  // cannot happen (the chosen bin always holds mass); keep everything
      if (tid == 0) { s.thr_key = 0; s.thr_idx = 0x7FFFFFFF; s.kept = tot; stats[r] = s; }
      return;
    }
    const double wt = exp(((double)z[s_anyi] - (double)zmax) / (double)T);
    double need = (target - above) / wt;
    int c = (int)ceil(need);
    if (c < 1) c = 1;
    // c-th smallest tied index: contiguous chunks keep index order
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
      s_anyi = c;  // reuse as the target count
    }
    __syncthreads();
    c = s_anyi;
    int idx = -1;
    {
      int run = s_cnt[tid];
      if (run < c) {
        for (int i = lo; i < hi; ++i) {
          if (float_key(z[i]) == prefix) {
            ++run;
            if (run == c) { idx = i; break; }
          }
        }
      }
    }
    __syncthreads();
    if (idx >= 0) s_anyi = idx;
    __syncthreads();
    s.thr_key = prefix;
    s.thr_idx = s_anyi;
    s.kept = above + (double)c * wt;
  }
  if (tid == 0) stats[r] = s;
}

int launch_row_stats(const float* logits, int rows, int V, long ld, float T, float top_p, RowStats* stats,
                     hipStream_t st) {
  if (rows <= 0) return 0;
  hipLaunchKernelGGL(k_row_stats, dim3(rows), dim3(SB), 0, st, logits, V, ld, T, top_p, stats);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Inverse-CDF draw over a weight function in vocabulary order: the smallest i
// with sum_{k<=i} w_k >= u * sum_k w_k.  Wave w scans the contiguous range
// [w*span, (w+1)*span) in 64-wide tiles; the first pass forms the wave totals,
// the wave holding the crossing rescans with the same additions in the same
// order and finds the lane by an inclusive shuffle scan.
template <class WF>
ER_DEV int draw_inverse_cdf(const WF& wf, int V, double u, double* red, int* s_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int span = ((V + 4 * 64 - 1) / (4 * 64)) * 64;
  const int lo = wave * span, hi = min(V, lo + span);
  double run = 0.0;
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    const double w = (i < hi) ? wf(i) : 0.0;
    run += wave_sum_d(w);
  }
  __syncthreads();
  if (lane == 0) red[wave] = run;
  if (tid == 0) *s_out = -1;
  __syncthreads();
  const double tot = red[0] + red[1] + red[2] + red[3];
  const double target = u * tot;
  // wave holding the crossing; if rounding leaves none, the last wave with mass
  double pre = 0.0, pre_last = 0.0;
  int cw = -1, last_w = 0;
  for (int w = 0; w < 4; ++w) {
    if (red[w] > 0.0) {
      if (pre + red[w] >= target) { cw = w; break; }
      last_w = w;
      pre_last = pre;
    }
    pre += red[w];
  }
  if (cw < 0) { cw = last_w; pre = pre_last; }
  if (wave == cw) {
    double r = pre;
    int found = -1;
    int last_nz = -1;
    for (int base = lo; base < hi && found < 0; base += 64) {
      const int i = base + lane;
      const double w = (i < hi) ? wf(i) : 0.0;
      const double ts = wave_sum_d(w);
      if (w > 0.0) last_nz = i;
      if (r + ts >= target) {
        double sc = w;  // inclusive scan
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const double t = __shfl_up(sc, o, 64);
          if (lane >= o) sc += t;
        }
        const bool hit = (r + sc >= target) && (w > 0.0);
        const unsigned long long m = __ballot(hit);
        if (m) found = base + __ffsll(m) - 1;
      }
      r += ts;
    }
    // reduce last non-zero over the wave (fallback when rounding leaves no hit)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) last_nz = max(last_nz, __shfl_xor(last_nz, o, 64));
    if (lane == 0) *s_out = found >= 0 ? found : last_nz;
  }
  __syncthreads();
  int res = *s_out;
  if (res < 0) res = 0;
  return res;
}

struct RowWeight {
  const float* z;
  RowStats s;
  float T;
  ER_DEV double operator()(int i) const { return tok_weight(z, i, s, T); }
};

__global__ __launch_bounds__(SB) void k_sample_rows(const float* __restrict__ logits, const RowStats* __restrict__ stats,
                                                    int V, long ld, float T, uint64_t seed,
                                                    const int32_t* __restrict__ seq_id, const int32_t* __restrict__ pos,
                                                    int didx, int purpose, int32_t* __restrict__ out, int out_stride,
                                                    const int32_t* __restrict__ row_map) {
  const int r = blockIdx.x;
  const long lr = row_map ? row_map[r] : r;
  __shared__ double red[4];
  __shared__ int s_out;
  RowWeight wf{logits + lr * ld, stats[lr], T};
  if (T == 0.0f) {
    if (threadIdx.x == 0) out[(long)r * out_stride] = wf.s.argmax;
    return;
  }
  const double u = philox_uniform(seed, (uint32_t)seq_id[r], (uint32_t)pos[r], (uint32_t)didx, (uint32_t)purpose);
  const int t = draw_inverse_cdf(wf, V, u, red, &s_out);
  if (threadIdx.x == 0) out[(long)r * out_stride] = t;
}

int launch_sample_rows(const float* logits, const RowStats* stats, int rows, int V, long ld, float T, uint64_t seed,
                       const int32_t* seq_id, const int32_t* pos, int didx, int purpose, int32_t* out, int out_stride,
                       const int32_t* row_map, hipStream_t st) {
  if (rows <= 0) return 0;
  hipLaunchKernelGGL(k_sample_rows, dim3(rows), dim3(SB), 0, st, logits, stats, V, ld, T, seed, seq_id, pos, didx,
                     purpose, out, out_stride, row_map);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

struct ResidualWeight {
  const float* zp;
  const float* zq;
  RowStats sp, sq;
  float T;
  ER_DEV double operator()(int i) const {
    const double p = tok_weight(zp, i, sp, T) / sp.kept;
    const double q = tok_weight(zq, i, sq, T) / sq.kept;
    return p > q ? p - q : 0.0;
  }
};

__global__ __launch_bounds__(SB) void k_spec_decide(const float* __restrict__ p_logits, const RowStats* __restrict__ p_stats,
                                                    const float* __restrict__ q_logits, const RowStats* __restrict__ q_stats,
                                                    const int32_t* __restrict__ tokens, int gamma, int V, float T,
                                                    uint64_t seed, const int32_t* __restrict__ seq_id,
                                                    const int32_t* __restrict__ pos0, int32_t* __restrict__ out_tok,
                                                    int32_t* __restrict__ n_acc) {
  const int b = blockIdx.x;
  const int G1 = gamma + 1;
  __shared__ double red[4];
  __shared__ int s_out;
  const uint32_t sid = (uint32_t)seq_id[b];
  const uint32_t n = (uint32_t)pos0[b];
  const int32_t* drafts = tokens + (long)b * G1 + 1;
  for (int j = 1; j <= gamma; ++j) {
    const long prow = (long)b * G1 + (j - 1);
    const long qrow = (long)(j - 1) * gridDim.x + b;  // drafter rows are [gamma][B]
    const float* zp = p_logits + prow * V;
    const float* zq = q_logits + qrow * V;
    const RowStats sp = p_stats[prow], sq = q_stats[qrow];
    const int d = drafts[j - 1];
    const double pd = tok_weight(zp, d, sp, T) / sp.kept;
    const double qd = tok_weight(zq, d, sq, T) / sq.kept;
    const double u = philox_uniform(seed, sid, n + j, (uint32_t)j, PURPOSE_ACCEPT);
    if (!(u * qd <= pd)) {
      const double u2 = philox_uniform(seed, sid, n + j, (uint32_t)j, PURPOSE_RESIDUAL);
      ResidualWeight rw{zp, zq, sp, sq, T};
      // zero residual mass (p == q on every token) falls back to p
      double part = 0.0;
      for (int i = threadIdx.x; i < V; i += SB) part += rw(i);
      __shared__ double red2[4];
      const double rs = block_sum_d(part, red2);
      int t;
      if (rs > 0.0) t = draw_inverse_cdf(rw, V, u2, red, &s_out);
      else t = draw_inverse_cdf(RowWeight{zp, sp, T}, V, u2, red, &s_out);
      if (threadIdx.x == 0) {
        for (int i = 0; i < j - 1; ++i) out_tok[(long)b * G1 + i] = drafts[i];
        out_tok[(long)b * G1 + j - 1] = t;
        n_acc[b] = j - 1;
      }
      return;
    }
  }
  const long prow = (long)b * G1 + gamma;
  const double u = philox_uniform(seed, sid, n + gamma + 1, (uint32_t)(gamma + 1), PURPOSE_RESIDUAL);
  const int t = draw_inverse_cdf(RowWeight{p_logits + prow * V, p_stats[prow], T}, V, u, red, &s_out);
  if (threadIdx.x == 0) {
    for (int i = 0; i < gamma; ++i) out_tok[(long)b * G1 + i] = drafts[i];
    out_tok[(long)b * G1 + gamma] = t;
    n_acc[b] = gamma;
  }
}

int launch_spec_decide(const float* p_logits, const RowStats* p_stats, const float* q_logits, const RowStats* q_stats,
                       const int32_t* tokens, int B, int gamma, int V, float T, uint64_t seed, const int32_t* seq_id,
                       const int32_t* pos0, int32_t* out_tok, int32_t* n_acc, hipStream_t st) {
  if (B <= 0) return 0;
  hipLaunchKernelGGL(k_spec_decide, dim3(B), dim3(SB), 0, st, p_logits, p_stats, q_logits, q_stats, tokens, gamma, V,
                     T, seed, seq_id, pos0, out_tok, n_acc);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace er
