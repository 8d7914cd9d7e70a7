// Paged grouped-query attention for decode (1 query per sequence), verify
// (gamma+1 causal queries per sequence) and prefill chunks.
//
// The verify pass scores every drafted position in one forward (TLT reading
// notes, section 1: the target checks d1..dk in one pass; a failed position
// invalidates everything after it, which the sampler handles).  The drafter
// reads the same KV pool: target-written entries for committed positions and
// its own provisional entries for draft positions (EfficientRollout "关键模块"
// item 1: the drafter shares the target's KV cache).
//
// One work-group = (item, kv head, KV split).  All grp = hq/hkv query heads of
// the KV head and all query positions of the item are handled together, so a
// K/V block is read from HBM once per (item, kv head) and reused from LDS by
// every query row.  Softmax is the online (running max / running sum) form;
// long contexts are split over work-groups and merged by k_attn_combine in a
// fixed order (deterministic).

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace er {

constexpr int ATT_MAXQ = 64 * 128;  // floats of the query tile in LDS (rows * hd)

template <bool BF>
__global__ __launch_bounds__(256) void k_attn(AttnArgs a, int nsplit, int bps) {
  const int item = blockIdx.x;
  const int g = blockIdx.y;
  const int sp = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hd = a.hd, grp = a.hq / a.hkv;
  const int qc = a.item_q_count[item];
  const int pos0 = a.item_q_pos0[item];
  const int qrow0 = a.item_q_row0[item];
  const int R = grp * qc;
  const int nkeys = pos0 + qc;                 // keys 0..pos0+qc-1
  const int nblk = (nkeys + 15) >> 4;
  const int b0 = sp * bps;
  const int b1 = min(nblk, b0 + bps);
  const float scale = 1.0f / sqrtf((float)hd);

  __shared__ float qs[ATT_MAXQ];
  __shared__ float ks[16 * 128];
  __shared__ float vs[16 * 128];

  typedef typename Act<BF>::T T;
  const T* q = (const T*)a.q;
  for (int idx = tid; idx < R * hd; idx += 256) {
    const int r = idx / hd, e = idx - r * hd;
    const int qi = r / grp, hh = g * grp + (r - qi * grp);
    qs[idx] = Act<BF>::ld(q, ((long)(qrow0 + qi) * a.hq + hh) * hd + e) * scale;
  }

  // per-row running state, rows r = wave + 4 * j
  constexpr int RMAX = 16;
  float mrun[RMAX], lrun[RMAX], acc0[RMAX], acc1[RMAX];
#pragma unroll
  for (int j = 0; j < RMAX; ++j) { mrun[j] = -INFINITY; lrun[j] = 0.f; acc0[j] = 0.f; acc1[j] = 0.f; }

  const int t = lane & 15, sl = lane >> 4;
  const int slw = hd >> 2;  // elements per slice
  const T* pool = (const T*)a.kv_pool;
  const int* bt = a.block_table + (long)a.item_bt_row[item] * a.bt_stride;

  for (int blk = b0; blk < b1; ++blk) {
    __syncthreads();
    const long phys = bt[blk];
    const long kb = ((((phys * a.n_layers + a.layer) * 2 + 0) * a.hkv + g) * 16) * hd;
    const long vb = ((((phys * a.n_layers + a.layer) * 2 + 1) * a.hkv + g) * 16) * hd;
    for (int idx = tid; idx < 16 * hd; idx += 256) {
      ks[idx] = Act<BF>::ld(pool, kb + idx);
      vs[idx] = Act<BF>::ld(pool, vb + idx);
    }
    __syncthreads();
    const int kpos = blk * 16 + t;
#pragma unroll
    for (int j = 0; j < RMAX; ++j) {
      const int r = wave + 4 * j;
      if (r >= R) break;
      const int qi = r / grp;
      const int qpos = pos0 + qi;
      float s = 0.f;
      const float* qr = qs + r * hd + sl * slw;
      const float* kr = ks + t * hd + sl * slw;
      for (int e = 0; e < slw; ++e) s = fmaf(qr[e], kr[e], s);
      s += __shfl_xor(s, 16, 64);
      s += __shfl_xor(s, 32, 64);
      if (kpos > qpos) s = -INFINITY;
      float mb = s;
      mb = fmaxf(mb, __shfl_xor(mb, 1, 64));
      mb = fmaxf(mb, __shfl_xor(mb, 2, 64));
      mb = fmaxf(mb, __shfl_xor(mb, 4, 64));
      mb = fmaxf(mb, __shfl_xor(mb, 8, 64));
      const float mnew = fmaxf(mrun[j], mb);
      if (mnew == -INFINITY) continue;  // whole block masked for this row (and nothing before)
      const float corr = expf(mrun[j] - mnew);
      const float p = (s == -INFINITY) ? 0.f : expf(s - mnew);
      float ps = p;
      ps += __shfl_xor(ps, 1, 64);
      ps += __shfl_xor(ps, 2, 64);
      ps += __shfl_xor(ps, 4, 64);
      ps += __shfl_xor(ps, 8, 64);
      lrun[j] = lrun[j] * corr + ps;
      float a0 = acc0[j] * corr, a1 = acc1[j] * corr;
      for (int tt = 0; tt < 16; ++tt) {
        const float pt = __shfl(p, tt, 64);
        a0 = fmaf(pt, vs[tt * hd + lane], a0);
        if (hd > 64) a1 = fmaf(pt, vs[tt * hd + 64 + lane], a1);
      }
      acc0[j] = a0;
      acc1[j] = a1;
      mrun[j] = mnew;
    }
  }

  // write out
  T* out = (T*)a.out;
#pragma unroll
  for (int j = 0; j < RMAX; ++j) {
    const int r = wave + 4 * j;
    if (r >= R) break;
    const int qi = r / grp, hh = g * grp + (r - qi * grp);
    if (nsplit == 1) {
      const float inv = lrun[j] > 0.f ? 1.0f / lrun[j] : 0.f;
      const long o = ((long)(qrow0 + qi) * a.hq + hh) * hd;
      if (lane < hd) Act<BF>::st(out, o + lane, acc0[j] * inv);
      if (hd > 64) Act<BF>::st(out, o + 64 + lane, acc1[j] * inv);
    } else {
      // partial: [item][g][sp][r][hd + 2]
      float* pp = a.ws + ((((long)item * a.hkv + g) * nsplit + sp) * (long)(grp * a.max_q_count) + r) * (hd + 2);
      if (lane < hd) pp[lane] = acc0[j];
      if (hd > 64) pp[64 + lane] = acc1[j];
      if (lane == 0) { pp[hd] = mrun[j]; pp[hd + 1] = lrun[j]; }
    }
  }
}

template <bool BF>
__global__ __launch_bounds__(128) void k_attn_combine(AttnArgs a, int nsplit) {
  const int item = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const int grp = a.hq / a.hkv, hd = a.hd;
  const int qc = a.item_q_count[item];
  if (r >= grp * qc) return;
  const long stride_sp = (long)(grp * a.max_q_count) * (hd + 2);
  const float* base = a.ws + ((((long)item * a.hkv + g) * nsplit) * (long)(grp * a.max_q_count) + r) * (hd + 2);
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, base[s * stride_sp + hd]);
  const int e = threadIdx.x;
  if (e >= hd) return;
  float num = 0.f, den = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < nsplit; ++s) {
      const float ms = base[s * stride_sp + hd];
      if (ms == -INFINITY) continue;
      const float w = expf(ms - M);
      num = fmaf(w, base[s * stride_sp + e], num);
      den = fmaf(w, base[s * stride_sp + hd + 1], den);
    }
  }
  const int qi = r / grp, hh = g * grp + (r - qi * grp);
  const long o = ((long)(a.item_q_row0[item] + qi) * a.hq + hh) * hd + e;
  typedef typename Act<BF>::T T;
  Act<BF>::st((T*)a.out, o, den > 0.f ? num / den : 0.f);
}

int launch_attention(const AttnArgs& a, hipStream_t st) {
  if (a.n_items <= 0) return 0;
  const int grp = a.hq / a.hkv;
  if ((a.hd != 64 && a.hd != 128) || a.hq % a.hkv != 0) return -1;
  if (grp * a.max_q_count > 64 || grp * a.max_q_count * a.hd > ATT_MAXQ) return -1;
  const int maxblk = (a.max_ctx + 15) / 16;
  long base = (long)a.n_items * a.hkv;
  int nsplit = (int)std::max(1L, std::min((long)(maxblk + 3) / 4, (512 + base - 1) / base));
  const int bps = (maxblk + nsplit - 1) / nsplit;
  nsplit = (maxblk + bps - 1) / bps;
  if (nsplit > 1) {
    const size_t need = (size_t)a.n_items * a.hkv * nsplit * grp * a.max_q_count * (a.hd + 2);
    if (need > a.ws_floats) return -2;
  }
  dim3 grid(a.n_items, a.hkv, nsplit);
  if (a.bf16) hipLaunchKernelGGL(k_attn<true>, grid, dim3(256), 0, st, a, nsplit, bps);
  else hipLaunchKernelGGL(k_attn<false>, grid, dim3(256), 0, st, a, nsplit, bps);
  if (hipGetLastError() != hipSuccess) return -3;
  if (nsplit > 1) {
    dim3 g2(a.n_items, a.hkv, grp * a.max_q_count);
    if (a.bf16) hipLaunchKernelGGL(k_attn_combine<true>, g2, dim3(128), 0, st, a, nsplit);
    else hipLaunchKernelGGL(k_attn_combine<false>, g2, dim3(128), 0, st, a, nsplit);
    if (hipGetLastError() != hipSuccess) return -3;
  }
  return 0;
}

}  // namespace er
