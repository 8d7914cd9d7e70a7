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
// KV block layout (16 positions): K as [16][hd], V transposed as [hd][16], so
// that both MFMA operands load as contiguous 16/8-byte pieces.
//
// bf16 path (k_attn_mfma): one work-group = (item, kv head, KV split); the
// grp = hq/hkv query heads of the KV head times the item's query positions
// form up to 64 "rows", 16 per wave.  Scores are computed transposed,
// S^T[token][row] = K . Q^T with v_mfma_f32_16x16x32_bf16, which leaves each
// lane holding 4 consecutive tokens of one row: exactly the A operand of the
// P.V product (v_mfma_f32_16x16x16_bf16 with V^T as B).  Softmax is the online
// (running max / running sum) form in fp32; the P operand is rounded to bf16.
// When the rows fill fewer than 4 waves, the spare waves take interleaved KV
// blocks and the partial results merge in LDS; long contexts also split over
// work-groups and merge in k_attn_combine.  All merges run in a fixed order.
//
// fp32 path (k_attn_valu): a plain per-row online softmax, one wavefront per
// row, for the fp32 model (small shapes only).

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace er {

typedef short __attribute__((ext_vector_type(4))) bf16x4s_t;
typedef __bf16 __attribute__((ext_vector_type(2))) bf16x2_t;

// Most KV blocks one work unit covers (its block ids are staged in LDS).
constexpr int kAttnMaxUnitBlocks = 1024;

ER_DEV long kv_block_base(long phys, int layer, int L, int kv, int hkv, int head, int hd) {
  return ((((phys * L + layer) * 2 + kv) * hkv + head) * 16) * (long)hd;
}

// Split partial record of one row of work unit u: [hd] unnormalised output,
// then running max, then running sum.
ER_DEV float* partial_row(const AttnArgs& a, long u, int g, int r) {
  const int grp = a.hq / a.hkv;
  return a.ws + (((long)u * a.hkv + g) * (long)(grp * a.max_q_count) + r) * (a.hd + 2);
}

// Work unit u: its item, its index among the item's units, how many units the
// item has, and its first block.  With a unit table, item i owns units
// unit_start[i] .. of unit_start[n_items + 1 + i] blocks each; otherwise every item
// has nsplit units of bps blocks (unit = item * nsplit + split).
struct Unit {
  int item, sp, nu, b0, bps;
};
ER_DEV Unit unit_of(const AttnArgs& a, int u, int nsplit, int bps) {
  Unit w;
  if (a.unit_start) {
    int lo = 0, hi = a.n_items;  // largest i with unit_start[i] <= u
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.unit_start[mid] <= u) lo = mid; else hi = mid;
    }
    w.item = lo;
    w.sp = u - a.unit_start[lo];
    w.nu = a.unit_start[lo + 1] - a.unit_start[lo];
    w.bps = a.unit_start[a.n_items + 1 + lo];
  } else {
    w.item = u / nsplit;
    w.sp = u - w.item * nsplit;
    w.nu = nsplit;
    w.bps = bps;
  }
  w.b0 = w.sp * w.bps;
  return w;
}

// D: stages of the K/V register ring (block t + D - 1 is loaded while block
// t is scored).  D = 2 fits 168 registers, three waves per SIMD (three
// work-groups per CU); D = 1 fits 128, four (LDS allows four work-groups per
// CU).  The three-stage ring needed ~221, two work-groups per CU.
template <int HD, int NW, int D>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(D == 2 ? 3 : 4)))
void k_attn_mfma(AttnArgs a, int nsplit, int bps) {
  constexpr int NC = HD / 16;   // 16-column output tiles
  constexpr int NQ = HD / 32;   // 32-wide k slices of the score MFMA
  const int u = blockIdx.x, g = blockIdx.y;
  if (a.unit_start && u >= a.n_units) return;
  // The unit's item, split and query/block-table fields: one uniform 32-byte
  // load of its record when the host wrote records, else a search of the
  // unit table and loads from the item arrays (a chain of dependent loads).
  Unit w;
  int qc, pos0, qrow0, btrow;
  if (a.unit_rec) {
    const int4* rp = reinterpret_cast<const int4*>(a.unit_rec) + 2 * (long)u;
    const int4 r0 = rp[0], r1 = rp[1];
    w.item = r0.x;
    w.sp = r0.y & 0xFFFF;
    w.nu = r0.y >> 16;
    w.b0 = r0.z;
    w.bps = r0.w;
    qc = r1.x;
    pos0 = r1.y;
    qrow0 = r1.z;
    btrow = r1.w;
  } else {
    w = unit_of(a, u, nsplit, bps);
    qc = a.item_q_count[w.item];
    pos0 = a.item_q_pos0[w.item];
    qrow0 = a.item_q_row0[w.item];
    btrow = a.item_bt_row[w.item];
  }
  // the wave index through readfirstlane, so that everything derived from it
  // (this wave's block list, its block-id loads) is known to be wave-uniform
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, kb = lane >> 4;
  const int grp = a.hq / a.hkv;
  const int R = grp * qc;
  const int rgroups = (R + 15) >> 4;
  const int rgn = rgroups == 1 ? 1 : (rgroups == 2 ? 2 : 4);
  const int s_in = NW / rgn;                 // waves sharing one row group
  const int rgi = wave / s_in, sin = wave % s_in;
  const int nblk = (pos0 + qc + 15) >> 4;
  const int b0 = w.b0;
  const int b1 = min(min(nblk, b0 + w.bps), b0 + kAttnMaxUnitBlocks);
  // scores in the log2 domain: s * log2(e) / sqrt(hd), so that every
  // exponential is one v_exp_f32 (exp2); the running maxima, the partial
  // records and the merges all use that domain
  const float scale = 1.4426950408889634f / sqrtf((float)HD);

  constexpr int OS = HD + 4;   // padded row stride of the merge area (rows 4 apart hit other banks)
  __shared__ float o_sh[NW][16 * OS];
  __shared__ float ml_sh[NW][2][16];

  // this lane's query row (as the MFMA column n = l16)
  const int r_q = rgi * 16 + l16;
  const bool q_ok = rgi < rgroups && r_q < R;
  const int qi_q = q_ok ? r_q / grp : 0;
  const int hh_q = g * grp + (q_ok ? r_q % grp : 0);
  const int qpos_q = pos0 + qi_q;

  // Q^T fragments (B operand): k = 8*kb .. +8 of slice i
  bf16x8_t qf[NQ];
  {
    const uint16_t* qp = (const uint16_t*)a.q + ((long)(qrow0 + qi_q) * a.hq + hh_q) * HD;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const uint4 v = q_ok ? *(const uint4*)(qp + 32 * i + 8 * kb) : uint4{0u, 0u, 0u, 0u};
      qf[i] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  f32x4_t o[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) o[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const uint16_t* pool = (const uint16_t*)a.kv_pool;
  const int32_t* bt = a.block_table + (long)btrow * a.bt_stride;

  // the unit's block ids, staged once (the launcher keeps a unit at most
  // kAttnMaxUnitBlocks blocks long)
  __shared__ int ids_sh[kAttnMaxUnitBlocks];
  for (int j = tid; j < b1 - b0; j += NW * 64) ids_sh[j] = bt[b0 + j];
  __syncthreads();

  if (rgi < rgroups) {
    // This wave's blocks are first + s_in * t, t < nb.  Their K and V
    // fragments go through a ring of D register stages (loads of blocks t+1
    // and t+2 are in flight while block t is scored).  The block ids come
    // from LDS one iteration ahead: LDS reads are counted apart from the
    // vector-memory loads, so reading an id never waits on K/V loads in
    // flight (an id from a global or scalar load issued in the loop either
    // stalls on that load's latency or makes the compiler drain the ring).
    // Every load is unconditional (indices clamped to the last block):
    // conditional loads would make the compiler drain the whole load counter
    // at each use.
    const int first = b0 + sin;
    const int nb = first < b1 ? (b1 - first + s_in - 1) / s_in : 0;
    const int tl = nb > 0 ? nb - 1 : 0;
    uint4 kq[D][NQ];
    uint2 vq[D][NC];
    auto bid = [&](int t) -> long {
      return (long)__builtin_amdgcn_readfirstlane(ids_sh[sin + s_in * min(t, tl)]);
    };
    auto fetch = [&](int slot, long phys) {
      const uint16_t* kp = pool + kv_block_base(phys, a.layer, a.n_layers, 0, a.hkv, g, HD);
      const uint16_t* vp = pool + kv_block_base(phys, a.layer, a.n_layers, 1, a.hkv, g, HD);
#pragma unroll
      for (int i = 0; i < NQ; ++i) kq[slot][i] = *(const uint4*)(kp + l16 * HD + 32 * i + 8 * kb);
#pragma unroll
      for (int c = 0; c < NC; ++c) vq[slot][c] = *(const uint2*)(vp + (16 * c + l16) * 16 + 4 * kb);
    };
    auto process = [&](int slot, int blk) {
      const uint4* kc = kq[slot];
      const uint2* vc = vq[slot];
      // S^T = K . Q^T: A = K rows (token l16), k = 8*kb + 32*i
      f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const bf16x8_t kf = __builtin_bit_cast(bf16x8_t, kc[i]);
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[i], s, 0, 0, 0);
      }
      // lane holds tokens 4*kb + r of row l16
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kpos = blk * 16 + 4 * kb + r;
        float v = s[r] * scale;
        if (!q_ok || kpos > qpos_q) v = -INFINITY;
        s[r] = v;
        mx = fmaxf(mx, v);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      // P enters the P.V product as two bf16 terms, p = hi + lo (hi = bf16(p),
      // lo = bf16(p - hi)): V is exact in bf16, so the product keeps ~16
      // mantissa bits of p instead of 8 at the cost of a second small MFMA.
      float corr, psum = 0.f;
      uint32_t pk[2], pl[2];
      if (m_new == -INFINITY) {
        corr = 1.f;
        pk[0] = pk[1] = pl[0] = pl[1] = 0u;
      } else {
        corr = __builtin_amdgcn_exp2f(m_run - m_new);
        float p[4], lo[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[r] = __builtin_amdgcn_exp2f(s[r] - m_new);   // exp2(-inf) = 0 for masked keys
          psum += p[r];
        }
        // bf16 pairs by the hardware conversion (round to nearest even)
        const bf16x2_t h01 = {(__bf16)p[0], (__bf16)p[1]}, h23 = {(__bf16)p[2], (__bf16)p[3]};
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          lo[r] = p[r] - (float)h01[r];
          lo[2 + r] = p[2 + r] - (float)h23[r];
        }
        const bf16x2_t l01 = {(__bf16)lo[0], (__bf16)lo[1]}, l23 = {(__bf16)lo[2], (__bf16)lo[3]};
        pk[0] = __builtin_bit_cast(uint32_t, h01);
        pk[1] = __builtin_bit_cast(uint32_t, h23);
        pl[0] = __builtin_bit_cast(uint32_t, l01);
        pl[1] = __builtin_bit_cast(uint32_t, l23);
      }
      psum += __shfl_xor(psum, 16, 64);
      psum += __shfl_xor(psum, 32, 64);
      l_run = l_run * corr + psum;
      m_run = m_new;
      // rescale O rows (rows 4*kb + r live in lanes l16 == 4*kb + r of the
      // score layout) -- skipped when no row's maximum moved, where every
      // factor is exactly 1
      if (__builtin_amdgcn_ballot_w64(corr != 1.0f) != 0) {
        float cr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) cr[r] = __shfl(corr, 4 * kb + r, 64);
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[c][r] *= cr[r];
      }
      const bf16x4s_t pa = __builtin_bit_cast(bf16x4s_t, *(const uint2*)pk);
      const bf16x4s_t pb = __builtin_bit_cast(bf16x4s_t, *(const uint2*)pl);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        // B = V^T: n = column 16c + l16, k = tokens 4*kb .. +4
        const bf16x4s_t vf = __builtin_bit_cast(bf16x4s_t, vc[c]);
        o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vf, o[c], 0, 0, 0);
        o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pb, vf, o[c], 0, 0, 0);
      }
    };
    if (nb > 0) {
#pragma unroll
      for (int d = 0; d < D - 1; ++d) fetch(d, bid(d));
      long idn = bid(D - 1);
      for (int t0 = 0; t0 < nb; t0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
          const int t = t0 + d;
          fetch((d + D - 1) % D, idn);  // block t + D - 1 (re-loads of the last block past the end)
          idn = bid(t + D);
          if (t < nb) process(d, first + s_in * t);
        }
      }
    }
  }

  // Merge the s_in waves of each row group in LDS (sources in a fixed
  // order).  Each of them then finishes the column tiles c with
  // c % s_in == sin, so the merge costs every wave only its share.
  float rl[4], rm[4];
  if (s_in > 1) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) o_sh[wave][(4 * kb + r) * OS + 16 * c + l16] = o[c][r];
    if (kb == 0) { ml_sh[wave][0][l16] = m_run; ml_sh[wave][1][l16] = l_run; }
    __syncthreads();
    const int w0 = rgi * s_in;
    float f[4][NW];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * kb + r;
      float mr[NW], M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        mr[w] = w < s_in ? ml_sh[w0 + w][0][row] : -INFINITY;
        M = fmaxf(M, mr[w]);
      }
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        f[r][w] = (mr[w] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mr[w] - M);
        if (w < s_in) L = fmaf(f[r][w], ml_sh[w0 + w][1][row], L);
      }
      rm[r] = M;
      rl[r] = L;
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c % s_in != sin) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w)
          if (w < s_in) v = fmaf(f[r][w], o_sh[w0 + w][(4 * kb + r) * OS + 16 * c + l16], v);
        o[c][r] = v;
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      rl[r] = __shfl(l_run, 4 * kb + r, 64);
      rm[r] = __shfl(m_run, 4 * kb + r, 64);
    }
  }
  if (rgi >= rgroups) return;

#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int rr = rgi * 16 + 4 * kb + r;
    if (rr >= R) continue;
    const int qi = rr / grp, hh = g * grp + rr % grp;
    if (w.nu == 1) {
      const float inv = rl[r] > 0.f ? 1.0f / rl[r] : 0.f;
      uint16_t* out = (uint16_t*)a.out + ((long)(qrow0 + qi) * a.hq + hh) * HD;
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (c % s_in == sin) out[16 * c + l16] = (uint16_t)f2bf(o[c][r] * inv);
    } else {
      float* pp = partial_row(a, u, g, rr);
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (c % s_in == sin) pp[16 * c + l16] = o[c][r];
      if (sin == 0 && l16 == 0) { pp[HD] = rm[r]; pp[HD + 1] = rl[r]; }
    }
  }
}

// fp32 (small models): one wavefront per row, keys streamed from the pool.
__global__ __launch_bounds__(256) void k_attn_valu(AttnArgs a, int nsplit, int bps) {
  const int u = blockIdx.x, g = blockIdx.y;
  if (a.unit_start && u >= a.n_units) return;
  const Unit w = unit_of(a, u, nsplit, bps);
  const int item = w.item;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hd = a.hd, grp = a.hq / a.hkv;
  const int qc = a.item_q_count[item], pos0 = a.item_q_pos0[item], qrow0 = a.item_q_row0[item];
  const int R = grp * qc;
  const int nkeys = pos0 + qc;
  const int k0 = w.b0 * 16;
  const int k1 = min(nkeys, k0 + w.bps * 16);
  const float scale = 1.0f / sqrtf((float)hd);
  const float* pool = (const float*)a.kv_pool;
  const int32_t* bt = a.block_table + (long)a.item_bt_row[item] * a.bt_stride;
  for (int r = wave; r < R; r += 4) {
    const int qi = r / grp, hh = g * grp + r % grp;
    const int qpos = pos0 + qi;
    const float* q = (const float*)a.q + ((long)(qrow0 + qi) * a.hq + hh) * hd;
    const float q0 = lane < hd ? q[lane] : 0.f;
    const float q1 = lane + 64 < hd ? q[lane + 64] : 0.f;
    float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
    const int kend = min(k1, qpos + 1);
    for (int k = k0; k < kend; ++k) {
      const long phys = bt[k >> 4];
      const int t = k & 15;
      const float* kr = pool + kv_block_base(phys, a.layer, a.n_layers, 0, a.hkv, g, hd) + t * hd;
      const float* vb = pool + kv_block_base(phys, a.layer, a.n_layers, 1, a.hkv, g, hd);
      float s = (lane < hd ? q0 * kr[lane] : 0.f) + (lane + 64 < hd ? q1 * kr[lane + 64] : 0.f);
      s = wave_sum(s) * scale;
      const float mn = fmaxf(m, s);
      const float c = expf(m - mn), p = expf(s - mn);
      l = l * c + p;
      if (lane < hd) o0 = o0 * c + p * vb[lane * 16 + t];
      if (lane + 64 < hd) o1 = o1 * c + p * vb[(lane + 64) * 16 + t];
      m = mn;
    }
    if (w.nu == 1) {
      float* out = (float*)a.out + ((long)(qrow0 + qi) * a.hq + hh) * hd;
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      if (lane < hd) out[lane] = o0 * inv;
      if (lane + 64 < hd) out[lane + 64] = o1 * inv;
    } else {
      float* pp = partial_row(a, u, g, r);
      if (lane < hd) pp[lane] = o0;
      if (lane + 64 < hd) pp[lane + 64] = o1;
      if (lane == 0) { pp[hd] = m; pp[hd + 1] = l; }
    }
  }
}

// Combine of an item's units for one (KV head, row): the units' maxima and
// weights exp(m_s - M) (weights kept in LDS), then blockDim / hd thread
// groups each sum a strided subset of the units for one output element per
// thread, and the groups add in a fixed order.  Every load of the first
// nt units' (max, sum) and of each group's first eight strided partials is
// issued before anything waits, so an item of up to 8 * ng units costs one
// memory round trip (the maxima, the weights and the partial sums were three
// dependent trips).  The sums run in the same order either way.
constexpr int kCombineMaxUnits = 4096;
template <bool BF>
__global__ __launch_bounds__(1024) void k_attn_combine(AttnArgs a, int nsplit) {
  __shared__ float w_sh[kCombineMaxUnits];
  __shared__ float red[2][16];
  __shared__ float acc_sh[1024];
  const int item = a.unit_start ? a.split_items[blockIdx.x] : blockIdx.x;
  const int g = blockIdx.y, r = blockIdx.z;
  const int grp = a.hq / a.hkv, hd = a.hd;
  const int qc = a.item_q_count[item];
  if (r >= grp * qc) return;
  const int u0 = a.unit_start ? a.unit_start[item] : item * nsplit;
  const int nu = a.unit_start ? a.unit_start[item + 1] - u0 : nsplit;
  if (nu == 1) return;  // written directly by its only unit
  const long stride_sp = (long)a.hkv * (grp * a.max_q_count) * (hd + 2);
  const float* base = partial_row(a, u0, g, r);
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6, nw = nt >> 6;
  const int ng = nt / hd, gi = tid / hd, e = tid - gi * hd;

  // the round trip: (max, sum) of unit tid and this group's first eight partials
  const int s_own = min(tid, nu - 1);
  const float m_own = base[s_own * stride_sp + hd];
  const float l_own = base[s_own * stride_sp + hd + 1];
  float p0[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) p0[j] = base[min(gi + j * ng, nu - 1) * stride_sp + e];

  float mx = tid < nu ? m_own : -INFINITY;
  for (int s = tid + nt; s < nu; s += nt) mx = fmaxf(mx, base[s * stride_sp + hd]);
  mx = wave_max(mx);
  if (lane == 0) red[0][wave] = mx;
  __syncthreads();
  float M = -INFINITY;
  for (int w = 0; w < nw; ++w) M = fmaxf(M, red[0][w]);
  // the bf16 kernel's partial maxima are in the log2 domain, the fp32 one's natural
  auto weight = [&](float ms) { return (ms == -INFINITY) ? 0.f : (BF ? __builtin_amdgcn_exp2f(ms - M) : expf(ms - M)); };
  float dl = 0.f;
  if (tid < nu) {
    const float wt = weight(m_own);
    w_sh[tid] = wt;
    dl = wt * l_own;   // fmaf(wt, l, 0)
  }
  for (int s = tid + nt; s < nu; s += nt) {
    const float wt = weight(base[s * stride_sp + hd]);
    w_sh[s] = wt;
    dl = fmaf(wt, base[s * stride_sp + hd + 1], dl);
  }
  dl = wave_sum(dl);
  if (lane == 0) red[1][wave] = dl;
  __syncthreads();
  float den = 0.f;
  for (int w = 0; w < nw; ++w) den += red[1][w];

  float num = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (gi + j * ng < nu) num = fmaf(w_sh[gi + j * ng], p0[j], num);
  int s = gi + 8 * ng;
  for (; s + 7 * ng < nu; s += 8 * ng) {
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = base[(s + j * ng) * stride_sp + e];
#pragma unroll
    for (int j = 0; j < 8; ++j) num = fmaf(w_sh[s + j * ng], p[j], num);
  }
  for (; s < nu; s += ng) num = fmaf(w_sh[s], base[s * stride_sp + e], num);
  acc_sh[tid] = num;
  __syncthreads();
  if (gi != 0) return;
  for (int k = 1; k < ng; ++k) num += acc_sh[k * hd + e];
  const int qi = r / grp, hh = g * grp + (r - qi * grp);
  const long o = ((long)(a.item_q_row0[item] + qi) * a.hq + hh) * hd + e;
  typedef typename Act<BF>::T T;
  Act<BF>::st((T*)a.out, o, den > 0.f ? num / den : 0.f);
}

// The split without a unit table: every item gets nsplit units of bps
// blocks.  Keys are split over work-groups until each wave walks at most 4
// blocks, but no further than ~512 groups in flight.
struct UniformSplit {
  int nsplit, bps;
};
static UniformSplit uniform_split(const AttnArgs& a) {
  const int grp = a.hq / a.hkv;
  const int maxblk = (a.max_ctx + 15) / 16;
  const long base = (long)a.n_items * a.hkv;
  // Waves of a work-group that share its KV range (the rest hold other query
  // rows): 4 when the rows fit one 16-row group, 2 for two, else 1.
  const int rows = grp * a.max_q_count;
  const int rgroups = (rows + 15) / 16;
  const int s_in = (rgroups == 1 ? 4 : (rgroups == 2 ? 2 : 1)) * (kAttnWaves / 4);
  const int per_wg = 4 * s_in;
  int nsplit = 1;
  if (maxblk > per_wg)
    nsplit = (int)std::max(1L, std::min((long)(maxblk + per_wg - 1) / per_wg, (512 + base - 1) / base));
  if ((maxblk + nsplit - 1) / nsplit > kAttnMaxUnitBlocks) nsplit = (maxblk + kAttnMaxUnitBlocks - 1) / kAttnMaxUnitBlocks;
  const int bps = std::max(1, (maxblk + nsplit - 1) / nsplit);
  return UniformSplit{std::max(1, (maxblk + bps - 1) / bps), bps};
}

// Ring depth of the scoring kernel for a launch: units of at most
// kAttnShortUnit blocks (about 12 per wave) take the one-stage ring at four
// work-groups per CU, longer ones the two-stage ring at three.  Measured on
// the rollout's batch bins (against the three-stage ring at two work-groups
// per CU): batch 1-11 16-19 % faster with one stage (21.6 -> 17.1 us at
// batch 1, 44.8 -> 35.1 at batch 6) where two stages gave 11-17 %, batch
// 46-204 1-2 % faster with two stages where one stage gave 0-6 % slower.
constexpr long kAttnShortUnit = 48;
int attn_ring(const AttnArgs& a) {
  const int maxblk = (a.max_ctx + 15) / 16;
  long units, bpu;
  if (a.unit_start) {
    units = std::max(1, a.n_units);
    bpu = ((long)maxblk * a.n_items + units - 1) / units;
  } else {
    bpu = uniform_split(a).bps;
  }
  return bpu <= kAttnShortUnit ? 1 : 2;
}

int launch_attention(const AttnArgs& a, hipStream_t st, int phase, int* combined) {
  if (a.n_items <= 0) return 0;
  const int grp = a.hq / a.hkv;
  if ((a.hd != 64 && a.hd != 128) || a.hq % a.hkv != 0) return -1;
  if (grp * a.max_q_count > 64) return -1;
  const int maxblk = (a.max_ctx + 15) / 16;
  const UniformSplit us = uniform_split(a);
  int nsplit = us.nsplit;
  const int bps = us.bps;
  const long units = a.unit_start ? (long)a.n_units : (long)a.n_items * nsplit;
  const bool combine = a.unit_start ? a.n_split > 0 : nsplit > 1;
  if (combine && (a.unit_start ? (maxblk + 7) / 8 : nsplit) > kCombineMaxUnits) return -1;
  if (combine) {
    const size_t need = (size_t)units * a.hkv * grp * a.max_q_count * (a.hd + 2);
    if (need > a.ws_floats) return -2;
  }
  if (combined) *combined = combine ? 1 : 0;
  if (units <= 0) return 0;
  dim3 grid((unsigned)units, a.hkv, 1);
  if (phase != 2) {
  if (a.bf16) {
    if (attn_ring(a) == 1) {
      if (a.hd == 128) hipLaunchKernelGGL((k_attn_mfma<128, kAttnWaves, 1>), grid, dim3(kAttnWaves * 64), 0, st, a, nsplit, bps);
      else hipLaunchKernelGGL((k_attn_mfma<64, kAttnWaves, 1>), grid, dim3(kAttnWaves * 64), 0, st, a, nsplit, bps);
    } else {
      if (a.hd == 128) hipLaunchKernelGGL((k_attn_mfma<128, kAttnWaves, 2>), grid, dim3(kAttnWaves * 64), 0, st, a, nsplit, bps);
      else hipLaunchKernelGGL((k_attn_mfma<64, kAttnWaves, 2>), grid, dim3(kAttnWaves * 64), 0, st, a, nsplit, bps);
    }
  } else {
    hipLaunchKernelGGL(k_attn_valu, grid, dim3(256), 0, st, a, nsplit, bps);
  }
  if (hipGetLastError() != hipSuccess) return -3;
  }
  if (combine && phase != 1) {
    // threads: hd per group, about one group per 8 units of the largest item
    const int mu = a.unit_start ? (a.max_units > 0 ? a.max_units : (maxblk + 7) / 8) : nsplit;
    int ngr = 1;
    while (ngr < 1024 / a.hd && ngr * 8 < mu) ngr *= 2;
    dim3 g2(a.unit_start ? a.n_split : a.n_items, a.hkv, grp * a.max_q_count);
    if (a.bf16) hipLaunchKernelGGL(k_attn_combine<true>, g2, dim3(ngr * a.hd), 0, st, a, nsplit);
    else hipLaunchKernelGGL(k_attn_combine<false>, g2, dim3(ngr * a.hd), 0, st, a, nsplit);
    if (hipGetLastError() != hipSuccess) return -3;
  }
  return 0;
}

}  // namespace er
