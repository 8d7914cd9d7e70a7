// Persistent decode forward: one cooperative launch runs a whole small-batch
// forward of a bf16 model (the target, or the W4/W8 self-drafter) from the
// embedding gather to the final residual stream, for up to 16 rows (decode
// and drafting at batch <= 16, verify at batch * (gamma + 1) <= 16).
//
// Why: in the memory-bound tail each decoder layer is five small projections
// and an attention pass; launched one kernel each, their ramp-up and drain
// (several microseconds per launch, ~170 launches per forward) cost more than
// the bytes they stream.  The drafter of the EfficientRollout page ("关键模块"
// item 1: the target's own weights quantized, sharing its KV cache) only pays
// if a W4 forward costs close to its 0.26x share of the target's bytes.
//
// Structure: one work-group of 8 waves per compute unit, all resident
// (cooperative launch).  Phases per layer, separated by a grid barrier:
//   QKV  x' = RMSNorm(h) formed while staging, RoPE + paged-KV append epilogue
//   ATT  paged GQA attention over work units (sequence, key range) x KV head
//   COMB merge of the units of sequences whose keys were split (if any)
//   O    attention output projection, residual add into h
//   GU   x' = RMSNorm(h), gate/up projection with the SwiGLU epilogue
//   DOWN down projection, residual add into h
// A linear phase is a list of tasks (128-row output tile, K slice) dealt to
// the work-groups in order; the 8 waves of a task each own 16 output rows and
// stream their weights through a register ring, with the task's x' slice
// staged once in LDS.  When K is split, each slice's partial tile goes to a
// workspace and the last slice to finish (a counter per tile) sums the slices
// in slice order and applies the epilogue, so results do not depend on which
// work-group finishes last.  The sums of squares of h for the next RMSNorm are
// added per (tile, row) as 64-bit fixed point (exact, order-free).
//
// Memory visibility across the 8 L2 caches: every value produced inside the
// kernel and read by another work-group is written with device-scope stores
// (sc1: through to memory) and read with device-scope loads, and each wave
// waits for its stores before arriving at a barrier or a tile counter.  The
// paged KV entries written in QKV are read with ordinary loads in ATT: each
// (layer, slot) entry is written once per forward and no cache holds it before
// (caches are invalidated at kernel start, and earlier phases read other
// layers).  The grid barrier spreads arrivals over 8 counters (a 256-group
// barrier on one counter serializes at ~15 ns per atomic) and releases the
// waiters through one generation word; every wait is bounded and reports a
// time-out through an error flag instead of hanging.

#include <algorithm>
#include <cstdio>

#include "common.h"
#include "kernels.h"
#include "linear_dev.h"

namespace er {

constexpr int DT = 512;      // threads per work-group
constexpr int DW = 8;        // waves per work-group

// Barrier words (see DecodeArgs::bar): 8 arrival counters, the arrival count
// of the last groups, the generation; each on its own 128-byte line.
constexpr int BAR_ARRIVE = 0, BAR_TOP = 8 * 32, BAR_GEN = 9 * 32;

// ---- device-scope (cross-L2 coherent) loads and stores ---------------------
// Bulk values go through buffer instructions with the sc1 cache policy
// (device scope: stores write through, loads miss stale L2 lines), which the
// compiler can keep many of in flight; atomic loads of the same scope are
// issued one at a time (each waits out a memory round trip), so atomics are
// used only for counters and flags.
constexpr int kBufCfg = 0x00020000;  // raw buffer, dword 3 of the resource on the gfx9 family
constexpr int kSC1 = 16;             // cache policy bits: sc1
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
ER_DEV Rsrc rsrc(const void* base) { return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7FFFFFFF, kBufCfg); }
ER_DEV uint4 bld128(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSC1));
}
ER_DEV uint32_t bld32(Rsrc r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kSC1); }
ER_DEV unsigned long long bld64(Rsrc r, uint32_t off) {
  typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kSC1);
  return (unsigned long long)v.x | ((unsigned long long)v.y << 32);
}
ER_DEV float bldf(Rsrc r, uint32_t off) { return __uint_as_float(bld32(r, off)); }
ER_DEV void bst128(Rsrc r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, kSC1);
}
ER_DEV void bst32(Rsrc r, uint32_t off, uint32_t v) { __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kSC1); }
ER_DEV void bstf(Rsrc r, uint32_t off, float v) { bst32(r, off, __float_as_uint(v)); }
ER_DEV void bst16(Rsrc r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, off, 0, kSC1);
}
ER_DEV uint32_t ld_dev32(const void* p) {
  return __hip_atomic_load((uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
ER_DEV unsigned long long ld_dev64(const void* p) {
  return __hip_atomic_load((unsigned long long*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
ER_DEV void st_dev32(void* p, uint32_t v) {
  __hip_atomic_store((uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
ER_DEV void st_dev64(void* p, unsigned long long v) {
  __hip_atomic_store((unsigned long long*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-bit store written through to memory, for the paged KV pool (which can
// exceed a buffer resource's 32-bit range).
ER_DEV void st_dev16(void* p, uint32_t v) {
  asm volatile("global_store_short %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
}
ER_DEV unsigned atomic_add_dev(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
ER_DEV void atomic_add_dev64(unsigned long long* p, unsigned long long v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this wave issued has completed.
ER_DEV void wait_mem() { __builtin_amdgcn_s_waitcnt(0); }

// Grid barrier.  Returns false after a time-out or when another group
// reported one (the caller then leaves the kernel).
ER_DEV bool grid_barrier(const DecodeArgs& a, unsigned& gen, int& nbar) {
  __shared__ int s_ok;
  wait_mem();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long* tr = (a.trace && nbar < a.trace_max) ? a.trace + ((long)nbar * gridDim.x + blockIdx.x) * 2 : nullptr;
    if (tr) tr[0] = __builtin_amdgcn_s_memrealtime();
    unsigned* bar = a.bar;
    const int G = (int)gridDim.x;
    const int slots = G < 8 ? G : 8;
    const int slot = (int)blockIdx.x & 7;
    const unsigned n_slot = (unsigned)(G >> 3) + ((slot < (G & 7)) ? 1u : 0u);
    if (atomic_add_dev(bar + BAR_ARRIVE + 32 * slot, 1u) == n_slot - 1u) {
      st_dev32(bar + BAR_ARRIVE + 32 * slot, 0u);
      wait_mem();
      if (atomic_add_dev(bar + BAR_TOP, 1u) == (unsigned)slots - 1u) {
        st_dev32(bar + BAR_TOP, 0u);
        wait_mem();
        st_dev32(bar + BAR_GEN, gen + 1u);
      }
    }
    int ok = 1;
    long spins = 0;
    while (ld_dev32(bar + BAR_GEN) == gen) {
      if (++spins > a.spin_limit || ((spins & 63) == 0 && ld_dev32(a.err) != 0)) {
        st_dev32(a.err, 1u);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (tr) tr[1] = __builtin_amdgcn_s_memrealtime();
    s_ok = ok;
  }
  __syncthreads();
  gen += 1u;
  ++nbar;
  return s_ok != 0;
}

// ---- linear phases -----------------------------------------------------------
// Values loaded from device memory (the layer descriptors) are not known to
// be wave-uniform, so every loop bound and address derived from them would be
// treated as divergent (exec-masked loads, after which the compiler drains
// the whole load counter at each use).  They are moved to scalar registers.
ER_DEV int sgpr(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <class T>
ER_DEV T* sgpr_ptr(T* p) {
  const unsigned long long u = (unsigned long long)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)u), hi = __builtin_amdgcn_readfirstlane((unsigned)(u >> 32));
  return (T*)(((unsigned long long)hi << 32) | lo);
}
ER_DEV LinearW sgpr_w(const LinearW& w) {
  LinearW o;
  o.fmt = sgpr(w.fmt);
  o.w = sgpr_ptr(w.w);
  o.scale = sgpr_ptr(w.scale);
  o.zero = sgpr_ptr(w.zero);
  o.N = sgpr(w.N);
  o.K = sgpr(w.K);
  return o;
}
enum { DEPI_QKV = 0, DEPI_RESID = 1, DEPI_SWIGLU = 2 };

// Physical weight row of logical row 16 * s + l16 (pairs of the RoPE / SwiGLU
// epilogues in lanes l16 and l16 ^ 8 of one 16-row subtile).
template <int EPI>
ER_DEV int dec_row(int F, int hd, int s, int l16) {
  if constexpr (EPI == DEPI_SWIGLU) {
    const int f = s * 8 + (l16 & 7);
    return (l16 & 8) ? F + f : f;
  } else if constexpr (EPI == DEPI_QKV) {
    const int per_head = hd >> 4;
    const int h = s / per_head, pb = (s - h * per_head) * 8;
    return h * hd + pb + (l16 & 7) + ((l16 & 8) ? (hd >> 1) : 0);
  } else {
    return 16 * s + l16;
  }
}

// Global-address-space views, so that loads through pointers taken from
// device memory compile to global (not flat) loads: a flat load counts on
// both the vector-memory and the LDS counters, and every wait on it would
// also wait for the other.
#define ER_G __attribute__((address_space(1)))
template <class T>
ER_DEV const ER_G T* gptr(const void* p) { return (const ER_G T*)p; }
ER_DEV uint4 ldg128(const void* p) { return __builtin_bit_cast(uint4, *(const ER_G u32x4_t*)p); }

// LDS carve of a linear phase: x' of every row for the whole K when the
// phase normalizes on load ([16][K + 8] bf16, staged once per phase), the
// per-chunk row sums of that x' for the quantized zero points, and the area
// where the K-splitting waves of a row group add their partial tiles.
constexpr int LIN_RED = DW * 64 * 16;                     // [8 waves][64 lanes] f32x4
ER_DEV int lin_xs_bytes(int M, int K) { return M * (K + 8) * 2; }
ER_DEV int lin_xsum_bytes(int K) { return (K / 128) * 16 * 4; }

template <int FMT> struct DStage { static constexpr int NW = (FMT == FMT_BF16) ? 4 : (FMT == FMT_W8 ? 2 : 1); };
// register ring depth: weights (and, from global memory, x') of DEPTH chunks in flight
template <int FMT, bool XG> struct DDepth {
  static constexpr int D = (FMT == FMT_BF16) ? (XG ? 3 : 4) : (FMT == FMT_W8) ? (XG ? 4 : 6) : (XG ? 4 : 8);
};

// One linear phase.  Tasks of 16 * RG output rows (RG = 8 / KS row groups of
// 16), the KS waves of a row group taking the K chunks ks, ks + KS, ...; a
// work-group's tasks t = blockIdx.x + G j form one stream of (task, chunk)
// items per wave, so the register ring runs on across task boundaries and a
// task's epilogue overlaps the next task's loads.  x' comes from LDS (XLDS:
// RMSNorm(h) staged once per phase) or straight from global memory (a bf16
// activation buffer written earlier in this forward, read through L2).
template <int FMT, int EPI, int KS, bool XLDS>
__device__ __noinline__ void lin_phase(const DecodeArgs& a, const LinearW& W_, int layer, const void* gnorm_,
                                       const float* h_in, const unsigned long long* ssq_in, const uint16_t* x_in,
                                       float* h_out, unsigned long long* ssq_out, long ssq_out_stride, char* lds) {
  const LinearW W = sgpr_w(W_);
  const void* gnorm = sgpr_ptr(gnorm_);
  // every scalar of the descriptor in scalar registers (a is a reference here)
  const int M = sgpr(a.M), F_ = sgpr(a.F), hd_ = sgpr(a.hd), d_ = sgpr(a.d), hq_ = sgpr(a.hq), hkv_ = sgpr(a.hkv);
  const int L_ = sgpr(a.L), slots_ = sgpr(a.ssq_slots);
  const float eps_ = __uint_as_float(sgpr(__float_as_uint(a.eps)));
  const int32_t* pos_ = sgpr_ptr(a.pos);
  const int64_t* slot_ = sgpr_ptr(a.slot);
  const float2* cs_ = sgpr_ptr(a.cs);
  void* kv_ = sgpr_ptr(a.kv_pool);
  uint16_t* qbuf_ = sgpr_ptr(a.qbuf);
  uint16_t* act_ = sgpr_ptr(a.act);
  h_in = sgpr_ptr(h_in);
  x_in = sgpr_ptr(x_in);
  h_out = sgpr_ptr(h_out);
  ssq_in = sgpr_ptr(ssq_in);
  ssq_out = sgpr_ptr(ssq_out);
  constexpr int RG = DW / KS;
  constexpr int NW = DStage<FMT>::NW;
  constexpr int DEPTH = DDepth<FMT, !XLDS>::D;
  constexpr int XW = XLDS ? 1 : 4;   // x' registers per stage when x' comes from global memory
  const int N = W.N, K = W.K;
  const int nc = K >> 7;
  const long G = nc;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int rg = wave / KS, ks = wave % KS;
  const int kb = lane >> 4, l16 = lane & 15;
  const int xr_row = l16 < M ? l16 : M - 1;
  const int ldsx = K + 8;
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds + LIN_RED);
  float* xsum = reinterpret_cast<float*>(lds + LIN_RED + (XLDS ? lin_xs_bytes(M, K) : 0));
  f32x4_t* red = reinterpret_cast<f32x4_t*>(lds);
  __shared__ float rs_sh[16];

  if constexpr (XLDS) {
    // x' = bf16(h * rstd * g) for all rows and the whole K, and its per-chunk row sums
    // 16 lanes per row, one slot each, all loads in flight at once (the slots
    // are updated by device-scope atomics: device-scope loads)
    if (tid < 16 * M) {
      const int m = tid >> 4, sl = tid & 15;
      unsigned long long t = sl < slots_ ? bld64(rsrc(ssq_in), (uint32_t)((sl * 16 + m) * 8)) : 0ull;
      t += __shfl_xor(t, 1, 64);
      t += __shfl_xor(t, 2, 64);
      t += __shfl_xor(t, 4, 64);
      t += __shfl_xor(t, 8, 64);
      if (sl == 0) rs_sh[m] = 1.0f / sqrtf((float)((double)t / SSQ_SCALE) / (float)K + eps_);
    }
    __syncthreads();
    const int K8 = K >> 3, tot = M * K8;
    for (int e0 = 0; e0 < tot; e0 += 4 * DT) {
      uint4 hv[4][2], gv[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int e = min(e0 + tid + p * DT, tot - 1);
        const int m = e / K8, k8 = e - m * K8;
        const ER_G float* hp = gptr<float>(h_in) + (long)m * K + (long)k8 * 8;
        hv[p][0] = ldg128((const void*)hp);
        hv[p][1] = ldg128((const void*)(hp + 4));
        gv[p] = ldg128((const void*)(gptr<uint16_t>(gnorm) + (long)k8 * 8));
      }
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int e = e0 + tid + p * DT;
        if (e >= tot) continue;
        const int m = e / K8, k8 = e - m * K8;
        const float rs = rs_sh[m];
        const uint4 h0 = hv[p][0], h1 = hv[p][1], g = gv[p];
        uint4 o;
        o.x = f2bf(__uint_as_float(h0.x) * rs * bf_lo(g.x)) | (f2bf(__uint_as_float(h0.y) * rs * bf_hi(g.x)) << 16);
        o.y = f2bf(__uint_as_float(h0.z) * rs * bf_lo(g.y)) | (f2bf(__uint_as_float(h0.w) * rs * bf_hi(g.y)) << 16);
        o.z = f2bf(__uint_as_float(h1.x) * rs * bf_lo(g.z)) | (f2bf(__uint_as_float(h1.y) * rs * bf_hi(g.z)) << 16);
        o.w = f2bf(__uint_as_float(h1.z) * rs * bf_lo(g.w)) | (f2bf(__uint_as_float(h1.w) * rs * bf_hi(g.w)) << 16);
        *(uint4*)(xs + m * ldsx + k8 * 8) = o;
      }
    }
    __syncthreads();
    if constexpr (FMT != FMT_BF16) {
      for (int e = tid; e < 16 * nc; e += DT) {
        const int c = e >> 4, m = e & 15;
        float sm = 0.f;
        if (m < M) {
          const uint4* p = (const uint4*)(xs + m * ldsx + c * 128);
          for (int q = 0; q < 16; ++q) {
            const uint4 v = p[q];
            sm += bf_lo(v.x) + bf_hi(v.x) + bf_lo(v.y) + bf_hi(v.y) + bf_lo(v.z) + bf_hi(v.z) + bf_lo(v.w) + bf_hi(v.w);
          }
        }
        xsum[e] = sm;
      }
      __syncthreads();
    }
  }

  const int R = 16 * RG;
  const int ntask = (N + R - 1) / R;
  const int Gw = (int)gridDim.x;
  const int my_tasks = (int)blockIdx.x < ntask ? (ntask - (int)blockIdx.x + Gw - 1) / Gw : 0;
  const int n_it = (nc - ks + KS - 1) / KS;   // this wave's chunks per task
  const int T = my_tasks * n_it;              // this wave's items
  const int last = T > 0 ? T - 1 : 0;

  // weight row of this lane in task j
  auto row_of = [&](int j, bool* in) -> int {
    const int s = ((int)blockIdx.x + Gw * j) * RG + rg;
    *in = 16 * s + l16 < N;
    return *in ? dec_row<EPI>(F_, hd_, s, l16) : N - 1;
  };

  uint4 wreg[DEPTH][NW];
  uint4 xreg[DEPTH][XW];
  uint32_t scr[DEPTH], zcr[DEPTH];
  auto issue = [&](int q, int slot) {
    q = min(q, last);
    const int j = q / n_it, it = q - j * n_it;
    const long c = ks + (long)KS * it;
    bool in;
    const long nrow = row_of(j, &in);
    if constexpr (FMT == FMT_BF16) {
      const ER_G uint16_t* p = gptr<uint16_t>(W.w) + nrow * K + c * 128 + 8 * kb;
#pragma unroll
      for (int i = 0; i < 4; ++i) wreg[slot][i] = ldg128((const void*)(p + 32 * i));
    } else if constexpr (FMT == FMT_W8) {
      const ER_G int8_t* p = gptr<int8_t>(W.w) + nrow * K + c * 128 + 16 * kb;
#pragma unroll
      for (int h = 0; h < 2; ++h) wreg[slot][h] = ldg128((const void*)(p + 64 * h));
    } else {
      wreg[slot][0] = ldg128((const void*)(gptr<uint8_t>(W.w) + w4_piece(nrow, c, W.N, K) + 16 * kb));
      // raw codes: converting here would make the issue wait for its own loads
      scr[slot] = gptr<uint16_t>(W.scale)[nrow * G + c];
      zcr[slot] = gptr<uint8_t>(W.zero)[nrow * G + c];
    }
    if constexpr (!XLDS) {
      const ER_G uint16_t* xp = gptr<uint16_t>(x_in) + (long)xr_row * K + c * 128;
#pragma unroll
      for (int i = 0; i < 4; ++i) xreg[slot][i] = ldg128((const void*)(xp + kcol<FMT>(i, kb)));
    }
  };

  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int q, int slot) {
    const int j = q / n_it, it = q - j * n_it;
    const int c = ks + KS * it;
    bf16x8_t xa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (XLDS)
        xa[i] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(xs + xr_row * ldsx + c * 128 + kcol<FMT>(i, kb)));
      else
        xa[i] = __builtin_bit_cast(bf16x8_t, xreg[slot][i]);
    }
    if constexpr (FMT == FMT_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[i], __builtin_bit_cast(bf16x8_t, wreg[slot][i]), acc, 0, 0, 0);
    } else {
      f32x4_t accg = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x8_t bw;
        if constexpr (FMT == FMT_W8) {
          const uint4 v = wreg[slot][i >> 1];
          bw = (i & 1) ? w8_to_bf16(v.z, v.w) : w8_to_bf16(v.x, v.y);
        } else {
          const uint4 v = wreg[slot][0];
          const uint32_t word = (i == 0) ? v.x : (i == 1) ? v.y : (i == 2) ? v.z : v.w;
          bw = w4_to_bf16(word);
        }
        accg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[i], bw, accg, 0, 0, 0);
      }
      // per-chunk row sums of x' for the zero point: from LDS, or from the
      // fragments (lanes l16 = m hold row m's 128 values over the 4 kb groups)
      float xsm[4];
      if constexpr (XLDS) {
        const float4 v = *reinterpret_cast<const float4*>(xsum + c * 16 + 4 * kb);
        xsm[0] = v.x; xsm[1] = v.y; xsm[2] = v.z; xsm[3] = v.w;
      } else {
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 v = xreg[slot][i];
          t += bf_lo(v.x) + bf_hi(v.x) + bf_lo(v.y) + bf_hi(v.y) + bf_lo(v.z) + bf_hi(v.z) + bf_lo(v.w) + bf_hi(v.w);
        }
        t += __shfl_xor(t, 16, 64);
        t += __shfl_xor(t, 32, 64);
#pragma unroll
        for (int r = 0; r < 4; ++r) xsm[r] = __shfl(t, 4 * kb + r, 64);
      }
      if constexpr (FMT == FMT_W8) {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += accg[r] - 128.0f * xsm[r];
      } else {
        const float sx = bf2f(scr[slot]), sy = 128.0f + (float)zcr[slot];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = fmaf(sx, fmaf(-sy, xsm[r], accg[r]), acc[r]);
      }
    }
  };

  // End of task j, inside the streaming loop: only LDS traffic here (the
  // KS partial tiles of each row group added in a fixed order, the row
  // group's M x 16 results parked), so the register ring's load counts stay
  // the same on both sides of the branch; every global store happens after
  // the loop.
  float* park = reinterpret_cast<float*>(lds + LIN_RED + (XLDS ? lin_xs_bytes(M, K) + lin_xsum_bytes(K) : 0));
  auto task_end = [&](int j) {
    if constexpr (KS > 1) {
      red[wave * 64 + lane] = acc;
      lds_barrier();
      if (ks == 0) {
#pragma unroll
        for (int s2 = 1; s2 < KS; ++s2) {
          const f32x4_t o = red[(wave + s2) * 64 + lane];
          acc[0] += o[0]; acc[1] += o[1]; acc[2] += o[2]; acc[3] += o[3];
        }
      }
      lds_barrier();  // the partials are read before the next task writes them
    }
    if (ks == 0) {
      // park[((j * RG + rg) * 16 + l16) * 16 + m]
      float* pp = park + ((j * RG + rg) * 16 + l16) * 16 + 4 * kb;
      *reinterpret_cast<f32x4_t*>(pp) = acc;
    }
    acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };

#pragma unroll
  for (int d = 0; d < DEPTH - 1; ++d) issue(d, d);
  {
    int it = 0, j = 0;
    for (int i0 = 0; i0 < T; i0 += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        const int q = i0 + d;
        issue(q + DEPTH - 1, (d + DEPTH - 1) % DEPTH);
        if (q < T) {
          compute(q, d);
          if (++it == n_it) {
            task_end(j);
            it = 0;
            ++j;
          }
        }
      }
    }
  }
  __syncthreads();

  // Epilogue of every parked result: one thread per (task, row group, row,
  // input row m), 16 consecutive threads over the 16 output rows of a group
  // (RoPE / SwiGLU partners at lane ^ 8, sums of squares over the 16 lanes).
  const int ent = my_tasks * RG * 16 * 16;
  for (int e0 = 0; e0 < ent; e0 += DT) {
    const int e = e0 + tid;
    const bool ok_e = e < ent;
    const int ee = ok_e ? e : ent - 1;
    const int l = ee & 15, m = (ee >> 4) & 15, grp = ee >> 8;  // grp = j * RG + rg
    const int j = grp / RG, rgi = grp - j * RG;
    const int s = ((int)blockIdx.x + Gw * j) * RG + rgi;
    const bool in = 16 * s + l < N;
    const int n = in ? dec_row<EPI>(F_, hd_, s, l) : N;
    float v = park[(grp * 16 + l) * 16 + m];
    float pv = park[(grp * 16 + (l ^ 8)) * 16 + m];
    if constexpr (FMT == FMT_W8) {
      // the W8 row scale applies to the whole dot product (each row its own)
      const int np = dec_row<EPI>(F_, hd_, s, l ^ 8);
      v *= gptr<float>(W.scale)[in ? n : N - 1];
      pv *= gptr<float>(W.scale)[(16 * s + (l ^ 8) < N) ? np : N - 1];
    }
    const bool w_ok = ok_e && m < M && in;
    if constexpr (EPI == DEPI_QKV) {
      if (w_ok) {
        const int hd = hd_, half = hd >> 1;
        const int head = n / hd, i = n - head * hd;
        const long sl = slot_[m];
        const long blk = sl >> 4;
        if (head < hq_ + hkv_) {
          const float2 cs = cs_[(long)pos_[m] * half + (i & (half - 1))];
          const float rv = (i < half) ? v * cs.x - pv * cs.y : v * cs.x + pv * cs.y;
          if (head < hq_) {
            bst16(rsrc(qbuf_ + (long)layer * 16 * hq_ * hd), (uint32_t)((((long)m * hq_ + head) * hd + i) * 2),
                  f2bf(rv));
          } else {
            const long o = ((((blk * L_ + layer) * 2 + 0) * hkv_ + (head - hq_)) * 16 + (sl & 15)) * hd + i;
            st_dev16((uint16_t*)kv_ + o, f2bf(rv));
          }
        } else {
          const int g = head - hq_ - hkv_;
          const long o = ((((blk * L_ + layer) * 2 + 1) * hkv_ + g) * 16) * (long)hd + (long)i * 16 + (sl & 15);
          st_dev16((uint16_t*)kv_ + o, f2bf(v));
        }
      }
    } else if constexpr (EPI == DEPI_SWIGLU) {
      if (w_ok && !(l & 8))
        bst16(rsrc(act_ + (long)layer * 16 * F_), (uint32_t)(((long)m * F_ + n) * 2),
              f2bf(v / (1.0f + expf(-v)) * pv));
    } else {
      float x = 0.f;
      if (w_ok) {
        const float hn = gptr<float>(h_in)[(long)m * d_ + n] + v;
        bstf(rsrc(h_out), (uint32_t)(((long)m * d_ + n) * 4), hn);
        x = hn * hn;
      }
      x += __shfl_xor(x, 1, 64);
      x += __shfl_xor(x, 2, 64);
      x += __shfl_xor(x, 4, 64);
      x += __shfl_xor(x, 8, 64);
      if (l == 0 && ok_e && m < M)
        atomic_add_dev64(ssq_out + (s % slots_) * ssq_out_stride + m,
                         (unsigned long long)rint((double)x * SSQ_SCALE));
    }
  }
  wait_mem();
}

// ---- attention ---------------------------------------------------------------
typedef short __attribute__((ext_vector_type(4))) dbf16x4_t;

ER_DEV long dec_kv_base(long phys, int layer, int L, int kv, int hkv, int head, int hd) {
  return ((((phys * L + layer) * 2 + kv) * hkv + head) * 16) * (long)hd;
}

// Offset (floats) of the split partial record of row r of unit u, KV head g:
// [hd] unnormalized output, running max, running sum.
ER_DEV long dec_partial_off(const DecodeArgs& a, long u, int g, int r) {
  const int grp = a.hq / a.hkv;
  return (((long)u * a.hkv + g) * (long)(grp * a.max_q) + r) * (a.hd + 2);
}

// One (work unit, KV head): the query rows of the unit's item (grp query
// heads x its query positions, up to 64) against its key blocks.  Row groups
// of 16 rows; the 8 / (row groups) waves of a row group take interleaved
// blocks and merge in LDS.
template <int HD>
__device__ __noinline__ void attn_task(const DecodeArgs& a, int layer, int u, int g, char* lds) {
  constexpr int NC = HD / 16;
  constexpr int NQ = HD / 32;
  constexpr int OS = HD + 4;
  float* o_sh = reinterpret_cast<float*>(lds);                       // [DW][16 * OS]
  float* ml_sh = reinterpret_cast<float*>(lds + DW * 16 * OS * 4);   // [DW][2][16]

  const int4* rp = reinterpret_cast<const int4*>(a.unit_rec) + 2 * (long)u;
  const int4 r0 = rp[0], r1 = rp[1];
  const int nu = r0.y >> 16, b0 = r0.z, bps = r0.w;
  const int qc = r1.x, pos0 = r1.y, qrow0 = r1.z, btrow = r1.w;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int l16 = lane & 15, kb = lane >> 4;
  const int grp = a.hq / a.hkv;
  const int R = grp * qc;
  const int rgroups = (R + 15) >> 4;
  const int rgn = rgroups == 1 ? 1 : (rgroups == 2 ? 2 : 4);
  const int s_in = DW / rgn;
  const int rgi = wave / s_in, sin = wave % s_in;
  const int nblk = (pos0 + qc + 15) >> 4;
  const int b1 = min(nblk, b0 + bps);
  const float scale = 1.0f / sqrtf((float)HD);

  const int r_q = rgi * 16 + l16;
  const bool q_ok = rgi < rgroups && r_q < R;
  const int qi_q = q_ok ? r_q / grp : 0;
  const int hh_q = g * grp + (q_ok ? r_q % grp : 0);
  const int qpos_q = pos0 + qi_q;

  bf16x8_t qf[NQ];
  {
    // q of this layer: written once in this forward, by the QKV phase
    const uint16_t* qp = a.qbuf + (long)layer * 16 * a.hq * HD + ((long)(qrow0 + qi_q) * a.hq + hh_q) * HD;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const uint4 v = *(const uint4*)(qp + 32 * i + 8 * kb);
      qf[i] = __builtin_bit_cast(bf16x8_t, q_ok ? v : uint4{0u, 0u, 0u, 0u});
    }
  }

  f32x4_t o[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) o[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const uint16_t* pool = (const uint16_t*)a.kv_pool;
  const int32_t* bt = a.block_table + (long)btrow * a.bt_stride;

  __syncthreads();  // the previous task's LDS reads are done
  if (rgi < rgroups) {
    constexpr int D = 3;
    const int first = b0 + sin;
    const int nb = first < b1 ? (b1 - first + s_in - 1) / s_in : 0;
    const int tl = nb > 0 ? nb - 1 : 0;
    uint4 kq[D][NQ];
    uint2 vq[D][NC];
    auto bid = [&](int t) -> long { return (long)bt[first + s_in * min(t, tl)]; };
    auto fetch = [&](int slot, long phys) {
      const uint16_t* kp = pool + dec_kv_base(phys, layer, a.L, 0, a.hkv, g, HD);
      const uint16_t* vp = pool + dec_kv_base(phys, layer, a.L, 1, a.hkv, g, HD);
#pragma unroll
      for (int i = 0; i < NQ; ++i) kq[slot][i] = *(const uint4*)(kp + l16 * HD + 32 * i + 8 * kb);
#pragma unroll
      for (int c = 0; c < NC; ++c) vq[slot][c] = *(const uint2*)(vp + (16 * c + l16) * 16 + 4 * kb);
    };
    auto process = [&](int slot, int blk) {
      f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NQ; ++i)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kq[slot][i]), qf[i], s, 0, 0, 0);
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
      float corr, psum = 0.f;
      uint32_t pk[2], pl[2];
      if (m_new == -INFINITY) {
        corr = 1.f;
        pk[0] = pk[1] = pl[0] = pl[1] = 0u;
      } else {
        corr = expf(m_run - m_new);
        uint32_t hb[4], lb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = (s[r] == -INFINITY) ? 0.f : expf(s[r] - m_new);
          psum += p;
          hb[r] = f2bf(p);
          lb[r] = f2bf(p - bf2f((uint16_t)hb[r]));
        }
        pk[0] = hb[0] | (hb[1] << 16);
        pk[1] = hb[2] | (hb[3] << 16);
        pl[0] = lb[0] | (lb[1] << 16);
        pl[1] = lb[2] | (lb[3] << 16);
      }
      psum += __shfl_xor(psum, 16, 64);
      psum += __shfl_xor(psum, 32, 64);
      l_run = l_run * corr + psum;
      m_run = m_new;
      float cr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) cr[r] = __shfl(corr, 4 * kb + r, 64);
      const dbf16x4_t pa = __builtin_bit_cast(dbf16x4_t, *(const uint2*)pk);
      const dbf16x4_t pb = __builtin_bit_cast(dbf16x4_t, *(const uint2*)pl);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int r = 0; r < 4; ++r) o[c][r] *= cr[r];
        const dbf16x4_t vf = __builtin_bit_cast(dbf16x4_t, vq[slot][c]);
        o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vf, o[c], 0, 0, 0);
        o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pb, vf, o[c], 0, 0, 0);
      }
    };
    if (nb > 0) {
      fetch(0, bid(0));
      fetch(1, bid(1));
      long idn = bid(2);
      for (int t0 = 0; t0 < nb; t0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
          const int t = t0 + d;
          fetch((d + 2) % D, idn);
          idn = bid(t + 3);
          if (t < nb) process(d, first + s_in * t);
        }
      }
    }
  }

  // merge the s_in waves of each row group (sources in a fixed order); each
  // wave finishes the column tiles c with c % s_in == sin
  float rl[4], rm[4];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) o_sh[wave * 16 * OS + (4 * kb + r) * OS + 16 * c + l16] = o[c][r];
  if (kb == 0) {
    ml_sh[(wave * 2 + 0) * 16 + l16] = m_run;
    ml_sh[(wave * 2 + 1) * 16 + l16] = l_run;
  }
  __syncthreads();
  if (rgi >= rgroups) return;
  const int w0 = rgi * s_in;
  float f[4][DW];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * kb + r;
    float mr[DW], Mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < DW; ++w) {
      mr[w] = w < s_in ? ml_sh[((w0 + w) * 2 + 0) * 16 + row] : -INFINITY;
      Mx = fmaxf(Mx, mr[w]);
    }
    float Ls = 0.f;
#pragma unroll
    for (int w = 0; w < DW; ++w) {
      f[r][w] = (mr[w] == -INFINITY) ? 0.f : expf(mr[w] - Mx);
      if (w < s_in) Ls = fmaf(f[r][w], ml_sh[((w0 + w) * 2 + 1) * 16 + row], Ls);
    }
    rm[r] = Mx;
    rl[r] = Ls;
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (c % s_in != sin) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < DW; ++w)
        if (w < s_in) v = fmaf(f[r][w], o_sh[(w0 + w) * 16 * OS + (4 * kb + r) * OS + 16 * c + l16], v);
      o[c][r] = v;
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int rr = rgi * 16 + 4 * kb + r;
    if (rr >= R) continue;
    const int qi = rr / grp, hh = g * grp + rr % grp;
    if (nu == 1) {
      const float inv = rl[r] > 0.f ? 1.0f / rl[r] : 0.f;
      const Rsrc ro = rsrc(a.abuf + (long)layer * 16 * a.hq * HD);
      const uint32_t ooff = (uint32_t)(((long)(qrow0 + qi) * a.hq + hh) * HD * 2);
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (c % s_in == sin) bst16(ro, ooff + (uint32_t)(16 * c + l16) * 2, f2bf(o[c][r] * inv));
    } else {
      const Rsrc rp = rsrc(a.apart);
      const uint32_t poff = (uint32_t)(dec_partial_off(a, u, g, rr) * 4);
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (c % s_in == sin) bstf(rp, poff + (uint32_t)(16 * c + l16) * 4, o[c][r]);
      if (sin == 0 && l16 == 0) {
        bstf(rp, poff + HD * 4, rm[r]);
        bstf(rp, poff + (HD + 1) * 4, rl[r]);
      }
    }
  }
}

template <int HD>
ER_DEV void attn_phase(const DecodeArgs& a, int layer, char* lds) {
  const int tasks = a.n_units * a.hkv;
  for (int t = blockIdx.x; t < tasks; t += gridDim.x) attn_task<HD>(a, layer, t / a.hkv, t % a.hkv, lds);
  wait_mem();
}

// Merge the units of split items: one wave per (split item, KV head, row);
// lanes first take units (maxima and weights exp(m_s - M) in chunks of 64),
// then output elements (HD / 64 per lane), adding the units in order.
template <int HD>
__device__ __noinline__ void comb_phase(const DecodeArgs& a, int layer) {
  constexpr int PE = HD / 64;
  const int grp = a.hq / a.hkv;
  const int Rmax = grp * a.max_q;
  const int lane = threadIdx.x & 63;
  const long tasks = (long)a.n_split * a.hkv * Rmax;
  const long stride_u = (long)a.hkv * Rmax * (HD + 2);
  for (long t = (long)blockIdx.x * DW + wave_id(); t < tasks; t += (long)gridDim.x * DW) {
    const int si = (int)(t / ((long)a.hkv * Rmax));
    const int g = (int)((t / Rmax) % a.hkv);
    const int r = (int)(t % Rmax);
    const int item = a.split_items[si];
    const int qc = a.item_q_count[item];
    if (r >= grp * qc) continue;
    const int u0 = a.unit_start[item];
    const int nu = a.unit_start[item + 1] - u0;
    const Rsrc rp = rsrc(a.apart);
    const uint32_t base = (uint32_t)(dec_partial_off(a, u0, g, r) * 4);
    const uint32_t su = (uint32_t)(stride_u * 4);
    float mx = -INFINITY;
    for (int s = lane; s < nu; s += 64) mx = fmaxf(mx, bldf(rp, base + (uint32_t)s * su + HD * 4));
    mx = wave_max(mx);
    float num[PE];
#pragma unroll
    for (int e = 0; e < PE; ++e) num[e] = 0.f;
    float den = 0.f;
    for (int s0 = 0; s0 < nu; s0 += 64) {
      const int s = s0 + lane;
      float w = 0.f;
      if (s < nu) {
        const float ms = bldf(rp, base + (uint32_t)s * su + HD * 4);
        w = (ms == -INFINITY) ? 0.f : expf(ms - mx);
        den = fmaf(w, bldf(rp, base + (uint32_t)s * su + (HD + 1) * 4), den);
      }
      const int cnt = min(64, nu - s0);
      // eight units' elements in flight at once, added in unit order
      for (int k0 = 0; k0 < cnt; k0 += 8) {
        float v[8][PE];
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
          for (int e = 0; e < PE; ++e)
            v[q][e] = bldf(rp, base + (uint32_t)(s0 + min(k0 + q, cnt - 1)) * su + (uint32_t)(lane + 64 * e) * 4);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float wk = __shfl(w, min(k0 + q, 63), 64);
          if (k0 + q < cnt) {
#pragma unroll
            for (int e = 0; e < PE; ++e) num[e] = fmaf(wk, v[q][e], num[e]);
          }
        }
      }
    }
    den = wave_sum(den);
    const int qi = r / grp, hh = g * grp + (r - qi * grp);
    const Rsrc ro = rsrc(a.abuf + (long)layer * 16 * a.hq * HD);
    const uint32_t ooff = (uint32_t)(((long)(a.item_q_row0[item] + qi) * a.hq + hh) * HD * 2);
#pragma unroll
    for (int e = 0; e < PE; ++e) bst16(ro, ooff + (uint32_t)(lane + 64 * e) * 2, f2bf(den > 0.f ? num[e] / den : 0.f));
  }
  wait_mem();
}

// ---- embedding -----------------------------------------------------------------
// h[m] = embed[token m] (one work-group per row) with its fixed-point sum of
// squares; every other group clears the sums of squares the later phases
// accumulate into.
ER_DEV void embed_phase(const DecodeArgs& a, char* lds) {
  float* red = reinterpret_cast<float*>(lds);
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int M = a.M, d = a.d;
  {
    // sums of squares: every slot of every phase (row 0..15), then the final ones in the
    // lm_head's layout; slot 0 of phase 0 is written below
    const long nz = (long)(2 * a.L) * a.ssq_slots * 16;
    for (long e = (long)blockIdx.x * DT + tid; e < nz; e += (long)gridDim.x * DT)
      if (e >= 16 || e % 16 >= M) st_dev64(a.ssq + e, 0ull);
    for (long e = (long)blockIdx.x * DT + tid; e < (long)a.ssq_slots * M; e += (long)gridDim.x * DT)
      st_dev64(a.ssq_out + (e / M) * a.ssq_stride + e % M, 0ull);
  }
  const Rsrc rh = rsrc(a.hbuf);
  for (int m = blockIdx.x; m < M; m += gridDim.x) {
    const long tok = a.tokens[(long)m * a.tok_stride];
    const uint16_t* er = (const uint16_t*)a.embed + tok * d;
    float sq = 0.f;
    for (int k = tid * 4; k < d; k += DT * 4) {
      const uint2 v = *(const uint2*)(er + k);
      const float e0 = bf_lo(v.x), e1 = bf_hi(v.x), e2 = bf_lo(v.y), e3 = bf_hi(v.y);
      bst128(rh, (uint32_t)(((long)m * d + k) * 4),
             uint4{__float_as_uint(e0), __float_as_uint(e1), __float_as_uint(e2), __float_as_uint(e3)});
      sq = fmaf(e0, e0, sq);
      sq = fmaf(e1, e1, sq);
      sq = fmaf(e2, e2, sq);
      sq = fmaf(e3, e3, sq);
    }
    sq = wave_sum(sq);
    __syncthreads();
    if (lane == 0) red[wave] = sq;
    __syncthreads();
    if (tid == 0) {
      float t = 0.f;
      for (int w = 0; w < DW; ++w) t += red[w];
      st_dev64(a.ssq + m, (unsigned long long)rint((double)t * SSQ_SCALE));
    }
  }
  wait_mem();
}

// Linear phase with the K split chosen at run time.
template <int FMT, int EPI, bool XLDS>
ER_DEV void lin_phase_ks(int ks, const DecodeArgs& a, const LinearW& W, int layer, const void* gnorm,
                         const float* h_in, const unsigned long long* ssq_in, const uint16_t* x_in, float* h_out,
                         unsigned long long* ssq_out, long ssq_out_stride, char* lds) {
  // every wave of a row group must own at least one chunk (the host keeps ks <= K / 128)
  if (ks == 8) lin_phase<FMT, EPI, 8, XLDS>(a, W, layer, gnorm, h_in, ssq_in, x_in, h_out, ssq_out, ssq_out_stride, lds);
  else if (ks == 4) lin_phase<FMT, EPI, 4, XLDS>(a, W, layer, gnorm, h_in, ssq_in, x_in, h_out, ssq_out, ssq_out_stride, lds);
  else lin_phase<FMT, EPI, 2, XLDS>(a, W, layer, gnorm, h_in, ssq_in, x_in, h_out, ssq_out, ssq_out_stride, lds);
}

template <int FMT, int HD>
__global__ __launch_bounds__(DT) void k_decode(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ unsigned s_gen;
  if (threadIdx.x == 0) s_gen = ld_dev32(a.bar + BAR_GEN);
  __syncthreads();
  unsigned gen = s_gen;
  int nbar = 0;
  if (a.trace && threadIdx.x == 0) a.trace[(long)a.trace_max * 2 * gridDim.x + blockIdx.x] = __builtin_amdgcn_s_memrealtime();

  embed_phase(a, lds);
  if (!grid_barrier(a, gen, nbar)) return;
  const long hstride = 16L * a.d;                 // one phase's rows of h
  const long sstride = (long)a.ssq_slots * 16;    // one phase's sums of squares
  for (int l = 0; l < a.L; ++l) {
    const DecLayerW& w = a.layers[l];
    const float* h0 = a.hbuf + (2 * l) * hstride;        // h entering the layer
    float* h1 = a.hbuf + (2 * l + 1) * hstride;          // after the attention block
    const unsigned long long* s0 = a.ssq + (2 * l) * sstride;
    unsigned long long* s1 = a.ssq + (2 * l + 1) * sstride;
    lin_phase_ks<FMT, DEPI_QKV, true>(a.ks[0], a, w.qkv, l, w.attn_norm, h0, s0, nullptr, nullptr, nullptr, 0, lds);
    if (!grid_barrier(a, gen, nbar)) return;
    attn_phase<HD>(a, l, lds);
    if (!grid_barrier(a, gen, nbar)) return;
    if (a.n_split > 0) {
      comb_phase<HD>(a, l);
      if (!grid_barrier(a, gen, nbar)) return;
    }
    lin_phase_ks<FMT, DEPI_RESID, false>(a.ks[1], a, w.o, l, nullptr, h0, nullptr, a.abuf + (long)l * 16 * a.hq * a.hd, h1,
                                         s1, 16, lds);
    if (!grid_barrier(a, gen, nbar)) return;
    lin_phase_ks<FMT, DEPI_SWIGLU, true>(a.ks[2], a, w.gu, l, w.mlp_norm, h1, s1, nullptr, nullptr, nullptr, 0, lds);
    if (!grid_barrier(a, gen, nbar)) return;
    const bool lastl = l + 1 == a.L;
    float* h2 = lastl ? a.h_final : a.hbuf + (2 * l + 2) * hstride;
    unsigned long long* s2 = lastl ? a.ssq_out : a.ssq + (2 * l + 2) * sstride;
    lin_phase_ks<FMT, DEPI_RESID, false>(a.ks[3], a, w.down, l, nullptr, h1, nullptr, a.act + (long)l * 16 * a.F, h2, s2,
                                         lastl ? a.ssq_stride : 16, lds);
    if (!lastl && !grid_barrier(a, gen, nbar)) return;
  }
}

// ---- host ------------------------------------------------------------------------
// Dynamic LDS of a launch: the largest of the attention merge area and a
// normalizing linear phase's x' (M rows of the d_model-wide input).
size_t decode_lds_bytes(int hd, int M, int d, int n_max, int nwg) {
  const size_t attn = (size_t)DW * 16 * (hd + 4) * 4 + (size_t)DW * 2 * 16 * 4;
  // parked results: one 16 x 16 fp32 block per row group of 16 output rows a work-group owns
  const size_t park = (size_t)((n_max / 16 + nwg - 1) / nwg + DW) * 16 * 16 * 4;
  const size_t lin = (size_t)LIN_RED + (size_t)M * (d + 8) * 2 + (size_t)(d / 128) * 16 * 4 + park;
  return std::max(attn, lin);
}
// Dynamic LDS ceiling: 160 KB per compute unit, less room for the kernel's
// static shared variables.
constexpr size_t kDecodeLdsMax = 150 * 1024;

// Waves splitting K in a projection [N, K] (tasks of 16 * 8 / ks rows): the
// choice among 8, 4 and 2 (at most K / 128) that minimizes tasks per
// work-group times chunks per wave and task; 0 when K has fewer than two
// 128-wide chunks.
int decode_ksplit(int N, int K, int nwg, int fmt) {
  (void)fmt;
  const int nc = K / 128;
  int best = 0;
  long best_cost = -1;
  for (int ks : {8, 4, 2}) {
    if (nc < ks) continue;
    const long ntask = (N + 16 * (8 / ks) - 1) / (16 * (8 / ks));
    const long cost = ((ntask + nwg - 1) / nwg) * ((nc + ks - 1) / ks);
    if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = ks; }
  }
  return best;
}

template <int FMT, int HD>
static int grid_t() {
  static int cached = -1;
  if (cached < 0) {
    cached = 0;
    const size_t lds = kDecodeLdsMax;
    int per_cu = 0, dev = 0, coop = 0, cus = 0;
    if (hipFuncSetAttribute((const void*)k_decode<FMT, HD>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) !=
            hipSuccess ||
        hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_decode<FMT, HD>, DT, lds) != hipSuccess) {
      (void)hipGetLastError();
      return 0;
    }
    if (coop && per_cu >= 1) cached = cus;  // one work-group per compute unit, all resident
  }
  return cached;
}

int decode_grid(int fmt, int hd) {
  if (hd != 128) return 0;
  switch (fmt) {
    case FMT_BF16: return grid_t<FMT_BF16, 128>();
    case FMT_W8: return grid_t<FMT_W8, 128>();
    case FMT_W4: return grid_t<FMT_W4, 128>();
  }
  return 0;
}

template <int FMT, int HD>
static int launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  const int G = grid_t<FMT, HD>();
  if (G <= 0 || a.n_wg != G) return -1;
  DecodeArgs b = a;
  void* args[] = {&b};
  const size_t lds = decode_lds_bytes(HD, a.M, a.d, std::max({(a.hq + 2 * a.hkv) * a.hd, a.d, 2 * a.F}), G);
  if (lds > kDecodeLdsMax) return -1;
  if (hipLaunchCooperativeKernel((const void*)k_decode<FMT, HD>, dim3((unsigned)G), dim3(DT), args, lds, st) !=
      hipSuccess)
    return -3;
  return 0;
}

int launch_decode(const DecodeArgs& a, int fmt, hipStream_t st) {
  if (a.M < 1 || a.M > 16 || a.hd != 128 || a.hq % a.hkv) return -1;
  if ((a.hq / a.hkv) * a.max_q > 64) return -1;
  if (a.d % 128 || a.F % 128 || (a.hq * a.hd) % 128) return -1;
  const int nck[4] = {a.d / 128, a.hq * a.hd / 128, a.d / 128, a.F / 128};
  for (int i = 0; i < 4; ++i)
    if ((a.ks[i] != 8 && a.ks[i] != 4 && a.ks[i] != 2) || a.ks[i] > nck[i]) return -1;
  if (a.ssq_slots < 1 || a.ssq_slots > 16) return -1;
  switch (fmt) {
    case FMT_BF16: return launch_decode_t<FMT_BF16, 128>(a, st);
    case FMT_W8: return launch_decode_t<FMT_W8, 128>(a, st);
    case FMT_W4: return launch_decode_t<FMT_W4, 128>(a, st);
  }
  return -1;
}

}  // namespace er
