// Linear layers of the target (bf16/fp32) and of the quantized self-drafter
// (W8 per-channel, W4 group-128): y[m, n] = sum_k x[m, k] * W[n, k].
//
// Two paths:
//  * k_linear_valu: one wavefront per output row, lanes stride over K, fp32
//    FMAs.  Used for fp32 models and for shapes the MFMA path does not take.
//  * k_linear_mfma: bf16 activations through LDS, weights streamed from HBM
//    straight into registers and fed to v_mfma_f32_16x16x32_bf16.  Quantized
//    codes are turned into bf16 with exponent-field tricks (no per-element
//    int->float conversion for W4), and the zero points are folded out per
//    128-wide K chunk with row sums of x.  Narrow projections split K across
//    the 8 waves of a work-group and reduce in LDS (deterministic, and no
//    device-scope fence: on gfx950 one costs an L2 write-back per group);
//    the block index is remapped so that the m-tiles sharing a weight tile
//    land on the same XCD (and its L2).
//
// The drafter kernels are the dequant-fused GEMV/skinny-GEMM of the
// EfficientRollout page ("关键模块" item 1: W4/W8 drafter from the target's own
// weights); the verify kernels are the target's linears at M = B * (gamma+1).

#include <algorithm>
#include <cstdio>

#include "common.h"
#include "kernels.h"
#include "linear_dev.h"

namespace er {

// ----------------------------------------------------------------------------
// Dequantized weight element (kernel-order W4 layout), fp32.
// ----------------------------------------------------------------------------
template <int FMT>
ER_DEV float w_elem(const void* __restrict__ w, const void* __restrict__ s, const void* __restrict__ z,
                    long n, long k, long K, long N) {
  if constexpr (FMT == FMT_F32) {
    return ((const float*)w)[n * K + k];
  } else if constexpr (FMT == FMT_BF16) {
    return bf2f(((const uint16_t*)w)[n * K + k]);
  } else if constexpr (FMT == FMT_W8) {
    return (float)((const int8_t*)w)[n * K + k] * ((const float*)s)[n];
  } else {
    const uint32_t word = ((const uint32_t*)w)[(w4_piece(n, k >> 7, N, K) + ((k & 127) >> 1)) >> 2];
    const int j = (int)(k & 7);
    const int bit = (j & 1) ? 16 + 4 * (j >> 1) : 4 * (j >> 1);
    const int q = (int)((word >> bit) & 15u);
    const long G = K >> 7;
    const float sc = bf2f(((const uint16_t*)s)[n * G + (k >> 7)]);
    const int zz = ((const uint8_t*)z)[n * G + (k >> 7)];
    return (float)(q - zz) * sc;
  }
}

template <int FMT, bool XBF>
__global__ __launch_bounds__(256) void k_linear_valu(const void* __restrict__ xv, int ldx, int M,
                                                     const void* __restrict__ w, const void* __restrict__ s,
                                                     const void* __restrict__ z, int N, int K,
                                                     void* __restrict__ yv, int ldy, int epi) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = blockIdx.x * 4 + wave;
  const int m0 = blockIdx.y * 4;
  if (n >= N) return;
  typedef typename Act<XBF>::T XT;
  const XT* x = (const XT*)xv;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k = lane * 4; k < K; k += 256) {
    float wv[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) wv[t] = w_elem<FMT>(w, s, z, n, k + t, K, N);
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      if (m0 + mm < M) {
        const long base = (long)(m0 + mm) * ldx + k;
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[mm] = fmaf(Act<XBF>::ld(x, base + t), wv[t], acc[mm]);
      }
    }
  }
#pragma unroll
  for (int mm = 0; mm < 4; ++mm) acc[mm] = wave_sum(acc[mm]);
  if (lane == 0) {
    for (int mm = 0; mm < 4 && m0 + mm < M; ++mm) {
      const long o = (long)(m0 + mm) * ldy + n;
      if (epi == EPI_RESID) ((float*)yv)[o] += acc[mm];
      else if (epi == EPI_ACT && XBF) ((uint16_t*)yv)[o] = (uint16_t)f2bf(acc[mm]);
      else ((float*)yv)[o] = acc[mm];
    }
  }
}

// ----------------------------------------------------------------------------
// MFMA linears (bf16 activations) with fused prologue / epilogue.
// ----------------------------------------------------------------------------
template <int FMT> struct WRegs { static constexpr int n = (FMT == FMT_BF16) ? 4 : (FMT == FMT_W8 ? 2 : 1); };

// Physical weight row of logical row 16*s + l16.  Paired epilogues need the
// two operands of each pair in lanes l16 and l16 ^ 8 of one 16-row subtile:
// SwiGLU pairs gate row f with up row F + f; RoPE pairs rows i and i + hd/2
// of a head.  Other epilogues use the identity.
ER_DEV int phys_row(const LinArgs& a, int s, int l16) {
  if (a.epi == EPI_SWIGLU) {
    const int f = s * 8 + (l16 & 7);
    return (l16 & 8) ? a.F + f : f;
  }
  if (a.epi == EPI_QKV) {
    const int per_head = a.hd >> 4;  // subtiles per head
    const int h = s / per_head, pb = (s - h * per_head) * 8;
    return h * a.hd + pb + (l16 & 7) + ((l16 & 8) ? (a.hd >> 1) : 0);
  }
  return 16 * s + l16;
}

ER_DEV int ssq_nslots(const LinArgs& a) { return a.ssq_slots > 1 ? a.ssq_slots : 1; }

constexpr int kMaxSsqSlots = 16;

ER_DEV float rstd_of(const LinArgs& a, long hrow) {
  // all slots' loads in flight at once (a rolled loop would wait out one
  // load latency per slot)
  const int ns = ssq_nslots(a);
  unsigned long long v[kMaxSsqSlots];
#pragma unroll
  for (int i = 0; i < kMaxSsqSlots; ++i) v[i] = i < ns ? a.ssq_in[(long)i * a.ssq_stride + hrow] : 0ull;
  unsigned long long t = 0;
#pragma unroll
  for (int i = 0; i < kMaxSsqSlots; ++i) t += v[i];
  const double ss = (double)t / SSQ_SCALE;
  return 1.0f / sqrtf((float)ss / (float)a.W.K + a.eps);
}

// 8 consecutive x' values (bf16) of row m at column k0.
ER_DEV uint4 load_x8(const LinArgs& a, long hrow, float rs, long k0) {
  if (!a.xnorm) return *(const uint4*)((const uint16_t*)a.x + hrow * a.ldx + k0);
  const float* hp = (const float*)a.x + hrow * a.ldx + k0;
  const float4 h0 = *(const float4*)hp, h1 = *(const float4*)(hp + 4);
  const uint4 g = *(const uint4*)((const uint16_t*)a.gnorm + k0);
  uint4 o;
  o.x = f2bf(h0.x * rs * bf_lo(g.x)) | (f2bf(h0.y * rs * bf_hi(g.x)) << 16);
  o.y = f2bf(h0.z * rs * bf_lo(g.y)) | (f2bf(h0.w * rs * bf_hi(g.y)) << 16);
  o.z = f2bf(h1.x * rs * bf_lo(g.z)) | (f2bf(h1.y * rs * bf_hi(g.z)) << 16);
  o.w = f2bf(h1.z * rs * bf_lo(g.w)) | (f2bf(h1.w * rs * bf_hi(g.w)) << 16);
  return o;
}

// Epilogue for the value v of (row m, physical column n); partner = the value
// of lane l16 ^ 8 (the other half of a SwiGLU / RoPE pair).  `write` is false
// for lanes whose m or n is out of range (they still provide partners).
ER_DEV void epilogue(const LinArgs& a, int m, int n, float v, float partner, bool write, int l16) {
  if (!write) return;
  if (a.epi == EPI_SWIGLU) {
    if (l16 & 8) return;  // gate lane writes silu(g) * u
    const float r = v / (1.0f + expf(-v)) * partner;
    ((uint16_t*)a.y)[(long)m * a.ldy + n] = (uint16_t)f2bf(r);
    return;
  }
  if (a.epi == EPI_QKV) {
    const int hd = a.hd, half = hd >> 1;
    const int head = n / hd, i = n - head * hd;
    const long sl = a.slot[m];
    if (head < a.hq + a.hkv) {
      const int ip = i & (half - 1);
      const float2 c = a.cs[(long)a.pos[m] * half + ip];
      const float r = (i < half) ? v * c.x - partner * c.y : v * c.x + partner * c.y;
      if (head < a.hq) {
        ((uint16_t*)a.qout)[((long)m * a.hq + head) * hd + i] = (uint16_t)f2bf(r);
      } else {
        const long blk = sl >> 4;
        const long o = ((((blk * a.n_layers + a.layer) * 2 + 0) * a.hkv + (head - a.hq)) * 16 + (sl & 15)) * hd + i;
        ((uint16_t*)a.kv_pool)[o] = (uint16_t)f2bf(r);
      }
    } else {
      const long blk = sl >> 4;
      const int g = head - a.hq - a.hkv;
      const long o = ((((blk * a.n_layers + a.layer) * 2 + 1) * a.hkv + g) * 16) * (long)hd + (long)i * 16 + (sl & 15);
      ((uint16_t*)a.kv_pool)[o] = (uint16_t)f2bf(v);
    }
    return;
  }
  const long o = (long)m * a.ldy + n;
  if (a.epi == EPI_RESID) ((float*)a.y)[o] += v;
  else if (a.epi == EPI_ACT && a.act_bf16) ((uint16_t*)a.y)[o] = (uint16_t)f2bf(v);
  else ((float*)a.y)[o] = v;
}

// Out-of-line epilogue for kernels with large accumulator tiles: keeps the
// fully unrolled store loop small enough that the tile stays in registers.
__device__ __noinline__ void epilogue_call(const LinArgs& a, int m, int n, float v, float partner, bool write, int l16) {
  epilogue(a, m, n, v, partner, write, l16);
}

// Sum of squares of the updated residual rows: `sq` is this lane's
// contribution to row m; the 16 lanes of each lane group (lane / 16) are
// summed and the group's lane `lead` adds the total (callers whose row spans
// several groups reduce across them first and pass one leader).
// This work-group's slot of row m's running sum of squares.
ER_DEV unsigned long long* ssq_slot(const LinArgs& a, int m) {
  return a.ssq_acc + (long)(blockIdx.x % ssq_nslots(a)) * a.ssq_stride + m;
}

// Clear rows [0, M) of ssq_zero in every slot.
ER_DEV void ssq_clear(const LinArgs& a, int tid, int nt) {
  const int M = a.M, tot = ssq_nslots(a) * M;
  for (int e = tid; e < tot; e += nt) a.ssq_zero[(long)(e / M) * a.ssq_stride + e % M] = 0ull;
}

ER_DEV void ssq_add(const LinArgs& a, int m, float sq, bool lead, bool mok) {
  sq += __shfl_xor(sq, 1, 64);
  sq += __shfl_xor(sq, 2, 64);
  sq += __shfl_xor(sq, 4, 64);
  sq += __shfl_xor(sq, 8, 64);
  if (lead && mok) atomicAdd(ssq_slot(a, m), (unsigned long long)rint((double)sq * SSQ_SCALE));
}

// ----------------------------------------------------------------------------
// Skinny MFMA linear (M <= 32).  One work-group = 8 waves over
// R = 16 * NR * (8 / KS) output rows and one m-tile of MT rows of x.  Wave w
// owns the 16*NR rows starting at 16 * NR * (w / KS) and the K chunks
// c = w % KS, w % KS + KS, ... (128 inputs per chunk); the KS partial tiles
// of a row group are summed in LDS in a fixed order, so the result is
// deterministic and no device-scope fence is needed (on gfx950 one costs an
// L2 write-back per work-group).  Weights and x fragments are loaded straight
// into registers (x is L1/L2 resident at these M; rows >= M are not loaded);
// each x fragment feeds NR weight subtiles, and the next chunk is in flight
// while the current one is multiplied.  The block index is remapped so that
// the m-tiles sharing a weight tile land on the same XCD (and its L2).
// ----------------------------------------------------------------------------
template <int FMT, int MT, int NR, int KS>
__global__ __launch_bounds__(512) void k_linear_mfma(LinArgs a, int mtiles) {
  constexpr int MI = MT / 16;
  constexpr int RG = 8 / KS;
  constexpr int R = 16 * NR * RG;
  constexpr int WR = WRegs<FMT>::n;
  __shared__ f32x4_t red[(KS > 1) ? 8 * MI * NR * 64 : 1];

  const int b = blockIdx.x, nwg = gridDim.x;
  const int xcd = b & 7, loc = b >> 3, per = nwg >> 3, rem = nwg & 7;
  const int L = (xcd < rem) ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
  const int mt = L % mtiles;
  const int nt = L / mtiles;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int rg = wave / KS, ks = wave % KS;
  const int kb = lane >> 4, l16 = lane & 15;
  const int m0 = mt * MT;
  const int M = a.M, N = a.W.N, K = a.W.K;
  const int nchunks = K >> 7;
  const long G = K >> 7;
  const void* __restrict__ wv = a.W.w;
  const void* __restrict__ sv = a.W.scale;
  const void* __restrict__ zv = a.W.zero;

  if (b == 0 && a.ssq_zero)
    ssq_clear(a, tid, 512);

  int n_lane[NR];
  long nrow[NR];
#pragma unroll
  for (int ni = 0; ni < NR; ++ni) {
    const int s = (nt * RG + rg) * NR + ni;  // logical 16-row subtile
    const bool in = 16 * s + l16 < N;
    n_lane[ni] = in ? phys_row(a, s, l16) : N;
    nrow[ni] = in ? n_lane[ni] : N - 1;      // clamp loads; results past N are dropped
  }

  f32x4_t acc[MI][NR];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NR; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  long xrow[MI];
  bool xok[MI];
  float xrs[MI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int m = m0 + mi * 16 + l16;
    xok[mi] = m < M;
    xrow[mi] = xok[mi] ? (a.xrow ? a.xrow[m] : m) : 0;
    xrs[mi] = (a.xnorm && xok[mi]) ? rstd_of(a, xrow[mi]) : 1.f;
  }

  uint4 wreg[2][NR][WR];
  uint4 xreg[2][MI][4];
  float wsc[2][NR], wz[2][NR];

  auto load = [&](int c, int buf) {
#pragma unroll
    for (int ni = 0; ni < NR; ++ni) {
      if constexpr (FMT == FMT_BF16) {
        const uint16_t* p = (const uint16_t*)wv + nrow[ni] * K + (long)c * 128;
#pragma unroll
        for (int i = 0; i < 4; ++i) wreg[buf][ni][i] = *(const uint4*)(p + kcol<FMT>(i, kb));
      } else if constexpr (FMT == FMT_W8) {
        const int8_t* p = (const int8_t*)wv + nrow[ni] * K + (long)c * 128;
#pragma unroll
        for (int h = 0; h < 2; ++h) wreg[buf][ni][h] = *(const uint4*)(p + 64 * h + 16 * kb);
      } else {
        const uint8_t* p = (const uint8_t*)wv + w4_piece(nrow[ni], c, N, K);
        wreg[buf][ni][0] = *(const uint4*)(p + 16 * kb);
        wsc[buf][ni] = bf2f(((const uint16_t*)sv)[nrow[ni] * G + c]);
        wz[buf][ni] = 128.0f + (float)((const uint8_t*)zv)[nrow[ni] * G + c];
      }
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint4 v = uint4{0u, 0u, 0u, 0u};
        if (xok[mi]) v = load_x8(a, xrow[mi], xrs[mi], (long)c * 128 + kcol<FMT>(i, kb));
        xreg[buf][mi][i] = v;
      }
    }
  };

  auto compute = [&](int buf) {
    f32x4_t accg[MI][NR];
    if constexpr (FMT != FMT_BF16) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NR; ++ni) accg[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x8_t bw[NR];
#pragma unroll
      for (int ni = 0; ni < NR; ++ni) {
        if constexpr (FMT == FMT_BF16) {
          bw[ni] = __builtin_bit_cast(bf16x8_t, wreg[buf][ni][i]);
        } else if constexpr (FMT == FMT_W8) {
          const uint4 v = wreg[buf][ni][i >> 1];
          bw[ni] = (i & 1) ? w8_to_bf16(v.z, v.w) : w8_to_bf16(v.x, v.y);
        } else {
          const uint4 v = wreg[buf][ni][0];
          const uint32_t word = (i == 0) ? v.x : (i == 1) ? v.y : (i == 2) ? v.z : v.w;
          bw[ni] = w4_to_bf16(word);
        }
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const bf16x8_t xa = __builtin_bit_cast(bf16x8_t, xreg[buf][mi][i]);
#pragma unroll
        for (int ni = 0; ni < NR; ++ni) {
          if constexpr (FMT == FMT_BF16)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bw[ni], acc[mi][ni], 0, 0, 0);
          else
            accg[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bw[ni], accg[mi][ni], 0, 0, 0);
        }
      }
    }
    if constexpr (FMT != FMT_BF16) {
      // zero-point / offset correction needs the chunk's row sums of x':
      // this lane holds 32 of row l16's 128 values; 4 lanes (kb) hold the rest.
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        float sm = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 v = xreg[buf][mi][i];
          sm += bf_lo(v.x) + bf_hi(v.x) + bf_lo(v.y) + bf_hi(v.y) + bf_lo(v.z) + bf_hi(v.z) + bf_lo(v.w) + bf_hi(v.w);
        }
        sm += __shfl_xor(sm, 16, 64);
        sm += __shfl_xor(sm, 32, 64);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float xsm = __shfl(sm, 4 * kb + r, 64);  // row 4*kb + r of this m-subtile
#pragma unroll
          for (int ni = 0; ni < NR; ++ni) {
            if constexpr (FMT == FMT_W8)
              acc[mi][ni][r] += accg[mi][ni][r] - 128.0f * xsm;
            else
              acc[mi][ni][r] = fmaf(wsc[buf][ni], fmaf(-wz[buf][ni], xsm, accg[mi][ni][r]), acc[mi][ni][r]);
          }
        }
      }
    }
  };

  if (ks < nchunks) {
    load(ks, 0);
    int buf = 0;
    for (int c = ks; c < nchunks; c += KS) {
      const bool nxt = c + KS < nchunks;
      if (nxt) { if (buf == 0) load(c + KS, 1); else load(c + KS, 0); }
      if (buf == 0) compute(0); else compute(1);
      buf ^= 1;
    }
  }

  if constexpr (FMT == FMT_W8) {
#pragma unroll
    for (int ni = 0; ni < NR; ++ni) {
      const float sc = ((const float*)sv)[nrow[ni]];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mi][ni][r] *= sc;
    }
  }

  if constexpr (KS > 1) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NR; ++ni) red[((wave * MI + mi) * NR + ni) * 64 + lane] = acc[mi][ni];
    __syncthreads();
    if (ks != 0) return;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NR; ++ni) {
        f32x4_t v = red[((wave * MI + mi) * NR + ni) * 64 + lane];
#pragma unroll
        for (int s = 1; s < KS; ++s) {
          const f32x4_t o = red[(((wave + s) * MI + mi) * NR + ni) * 64 + lane];
          v[0] += o[0]; v[1] += o[1]; v[2] += o[2]; v[3] += o[3];
        }
        acc[mi][ni] = v;
      }
  }

  const bool want_ssq = a.epi == EPI_RESID && a.ssq_acc;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + mi * 16 + 4 * kb + r;
      const bool mok = m < M;
      float sq = 0.f;
#pragma unroll
      for (int ni = 0; ni < NR; ++ni) {
        const float v = acc[mi][ni][r];
        const float partner = __shfl_xor(v, 8, 64);
        const bool ok = mok && n_lane[ni] < N;
        epilogue(a, m, n_lane[ni], v, partner, ok, l16);
        if (want_ssq && ok) {
          const float hn = ((const float*)a.y)[(long)m * a.ldy + n_lane[ni]];
          sq = fmaf(hn, hn, sq);
        }
      }
      if (want_ssq) ssq_add(a, m, sq, l16 == 0, mok);
    }
}

// ----------------------------------------------------------------------------
// Tiled bf16 GEMM for M > 32 (verify at moderate batch, AR at large batch,
// prefill): 128x128 output tile per work-group (4 waves, 64x64 each, 16x16x32
// MFMA), both operands staged through double-buffered LDS in 64-wide K steps,
// next step's global loads in flight during the current MFMAs.  Narrow
// outputs split K over work-groups; partial tiles then go to a workspace and
// k_splitk_reduce sums them in a fixed order and applies the epilogue.
// ----------------------------------------------------------------------------
constexpr int GB_M = 128, GB_N = 128, GB_K = 64, GB_LD = GB_K + 8;
constexpr size_t kSkinnyLdsMax = (size_t)160 << 10;

__global__ __launch_bounds__(256) void k_gemm_bf16(LinArgs a, float* __restrict__ part, int nsplit,
                                                   int ksteps_per_split, int mtiles) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * GB_M * GB_LD + 2 * GB_N * GB_LD];
  uint16_t (*As)[GB_M * GB_LD] = reinterpret_cast<uint16_t (*)[GB_M * GB_LD]>(smem);
  uint16_t (*Bs)[GB_N * GB_LD] = reinterpret_cast<uint16_t (*)[GB_N * GB_LD]>(smem + 2 * GB_M * GB_LD);
  __shared__ float rs_sh[GB_M];
  const int b = blockIdx.x, nwg = gridDim.x;
  const int xcd = b & 7, loc = b >> 3, per = nwg >> 3, rem = nwg & 7;
  const int L = (xcd < rem) ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
  const int mt = L % mtiles;
  const int t2 = L / mtiles;
  const int sp = t2 % nsplit;
  const int nt = t2 / nsplit;
  const int M = a.M, N = a.W.N, K = a.W.K;
  const int m0 = mt * GB_M, n0 = nt * GB_N;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int kb = lane >> 4, l16 = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;
  const int nsteps = K / GB_K;
  const int s0 = sp * ksteps_per_split;
  const int s1 = min(nsteps, s0 + ksteps_per_split);
  const uint16_t* __restrict__ W = (const uint16_t*)a.W.w;

  if (b == 0 && a.ssq_zero && nsplit == 1)
    ssq_clear(a, tid, 256);
  if (tid < GB_M) {
    const int m = m0 + tid;
    rs_sh[tid] = (a.xnorm && m < M) ? rstd_of(a, a.xrow ? a.xrow[m] : m) : 1.f;
  }
  __syncthreads();

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // weight tile rows: 16-row subtiles s = n0/16 + row/16 in the epilogue's row order
  long wrow[4];
  bool wok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (tid + 256 * i) >> 3;
    const int s = (n0 >> 4) + (row >> 4);
    wok[i] = n0 + row < N;
    wrow[i] = wok[i] ? phys_row(a, s, row & 15) : 0;
  }
  uint4 ra[4], rb[4];
  auto gload = [&](int st) {
    const long k0 = (long)st * GB_K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int row = idx >> 3, c8 = (idx & 7) * 8;
      const int m = m0 + row;
      ra[i] = uint4{0u, 0u, 0u, 0u};
      if (m < M) ra[i] = load_x8(a, a.xrow ? a.xrow[m] : m, rs_sh[row], k0 + c8);
      rb[i] = wok[i] ? *(const uint4*)(W + wrow[i] * K + k0 + c8) : uint4{0u, 0u, 0u, 0u};
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int row = idx >> 3, c8 = (idx & 7) * 8;
      *(uint4*)(&As[buf][row * GB_LD + c8]) = ra[i];
      *(uint4*)(&Bs[buf][row * GB_LD + c8]) = rb[i];
    }
  };
  auto mma = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = *(const bf16x8_t*)(&As[buf][(64 * wm + 16 * i + l16) * GB_LD + 32 * ks + 8 * kb]);
        bfr[i] = *(const bf16x8_t*)(&Bs[buf][(64 * wn + 16 * i + l16) * GB_LD + 32 * ks + 8 * kb]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  if (s0 < s1) {
    gload(s0);
    sstore(0);
    __syncthreads();
    int buf = 0;
    for (int st = s0; st < s1; ++st) {
      const bool nxt = st + 1 < s1;
      if (nxt) gload(st + 1);
      mma(buf);
      if (nxt) sstore(buf ^ 1);
      lds_barrier();
      buf ^= 1;
    }
  }

  // Stage the 128x128 tile through LDS (reusing the operand buffers) so the
  // epilogue walks it row-wise: coalesced stores, pair partners at column ^ 8,
  // one sum-of-squares partial per (row, 64 columns).
  // acc[i][j][r] is row 64 wm + 16 i + 4 kb + r, column 64 wn + 16 j + l16.
  float* Cs = reinterpret_cast<float*>(smem);
  constexpr int CLD = GB_N + 4;
  static_assert(sizeof(smem) >= sizeof(float) * GB_M * CLD, "C tile does not fit");
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) Cs[(64 * wm + 16 * i + 4 * kb + r) * CLD + 64 * wn + 16 * j + l16] = acc[i][j][r];
  __syncthreads();
  const bool want_ssq = a.epi == EPI_RESID && a.ssq_acc && nsplit == 1;
  for (int e = tid; e < GB_M * GB_N; e += 256) {
    const int row = e >> 7, col = e & 127;  // a wave covers 64 columns of one row
    const int m = m0 + row, nl = n0 + col;
    const bool mok = m < M, nok = nl < N;
    const int n = nok ? phys_row(a, nl >> 4, nl & 15) : N;
    const float v = Cs[row * CLD + col];
    float sq = 0.f;
    if (nsplit > 1) {
      if (mok && nok) part[((long)sp * M + m) * N + n] = v;
    } else {
      epilogue(a, m, n, v, Cs[row * CLD + (col ^ 8)], mok && nok, nl & 15);
      if (want_ssq && mok && nok) {
        const float hn = ((const float*)a.y)[(long)m * a.ldy + n];
        sq = hn * hn;
      }
    }
    if (want_ssq) {  // wave-uniform: all 64 lanes share the row
      sq += __shfl_xor(sq, 16, 64);
      sq += __shfl_xor(sq, 32, 64);
      ssq_add(a, m, sq, lane == 0, mok);
    }
  }
}

// Split-K reduction: one wave per (row, 64 logical columns); the partials are
// summed in split order, then the same epilogue as the unsplit kernel.  The
// four waves of a work-group cover consecutive column groups, mostly of one
// row, so a residual epilogue's sum of squares is added once per (work-group,
// row) after an LDS pre-sum instead of once per wave (fewer same-address
// atomics).
__global__ __launch_bounds__(256) void k_splitk_reduce(LinArgs a, const float* __restrict__ part, int nsplit) {
  __shared__ float ssq_sh[4];
  __shared__ int row_sh[4];
  const int M = a.M, N = a.W.N;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const long wid = (long)blockIdx.x * 4 + wave;
  const long ngroups = (N + 63) / 64;
  if (blockIdx.x == 0 && a.ssq_zero)
    ssq_clear(a, threadIdx.x, 256);
  const bool want_ssq = a.epi == EPI_RESID && a.ssq_acc;
  const bool live = wid < (long)M * ngroups;
  if (!live && !want_ssq) return;
  float sq = 0.f;
  int m = -1;
  if (live) {
    m = (int)(wid / ngroups);
    const int nl = (int)(wid - (long)m * ngroups) * 64 + lane;
    const bool nok = nl < N;
    const int l16 = lane & 15;
    const int n = nok ? phys_row(a, nl >> 4, l16) : 0;
    float v = 0.f;
    if (nok)
      for (int s = 0; s < nsplit; ++s) v += part[((long)s * M + m) * N + n];
    const float partner = __shfl_xor(v, 8, 64);
    epilogue(a, m, n, v, partner, nok, l16);
    if (want_ssq && nok) {
      const float hn = ((const float*)a.y)[(long)m * a.ldy + n];
      sq = hn * hn;
    }
  }
  if (!want_ssq) return;
  sq = wave_sum(sq);
  if (lane == 0) {
    ssq_sh[wave] = sq;
    row_sh[wave] = m;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int cur = -1;
    float acc = 0.f;
    for (int w = 0; w < 4; ++w) {
      const int r = row_sh[w];
      if (r != cur) {
        if (cur >= 0) atomicAdd(ssq_slot(a, cur), (unsigned long long)rint((double)acc * SSQ_SCALE));
        cur = r;
        acc = 0.f;
      }
      acc += ssq_sh[w];
    }
    if (cur >= 0) atomicAdd(ssq_slot(a, cur), (unsigned long long)rint((double)acc * SSQ_SCALE));
  }
}

static int run_gemm(const LinArgs& a, const LinearWs& ws, hipStream_t st, LinearInfo* info) {
  const int M = a.M;
  const int mtiles = (M + GB_M - 1) / GB_M;
  const int ntiles = (a.W.N + GB_N - 1) / GB_N;
  const int nsteps = a.W.K / GB_K;
  const long base = (long)mtiles * ntiles;
  int nsplit = 1;
  while (base * nsplit < 256 && nsteps / (nsplit * 2) >= 4 &&
         (size_t)(nsplit * 2) * M * a.W.N <= ws.partial_floats)
    nsplit *= 2;
  const int kps = (nsteps + nsplit - 1) / nsplit;
  nsplit = (nsteps + kps - 1) / kps;
  if (info) {
    snprintf(info->name, sizeof info->name, "er::k_gemm_bf16");
    info->nsplit = nsplit;
  }
  hipLaunchKernelGGL(k_gemm_bf16, dim3((unsigned)(base * nsplit)), dim3(256), 0, st, a, ws.partial, nsplit, kps,
                     mtiles);
  if (hipGetLastError() != hipSuccess) return -3;
  if (nsplit > 1) {
    const long waves = (long)M * ((a.W.N + 63) / 64);
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, a, ws.partial, nsplit);
    if (hipGetLastError() != hipSuccess) return -3;
  }
  return 0;
}

// ----------------------------------------------------------------------------
// Streaming skinny linear for M <= 16 (decode, drafting, small verify).
// x' (M rows x K, bf16, formed from the fp32 residual when normalizing) is
// staged once per work-group in LDS; each wave then streams its weight rows
// from HBM through a register ring DEPTH stages deep.  LDS reads are counted
// apart from vector-memory loads, so reading x' never waits on weights still
// in flight, and a normalizing prologue does not serialize the weight stream.
// A stage is 128 k of one 16-row subtile per lane group: bf16 4 x 16 B per
// lane, W8 2 x 16 B, W4 1 x 16 B (one quantization group).  For the quantized
// formats the per-group row sums of x' (zero-point terms) are formed in the
// prologue from the x' pieces themselves.  Waves split K (KS) within the
// work-group and reduce in LDS in a fixed order; the first DEPTH-1 weight
// stages, the W4 scale / zero staging loads and the x' loads all go out
// before the prologue's first wait, so that they overlap (the prologue once
// took ~4 us of a 17-21 us W4 launch at M = 1 with three dependent trips).
// ----------------------------------------------------------------------------
template <int FMT> struct StageW { static constexpr int NW = (FMT == FMT_BF16) ? 4 : (FMT == FMT_W8 ? 2 : 1); };

// LDS of k_skinny: x' [M][K+8] bf16; quantized formats add per-chunk row sums
// of x' [K/128][16] (rows < M written; the others feed only output rows that
// are never stored) and the work-group's scale/zero pairs [R][K/128]
// (float2); then the KS reduction area.
struct SkinnyLds {
  size_t xsum, sz, red, total;
};
static inline SkinnyLds skinny_lds(int fmt, int M, int K, int NR, int KS) {
  SkinnyLds L;
  const size_t nch = (size_t)K / 128;
  const size_t R = (size_t)16 * NR * (8 / KS);
  size_t b = (size_t)M * ((size_t)K + 8) * 2;
  b = (b + 15) & ~(size_t)15;
  L.xsum = b;
  if (fmt != FMT_BF16) b += nch * 16 * 4;
  L.sz = b;
  if (fmt == FMT_W4) b += R * nch * 8;
  // the KS reduction runs after every wave is done with x' and reuses its space
  L.red = 0;
  const size_t red = KS > 1 ? (size_t)8 * NR * 64 * 16 : 0;
  L.total = std::max(b, red);
  return L;
}

template <int FMT, int NR, int KS, int DEPTH>
__global__ __launch_bounds__(512) void k_skinny(LinArgs a, SkinnyLds L) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  constexpr int RG = 8 / KS;
  constexpr int R = 16 * NR * RG;
  constexpr int NW = StageW<FMT>::NW;
  const int M = a.M, N = a.W.N, K = a.W.K;
  const int ldsx = K + 8;
  const int nchunks = K >> 7;
  char* lds = reinterpret_cast<char*>(xs);
  float* xsum = reinterpret_cast<float*>(lds + L.xsum);   // [nchunks][16] row sums of x' per chunk
  float2* szl = reinterpret_cast<float2*>(lds + L.sz);    // [R][nchunks] (scale, 128 + zero), W4
  f32x4_t* red = reinterpret_cast<f32x4_t*>(lds + L.red);

  const int b = blockIdx.x, nwg = gridDim.x;
  const int xcd = b & 7, loc = b >> 3, per = nwg >> 3, rem = nwg & 7;
  const int nt = (xcd < rem) ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int rg = wave / KS, ks = wave % KS;
  const int kb = lane >> 4, l16 = lane & 15;
  const long G = K >> 7;
  const void* __restrict__ wv = a.W.w;
  const void* __restrict__ sv = a.W.scale;
  const void* __restrict__ zv = a.W.zero;

  if (b == 0 && a.ssq_zero)
    ssq_clear(a, tid, 512);

  int n_lane[NR];
  long nrow[NR];
#pragma unroll
  for (int ni = 0; ni < NR; ++ni) {
    const int s = (nt * RG + rg) * NR + ni;
    const bool in = 16 * s + l16 < N;
    n_lane[ni] = in ? phys_row(a, s, l16) : N;
    nrow[ni] = in ? n_lane[ni] : N - 1;
  }

  // this wave's stages: chunks ks, ks + KS, ...
  const int n_it = (nchunks - ks + KS - 1) / KS;
  uint4 wreg[DEPTH][NR][NW];

  auto issue = [&](int it, int slot) {
    const long c = min(ks + (long)KS * it, (long)nchunks - 1);
#pragma unroll
    for (int ni = 0; ni < NR; ++ni) {
      if constexpr (FMT == FMT_BF16) {
        const uint16_t* p = (const uint16_t*)wv + nrow[ni] * K + c * 128 + 8 * kb;
#pragma unroll
        for (int i = 0; i < 4; ++i) wreg[slot][ni][i] = *(const uint4*)(p + 32 * i);
      } else if constexpr (FMT == FMT_W8) {
        const int8_t* p = (const int8_t*)wv + nrow[ni] * K + c * 128 + 16 * kb;
#pragma unroll
        for (int h = 0; h < 2; ++h) wreg[slot][ni][h] = *(const uint4*)(p + 64 * h);
      } else {
        const uint8_t* p = (const uint8_t*)wv + w4_piece(nrow[ni], c, N, K) + 16 * kb;
        wreg[slot][ni][0] = *(const uint4*)p;
      }
    }
  };

  f32x4_t acc[NR];
#pragma unroll
  for (int ni = 0; ni < NR; ++ni) acc[ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // lanes of rows >= M read row M-1 instead (their outputs are never stored):
  // no predicated LDS reads in the loop
  const int xr_row = l16 < M ? l16 : M - 1;
  auto compute = [&](int it, int slot) {
    const int c = ks + KS * it;
    bf16x8_t xa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      xa[i] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(xs + xr_row * ldsx + c * 128 + kcol<FMT>(i, kb)));
    f32x4_t accg[NR];
    if constexpr (FMT != FMT_BF16) {
#pragma unroll
      for (int ni = 0; ni < NR; ++ni) accg[ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int ni = 0; ni < NR; ++ni) {
        bf16x8_t bw;
        if constexpr (FMT == FMT_BF16) {
          bw = __builtin_bit_cast(bf16x8_t, wreg[slot][ni][i]);
          acc[ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[i], bw, acc[ni], 0, 0, 0);
        } else {
          if constexpr (FMT == FMT_W8) {
            const uint4 v = wreg[slot][ni][i >> 1];
            bw = (i & 1) ? w8_to_bf16(v.z, v.w) : w8_to_bf16(v.x, v.y);
          } else {
            const uint4 v = wreg[slot][ni][0];
            const uint32_t word = (i == 0) ? v.x : (i == 1) ? v.y : (i == 2) ? v.z : v.w;
            bw = w4_to_bf16(word);
          }
          accg[ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[i], bw, accg[ni], 0, 0, 0);
        }
      }
    }
    if constexpr (FMT != FMT_BF16) {
      const float4 xs4 = *reinterpret_cast<const float4*>(xsum + c * 16 + 4 * kb);  // rows 4kb .. 4kb+3
      const float xsm[4] = {xs4.x, xs4.y, xs4.z, xs4.w};
      float2 sz[NR];
      if constexpr (FMT == FMT_W4) {
#pragma unroll
        for (int ni = 0; ni < NR; ++ni) sz[ni] = szl[(rg * NR + ni) * 16 * nchunks + l16 * nchunks + c];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int ni = 0; ni < NR; ++ni) {
          if constexpr (FMT == FMT_W8)
            acc[ni][r] += accg[ni][r] - 128.0f * xsm[r];
          else
            acc[ni][r] = fmaf(sz[ni].x, fmaf(-sz[ni].y, xsm[r], accg[ni][r]), acc[ni][r]);
        }
      }
    }
  };

  // Weights for the first stages go out before the x' fill.  Every loop
  // iteration issues exactly one stage (clamped to the last one: re-reads hit
  // the cache), so the compiler can keep DEPTH - 1 stages in flight instead
  // of draining the load counter at each use.
  const int last_it = n_it > 0 ? n_it - 1 : 0;
#pragma unroll
  for (int d = 0; d < DEPTH - 1; ++d) issue(min(d, last_it), d);

  {
    // Prologue, one memory round trip before the first barrier: the first
    // pass of the W4 scale / zero staging, the rows' 1/rms (from one slot
    // load per (row, slot) lane summed over 16 lanes) and the first x' pieces
    // are all issued before anything waits.  x' fill: XF 16-byte pieces per
    // thread in flight at once (with the norm on load each piece is three
    // loads; two pieces keep the kernel at 65 VGPRs, three 512-thread
    // work-groups per CU, where four pieces took 91 and two work-groups).
    // The per-chunk row sums of x' (zero-point terms of the quantized
    // formats) come from the pieces themselves: the 16 pieces of one
    // (row, chunk) are 16 consecutive threads (K is a multiple of 128), summed
    // by shuffles.
    constexpr int XF = 2;
    constexpr int SZJ = 2;  // scale / zero entries per thread per staging pass (4 measured no better)
    __shared__ float rs_sh[16];
    const int sz_total = (FMT == FMT_W4) ? R * nchunks : 0;
    uint32_t sc[SZJ], zc[SZJ];
    auto sz_load = [&](int e0) {
#pragma unroll
      for (int j = 0; j < SZJ; ++j) {
        const int e = min(e0 + tid + 512 * j, sz_total - 1);
        const int rr = e / nchunks, c = e - rr * nchunks;
        const int s2 = nt * RG * NR + (rr >> 4);
        const int l = rr & 15;
        const long n = (16 * s2 + l < N) ? phys_row(a, s2, l) : N - 1;
        sc[j] = ((const uint16_t*)sv)[n * G + c];
        zc[j] = ((const uint8_t*)zv)[n * G + c];
      }
    };
    auto sz_store = [&](int e0) {
#pragma unroll
      for (int j = 0; j < SZJ; ++j) {
        const int e = e0 + tid + 512 * j;
        if (e < sz_total) szl[e] = make_float2(bf2f((uint16_t)sc[j]), 128.0f + (float)zc[j]);
      }
    };
    if constexpr (FMT == FMT_W4) sz_load(0);
    if (a.xnorm && tid < 16 * M) {
      const int m = tid >> 4, sl = tid & 15;
      const long hrow = a.xrow ? a.xrow[m] : m;
      unsigned long long t = sl < ssq_nslots(a) ? a.ssq_in[(long)sl * a.ssq_stride + hrow] : 0ull;
      t += __shfl_xor(t, 1, 64);
      t += __shfl_xor(t, 2, 64);
      t += __shfl_xor(t, 4, 64);
      t += __shfl_xor(t, 8, 64);
      if (sl == 0) rs_sh[m] = 1.0f / sqrtf((float)((double)t / SSQ_SCALE) / (float)K + a.eps);
    }
    const int K8 = K >> 3, tot = M * K8;
    for (int e0 = 0; e0 < tot; e0 += XF * 512) {
      uint4 v[XF], h1[XF], g[XF];
#pragma unroll
      for (int j = 0; j < XF; ++j) {
        const int e = min(e0 + tid + 512 * j, tot - 1);
        const int m = e / K8, k8 = e - m * K8;
        const long hrow = a.xrow ? a.xrow[m] : m;
        if (a.xnorm) {
          const float* hp = (const float*)a.x + hrow * a.ldx + (long)k8 * 8;
          v[j] = *(const uint4*)hp;
          h1[j] = *(const uint4*)(hp + 4);
          g[j] = *(const uint4*)((const uint16_t*)a.gnorm + (long)k8 * 8);
        } else {
          v[j] = *(const uint4*)((const uint16_t*)a.x + hrow * a.ldx + (long)k8 * 8);
        }
      }
      if (a.xnorm && e0 == 0) __syncthreads();  // rs_sh
#pragma unroll
      for (int j = 0; j < XF; ++j) {
        const int e = e0 + tid + 512 * j;
        const bool in = e < tot;   // the same for the 16 lanes of one (row, chunk)
        const int m = e / K8, k8 = e - m * K8;
        uint4 o = v[j];
        if (a.xnorm) {
          const float rs = rs_sh[in ? m : 0];
          const uint4 h0 = v[j], hh = h1[j], gg = g[j];
          o.x = f2bf(__uint_as_float(h0.x) * rs * bf_lo(gg.x)) | (f2bf(__uint_as_float(h0.y) * rs * bf_hi(gg.x)) << 16);
          o.y = f2bf(__uint_as_float(h0.z) * rs * bf_lo(gg.y)) | (f2bf(__uint_as_float(h0.w) * rs * bf_hi(gg.y)) << 16);
          o.z = f2bf(__uint_as_float(hh.x) * rs * bf_lo(gg.z)) | (f2bf(__uint_as_float(hh.y) * rs * bf_hi(gg.z)) << 16);
          o.w = f2bf(__uint_as_float(hh.z) * rs * bf_lo(gg.w)) | (f2bf(__uint_as_float(hh.w) * rs * bf_hi(gg.w)) << 16);
        }
        if (in) *(uint4*)(xs + m * ldsx + k8 * 8) = o;
        if constexpr (FMT != FMT_BF16) {
          float sm = bf_lo(o.x) + bf_hi(o.x) + bf_lo(o.y) + bf_hi(o.y) + bf_lo(o.z) + bf_hi(o.z) + bf_lo(o.w) + bf_hi(o.w);
          sm += __shfl_xor(sm, 1, 64);
          sm += __shfl_xor(sm, 2, 64);
          sm += __shfl_xor(sm, 4, 64);
          sm += __shfl_xor(sm, 8, 64);
          if (in && (tid & 15) == 0) xsum[(k8 >> 4) * 16 + m] = sm;
        }
      }
    }
    if constexpr (FMT == FMT_W4) {
      // this work-group's rows: logical subtile (nt*RG + rg')*NR + ni, lane
      // row l16; SZJ entries per thread in flight at once
      sz_store(0);
      for (int e0 = SZJ * 512; e0 < sz_total; e0 += SZJ * 512) {
        sz_load(e0);
        sz_store(e0);
      }
    }
    __syncthreads();
  }

  for (int i0 = 0; i0 < n_it; i0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int it = i0 + d;
      issue(min(it + DEPTH - 1, last_it), (d + DEPTH - 1) % DEPTH);
      if (it < n_it) compute(it, d);
    }
  }

  if constexpr (FMT == FMT_W8) {
#pragma unroll
    for (int ni = 0; ni < NR; ++ni) {
      const float sc = ((const float*)sv)[nrow[ni]];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[ni][r] *= sc;
    }
  }

  if constexpr (KS > 1) {
    __syncthreads();  // the reduction area overlays x'
#pragma unroll
    for (int ni = 0; ni < NR; ++ni) red[(wave * NR + ni) * 64 + lane] = acc[ni];
    __syncthreads();
    if (ks != 0) return;
#pragma unroll
    for (int ni = 0; ni < NR; ++ni) {
      f32x4_t v = red[(wave * NR + ni) * 64 + lane];
#pragma unroll
      for (int s2 = 1; s2 < KS; ++s2) {
        const f32x4_t o = red[((wave + s2) * NR + ni) * 64 + lane];
        v[0] += o[0]; v[1] += o[1]; v[2] += o[2]; v[3] += o[3];
      }
      acc[ni] = v;
    }
  }

  const bool want_ssq = a.epi == EPI_RESID && a.ssq_acc;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * kb + r;
    const bool mok = m < M;
    float sq = 0.f;
#pragma unroll
    for (int ni = 0; ni < NR; ++ni) {
      const float v = acc[ni][r];
      const float partner = __shfl_xor(v, 8, 64);
      const bool ok = mok && n_lane[ni] < N;
      epilogue(a, m, n_lane[ni], v, partner, ok, l16);
      if (want_ssq && ok) {
        const float hn = ((const float*)a.y)[(long)m * a.ldy + n_lane[ni]];
        sq = fmaf(hn, hn, sq);
      }
    }
    if (want_ssq) ssq_add(a, m, sq, l16 == 0, mok);
  }
}

template <int FMT, int NR, int KS, int DEPTH>
static int run_skinny(const LinArgs& a, hipStream_t st, LinearInfo* info) {
  constexpr int R = 16 * NR * (8 / KS);
  const SkinnyLds L = skinny_lds(FMT, a.M, a.W.K, NR, KS);
  const size_t lds = L.total;
  if (a.M > 16 || lds > kSkinnyLdsMax) return -1;
  const long nwg = (a.W.N + R - 1) / R;
  if (info) {
    snprintf(info->name, sizeof info->name, "er::k_skinny<%d, %d, %d, %d>", FMT, NR, KS, DEPTH);
    info->nsplit = KS;
  }
  hipLaunchKernelGGL((k_skinny<FMT, NR, KS, DEPTH>), dim3((unsigned)nwg), dim3(512), lds, st, a, L);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Explicit streaming variant: code = 2000 + 100*NR + 10*KS + DEPTH.
template <int FMT>
static int run_skinny_variant(int code, const LinArgs& a, hipStream_t st, LinearInfo* info) {
  const int nr = (code / 100) % 10, ks = (code / 10) % 10, dp = code % 10;
#define ER_S(NR_, KS_, D_) \
  if (nr == NR_ && ks == KS_ && dp == D_) return run_skinny<FMT, NR_, KS_, D_>(a, st, info);
#define ER_SK(NR_, D_) ER_S(NR_, 2, D_) ER_S(NR_, 4, D_) ER_S(NR_, 8, D_)
  ER_SK(1, 2) ER_SK(1, 3) ER_SK(1, 4) ER_SK(2, 2) ER_SK(2, 3) ER_SK(2, 4)
  ER_S(1, 1, 2) ER_S(1, 1, 3) ER_S(1, 1, 4) ER_S(1, 1, 6) ER_S(1, 1, 8) ER_S(2, 1, 2) ER_S(2, 1, 3) ER_S(2, 1, 4)
  if constexpr (FMT != FMT_BF16) { ER_SK(4, 2) ER_SK(4, 3) ER_SK(4, 4) ER_SK(1, 6) ER_SK(2, 6) ER_SK(1, 8) }
#undef ER_SK
#undef ER_S
  return -1;
}

// ----------------------------------------------------------------------------
// Weight-streaming GEMM for 16 < M <= 256: large-batch decode and verify
// (bf16 weights) and drafting (W8 / W4 weights), where the layer is still
// bound by reading W once.  Each wave streams its own 16*NR weight rows
// through a register ring (DEPTH stages of 128 k); the M x (KS*128) window of
// x for the current step is staged in LDS and shared by every wave
// (double-buffered, one barrier per step).  Quantized weights are converted
// in registers once per stage and feed every m-subtile of the window (so each
// weight byte is read once whatever M is), as bf16 of (q + 128); the
// zero-point term uses the window's per-chunk row sums of x, formed once per
// work-group while the window is written to LDS (16 lanes per row and chunk,
// summed by shuffles): W4 adds s * (acc_chunk - (128 + z) * sum) per chunk,
// W8 acc_chunk - 128 * sum, scaled per row at the end.  The next
// window's loads are issued ahead of the weights so that writing it to LDS
// never waits on weight loads still in flight.  KS waves split each step's K
// range and reduce in LDS; nsplit > 1 splits K over work-groups, with the
// partial tiles summed in a fixed order by k_splitk_reduce.
// ----------------------------------------------------------------------------
template <int FMT, int MI, int NR, int KS, int DEPTH>
__global__ __launch_bounds__(512) void k_wgemm(LinArgs a, float* __restrict__ part, int nsplit, int cps, int mtiles) {
  constexpr int RG = 8 / KS;
  constexpr int MT = 16 * MI;
  constexpr int WK = KS * 128;           // k per step
  constexpr int LDX = WK + 8;            // LDS row stride (bf16)
  constexpr int XV = MT * WK / 8 / 512;  // uint4 of the x window per thread
  static_assert(MT * WK % (8 * 512) == 0, "x window must split evenly over the threads");
  constexpr int NW = StageW<FMT>::NW;   // uint4 of one stage of one subtile per lane
  constexpr bool Q = FMT != FMT_BF16;
  __shared__ __attribute__((aligned(16))) uint16_t xw[2][MT * LDX];
  __shared__ __attribute__((aligned(16))) float xsum_sh[Q ? 2 : 1][Q ? KS * MT : 1];  // [buf][chunk of window][row]

  const int b = blockIdx.x, nwg = gridDim.x;
  const int xcd = b & 7, loc = b >> 3, per = nwg >> 3, rem = nwg & 7;
  const int L = (xcd < rem) ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
  // the m-tiles of one weight tile are adjacent block indices (one XCD, one L2)
  const int mt = L % mtiles, sp = (L / mtiles) % nsplit, nt = L / mtiles / nsplit;
  const int m0 = mt * MT;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int rg = wave / KS, ks = wave % KS;
  const int kb = lane >> 4, l16 = lane & 15;
  const int M = a.M, N = a.W.N, K = a.W.K;
  const int nchunks = K >> 7;
  const int c0 = sp * cps, c1 = min(nchunks, c0 + cps);
  const int T = (c1 - c0 + KS - 1) / KS;  // steps
  const void* __restrict__ Wv = a.W.w;
  const uint16_t* __restrict__ X = (const uint16_t*)a.x;
  const long G = K >> 7;

  if (b == 0 && a.ssq_zero && nsplit == 1)
    ssq_clear(a, tid, 512);

  int n_lane[NR];
  long nrow[NR];
#pragma unroll
  for (int ni = 0; ni < NR; ++ni) {
    const int s = (nt * RG + rg) * NR + ni;
    const bool in = 16 * s + l16 < N;
    n_lane[ni] = in ? phys_row(a, s, l16) : N;
    nrow[ni] = in ? n_lane[ni] : N - 1;
  }

  uint4 wreg[DEPTH][NR][NW];
  float wsc[DEPTH][NR], wzp[DEPTH][NR];   // W4: scale and 128 + zero of (row, chunk)
  uint4 xr[XV];
  auto issue_w = [&](int t, int slot) {
    const long c = c0 + (long)t * KS + ks;
    if (c >= c1) return;
#pragma unroll
    for (int ni = 0; ni < NR; ++ni) {
      if constexpr (FMT == FMT_BF16) {
        const uint16_t* p = (const uint16_t*)Wv + nrow[ni] * K + c * 128 + 8 * kb;
#pragma unroll
        for (int i = 0; i < 4; ++i) wreg[slot][ni][i] = *(const uint4*)(p + 32 * i);
      } else if constexpr (FMT == FMT_W8) {
        const int8_t* p = (const int8_t*)Wv + nrow[ni] * K + c * 128 + 16 * kb;
#pragma unroll
        for (int h = 0; h < 2; ++h) wreg[slot][ni][h] = *(const uint4*)(p + 64 * h);
      } else {
        const uint8_t* p = (const uint8_t*)Wv + w4_piece(nrow[ni], c, N, K) + 16 * kb;
        wreg[slot][ni][0] = *(const uint4*)p;
        wsc[slot][ni] = bf2f(((const uint16_t*)a.W.scale)[nrow[ni] * G + c]);
        wzp[slot][ni] = 128.0f + (float)((const uint8_t*)a.W.zero)[nrow[ni] * G + c];
      }
    }
  };
  auto load_x = [&](int t) {
    const long k0 = (long)(c0 + t * KS) * 128;
#pragma unroll
    for (int v = 0; v < XV; ++v) {
      const int e = tid + 512 * v;
      const int m = e / (WK / 8), k8 = e - m * (WK / 8);
      uint4 val = uint4{0u, 0u, 0u, 0u};
      if (m0 + m < M && k0 + k8 * 8 < (long)c1 * 128) val = *(const uint4*)(X + (long)(m0 + m) * a.ldx + k0 + k8 * 8);
      xr[v] = val;
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int v = 0; v < XV; ++v) {
      const int e = tid + 512 * v;
      const int m = e / (WK / 8), k8 = e - m * (WK / 8);
      *(uint4*)(&xw[buf][m * LDX + k8 * 8]) = xr[v];
      if constexpr (Q) {
        // the 16 pieces of one (row, chunk) are 16 aligned consecutive threads
        const uint4 o = xr[v];
        float sm = bf_lo(o.x) + bf_hi(o.x) + bf_lo(o.y) + bf_hi(o.y) + bf_lo(o.z) + bf_hi(o.z) + bf_lo(o.w) + bf_hi(o.w);
        sm += __shfl_xor(sm, 1, 64);
        sm += __shfl_xor(sm, 2, 64);
        sm += __shfl_xor(sm, 4, 64);
        sm += __shfl_xor(sm, 8, 64);
        if ((k8 & 15) == 0) xsum_sh[buf][(k8 >> 4) * MT + m] = sm;
      }
    }
  };

  f32x4_t acc[MI][NR];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NR; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int t, int slot, int buf) {
    const int c = c0 + t * KS + ks;
    if (c >= c1) return;
    if constexpr (FMT == FMT_BF16) {
      const uint16_t* xb = &xw[buf][ks * 128 + 8 * kb];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          const bf16x8_t xa = *(const bf16x8_t*)(xb + (mi * 16 + l16) * LDX + 32 * i);
#pragma unroll
          for (int ni = 0; ni < NR; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, __builtin_bit_cast(bf16x8_t, wreg[slot][ni][i]),
                                                                  acc[mi][ni], 0, 0, 0);
        }
      }
    } else {
      // the stage's weights as bf16 of (q + 128), converted once for every m-subtile
      bf16x8_t bw[NR][4];
#pragma unroll
      for (int ni = 0; ni < NR; ++ni)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (FMT == FMT_W8) {
            const uint4 v = wreg[slot][ni][i >> 1];
            bw[ni][i] = (i & 1) ? w8_to_bf16(v.z, v.w) : w8_to_bf16(v.x, v.y);
          } else {
            const uint4 v = wreg[slot][ni][0];
            bw[ni][i] = w4_to_bf16((i == 0) ? v.x : (i == 1) ? v.y : (i == 2) ? v.z : v.w);
          }
        }
      const uint16_t* xb = &xw[buf][ks * 128];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        f32x4_t accg[NR];
#pragma unroll
        for (int ni = 0; ni < NR; ++ni) accg[ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8_t xa = *(const bf16x8_t*)(xb + (mi * 16 + l16) * LDX + kcol<FMT>(i, kb));
#pragma unroll
          for (int ni = 0; ni < NR; ++ni)
            accg[ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bw[ni][i], accg[ni], 0, 0, 0);
        }
        // rows mi*16 + 4kb + r of this chunk's row sums
        const float4 xs4 = *reinterpret_cast<const float4*>(&xsum_sh[buf][ks * MT + mi * 16 + 4 * kb]);
        const float xsm[4] = {xs4.x, xs4.y, xs4.z, xs4.w};
#pragma unroll
        for (int ni = 0; ni < NR; ++ni)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if constexpr (FMT == FMT_W8)
              acc[mi][ni][r] += accg[ni][r] - 128.0f * xsm[r];
            else
              acc[mi][ni][r] = fmaf(wsc[slot][ni], fmaf(-wzp[slot][ni], xsm[r], accg[ni][r]), acc[mi][ni][r]);
          }
      }
    }
  };

  // prologue: x window 0 first, then the first weight stages
  load_x(0);
#pragma unroll
  for (int d = 0; d < DEPTH - 1; ++d)
    if (d < T) issue_w(d, d);
  store_x(0);
  __syncthreads();

  for (int t0 = 0; t0 < T; t0 += 2 * DEPTH) {
#pragma unroll
    for (int d = 0; d < 2 * DEPTH; ++d) {
      const int t = t0 + d;
      if (t < T) {
        if (t + 1 < T) load_x(t + 1);
        if (t + DEPTH - 1 < T) issue_w(t + DEPTH - 1, (d + DEPTH - 1) % DEPTH);
        compute(t, d % DEPTH, d & 1);
        if (t + 1 < T) store_x((d + 1) & 1);
        lds_barrier();
      }
    }
  }

  if constexpr (FMT == FMT_W8) {
#pragma unroll
    for (int ni = 0; ni < NR; ++ni) {
      const float sc = ((const float*)a.W.scale)[nrow[ni]];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mi][ni][r] *= sc;
    }
  }

  // reduce the KS partial tiles (fixed order) through the x window's LDS
  if constexpr (KS > 1) {
    f32x4_t* red = reinterpret_cast<f32x4_t*>(&xw[0][0]);
    static_assert(sizeof(xw) >= sizeof(f32x4_t) * 8 * MI * NR * 64, "reduction area does not fit");
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NR; ++ni) red[((wave * MI + mi) * NR + ni) * 64 + lane] = acc[mi][ni];
    __syncthreads();
    if (ks != 0) return;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NR; ++ni) {
        f32x4_t v = red[((wave * MI + mi) * NR + ni) * 64 + lane];
#pragma unroll
        for (int s2 = 1; s2 < KS; ++s2) {
          const f32x4_t o = red[(((wave + s2) * MI + mi) * NR + ni) * 64 + lane];
          v[0] += o[0]; v[1] += o[1]; v[2] += o[2]; v[3] += o[3];
        }
        acc[mi][ni] = v;
      }
  }

  const bool want_ssq = a.epi == EPI_RESID && a.ssq_acc && nsplit == 1;
  if constexpr (MI * NR > 8) {
    // Large tiles: stage the (MT x R) result through LDS and walk it row-wise,
    // so that the fully unrolled register loop stays small.
    static_assert(KS == 1 && 16 * NR * RG == 128, "LDS epilogue expects 128-column tiles");
    constexpr int R = 128, CLD = R + 4;
    static_assert(sizeof(xw) >= sizeof(float) * MT * CLD, "result tile does not fit");
    float* Cs = reinterpret_cast<float*>(&xw[0][0]);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NR; ++ni)
#pragma unroll
        for (int r = 0; r < 4; ++r) Cs[(mi * 16 + 4 * kb + r) * CLD + (rg * NR + ni) * 16 + l16] = acc[mi][ni][r];
    __syncthreads();
    for (int e = tid; e < MT * R; e += 512) {
      const int row = e >> 7, col = e & 127;  // a wave covers 64 columns of one row
      const int m = m0 + row;
      const int sidx = (nt * RG) * NR + (col >> 4);
      const bool mok = m < M, nok = 16 * sidx + (col & 15) < N;
      const int n = nok ? phys_row(a, sidx, col & 15) : N;
      const float v = Cs[row * CLD + col];
      float sq = 0.f;
      if (nsplit > 1) {
        if (mok && nok) part[((long)sp * M + m) * N + n] = v;
      } else {
        epilogue(a, m, n, v, Cs[row * CLD + (col ^ 8)], mok && nok, col & 15);
        if (want_ssq && mok && nok) {
          const float hn = ((const float*)a.y)[(long)m * a.ldy + n];
          sq = hn * hn;
        }
      }
      if (want_ssq) {
        sq += __shfl_xor(sq, 16, 64);
        sq += __shfl_xor(sq, 32, 64);
        ssq_add(a, m, sq, lane == 0, mok);
      }
    }
    return;
  }
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + mi * 16 + 4 * kb + r;
      const bool mok = m < M;
      float sq = 0.f;
#pragma unroll
      for (int ni = 0; ni < NR; ++ni) {
        const float v = acc[mi][ni][r];
        const bool ok = mok && n_lane[ni] < N;
        if (nsplit > 1) {
          if (ok) part[((long)sp * M + m) * N + n_lane[ni]] = v;
          continue;
        }
        const float partner = __shfl_xor(v, 8, 64);
        epilogue(a, m, n_lane[ni], v, partner, ok, l16);
        if (want_ssq && ok) {
          const float hn = ((const float*)a.y)[(long)m * a.ldy + n_lane[ni]];
          sq = fmaf(hn, hn, sq);
        }
      }
      if (want_ssq) ssq_add(a, m, sq, l16 == 0, mok);
    }
}

template <int FMT, int MI, int NR, int KS, int DEPTH>
static int run_wgemm_fmt(const LinArgs& a, const LinearWs& ws, int want_wgs, hipStream_t st, LinearInfo* info) {
  constexpr int R = 16 * NR * (8 / KS);
  constexpr int MT = 16 * MI;
  // bf16 weights: one m-tile (the plan sends larger M to the tiled GEMMs); quantized weights are
  // re-read once per m-tile of up to MT rows
  if ((FMT == FMT_BF16 && a.M > MT) || a.W.fmt != FMT || a.xnorm) return -1;
  const int mtiles = (a.M + MT - 1) / MT;
  const int nchunks = a.W.K / 128;
  const long ntiles = (a.W.N + R - 1) / R;
  int nsplit = 1;
  // split K over work-groups while the grid is short of want_wgs and every
  // split keeps at least 4 steps
  while (ntiles * mtiles * nsplit * 2 <= want_wgs && nchunks / (nsplit * 2 * KS) >= 4 &&
         (size_t)(nsplit * 2) * a.M * a.W.N <= ws.partial_floats && ws.partial)
    nsplit *= 2;
  const int cps = (nchunks + nsplit - 1) / nsplit;
  nsplit = (nchunks + cps - 1) / cps;
  if (info) {
    if (FMT == FMT_BF16) snprintf(info->name, sizeof info->name, "er::k_wgemm<%d, %d, %d, %d>", MI, NR, KS, DEPTH);
    else snprintf(info->name, sizeof info->name, "er::k_wgemm<%d, %d, %d, %d, %d>", FMT, MI, NR, KS, DEPTH);
    info->nsplit = nsplit;
  }
  hipLaunchKernelGGL((k_wgemm<FMT, MI, NR, KS, DEPTH>), dim3((unsigned)(ntiles * nsplit * mtiles)), dim3(512), 0, st, a,
                     ws.partial, nsplit, cps, mtiles);
  if (hipGetLastError() != hipSuccess) return -3;
  if (nsplit > 1) {
    const long waves = (long)a.M * ((a.W.N + 63) / 64);
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, a, ws.partial, nsplit);
    if (hipGetLastError() != hipSuccess) return -3;
  }
  return 0;
}

// The weight-streaming GEMM for the weights' format.
template <int MI, int NR, int KS, int DEPTH>
static int run_wgemm(const LinArgs& a, const LinearWs& ws, int want_wgs, hipStream_t st, LinearInfo* info) {
  switch (a.W.fmt) {
    case FMT_BF16: return run_wgemm_fmt<FMT_BF16, MI, NR, KS, DEPTH>(a, ws, want_wgs, st, info);
    case FMT_W8: return run_wgemm_fmt<FMT_W8, MI, NR, KS, DEPTH>(a, ws, want_wgs, st, info);
    case FMT_W4: return run_wgemm_fmt<FMT_W4, MI, NR, KS, DEPTH>(a, ws, want_wgs, st, info);
  }
  return -1;
}

// Explicit weight-streaming variant: code = 3000 + 100*MI(1 digit: 2,4,8; 0 = 16) + 10*KS + 10000*NR... kept
// simple: code = 30000 + 1000*NR + 100*KS + 10*DEPTH + MI index (0: MI 2, 1: 4, 2: 8, 3: 16);
// want_wgs comes from the caller.
static int run_wgemm_variant(int code, const LinArgs& a, const LinearWs& ws, hipStream_t st, LinearInfo* info) {
  const int nr = (code / 1000) % 10, ks = (code / 100) % 10, dp = (code / 10) % 10, mix = code % 10;
  const int want = 512;
#define ER_W(MI_, NR_, KS_, D_, IX_) \
  if (mix == IX_ && nr == NR_ && ks == KS_ && dp == D_) return run_wgemm<MI_, NR_, KS_, D_>(a, ws, want, st, info);
  ER_W(2, 1, 4, 2, 0) ER_W(2, 1, 4, 3, 0) ER_W(2, 2, 4, 2, 0) ER_W(2, 1, 2, 3, 0)
  ER_W(4, 1, 2, 2, 1) ER_W(4, 1, 2, 3, 1) ER_W(4, 2, 2, 2, 1) ER_W(4, 1, 1, 3, 1)
  ER_W(8, 1, 1, 2, 2) ER_W(8, 1, 1, 3, 2)
  ER_W(16, 1, 1, 2, 3) ER_W(16, 1, 1, 3, 3)
#undef ER_W
  return -1;
}

// ----------------------------------------------------------------------------
// Deep-pipelined tiled GEMM for bf16 weights, M > 16: BM x 128 output tile
// per work-group of 8 waves (WM x WN waves, each (BM/WM) x (128/WN)), K steps
// of 64.  Both operands go global -> register ring (DEPTH steps ahead) ->
// LDS (double buffer) -> MFMA.  x and W of a step are issued together, so the
// wait before a step's LDS store never covers loads of later steps: DEPTH - 2
// steps of latency stay hidden.  Split-K partials go through
// k_splitk_reduce, as for k_gemm_bf16.
// ----------------------------------------------------------------------------
template <int BM, int WM, int DEPTH, int BK>
__global__ __launch_bounds__(512) void k_gemm2(LinArgs a, float* __restrict__ part, int nsplit, int sps, int mtiles) {
  constexpr int BN = 128, LDA = BK + 8;
  constexpr int KK = BK / 32;                 // 32-wide k slices per step
  constexpr int WN = 8 / WM;
  constexpr int TM = BM / WM, TN = BN / WN;   // wave tile
  constexpr int FM = TM / 16, FN = TN / 16;   // 16x16 fragments per wave
  constexpr int XV = BM * BK / 8 / 512;       // uint4 of x per thread per step
  constexpr int WV = BN * BK / 8 / 512;       // uint4 of W per thread per step
  constexpr int CPR = BK / 8;                 // 16-byte pieces per tile row
  static_assert(XV >= 1 && WV >= 1 && BK % 32 == 0, "tile does not split over 512 threads");
  // one LDS array, carved explicitly: the epilogue overlays its C tile on the
  // operand buffers, which needs their order and adjacency to be fixed
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * BM * LDA + 2 * BN * LDA];
  uint16_t (*As)[BM * LDA] = reinterpret_cast<uint16_t (*)[BM * LDA]>(smem);
  uint16_t (*Bs)[BN * LDA] = reinterpret_cast<uint16_t (*)[BN * LDA]>(smem + 2 * BM * LDA);

  const int b = blockIdx.x, nwg = gridDim.x;
  const int xcd = b & 7, loc = b >> 3, per = nwg >> 3, rem = nwg & 7;
  const int L = (xcd < rem) ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
  const int mt = L % mtiles;
  const int t2 = L / mtiles;
  const int sp = t2 % nsplit;
  const int nt = t2 / nsplit;
  const int M = a.M, N = a.W.N, K = a.W.K;
  const int m0 = mt * BM, n0 = nt * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int kb = lane >> 4, l16 = lane & 15;
  const int wm = wave / WN, wn = wave % WN;
  const int nsteps = K / BK;
  const int s0 = sp * sps;
  const int s1 = min(nsteps, s0 + sps);
  const int T = s1 - s0;
  const uint16_t* __restrict__ W = (const uint16_t*)a.W.w;
  const uint16_t* __restrict__ X = (const uint16_t*)a.x;

  if (b == 0 && a.ssq_zero && nsplit == 1)
    ssq_clear(a, tid, 512);

  // per-thread load slots: row = e / 8, 16-byte column c8 = e % 8
  long wsrc[WV];
  bool wok[WV];
#pragma unroll
  for (int v = 0; v < WV; ++v) {
    const int e = tid + 512 * v, row = e / CPR;
    wok[v] = n0 + row < N;
    // rows past the end load row N-1 (always in bounds) and are zeroed when stashed
    const int nr = wok[v] ? n0 + row : N - 1;
    wsrc[v] = (long)phys_row(a, nr >> 4, nr & 15) * K + (e % CPR) * 8;
  }
  long xsrc[XV];
  bool xok[XV];
#pragma unroll
  for (int v = 0; v < XV; ++v) {
    const int e = tid + 512 * v, row = e / CPR;
    const int m = m0 + row;
    xok[v] = m < M;
    const int mr = xok[v] ? m : M - 1;
    xsrc[v] = (long)(a.xrow ? a.xrow[mr] : mr) * a.ldx + (e % CPR) * 8;
  }

  uint4 wr[DEPTH][WV], xr[DEPTH][XV];
  // Loads are unpredicated (clamped rows, a clamped step index): exec-masked
  // loads inside the ring make the compiler drain the whole load counter at
  // every use instead of waiting for the oldest stage only.
  auto issue = [&](int t, int slot) {
    const long k0 = (long)(s0 + t) * BK;
#pragma unroll
    for (int v = 0; v < XV; ++v) xr[slot][v] = *(const uint4*)(X + xsrc[v] + k0);
#pragma unroll
    for (int v = 0; v < WV; ++v) wr[slot][v] = *(const uint4*)(W + wsrc[v] + k0);
  };
  // out-of-range rows are cleared with a mask (a select here would become a
  // select of addresses and push the ring into scratch memory)
  uint32_t xmask[XV], wmask[WV];
#pragma unroll
  for (int v = 0; v < XV; ++v) xmask[v] = xok[v] ? 0xFFFFFFFFu : 0u;
#pragma unroll
  for (int v = 0; v < WV; ++v) wmask[v] = wok[v] ? 0xFFFFFFFFu : 0u;
  auto and4 = [](uint4 q, uint32_t m) { return uint4{q.x & m, q.y & m, q.z & m, q.w & m}; };
  auto stash = [&](int slot, int buf) {
#pragma unroll
    for (int v = 0; v < XV; ++v) {
      const int e = tid + 512 * v;
      *(uint4*)(&As[buf][(e / CPR) * LDA + (e % CPR) * 8]) = and4(xr[slot][v], xmask[v]);
    }
#pragma unroll
    for (int v = 0; v < WV; ++v) {
      const int e = tid + 512 * v;
      *(uint4*)(&Bs[buf][(e / CPR) * LDA + (e % CPR) * 8]) = and4(wr[slot][v], wmask[v]);
    }
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto mma = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *(const bf16x8_t*)(&As[buf][(TM * wm + 16 * i + l16) * LDA + 32 * kk + 8 * kb]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *(const bf16x8_t*)(&Bs[buf][(TN * wn + 16 * j + l16) * LDA + 32 * kk + 8 * kb]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  if (T > 0) {
    const int tl = T - 1;
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d)
      if (d < T) issue(d, d);
    stash(0, 0);
    __syncthreads();
    // Whole groups of 2 * DEPTH steps run without any condition, so that the
    // load counter is the same on every path and each stash waits for its
    // own stage only.  Re-issues of the last stage and the stash after the
    // last step touch data nobody reads.
    int t0 = 0;
    for (; t0 + 2 * DEPTH <= T; t0 += 2 * DEPTH) {
#pragma unroll
      for (int d = 0; d < 2 * DEPTH; ++d) {
        issue(min(t0 + d + DEPTH - 1, tl), (d + DEPTH - 1) % DEPTH);
        __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the math
        mma(d & 1);
        stash((d + 1) % DEPTH, (d + 1) & 1);
        lds_barrier();
      }
    }
#pragma unroll
    for (int d = 0; d < 2 * DEPTH; ++d) {
      const int t = t0 + d;
      if (t < T) {
        if (t + DEPTH - 1 < T) issue(t + DEPTH - 1, (d + DEPTH - 1) % DEPTH);
        mma(d & 1);
        if (t + 1 < T) stash((d + 1) % DEPTH, (d + 1) & 1);
        lds_barrier();
      }
    }
  }

  // epilogue through LDS (overlaying the operand buffers): row-wise walk,
  // pair partners at column ^ 8, one sum-of-squares partial per (row, 64 cols)
  constexpr int CLD = BN + 4;
  // rows per pass so that the C tile fits in the operand buffers
  constexpr int NPASS0 = (sizeof(float) * BM * CLD + sizeof(smem) - 1) / sizeof(smem);
  constexpr int NPASS = NPASS0 <= 1 ? 1 : NPASS0 <= 2 ? 2 : NPASS0 <= 4 ? 4 : 8;  // a power of two divides BM
  constexpr int RP = BM / NPASS;
  static_assert(BM % NPASS == 0 && RP % TM == 0, "epilogue passes must hold whole wave tiles");
  static_assert(sizeof(float) * RP * CLD <= sizeof(smem), "C tile pass does not fit");
  float* Cs = reinterpret_cast<float*>(smem);
  const bool want_ssq = a.epi == EPI_RESID && a.ssq_acc && nsplit == 1;
#pragma unroll
  for (int pass = 0; pass < NPASS; ++pass) {
    if (pass > 0) __syncthreads();
    if ((TM * wm) / RP == pass) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            Cs[(TM * wm - pass * RP + 16 * i + 4 * kb + r) * CLD + TN * wn + 16 * j + l16] = acc[i][j][r];
    }
    __syncthreads();
    for (int e = tid; e < RP * BN; e += 512) {
      const int row = e >> 7, col = e & 127;
      const int m = m0 + pass * RP + row, nl = n0 + col;
      const bool mok = m < M, nok = nl < N;
      const int n = nok ? phys_row(a, nl >> 4, nl & 15) : N;
      const float v = Cs[row * CLD + col];
      float sq = 0.f;
      if (nsplit > 1) {
        if (mok && nok) part[((long)sp * M + m) * N + n] = v;
      } else {
        epilogue(a, m, n, v, Cs[row * CLD + (col ^ 8)], mok && nok, nl & 15);
        if (want_ssq && mok && nok) {
          const float hn = ((const float*)a.y)[(long)m * a.ldy + n];
          sq = hn * hn;
        }
      }
      if (want_ssq) {
        sq += __shfl_xor(sq, 16, 64);
        sq += __shfl_xor(sq, 32, 64);
        ssq_add(a, m, sq, lane == 0, mok);
      }
    }
  }
}

template <int BM, int WM, int DEPTH, int BK = 64>
static int run_gemm2(const LinArgs& a, const LinearWs& ws, int want_wgs, hipStream_t st, LinearInfo* info) {
  if (a.W.fmt != FMT_BF16 || a.xnorm || a.W.K % BK) return -1;
  const int mtiles = (a.M + BM - 1) / BM;
  const long ntiles = (a.W.N + 127) / 128;
  const int nsteps = a.W.K / BK;
  const long base = (long)mtiles * ntiles;
  int nsplit = 1;
  while (base * nsplit * 2 <= want_wgs && nsteps / (nsplit * 2) >= 512 / BK &&
         (size_t)(nsplit * 2) * a.M * a.W.N <= ws.partial_floats && ws.partial)
    nsplit *= 2;
  const int sps = (nsteps + nsplit - 1) / nsplit;
  nsplit = (nsteps + sps - 1) / sps;
  if (info) {
    snprintf(info->name, sizeof info->name, "er::k_gemm2<%d, %d, %d, %d>", BM, WM, DEPTH, BK);
    info->nsplit = nsplit;
  }
  hipLaunchKernelGGL((k_gemm2<BM, WM, DEPTH, BK>), dim3((unsigned)(base * nsplit)), dim3(512), 0, st, a, ws.partial,
                     nsplit, sps, mtiles);
  if (hipGetLastError() != hipSuccess) return -3;
  if (nsplit > 1) {
    const long waves = (long)a.M * ((a.W.N + 63) / 64);
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, a, ws.partial, nsplit);
    if (hipGetLastError() != hipSuccess) return -3;
  }
  return 0;
}

// Explicit deep-pipelined GEMM variant: code = 40000 + 100*ix + 10*DEPTH +
// want_wgs/256, ix = 1, 2, 3: BM = 64, 128, 256 with 64-wide k steps; ix = 5:
// BM = 128 with 32-wide k steps (deeper rings at the same register cost)
static int run_gemm2_variant(int code, const LinArgs& a, const LinearWs& ws, hipStream_t st, LinearInfo* info) {
  const int ix = (code / 100) % 10, dp = (code / 10) % 10, want = 256 * (code % 10);
#define ER_G(BM_, WM_, IX_, D_) \
  if (ix == IX_ && dp == D_) return run_gemm2<BM_, WM_, D_>(a, ws, want, st, info);
  ER_G(64, 1, 1, 4) ER_G(64, 1, 1, 6) ER_G(128, 2, 2, 3) ER_G(128, 2, 2, 4)
  ER_G(128, 2, 2, 6) ER_G(256, 4, 3, 3) ER_G(256, 4, 3, 4)
#undef ER_G
#define ER_G32(BM_, WM_, IX_, D_) \
  if (ix == IX_ && dp == D_) return run_gemm2<BM_, WM_, D_, 32>(a, ws, want, st, info);
  ER_G32(128, 2, 5, 6) ER_G32(128, 2, 5, 8)
#undef ER_G32
#define ER_G128(BM_, WM_, IX_, D_) \
  if (ix == IX_ && dp == D_) return run_gemm2<BM_, WM_, D_, 128>(a, ws, want, st, info);
  ER_G128(64, 1, 6, 2) ER_G128(64, 1, 6, 3) ER_G128(64, 1, 6, 4) ER_G128(128, 2, 7, 2) ER_G128(128, 2, 7, 3)
#undef ER_G128
  return -1;
}

// ----------------------------------------------------------------------------
template <int FMT, int MT, int NR, int KS>
static int run_mfma(const LinArgs& a, hipStream_t st, LinearInfo* info) {
  constexpr int R = 16 * NR * (8 / KS);
  const int mtiles = (a.M + MT - 1) / MT;
  const long ntiles = (a.W.N + R - 1) / R;
  const long nwg = ntiles * mtiles;
  if (nwg > 0x7FFFFFFF) return -1;
  if (info) {
    snprintf(info->name, sizeof info->name, "er::k_linear_mfma<%d, %d, %d, %d>", FMT, MT, NR, KS);
    info->nsplit = KS;
  }
  hipLaunchKernelGGL((k_linear_mfma<FMT, MT, NR, KS>), dim3((unsigned)nwg), dim3(512), 0, st, a, mtiles);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Explicit variant (tuning / tests): code = 1000 + 100*NR + 10*KS + MT/16.
template <int FMT>
static int run_variant(int code, const LinArgs& a, hipStream_t st, LinearInfo* info) {
  const int nr = (code / 100) % 10, ks = (code / 10) % 10, mt = 16 * (code % 10);
  if (a.M > mt) return -1;
#define ER_V(NR_, KS_, MT_) \
  if (nr == NR_ && ks == KS_ && mt == MT_) return run_mfma<FMT, MT_, NR_, KS_>(a, st, info);
#define ER_VK(NR_, MT_) ER_V(NR_, 1, MT_) ER_V(NR_, 2, MT_) ER_V(NR_, 4, MT_) ER_V(NR_, 8, MT_)
  ER_VK(1, 16) ER_VK(2, 16) ER_VK(4, 16) ER_VK(1, 32) ER_VK(2, 32)
#undef ER_VK
#undef ER_V
  return -1;
}

// Automatic choice, from a sweep of the 7B-shaped projections on MI355X:
// splitting K over all 8 waves wins at M <= 16 for every width; two 16-row
// subtiles per wave pay off for wide outputs (and for the quantized formats,
// whose x fragments are relatively expensive); M in 17..32 uses 32-row
// m-tiles; larger M goes to the tiled GEMM (bf16) .
template <int FMT>
static int dispatch_mfma(const LinArgs& a, hipStream_t st, LinearInfo* info) {
  const bool wide = a.W.N >= 16384;
  if (a.M <= 16) {
    if (wide || (FMT != FMT_BF16 && a.W.N >= 4096)) return run_mfma<FMT, 16, 2, 8>(a, st, info);
    return run_mfma<FMT, 16, 1, 8>(a, st, info);
  }
  if (wide) return run_mfma<FMT, 32, 2, 4>(a, st, info);
  return run_mfma<FMT, 32, 1, 8>(a, st, info);
}

// Automatic choice among the streaming variants, from a sweep of the Qwen2.5-7B
// projections on MI355X with weights rotating through more than the 256 MB
// last-level cache (M = 1 and 4): 2-deep rings for bf16 (its 16-byte stages
// already keep enough bytes in flight), K split over all 8 waves for narrow
// outputs and over 2 or 4 for wide ones; the W4 drafter wants 3-4 deep rings
// on its long-K and wide layers.
template <int FMT>
static int dispatch_skinny(const LinArgs& a, hipStream_t st, LinearInfo* info) {
  const int N = a.W.N, K = a.W.K;
  if constexpr (FMT == FMT_BF16) {
    if (N >= 65536) return a.M <= 2 ? run_skinny<FMT, 1, 2, 2>(a, st, info) : run_skinny<FMT, 2, 2, 2>(a, st, info);
    if (N >= 16384) return run_skinny<FMT, 1, 2, 2>(a, st, info);
    if (N >= 4096) return run_skinny<FMT, 1, 4, 2>(a, st, info);
    return run_skinny<FMT, 1, 8, 2>(a, st, info);
  } else {
    if (K >= 8192) return run_skinny<FMT, 1, 8, 4>(a, st, info);
    // 64 rows per work-group: their scale/zero pairs must fit beside x' (the caller checked 16 rows)
    if (N >= 8192 && skinny_lds(FMT, a.M, K, 1, 2).total <= kSkinnyLdsMax) return run_skinny<FMT, 1, 2, 3>(a, st, info);
    return run_skinny<FMT, 1, 8, 2>(a, st, info);
  }
}

// Automatic kernel choice (bf16 weights by M; the quantized drafter formats
// use the streaming kernel while x' fits in LDS).  From sweeps of the
// Qwen2.5-7B projections on MI355X with weights rotating through more than the
// 256 MB last-level cache: the streaming kernel up to M = 8 (and for the
// narrower layers up to 16), the deep-pipelined GEMM for long K and for the
// vocabulary projection from M = 9 and for everything from M = 33, the
// weight-streaming GEMM for the wide layers in between, and the register-fed
// kernel for the square attention output projection up to M = 32.
enum Plan { P_STREAM, P_SKINNY_OLD, P_WGEMM, P_GEMM2, P_GEMM };

static Plan plan_of(const LinArgs& a) {
  const int M = a.M, N = a.W.N, K = a.W.K;
  const size_t lds = skinny_lds(a.W.fmt, M, K, 1, 8).total;
  const bool stream_fits = M <= 16 && lds <= kSkinnyLdsMax;
  if (a.W.fmt != FMT_BF16) {
    if (stream_fits && (M <= 8 || N >= 65536 || (N >= 16384 && M <= 12))) return P_STREAM;
    // above 16 rows the weight-streaming GEMM (each quantized weight read once per 32- or 64-row
    // m-tile, converted once for the tile's rows; any M, in m-tiles), except the narrow square layers at <= 32 rows,
    // where the register-fed kernel was faster (W4 O projection at M = 22: 10.6 vs 14.4 us)
    if (M > 16 && !(M <= 32 && N <= 4096 && K <= 4096)) return P_WGEMM;
    return P_SKINNY_OLD;
  }
  if (M <= 8 && stream_fits) return P_STREAM;
  if (K % 64) return P_SKINNY_OLD;
  if (M <= 8) return P_GEMM2;  // long K (x' does not fit in LDS)
  if (M <= 32) {
    if (N < 4096) return K >= 8192 ? P_GEMM2 : P_SKINNY_OLD;
    if (N >= 65536) return P_GEMM2;
    if (M <= 16 && N < 16384 && stream_fits) return P_STREAM;
    return P_WGEMM;
  }
  if (M <= 256) return P_GEMM2;
  return P_GEMM;
}

template <int FMT>
static int run_stream_auto(const LinArgs& a, hipStream_t st, LinearInfo* info) {
  const int N = a.W.N, K = a.W.K, M = a.M;
  if constexpr (FMT == FMT_BF16) {
    if (M > 8) {
      if (N >= 65536) return run_skinny<FMT, 2, 2, 3>(a, st, info);
      if (N >= 16384) return run_skinny<FMT, 1, 2, 2>(a, st, info);
      return run_skinny<FMT, 1, 4, 2>(a, st, info);
    }
    return dispatch_skinny<FMT>(a, st, info);
  } else {
    if (M > 8) {
      // the work-group's scale/zero pairs grow with its rows (16 * NR * 8 / KS): take the widest
      // variant whose LDS still fits (the caller checked the 16-row one)
      auto fits = [&](int nr, int ks) { return skinny_lds(FMT, M, K, nr, ks).total <= kSkinnyLdsMax; };
      if (N >= 65536 && fits(2, 2)) return run_skinny<FMT, 2, 2, 3>(a, st, info);
      if (fits(4, 2)) return run_skinny<FMT, 4, 2, 3>(a, st, info);
      if (fits(2, 2)) return run_skinny<FMT, 2, 2, 3>(a, st, info);
      if (fits(1, 2)) return run_skinny<FMT, 1, 2, 3>(a, st, info);
      return run_skinny<FMT, 1, 8, 2>(a, st, info);
    }
    return dispatch_skinny<FMT>(a, st, info);
  }
}

static int run_auto(const LinArgs& a, const LinearWs& ws, Plan p, hipStream_t st, LinearInfo* info) {
  const int M = a.M, N = a.W.N, K = a.W.K;
  switch (p) {
    case P_STREAM:
      switch (a.W.fmt) {
        case FMT_BF16: return run_stream_auto<FMT_BF16>(a, st, info);
        case FMT_W8: return run_stream_auto<FMT_W8>(a, st, info);
        case FMT_W4: return run_stream_auto<FMT_W4>(a, st, info);
      }
      return -1;
    case P_WGEMM:
      if (a.W.fmt != FMT_BF16) {
        // W4 at the 7B shape (us; register-fed kernel / 32-row tiles, 64 rows per group / 64-row tiles,
        // 128 rows per group): QKV at M = 46 29.7 / 19.7 / 20.0, at 204 74.6 / 28.6 / 38.4; gate/up at
        // 22 60.3 / 49.1 / 57.8, at 46 110.0 / 72.7 / 60.5, at 204 354.1 / 211.9 / 167.6; down at 46
        // 82.6 / 40.1 / 33.1, at 204 268.2 / 119.4 / 86.5.  128-row tiles were slower still.
        if (M <= 32 || (N <= 8192 && K <= 4096)) return run_wgemm<2, 1, 2, 3>(a, ws, 512, st, info);
        return run_wgemm<4, 1, 1, 3>(a, ws, 512, st, info);
      }
      if (M <= 32) return run_wgemm<2, 1, 4, 3>(a, ws, 512, st, info);
      return run_wgemm<4, 1, 1, 3>(a, ws, 512, st, info);
    case P_GEMM2:
      // split K until about one wave of work-groups (256): more splits cost
      // more in the reduction than they gain in parallelism
      // 257..384 column tiles (7B gate/up: 296) overfill one wave of the chip
      // by a fraction: a two-way split evens the tail (8 % at M = 33).  Below
      // 256 tiles (14B gate/up: 216) the split costs 14 % instead.
      if (M <= 64) {
        const long nt = (N + 127) / 128;
        return run_gemm2<64, 1, 4>(a, ws, nt > 256 && nt <= 384 ? 768 : 256, st, info);
      }
      if (M <= 128) {
        if (K < 8192 && (N < 4096 || (N >= 16384 && N < 65536))) return run_gemm2<64, 1, 6>(a, ws, 256, st, info);
        return run_gemm2<128, 2, 3>(a, ws, 256, st, info);
      }
      if (K >= 8192) return run_gemm2<256, 4, 3>(a, ws, 256, st, info);
      if (N >= 65536) return run_gemm2<256, 4, 3>(a, ws, 512, st, info);
      if (N >= 16384) return run_gemm2<128, 2, 6, 32>(a, ws, 256, st, info);
      return run_gemm2<128, 2, 4>(a, ws, 256, st, info);
    case P_GEMM:
      return run_gemm(a, ws, st, info);
    case P_SKINNY_OLD:
      switch (a.W.fmt) {
        case FMT_BF16: return dispatch_mfma<FMT_BF16>(a, st, info);
        case FMT_W8: return dispatch_mfma<FMT_W8>(a, st, info);
        case FMT_W4: return dispatch_mfma<FMT_W4>(a, st, info);
      }
      return -1;
  }
  return -1;
}

// x' = bf16(RMSNorm(h[xrow[m]]) * g) materialized for the kernels that read
// bf16 x, with the row's 1/rms from the producers' fixed-point sums of
// squares (no second pass over h).  Work-group (m, c) covers 2048 columns of
// row m, 8 per thread; the h loads are issued before the barrier that
// publishes 1/rms.
__global__ __launch_bounds__(256) void k_xnorm(LinArgs a, uint16_t* __restrict__ xn) {
  __shared__ float rs_sh;
  const int m = blockIdx.x, tid = threadIdx.x;
  const int K = a.W.K;
  const long hrow = a.xrow ? a.xrow[m] : m;
  const int k0 = (blockIdx.y * 256 + tid) * 8;
  const bool ok = k0 < K;
  const int kc = ok ? k0 : 0;
  const float* hp = (const float*)a.x + hrow * a.ldx + kc;
  const uint4 h0 = *(const uint4*)hp, h1 = *(const uint4*)(hp + 4);
  const uint4 g = *(const uint4*)((const uint16_t*)a.gnorm + kc);
  if (tid < 16) {
    unsigned long long t = tid < ssq_nslots(a) ? a.ssq_in[(long)tid * a.ssq_stride + hrow] : 0ull;
    t += __shfl_xor(t, 1, 64);
    t += __shfl_xor(t, 2, 64);
    t += __shfl_xor(t, 4, 64);
    t += __shfl_xor(t, 8, 64);
    if (tid == 0) rs_sh = 1.0f / sqrtf((float)((double)t / SSQ_SCALE) / (float)K + a.eps);
  }
  __syncthreads();
  if (!ok) return;
  const float rs = rs_sh;
  uint4 o;
  o.x = f2bf(__uint_as_float(h0.x) * rs * bf_lo(g.x)) | (f2bf(__uint_as_float(h0.y) * rs * bf_hi(g.x)) << 16);
  o.y = f2bf(__uint_as_float(h0.z) * rs * bf_lo(g.y)) | (f2bf(__uint_as_float(h0.w) * rs * bf_hi(g.y)) << 16);
  o.z = f2bf(__uint_as_float(h1.x) * rs * bf_lo(g.z)) | (f2bf(__uint_as_float(h1.y) * rs * bf_hi(g.z)) << 16);
  o.w = f2bf(__uint_as_float(h1.z) * rs * bf_lo(g.w)) | (f2bf(__uint_as_float(h1.w) * rs * bf_hi(g.w)) << 16);
  *(uint4*)(xn + (long)m * K + k0) = o;
}

// After a library GEMM that added x W^T into h: each row's sum of squares
// into slot 0 of ssq_acc (partial sums of 256 threads, each converted to
// fixed point, added as integers, so the total does not depend on the order)
// and the consumed buffer ssq_zero cleared for the rows, as the fused
// residual epilogues do.
__global__ __launch_bounds__(256) void k_resid_ssq(LinArgs a) {
  const int m = blockIdx.x, tid = threadIdx.x;
  if (a.ssq_zero && tid < ssq_nslots(a)) a.ssq_zero[(long)tid * a.ssq_stride + m] = 0ull;
  if (!a.ssq_acc) return;
  const float* h = (const float*)a.y + (long)m * a.ldy;
  float sq = 0.f;
  for (int k = tid * 4; k < a.W.N; k += 256 * 4) {
    const float4 v = *(const float4*)(h + k);
    sq = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, sq))));
  }
  unsigned long long t = (unsigned long long)rint((double)sq * SSQ_SCALE);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o, 64);
  __shared__ unsigned long long part[4];
  if ((tid & 63) == 0) part[tid >> 6] = t;
  __syncthreads();
  if (tid == 0) atomicAdd(a.ssq_acc + m, part[0] + part[1] + part[2] + part[3]);
}

// Large-M bf16 projections through the library GEMM (blas.hip), with the
// epilogue as its own kernel: x' formed once (k_xnorm) when normalizing on
// load; QKV and gate/up land in fp32 in ws.blas_out for RoPE + the KV append
// and SwiGLU; the residual projections add into h (beta = 1) and then sum its
// squares; logits are written directly.  Returns 1 when the case does not
// apply (the hand-written kernels run): below the shape's row threshold
// (blas_wins, or a fixed blas_min_m; the long-K down projection always below
// 1024 rows), gathered rows without the norm, or while the stream is being
// captured (recorded graphs hold the hand-written kernels only).
// Rows from which the library's GEMM beats the hand-written kernels, by
// shape (same-box sweeps of the Qwen2.5-7B projections on MI355X, library
// time / hand-written time): output widths from 16384 (gate/up: 0.89 at 16
// rows, 0.61 at 96) from 16 rows; the vocabulary projection from 48 (0.93 at
// 46); widths from 4096 (QKV: 0.90 at 80) from 80; narrower ones (the square
// O projection) from 17: with the library's algorithm chosen by timing, the
// whole AR step ran 1.4-3.2 % faster at 17-32 rows and 1.1 % at 48-64 with
// the O projection on the library, and the same from 96 to 192; K from 8192
// (down: 1.5-2.6 below 1024 rows; the AR step 8-16 % slower with it on the
// library at 17-192 rows) from 1024.
static bool blas_wins(int M, int N, int K) {
  if (K >= 8192) return M >= 1024;
  if (N >= 65536) return M >= 48;
  if (N >= 16384) return M >= 16;
  if (N >= 4096) return M >= 80;
  return M >= 17;
}

static int run_blas(const LinArgs& a, const LinearWs& ws, hipStream_t st, LinearInfo* info) {
  const int M = a.M, N = a.W.N, K = a.W.K;
  if (!ws.blas || ws.blas_min_m == 0 || a.W.fmt != FMT_BF16 || !a.act_bf16) return 1;
  if (ws.blas_min_m < 0 ? !blas_wins(M, N, K) : (M < ws.blas_min_m || (K >= 8192 && M < 1024))) return 1;
  if (!a.xnorm && a.xrow) return 1;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) return 1;
  float* out = nullptr;
  int ldo = 0;
  float beta = 0.f;
  const char* what = nullptr;
  switch (a.epi) {
    case EPI_F32:
      if (a.ssq_zero || a.ssq_acc) return 1;
      out = (float*)a.y;
      ldo = a.ldy;
      what = "logits";
      break;
    case EPI_RESID:
      out = (float*)a.y;
      ldo = a.ldy;
      beta = 1.f;
      what = "residual";
      if (a.ldy % 4 != 0 || N % 4 != 0) return 1;
      break;
    case EPI_QKV:
    case EPI_SWIGLU:
      if (a.ssq_zero || a.ssq_acc || !ws.blas_out || (size_t)M * N > ws.blas_out_floats) return 1;
      if (a.epi == EPI_SWIGLU && a.ldy != a.F) return 1;
      out = ws.blas_out;
      ldo = N;
      what = a.epi == EPI_QKV ? "rope_kv" : "swiglu";
      break;
    default:
      return 1;
  }
  const void* x = a.x;
  int ldx = a.ldx;
  if (a.xnorm) {
    if (!ws.xn || (size_t)M * K > ws.xn_elems) return 1;
    hipLaunchKernelGGL(k_xnorm, dim3(M, (K + 2047) / 2048), dim3(256), 0, st, a, ws.xn);
    if (hipGetLastError() != hipSuccess) return -3;
    x = ws.xn;
    ldx = K;
  }
  const int r = blas_gemm(ws.blas, x, ldx, M, a.W.w, N, K, out, ldo, true, beta, st);
  if (r != 0) return r;  // 1: no algorithm for the shape, the hand-written kernels run
  int e = 0;
  if (a.epi == EPI_QKV)
    e = launch_rope_kv(ws.blas_out, M, a.hq, a.hkv, a.hd, a.pos, a.slot, a.cs, a.qout, a.kv_pool, a.layer,
                       a.n_layers, true, st);
  else if (a.epi == EPI_SWIGLU)
    e = launch_swiglu(ws.blas_out, M, a.F, a.y, true, st);
  else if (a.epi == EPI_RESID && (a.ssq_acc || a.ssq_zero)) {
    hipLaunchKernelGGL(k_resid_ssq, dim3(M), dim3(256), 0, st, a);
    e = hipGetLastError() == hipSuccess ? 0 : -3;
  }
  if (e) return e;
  if (info) {
    snprintf(info->name, sizeof info->name, "hipblaslt::gemm_bf16+%s", what);
    info->nsplit = 1;
  }
  return 0;
}

int launch_linear_fused(const LinArgs& a, const LinearWs& ws, int path, hipStream_t st, LinearInfo* info) {
  if (a.M <= 0 || a.W.N <= 0) return 0;
  if (a.ssq_slots > kMaxSsqSlots || (a.ssq_slots > 1 && a.ssq_stride < a.M)) return -1;
  if (a.W.K % 128 != 0 || (!a.xnorm && a.ldx % 8 != 0) || (a.xnorm && a.ldx % 4 != 0)) return -1;
  if ((a.epi == EPI_SWIGLU && a.W.N != 2 * a.F) ||
      (a.epi == EPI_QKV && (a.W.N != (a.hq + 2 * a.hkv) * a.hd || a.hd % 16 != 0)))
    return -1;
  if (a.epi == EPI_SWIGLU && a.F % 8 != 0) return -1;
  const bool gemm_ok = a.W.fmt == FMT_BF16 && a.W.K % GB_K == 0 && ws.partial != nullptr;
  if (path == 0) {
    const int r = run_blas(a, ws, st, info);
    if (r != 1) return r;
  }
  if (path == 3) {
    if (!gemm_ok) return -1;
    return run_gemm(a, ws, st, info);
  }
  if (path >= 40000) return run_gemm2_variant(path, a, ws, st, info);
  if (path >= 30000) return run_wgemm_variant(path, a, ws, st, info);
  if (path >= 2000) {
    switch (a.W.fmt) {
      case FMT_BF16: return run_skinny_variant<FMT_BF16>(path, a, st, info);
      case FMT_W8: return run_skinny_variant<FMT_W8>(path, a, st, info);
      case FMT_W4: return run_skinny_variant<FMT_W4>(path, a, st, info);
    }
    return -1;
  }
  if (path >= 1000) {
    switch (a.W.fmt) {
      case FMT_BF16: return run_variant<FMT_BF16>(path, a, st, info);
      case FMT_W8: return run_variant<FMT_W8>(path, a, st, info);
      case FMT_W4: return run_variant<FMT_W4>(path, a, st, info);
    }
    return -1;
  }
  if (path == 2) {  // the register-fed skinny kernel, any M (32-row m-tiles)
    switch (a.W.fmt) {
      case FMT_BF16: return dispatch_mfma<FMT_BF16>(a, st, info);
      case FMT_W8: return dispatch_mfma<FMT_W8>(a, st, info);
      case FMT_W4: return dispatch_mfma<FMT_W4>(a, st, info);
    }
    return -1;
  }
  Plan p = plan_of(a);
  if ((p == P_GEMM || p == P_GEMM2 || (p == P_WGEMM && a.W.fmt == FMT_BF16)) && !gemm_ok) p = P_SKINNY_OLD;
  if (p == P_WGEMM && !ws.partial) p = P_SKINNY_OLD;
  if (a.xnorm && p != P_STREAM) {
    // these kernels read bf16 x: form x' = RMSNorm(h) * g once, in the workspace
    if (ws.xn && (size_t)a.M * a.W.K <= ws.xn_elems) {
      hipLaunchKernelGGL(k_xnorm, dim3(a.M, (a.W.K + 2047) / 2048), dim3(256), 0, st, a, ws.xn);
      if (hipGetLastError() != hipSuccess) return -3;
      LinArgs b = a;
      b.x = ws.xn;
      b.ldx = a.W.K;
      b.xnorm = 0;
      b.xrow = nullptr;
      b.ssq_in = nullptr;
      return run_auto(b, ws, p, st, info);
    }
    if (p != P_SKINNY_OLD) p = (p == P_GEMM) ? P_GEMM : P_SKINNY_OLD;  // these two normalize on load themselves
    if (p == P_GEMM) return run_gemm(a, ws, st, info);
  }
  return run_auto(a, ws, p, st, info);
}

template <int FMT, bool XBF>
static int run_valu(const void* x, int ldx, int M, const LinearW& W, void* y, int ldy, int epi, hipStream_t st,
                    LinearInfo* info) {
  dim3 grid((W.N + 3) / 4, (M + 3) / 4);
  if (info) {
    snprintf(info->name, sizeof info->name, "er::k_linear_valu<%d, %s>", FMT, XBF ? "true" : "false");
    info->nsplit = 1;
  }
  hipLaunchKernelGGL((k_linear_valu<FMT, XBF>), grid, dim3(256), 0, st, x, ldx, M, W.w, W.scale, W.zero, W.N, W.K,
                     y, ldy, epi);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int launch_linear(const void* x, bool act_bf16, int ldx, int M, const LinearW& W, void* y, int ldy, int epi,
                  const LinearWs& ws, int path, hipStream_t st, LinearInfo* info) {
  if (M <= 0 || W.N <= 0) return 0;
  if (W.K % 4 != 0) return -1;
  if (W.fmt == FMT_W4 && W.K % 128 != 0) return -1;
  if (epi != EPI_F32 && epi != EPI_ACT && epi != EPI_RESID) return -1;
  const bool mfma_ok = act_bf16 && W.fmt != FMT_F32 && W.K % 128 == 0 && ldx % 8 == 0;
  if ((path >= 2) && !mfma_ok) return -1;
  if (mfma_ok && path != 1) {
    LinArgs a{};
    a.x = x;
    a.ldx = ldx;
    a.M = M;
    a.W = W;
    a.epi = epi;
    a.y = y;
    a.ldy = ldy;
    a.act_bf16 = act_bf16;
    return launch_linear_fused(a, ws, path, st, info);
  }
  if (act_bf16) {
    switch (W.fmt) {
      case FMT_F32: return run_valu<FMT_F32, true>(x, ldx, M, W, y, ldy, epi, st, info);
      case FMT_BF16: return run_valu<FMT_BF16, true>(x, ldx, M, W, y, ldy, epi, st, info);
      case FMT_W8: return run_valu<FMT_W8, true>(x, ldx, M, W, y, ldy, epi, st, info);
      case FMT_W4: return run_valu<FMT_W4, true>(x, ldx, M, W, y, ldy, epi, st, info);
    }
  } else {
    switch (W.fmt) {
      case FMT_F32: return run_valu<FMT_F32, false>(x, ldx, M, W, y, ldy, epi, st, info);
      case FMT_BF16: return run_valu<FMT_BF16, false>(x, ldx, M, W, y, ldy, epi, st, info);
      case FMT_W8: return run_valu<FMT_W8, false>(x, ldx, M, W, y, ldy, epi, st, info);
      case FMT_W4: return run_valu<FMT_W4, false>(x, ldx, M, W, y, ldy, epi, st, info);
    }
  }
  return -1;
}

}  // namespace er
