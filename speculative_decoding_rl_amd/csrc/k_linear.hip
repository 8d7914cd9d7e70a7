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
//    128-wide K chunk with row sums of x.  Split-K across work-groups with a
//    deterministic last-arriving-group reduction keeps >= ~4 groups per CU for
//    the narrow projections; the block index is remapped so that the m-tiles
//    sharing a weight tile land on the same XCD (and its L2).
//
// The drafter kernels are the dequant-fused GEMV/skinny-GEMM of the
// EfficientRollout page ("关键模块" item 1: W4/W8 drafter from the target's own
// weights); the verify kernels are the target's linears at M = B * (gamma+1).

#include "common.h"
#include "kernels.h"

namespace er {

// ----------------------------------------------------------------------------
// Dequantized weight element (kernel-order W4 layout), fp32.
// ----------------------------------------------------------------------------
template <int FMT>
ER_DEV float w_elem(const void* __restrict__ w, const void* __restrict__ s, const void* __restrict__ z,
                    long n, long k, long K) {
  if constexpr (FMT == FMT_F32) {
    return ((const float*)w)[n * K + k];
  } else if constexpr (FMT == FMT_BF16) {
    return bf2f(((const uint16_t*)w)[n * K + k]);
  } else if constexpr (FMT == FMT_W8) {
    return (float)((const int8_t*)w)[n * K + k] * ((const float*)s)[n];
  } else {
    const uint32_t word = ((const uint32_t*)w)[(n * K + k) >> 3];
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
    for (int t = 0; t < 4; ++t) wv[t] = w_elem<FMT>(w, s, z, n, k + t, K);
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
// MFMA skinny GEMM.
// ----------------------------------------------------------------------------
template <int FMT> struct WRegs { static constexpr int n = (FMT == FMT_BF16) ? 4 : (FMT == FMT_W8 ? 2 : 1); };

// LDS column (in bf16 elements within the 128-wide chunk) of the 8 k-slots that
// lane group kb feeds to MFMA number i; the same mapping decides which weight
// bytes a lane loads, so A and B agree on every k.
template <int FMT>
ER_DEV int kcol(int i, int kb) {
  if constexpr (FMT == FMT_BF16) return 32 * i + 8 * kb;
  else if constexpr (FMT == FMT_W8) return 64 * (i >> 1) + 16 * kb + 8 * (i & 1);
  else return 32 * kb + 8 * i;
}

// 8 int8 codes (two words) -> bf16 of (q + 128), exact.
ER_DEV bf16x8_t w8_to_bf16(uint32_t a, uint32_t b) {
  a ^= 0x80808080u;
  b ^= 0x80808080u;
  uint32_t r[4];
  const uint32_t src[2] = {a, b};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float f0 = (float)(src[h] & 0xFFu), f1 = (float)((src[h] >> 8) & 0xFFu);
    const float f2 = (float)((src[h] >> 16) & 0xFFu), f3 = (float)(src[h] >> 24);
    r[2 * h] = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
    r[2 * h + 1] = (__float_as_uint(f2) >> 16) | (__float_as_uint(f3) & 0xFFFF0000u);
  }
  return __builtin_bit_cast(bf16x8_t, *(const uint4*)r);
}

// One kernel-order W4 word (8 codes) -> bf16 of (q + 128), exact: the code
// lands in the mantissa of 128.0.
ER_DEV bf16x8_t w4_to_bf16(uint32_t w) {
  uint32_t r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = ((w >> (4 * j)) & 0x000F000Fu) | 0x43004300u;
  return __builtin_bit_cast(bf16x8_t, *(const uint4*)r);
}

template <int FMT, int MT, int NR>
__global__ __launch_bounds__(256) void k_linear_mfma(
    const uint16_t* __restrict__ x, int ldx, int M, const void* __restrict__ wv,
    const void* __restrict__ sv, const void* __restrict__ zv, int N, int K, void* __restrict__ yv,
    int ldy, int epi, int act_bf16, int mtiles, int nsplit, int cps, float* __restrict__ partial,
    int* __restrict__ counters) {
  constexpr int MI = MT / 16;
  constexpr int NT = 64 * NR;
  constexpr int LDSR = 136;  // 128 + 8 bf16 of padding per row
  constexpr int WR = WRegs<FMT>::n;
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][MT * LDSR];
  __shared__ float xsum[2][MT];
  __shared__ int s_last;

  // XCD-aware logical index: consecutive logical ids run on one XCD.
  const int b = blockIdx.x, nwg = gridDim.x;
  const int xcd = b & 7, loc = b >> 3, per = nwg >> 3, rem = nwg & 7;
  const int L = (xcd < rem) ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
  const int mt = L % mtiles;
  const int t2 = L / mtiles;
  const int sp = t2 % nsplit;
  const int nt = t2 / nsplit;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kb = lane >> 4, l16 = lane & 15;
  const int m0 = mt * MT;
  const int nchunks = K >> 7;
  const int c0 = sp * cps;
  const int c1 = min(nchunks, c0 + cps);
  const long G = K >> 7;

  int nrow[NR];
#pragma unroll
  for (int ni = 0; ni < NR; ++ni) {
    const int n = nt * NT + wave * 16 * NR + ni * 16 + l16;
    nrow[ni] = n < N ? n : N - 1;  // clamp loads; results past N are dropped
  }

  f32x4_t acc[MI][NR];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NR; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 wreg[2][NR][WR];
  float wsc[2][NR], wz[2][NR];
  uint4 xreg[MI];

  auto load_w = [&](int c, int buf) {
#pragma unroll
    for (int ni = 0; ni < NR; ++ni) {
      const long n = nrow[ni];
      if constexpr (FMT == FMT_BF16) {
        const uint16_t* p = (const uint16_t*)wv + n * K + (long)c * 128;
#pragma unroll
        for (int i = 0; i < 4; ++i) wreg[buf][ni][i] = *(const uint4*)(p + kcol<FMT>(i, kb));
      } else if constexpr (FMT == FMT_W8) {
        const int8_t* p = (const int8_t*)wv + n * K + (long)c * 128;
#pragma unroll
        for (int h = 0; h < 2; ++h) wreg[buf][ni][h] = *(const uint4*)(p + 64 * h + 16 * kb);
      } else {
        const uint8_t* p = (const uint8_t*)wv + (n * K + (long)c * 128) / 2;
        wreg[buf][ni][0] = *(const uint4*)(p + 16 * kb);
        wsc[buf][ni] = bf2f(((const uint16_t*)sv)[n * G + c]);
        wz[buf][ni] = 128.0f + (float)((const uint8_t*)zv)[n * G + c];
      }
    }
  };
  auto load_x = [&](int c) {
#pragma unroll
    for (int p = 0; p < MI; ++p) {
      const int row = p * 16 + (tid >> 4);
      const int m = m0 + row;
      if (m < M) xreg[p] = *(const uint4*)(x + (long)m * ldx + (long)c * 128 + (tid & 15) * 8);
      else xreg[p] = uint4{0u, 0u, 0u, 0u};
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int p = 0; p < MI; ++p) {
      const int row = p * 16 + (tid >> 4);
      *(uint4*)(&xs[buf][row * LDSR + (tid & 15) * 8]) = xreg[p];
      if constexpr (FMT != FMT_BF16) {
        const uint4 v = xreg[p];
        float sm = bf_lo(v.x) + bf_hi(v.x) + bf_lo(v.y) + bf_hi(v.y) + bf_lo(v.z) + bf_hi(v.z) +
                   bf_lo(v.w) + bf_hi(v.w);
        sm += __shfl_xor(sm, 1, 64);
        sm += __shfl_xor(sm, 2, 64);
        sm += __shfl_xor(sm, 4, 64);
        sm += __shfl_xor(sm, 8, 64);
        if ((tid & 15) == 0) xsum[buf][row] = sm;
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
        const bf16x8_t a = *(const bf16x8_t*)(&xs[buf][(mi * 16 + l16) * LDSR + kcol<FMT>(i, kb)]);
#pragma unroll
        for (int ni = 0; ni < NR; ++ni) {
          if constexpr (FMT == FMT_BF16)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bw[ni], acc[mi][ni], 0, 0, 0);
          else
            accg[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bw[ni], accg[mi][ni], 0, 0, 0);
        }
      }
    }
    if constexpr (FMT != FMT_BF16) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float xsm = xsum[buf][mi * 16 + 4 * kb + r];
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

  if (c0 < c1) {
    load_w(c0, 0);
    load_x(c0);
    store_x(0);
    __syncthreads();
    int buf = 0;
    for (int c = c0; c < c1; ++c) {
      const bool nxt = c + 1 < c1;
      if (nxt) {
        if (buf == 0) load_w(c + 1, 1); else load_w(c + 1, 0);
        load_x(c + 1);
      }
      if (buf == 0) compute(0); else compute(1);
      if (nxt) { if (buf == 0) store_x(1); else store_x(0); }
      __syncthreads();
      buf ^= 1;
    }
  }

  // W8: per-row scale.
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

  if (nsplit > 1) {
    const long tile = (long)mt + (long)mtiles * nt;
    float* pp = partial + (tile * nsplit + sp) * (long)(MT * NT);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NR; ++ni)
#pragma unroll
        for (int r = 0; r < 4; ++r) pp[(((wave * MI + mi) * NR + ni) * 4 + r) * 64 + lane] = acc[mi][ni][r];
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const int prev = atomicAdd(&counters[tile], 1);
      s_last = (prev == nsplit - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    const float* p0 = partial + tile * nsplit * (long)(MT * NT);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NR; ++ni)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const long o = (((wave * MI + mi) * NR + ni) * 4 + r) * 64 + lane;
          float v = 0.f;
          for (int q = 0; q < nsplit; ++q) v += __builtin_nontemporal_load(p0 + (long)q * (MT * NT) + o);
          acc[mi][ni][r] = v;
        }
    if (tid == 0) counters[tile] = 0;
  }

#pragma unroll
  for (int ni = 0; ni < NR; ++ni) {
    const int n = nt * NT + wave * 16 * NR + ni * 16 + l16;
    if (n >= N) continue;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + mi * 16 + 4 * kb + r;
        if (m >= M) continue;
        const long o = (long)m * ldy + n;
        const float v = acc[mi][ni][r];
        if (epi == EPI_RESID) ((float*)yv)[o] += v;
        else if (epi == EPI_ACT && act_bf16) ((uint16_t*)yv)[o] = (uint16_t)f2bf(v);
        else ((float*)yv)[o] = v;
      }
  }
}

// ----------------------------------------------------------------------------
template <int FMT, int MT, int NR>
static int run_mfma(const void* x, int ldx, int M, const LinearW& W, void* y, int ldy, int epi, bool act_bf16,
                    const LinearWs& ws, hipStream_t st) {
  constexpr int NT = 64 * NR;
  const int mtiles = (M + MT - 1) / MT;
  const int ntiles = (W.N + NT - 1) / NT;
  const int nchunks = W.K / 128;
  const long base = (long)mtiles * ntiles;
  int nsplit = 1;
  while (base * nsplit < 1024 && nchunks / (nsplit * 2) >= 2) nsplit *= 2;
  const int cps = (nchunks + nsplit - 1) / nsplit;
  nsplit = (nchunks + cps - 1) / cps;
  if (nsplit > 1) {
    if ((size_t)base * nsplit * MT * NT > ws.partial_floats || base > ws.n_counters) nsplit = 1;
  }
  const int cps2 = nsplit == 1 ? nchunks : cps;
  const long nwg = base * nsplit;
  if (nwg > 0x7FFFFFFF) return -1;
  hipLaunchKernelGGL((k_linear_mfma<FMT, MT, NR>), dim3((unsigned)nwg), dim3(256), 0, st, (const uint16_t*)x, ldx,
                     M, W.w, W.scale, W.zero, W.N, W.K, y, ldy, epi, (int)act_bf16, mtiles, nsplit, cps2, ws.partial,
                     ws.counters);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

template <int FMT>
static int dispatch_mfma(const void* x, int ldx, int M, const LinearW& W, void* y, int ldy, int epi, bool act_bf16,
                         const LinearWs& ws, hipStream_t st) {
  const bool wide = (W.N + 127) / 128 >= 512;
  if (M <= 16) return wide ? run_mfma<FMT, 16, 2>(x, ldx, M, W, y, ldy, epi, act_bf16, ws, st)
                           : run_mfma<FMT, 16, 1>(x, ldx, M, W, y, ldy, epi, act_bf16, ws, st);
  if (M <= 32) return wide ? run_mfma<FMT, 32, 2>(x, ldx, M, W, y, ldy, epi, act_bf16, ws, st)
                           : run_mfma<FMT, 32, 1>(x, ldx, M, W, y, ldy, epi, act_bf16, ws, st);
  return wide ? run_mfma<FMT, 64, 2>(x, ldx, M, W, y, ldy, epi, act_bf16, ws, st)
              : run_mfma<FMT, 64, 1>(x, ldx, M, W, y, ldy, epi, act_bf16, ws, st);
}

template <int FMT, bool XBF>
static int run_valu(const void* x, int ldx, int M, const LinearW& W, void* y, int ldy, int epi, hipStream_t st) {
  dim3 grid((W.N + 3) / 4, (M + 3) / 4);
  hipLaunchKernelGGL((k_linear_valu<FMT, XBF>), grid, dim3(256), 0, st, x, ldx, M, W.w, W.scale, W.zero, W.N, W.K,
                     y, ldy, epi);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int launch_linear(const void* x, bool act_bf16, int ldx, int M, const LinearW& W, void* y, int ldy, int epi,
                  const LinearWs& ws, int path, hipStream_t st) {
  if (M <= 0 || W.N <= 0) return 0;
  if (W.K % 4 != 0) return -1;
  if (W.fmt == FMT_W4 && W.K % 128 != 0) return -1;
  const bool mfma_ok = act_bf16 && W.fmt != FMT_F32 && W.K % 128 == 0 && ldx % 8 == 0;
  const bool use_mfma = mfma_ok && path != 1;
  if (path == 2 && !mfma_ok) return -1;
  if (use_mfma) {
    switch (W.fmt) {
      case FMT_BF16: return dispatch_mfma<FMT_BF16>(x, ldx, M, W, y, ldy, epi, act_bf16, ws, st);
      case FMT_W8: return dispatch_mfma<FMT_W8>(x, ldx, M, W, y, ldy, epi, act_bf16, ws, st);
      case FMT_W4: return dispatch_mfma<FMT_W4>(x, ldx, M, W, y, ldy, epi, act_bf16, ws, st);
    }
    return -1;
  }
  if (act_bf16) {
    switch (W.fmt) {
      case FMT_F32: return run_valu<FMT_F32, true>(x, ldx, M, W, y, ldy, epi, st);
      case FMT_BF16: return run_valu<FMT_BF16, true>(x, ldx, M, W, y, ldy, epi, st);
      case FMT_W8: return run_valu<FMT_W8, true>(x, ldx, M, W, y, ldy, epi, st);
      case FMT_W4: return run_valu<FMT_W4, true>(x, ldx, M, W, y, ldy, epi, st);
    }
  } else {
    switch (W.fmt) {
      case FMT_F32: return run_valu<FMT_F32, false>(x, ldx, M, W, y, ldy, epi, st);
      case FMT_BF16: return run_valu<FMT_BF16, false>(x, ldx, M, W, y, ldy, epi, st);
      case FMT_W8: return run_valu<FMT_W8, false>(x, ldx, M, W, y, ldy, epi, st);
      case FMT_W4: return run_valu<FMT_W4, false>(x, ldx, M, W, y, ldy, epi, st);
    }
  }
  return -1;
}

}  // namespace er
