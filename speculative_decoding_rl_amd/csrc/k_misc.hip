// Element-wise and per-row kernels of the decoder layer, the drafter
// quantizers and small utilities.
//
// Decoder layer (pre-norm, the Qwen2.5 / Llama-3 family the workloads name):
// embedding gather, RMSNorm (x / sqrt(mean(x^2) + eps) * g), rotate-half RoPE
// with KV append into the paged pool, SwiGLU (silu(gate) * up).
//
// Quantizers build the self-drafter from the target's own weights
// (EfficientRollout, "关键模块" item 1; W4A16 in "与现有工作流的接口"):
//  * W8 symmetric per output row: s = max|w| / 127 rounded up to fp32,
//    q = clamp(rint(w / s), -127, 127).
//  * W4 asymmetric per row and 128-wide group: lo = min(min w, 0),
//    hi = max(max w, 0), s = (hi - lo) / 15 rounded up to bf16,
//    z = clamp(rint(-lo / s), 0, 15), q = clamp(rint(w / s) + z, 0, 15).
// Scales and quotients are formed in fp64 so the codes are a deterministic
// function of the stored weights.

#include "common.h"
#include "kernels.h"
#include "linear_dev.h"

namespace er {

__global__ __launch_bounds__(256) void k_embed(const int32_t* __restrict__ tok, int stride, const void* __restrict__ E,
                                               int bf16, int d, float* __restrict__ h, unsigned long long* __restrict__ ssq,
                                               unsigned long long* __restrict__ ssq_zero, int slots, long sstride) {
  const int m = blockIdx.x;
  const long t = tok[(long)m * stride];
  float s = 0.f;
  if (bf16) {
    const uint16_t* e = (const uint16_t*)E + t * d;
    for (int i = threadIdx.x; i < d; i += blockDim.x) {
      const float v = bf2f(e[i]);
      h[(long)m * d + i] = v;
      s = fmaf(v, v, s);
    }
  } else {
    const float* e = (const float*)E + t * d;
    for (int i = threadIdx.x; i < d; i += blockDim.x) {
      const float v = e[i];
      h[(long)m * d + i] = v;
      s = fmaf(v, v, s);
    }
  }
  // every slot of the row: the sum in slot 0, the other slots cleared
  if (ssq_zero && (int)threadIdx.x < slots) ssq_zero[(long)threadIdx.x * sstride + m] = 0ull;
  if (!ssq) return;
  if (threadIdx.x > 0 && (int)threadIdx.x < slots) ssq[(long)threadIdx.x * sstride + m] = 0ull;
  s = wave_sum(s);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) ssq[m] = (unsigned long long)rint((double)(red[0] + red[1] + red[2] + red[3]) * SSQ_SCALE);
}

int launch_embed(const int32_t* tokens, int tok_stride, int M, const void* embed, bool bf16, int d, float* h,
                 unsigned long long* ssq, unsigned long long* ssq_zero, hipStream_t st, int ssq_slots,
                 long ssq_stride) {
  if (M <= 0) return 0;
  if (ssq_slots < 1) ssq_slots = 1;
  if (ssq_slots > 256) return -1;
  hipLaunchKernelGGL(k_embed, dim3(M), dim3(256), 0, st, tokens, tok_stride, embed, (int)bf16, d, h, ssq, ssq_zero,
                     ssq_slots, ssq_stride);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

__global__ __launch_bounds__(256) void k_rmsnorm(const float* __restrict__ h, int d, const void* __restrict__ g,
                                                 int bf16, float eps, void* __restrict__ x,
                                                 const int32_t* __restrict__ row_index) {
  const int m = blockIdx.x;
  const long src = row_index ? row_index[m] : m;
  const float* hr = h + src * d;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += blockDim.x) ss = fmaf(hr[i], hr[i], ss);
  ss = wave_sum(ss);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float r = 1.0f / sqrtf(tot / (float)d + eps);
  if (bf16) {
    const uint16_t* gg = (const uint16_t*)g;
    uint16_t* xr = (uint16_t*)x + (long)m * d;
    for (int i = threadIdx.x; i < d; i += blockDim.x) xr[i] = (uint16_t)f2bf(hr[i] * r * bf2f(gg[i]));
  } else {
    const float* gg = (const float*)g;
    float* xr = (float*)x + (long)m * d;
    for (int i = threadIdx.x; i < d; i += blockDim.x) xr[i] = hr[i] * r * gg[i];
  }
}

int launch_rmsnorm(const float* h, int M, int d, const void* g, bool bf16, float eps, void* x,
                   const int32_t* row_index, hipStream_t st) {
  if (M <= 0) return 0;
  hipLaunchKernelGGL(k_rmsnorm, dim3(M), dim3(256), 0, st, h, d, g, (int)bf16, eps, x, row_index);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// KV pool: block b (16 positions), layer l, head h holds K as [16][hd] at
// ((((b * L + l) * 2 + 0) * hkv + h) * 16) * hd and V transposed as [hd][16]
// at ((((b * L + l) * 2 + 1) * hkv + h) * 16) * hd.
ER_DEV long kv_base(long slot, int layer, int L, int kv, int hkv, int head, int hd) {
  const long block = slot >> 4;
  return ((((block * L + layer) * 2 + kv) * hkv + head) * 16) * (long)hd;
}

__global__ __launch_bounds__(256) void k_rope_kv(const float* __restrict__ qkv, int hq, int hkv, int hd,
                                                 const int32_t* __restrict__ pos, const int64_t* __restrict__ slot,
                                                 const float2* __restrict__ cs, void* __restrict__ qout,
                                                 void* __restrict__ pool, int layer, int L, int bf16) {
  const int m = blockIdx.x;
  const int half = hd >> 1;
  const int width = (hq + 2 * hkv) * hd;
  const float* row = qkv + (long)m * width;
  const long p = pos[m];
  const long sl = slot[m];
  const float2* csr = cs + p * half;
  const int npairs = (hq + hkv) * half;
  for (int idx = threadIdx.x; idx < npairs; idx += blockDim.x) {
    const int head = idx / half, i = idx - head * half;
    const float x1 = row[head * hd + i], x2 = row[head * hd + i + half];
    const float2 c = csr[i];
    const float r1 = x1 * c.x - x2 * c.y;
    const float r2 = x2 * c.x + x1 * c.y;
    if (head < hq) {
      const long o = ((long)m * hq + head) * hd;
      if (bf16) {
        ((uint16_t*)qout)[o + i] = (uint16_t)f2bf(r1);
        ((uint16_t*)qout)[o + i + half] = (uint16_t)f2bf(r2);
      } else {
        ((float*)qout)[o + i] = r1;
        ((float*)qout)[o + i + half] = r2;
      }
    } else {
      const long o = kv_base(sl, layer, L, 0, hkv, head - hq, hd) + (sl & 15) * hd;
      if (bf16) {
        ((uint16_t*)pool)[o + i] = (uint16_t)f2bf(r1);
        ((uint16_t*)pool)[o + i + half] = (uint16_t)f2bf(r2);
      } else {
        ((float*)pool)[o + i] = r1;
        ((float*)pool)[o + i + half] = r2;
      }
    }
  }
  for (int idx = threadIdx.x; idx < hkv * hd; idx += blockDim.x) {
    const int g = idx / hd, e = idx - g * hd;
    const float v = row[(hq + hkv) * hd + idx];
    const long o = kv_base(sl, layer, L, 1, hkv, g, hd) + (long)e * 16 + (sl & 15);
    if (bf16) ((uint16_t*)pool)[o] = (uint16_t)f2bf(v);
    else ((float*)pool)[o] = v;
  }
}

int launch_rope_kv(const float* qkv, int M, int hq, int hkv, int hd, const int32_t* pos, const int64_t* slot,
                   const float2* cs, void* qout, void* kv_pool, int layer, int n_layers, bool bf16, hipStream_t st) {
  if (M <= 0) return 0;
  hipLaunchKernelGGL(k_rope_kv, dim3(M), dim3(256), 0, st, qkv, hq, hkv, hd, pos, slot, cs, qout, kv_pool, layer,
                     n_layers, (int)bf16);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

__global__ __launch_bounds__(256) void k_swiglu(const float* __restrict__ gu, int F, void* __restrict__ act,
                                                int bf16) {
  const int m = blockIdx.y;
  const int f = blockIdx.x * blockDim.x + threadIdx.x;
  if (f >= F) return;
  const float g = gu[(long)m * 2 * F + f];
  const float u = gu[(long)m * 2 * F + F + f];
  const float v = g / (1.0f + expf(-g)) * u;
  if (bf16) ((uint16_t*)act)[(long)m * F + f] = (uint16_t)f2bf(v);
  else ((float*)act)[(long)m * F + f] = v;
}

int launch_swiglu(const float* gu, int M, int F, void* act, bool bf16, hipStream_t st) {
  if (M <= 0) return 0;
  hipLaunchKernelGGL(k_swiglu, dim3((F + 255) / 256, M), dim3(256), 0, st, gu, F, act, (int)bf16);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// ---------------------------------------------------------------------------
// Quantizers.
// ---------------------------------------------------------------------------
ER_DEV float f32_round_up(double v) {
  float t = (float)v;
  if ((double)t < v) t = nextafterf(t, __builtin_huge_valf());
  return t;
}
ER_DEV double bf16_round_up(double v) {
  const uint32_t u = __float_as_uint(f32_round_up(v));
  uint32_t hi = u >> 16;
  if (u & 0xFFFFu) hi += 1;
  return (double)__uint_as_float(hi << 16);
}

__global__ __launch_bounds__(256) void k_quant_w8(const void* __restrict__ W, int bf16, int K, int8_t* __restrict__ q,
                                                  float* __restrict__ scale) {
  const long n = blockIdx.x;
  auto ld = [&](long k) -> float {
    return bf16 ? bf2f(((const uint16_t*)W)[n * K + k]) : ((const float*)W)[n * K + k];
  };
  float amax = 0.f;
  for (int k = threadIdx.x; k < K; k += blockDim.x) amax = fmaxf(amax, fabsf(ld(k)));
  amax = wave_max(amax);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax > 0.f ? f32_round_up((double)amax / 127.0) : 1.0f;
  for (int k = threadIdx.x; k < K; k += blockDim.x) {
    double v = rint((double)ld(k) / (double)s);
    v = fmin(127.0, fmax(-127.0, v));
    q[n * K + k] = (int8_t)(int)v;
  }
  if (threadIdx.x == 0) scale[n] = s;
}

int launch_quantize_w8(const void* W, bool bf16, int N, int K, int8_t* q, float* scale, hipStream_t st) {
  if (N <= 0) return 0;
  hipLaunchKernelGGL(k_quant_w8, dim3(N), dim3(256), 0, st, W, (int)bf16, K, q, scale);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// One wave per (row, 128-group); lane l holds elements 2l and 2l+1 and writes
// their canonical byte (low nibble = even k).
__global__ __launch_bounds__(256) void k_quant_w4(const uint16_t* __restrict__ W, int N, int K,
                                                  uint8_t* __restrict__ packed, uint16_t* __restrict__ scale,
                                                  uint8_t* __restrict__ zero) {
  const int G = K >> 7;
  const long gid = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gid >= (long)N * G) return;
  const int lane = threadIdx.x & 63;
  const long n = gid / G;
  const int g = (int)(gid - n * G);
  const long k = (long)g * 128 + 2 * lane;
  const uint32_t pair = *(const uint32_t*)(W + n * K + k);
  const double w0 = (double)bf_lo(pair), w1 = (double)bf_hi(pair);
  double lo = fmin(w0, w1), hi = fmax(w0, w1);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = fmin(lo, __shfl_xor(lo, o, 64));
    hi = fmax(hi, __shfl_xor(hi, o, 64));
  }
  lo = fmin(lo, 0.0);
  hi = fmax(hi, 0.0);
  const double span = hi - lo;
  double s = 1.0, z = 0.0;
  if (span > 0.0) {
    s = bf16_round_up(span / 15.0);
    z = fmin(15.0, fmax(0.0, rint(-lo / s)));
  }
  const int q0 = (int)fmin(15.0, fmax(0.0, rint(w0 / s) + z));
  const int q1 = (int)fmin(15.0, fmax(0.0, rint(w1 / s) + z));
  packed[(n * K + k) >> 1] = (uint8_t)(q0 | (q1 << 4));
  if (lane == 0) {
    scale[n * G + g] = (uint16_t)(__float_as_uint((float)s) >> 16);
    zero[n * G + g] = (uint8_t)(int)z;
  }
}

int launch_quantize_w4(const void* W, int N, int K, uint8_t* packed_canon, uint16_t* scale, uint8_t* zero,
                       hipStream_t st) {
  if (N <= 0) return 0;
  if (K % 128 != 0) return -1;
  const long groups = (long)N * (K / 128);
  hipLaunchKernelGGL(k_quant_w4, dim3((unsigned)((groups + 3) / 4)), dim3(256), 0, st, (const uint16_t*)W, N, K,
                     packed_canon, scale, zero);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Canonical W4 (row-major bytes, k at bits 4k of each word) -> kernel order:
// within a word, k = 2i at bits 4i and k = 2i+1 at bits 16 + 4i; the words
// placed in the kernel layout (w4_piece: rows in groups of 8, a group's
// 64-byte pieces chunk after chunk).
__global__ __launch_bounds__(256) void k_w4_order(const uint32_t* __restrict__ in, long nwords, int N, int K,
                                                  uint32_t* __restrict__ out) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nwords) return;
  const uint32_t c = in[i];
  uint32_t r = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r |= ((c >> (8 * j)) & 0xFu) << (4 * j);
    r |= ((c >> (8 * j + 4)) & 0xFu) << (16 + 4 * j);
  }
  const long wpr = (long)K >> 3;             // words per row
  const long n = i / wpr, kw = i - n * wpr;  // kw: word within the row, 16 per 128-code chunk
  out[(w4_piece(n, kw >> 4, N, K) >> 2) + (kw & 15)] = r;
}

int launch_w4_to_kernel_order(const uint8_t* canon, int N, int K, uint8_t* out, hipStream_t st) {
  const long nwords = (long)N * K / 8;
  if (nwords <= 0) return 0;
  if (K % 128 != 0) return -1;
  hipLaunchKernelGGL(k_w4_order, dim3((unsigned)((nwords + 255) / 256)), dim3(256), 0, st, (const uint32_t*)canon,
                     nwords, N, K, (uint32_t*)out);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

__global__ void k_philox_uniform(uint64_t seed, const uint32_t* __restrict__ ctr, int n, double* __restrict__ u) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  u[i] = philox_uniform(seed, ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3]);
}

int launch_philox_uniform(uint64_t seed, const uint32_t* ctr4, int n, double* u, hipStream_t st) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_philox_uniform, dim3((n + 255) / 256), dim3(256), 0, st, seed, ctr4, n, u);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

__global__ __launch_bounds__(256) void k_stream_read(const uint4* __restrict__ p, size_t n, uint32_t* sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;  // keeps the loads alive
}

int launch_stream_read(const void* p, size_t bytes, uint32_t* sink, hipStream_t st) {
  hipLaunchKernelGGL(k_stream_read, dim3(2048), dim3(256), 0, st, (const uint4*)p, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace er
