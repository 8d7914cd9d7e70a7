// Shared device/host helpers for the gfx950 kernels of the self-speculative step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define ER_DEV __device__ __forceinline__

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// ---- bf16 <-> fp32 (bf16 held as raw uint16 bits) --------------------------
ER_DEV float bf2f(uint32_t b16) { return __uint_as_float(b16 << 16); }
ER_DEV float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
ER_DEV float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round to nearest even (NaN -> canonical quiet NaN).
ER_DEV uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Activation element load/store for fp32 or bf16 storage.
template <bool BF> struct Act;
template <> struct Act<false> {
  typedef float T;
  static ER_DEV float ld(const float* p, long i) { return p[i]; }
  static ER_DEV void st(float* p, long i, float v) { p[i] = v; }
};
template <> struct Act<true> {
  typedef uint16_t T;
  static ER_DEV float ld(const uint16_t* p, long i) { return bf2f(p[i]); }
  static ER_DEV void st(uint16_t* p, long i, float v) { p[i] = (uint16_t)f2bf(v); }
};

// ---- wave64 reductions -------------------------------------------------------
ER_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
ER_DEV double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
ER_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ---- Philox4x32-10 (Salmon et al., SC'11) ----------------------------------
// Round: multiply counter words 0 and 2 by the two Philox multipliers (keeping
// high and low halves), mix the high halves with words 1 and 3 and the round
// key; the key advances by the two Weyl increments between rounds.
ER_DEV void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) { k0 += W0; k1 += W1; }
    uint32_t hi0 = __umulhi(M0, c[0]), lo0 = M0 * c[0];
    uint32_t hi1 = __umulhi(M1, c[2]), lo1 = M1 * c[2];
    uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
  }
}

// Uniform in (0, 1] from the first output word; exact in fp32 (and fp64).
// Counter = (seq_id, pos, draft_idx, purpose); key = (seed lo, seed hi).
ER_DEV double philox_uniform(uint64_t seed, uint32_t seq, uint32_t pos, uint32_t didx, uint32_t purpose) {
  uint32_t c[4] = {seq, pos, didx, purpose};
  philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  return ((double)(c[0] >> 8) + 1.0) * (1.0 / 16777216.0);
}


// Order-preserving map of fp32 to uint32 (larger float -> larger key).
ER_DEV uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0) u = 0;  // -0 and +0 are the same logit
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Work-group barrier for LDS hand-offs only: waits for this wave's LDS
// operations (lgkmcnt(0); vmcnt and expcnt left at their maxima) and then
// meets the other waves.  Unlike __syncthreads() it carries no memory fence,
// so global loads issued ahead (software pipelines) stay in flight.
ER_DEV void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
}

// Index of this wave in its work-group, known to the compiler to be
// wave-uniform (so that branches and addresses derived from it stay scalar).
ER_DEV int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
