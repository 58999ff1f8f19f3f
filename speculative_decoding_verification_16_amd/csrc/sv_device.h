// sv_device.h -- device-side helpers shared by the verification kernels
// (gfx950, wave64): wave reductions, bf16 packing, the Philox4x32-10
// counter generator and the per-row target-distribution helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kWave = 64;
constexpr int kMaxNodes = 64;     // one 64-bit ancestor mask per node
constexpr int kChunk = 4096;      // vocabulary chunk of the sampler statistics
constexpr int kMaxVocab = 1 << 22;
constexpr int kMaxChunks = kMaxVocab / kChunk;

// Per (row, vocabulary chunk) statistics written by the row-statistics pass.
struct ChunkStat {
  float lmax;   // largest raw logit of the chunk (-inf if none finite)
  int32_t arg;  // lowest index attaining lmax (greedy argmax)
  double s;     // sum over the chunk of exp2((logit - lmax) * log2(e) / T)
};
static_assert(sizeof(ChunkStat) == 16, "ChunkStat layout");

// Per-row normalisation of the target distribution, merged from the row's
// chunk statistics: p(x) = exp2((logit - lmax) * log2(e) / T) / S.
struct RowStat {
  float lmax;   // largest raw logit of the row (-inf if none is finite)
  int32_t arg;  // lowest index attaining lmax (greedy argmax)
  double S;     // sum over the row of exp2((logit - lmax) * log2(e) / T)
};
static_assert(sizeof(RowStat) == 16, "RowStat layout");

// Data-error bits (same values as SV_STATUS_* in the public header).
constexpr int32_t kStTree = 0x01, kStPacking = 0x02, kStToken = 0x04, kStNonFinite = 0x08,
                  kStZeroResidual = 0x10, kStCtx = 0x20, kStSync = 0x40, kStBlock = 0x80;

__device__ __forceinline__ void flag(int32_t* status, int32_t bits) {
  if (status) atomicOr(status, bits);
}

// ---- wave reductions (fixed butterfly order: deterministic) ---------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
// max with the lowest index on ties
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o);
    int oi = __shfl_xor(i, o);
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
  }
}

// ---- bf16 ------------------------------------------------------------------
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // finite, non-negative inputs only
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// ---- Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) --------------------
// Ten rounds; each multiplies counter words 0 and 2 by the two Philox
// multipliers, mixes the high halves with the other words and the key, and
// bumps the key by the two Weyl constants between rounds.
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = M0 * c0, hi0 = __umulhi(M0, c0);
    const uint32_t lo1 = M1 * c2, hi1 = __umulhi(M1, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += W0; k1 += W1;
  }
  return c0;
}
// U(request, j, purpose) in (0,1): (w0 + 1/2) * 2^-32, exact in fp64.
__device__ __forceinline__ double uniform01(uint64_t seed, uint32_t rid, uint32_t j, uint32_t purpose,
                                            uint32_t step) {
  const uint32_t w = philox_word0(rid, j, purpose, step, (uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32));
  return ((double)w + 0.5) * (1.0 / 4294967296.0);
}

// ---- target distribution ---------------------------------------------------
// Unnormalised target weight of one logit relative to the row maximum:
// exp((logit - lmax) / T) evaluated as exp2((logit - lmax) * log2(e)/T) with
// the hardware v_exp_f32 (the argument is <= 0; weights below 2^-126 flush to
// zero, far below any probability the sampler can resolve).
__device__ __forceinline__ float target_weight(float logit, float lmax, float c) {
  return __builtin_amdgcn_exp2f((logit - lmax) * c);
}
// p(x) as an fp32 value; every kernel that needs p uses exactly this.
__device__ __forceinline__ float target_prob(float logit, float lmax, float c, float invS) {
  return target_weight(logit, lmax, c) * invS;
}

// Residual weight of one token, S * max(0, p - cc q), in fp32: the caller
// passes ccS = cc * S and divides sums of these weights by S in fp64. One fma
// and one max per token; the rounding (a few fp32 ulps of p) stays far below
// the 1e-6 CDF tolerance.
__device__ __forceinline__ float residual_weight(float logit, float q, float lmax, float c, float ccS) {
  return fmaxf(0.f, fmaf(-ccS, q, target_weight(logit, lmax, c)));
}

// Min-p truncation ([LOSSY] section 2.3): token x is in the allowed set iff
// logit - lmax >= theta with theta = fp32(T ln p_base) -- p(x) >= p_base
// max p written on the fp32 logit difference, the comparison every side of
// the library (and its checker) makes identically. TR = false: no truncation.
template <bool TR>
__device__ __forceinline__ float allowed(float w, float logit, float lmax, float theta) {
  return (!TR || logit - lmax >= theta) ? w : 0.f;
}

// Row normalisation from its chunk statistics, computed by one full wave
// (every lane returns the same values): lmax = max over chunks,
// S = sum_ch s_ch * exp2((lmax_ch - lmax) * c) in fp64, summed lane-strided
// then by butterfly, so every caller gets bitwise the same S.
__device__ __forceinline__ void row_norm(const ChunkStat* st, int nch, float c, float& lmax, double& S,
                                         int& arg, float& argval) {
  const int lane = threadIdx.x & (kWave - 1);
  float m = -INFINITY;
  float av = -INFINITY;
  int ai = 0x7fffffff;
  for (int ch = lane; ch < nch; ch += kWave) {
    const ChunkStat s = st[ch];
    m = fmaxf(m, s.lmax);
    if (s.lmax > av || (s.lmax == av && s.arg < ai)) { av = s.lmax; ai = s.arg; }
  }
  m = wave_max(m);
  wave_argmax(av, ai);
  double acc = 0.0;
  if (m != -INFINITY) {
    for (int ch = lane; ch < nch; ch += kWave) {
      const ChunkStat s = st[ch];
      if (s.lmax != -INFINITY) acc += s.s * exp2((double)(s.lmax - m) * (double)c);
    }
  }
  S = wave_sum(acc);
  lmax = m;
  arg = ai;
  argval = av;
}

}  // namespace sv
