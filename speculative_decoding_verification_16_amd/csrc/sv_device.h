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
  int32_t arg;  // lowest index attaining lmax (greedy argmax); -1: the chunk holds a NaN or +inf
  double s;     // sum over the chunk of exp2((logit - lmax) * log2(e) / T)
};
static_assert(sizeof(ChunkStat) == 16, "ChunkStat layout");

// Per-row normalisation of the target distribution, merged from the row's
// chunk statistics: p(x) = exp2((logit - lmax) * log2(e) / T) / S.
struct RowStat {
  float lmax;   // largest raw logit of the row (-inf if none is finite, or if one is NaN or +inf)
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

// 2^y for y <= 0 in fp64, within a few fp64 ulps: with k = floor(256 y),
// y = k / 256 + r / 256, r in [0, 1]; 2^y = 2^(k >> 8) * 2^((k & 255) / 256)
// * 2^(r / 256), the middle factor from a table of 256 doubles (tab[j],
// built with the fp64 exp2 of the math library), the last from its Taylor
// polynomial in t = r ln 2 / 256 (t <= 0.0028: the first term left out is
// below 1e-18), the first by exponent scaling. About 14 fp64 and integer
// operations against several times that for a general fp64 exp2. 0 below
// 2^-1074.
constexpr int kExp2Tab = 256;
__device__ __forceinline__ double exp2_neg_f64(double y, const double* tab) {
  if (!(y > -1075.0)) return 0.0;
  const double ys = y * 256.0;  // exact
  const double kf = floor(ys);
  const int k = (int)kf;
  const double t = (ys - kf) * (0.69314718055994530942 / 256.0);
  double q = 1.0 / 120.0;
  q = fma(q, t, 1.0 / 24.0);
  q = fma(q, t, 1.0 / 6.0);
  q = fma(q, t, 0.5);
  q = fma(q, t, 1.0);
  q = fma(q, t, 1.0);
  return ldexp(tab[k & (kExp2Tab - 1)] * q, k >> 8);  // k >> 8 = floor(k / 256), k & 255 = k mod 256
}

// Residual weight of one token, S * max(0, p - cc q), in fp32: the caller
// passes ccS = cc * S and divides sums of these weights by S in fp64. One fma
// and one max per token; the rounding (a few fp32 ulps of p) stays far below
// the 1e-6 CDF tolerance.
__device__ __forceinline__ float residual_weight(float logit, float q, float lmax, float c, float ccS) {
  return fmaxf(0.f, fmaf(-ccS, q, target_weight(logit, lmax, c)));
}

// Allowed set of truncation sampling ([LOSSY] section 2.3): token x is in it
// iff l_x - l_max >= th, with th the row's threshold in fp64 (T ln p_base for
// min-p; T (ln S + min(ln eps, ln delta - H)) for eta) -- p(x) >= p_base max p
// (or p(x) >= tau) written on the logit difference. The difference is formed
// in fp64 (exact for logits within a factor 2^29 of each other), but only for
// the rare tokens whose fp32 difference falls in the guard band [lo, hi): an
// fp32 difference d at or above hi implies the exact one is >= th, and one
// below lo implies it is < th (lo and hi are th -/+ 2^-20 |th| rounded
// outward to fp32, wider than the 2^-24 relative rounding of d). So the
// set is the definition's, decided exactly.
struct RowThr {
  double th;  // threshold on l_x - l_max
  float lo;   // fp32 guard band: d >= hi is in, d < lo is out
  float hi;
};
static_assert(sizeof(RowThr) == 16, "RowThr layout");

__host__ __device__ inline RowThr make_row_thr(double th) {
  RowThr t;
  t.th = th;
  const double g = ldexp(fabs(th), -20);
  float hi = (float)(th + g), lo = (float)(th - g);
  if ((double)hi < th + g) hi = nextafterf(hi, INFINITY);
  if ((double)lo > th - g) lo = nextafterf(lo, -INFINITY);
  t.lo = lo;
  t.hi = hi;
  return t;
}

// w if x is allowed (or TR is false: no truncation), else 0
template <bool TR>
__device__ __forceinline__ float allowed(float w, float logit, float lmax, const RowThr& t) {
  if (!TR) return w;
  const float d = logit - lmax;
  bool in = d >= t.hi;
  if (!in && d >= t.lo) in = (double)logit - (double)lmax >= t.th;
  return in ? w : 0.f;
}
template <bool TR>
__device__ __forceinline__ bool is_allowed(float logit, float lmax, const RowThr& t) {
  return allowed<TR>(1.f, logit, lmax, t) != 0.f;
}

// Row normalisation from its chunk statistics, computed by a group of 4
// lanes (lanes 4 k .. 4 k + 3 of a wave, all active; every lane of the group
// returns the same values): lmax = max over chunks,
// S = sum_ch s_ch * exp2((lmax_ch - lmax) * c) in fp64, summed group-strided
// then by a butterfly inside the group, so every caller gets bitwise the same
// S. A row with a NaN or +inf logit (a chunk whose arg is kBadChunk) has no
// distribution: it gets lmax = -inf, like a row whose logits are all -inf.
// A wave normalises 16 rows at once, so a workgroup of 256 threads covers
// the 65 rows of the largest request in two rounds and usually in one, each
// lane's chunk loads independent of each other.
constexpr int32_t kBadChunk = -1;
constexpr int kRowGroup = 4;
__device__ __forceinline__ bool group_any(bool v) {
  const uint64_t bal = __ballot(v);
  return ((bal >> ((threadIdx.x & (kWave - 1)) & ~(kRowGroup - 1))) & ((1ull << kRowGroup) - 1)) != 0;
}
__device__ __forceinline__ double group_sum(double v) {
#pragma unroll
  for (int o = kRowGroup / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
// (Up to kRowRegs chunks per lane -- 64 chunks, a vocabulary of 262144 --
// the statistics are read once into registers; beyond, twice.)
constexpr int kRowRegs = 16;
__device__ __forceinline__ void row_norm_acc(const ChunkStat& s, float& m, float& av, int& ai, bool& bad) {
  bad |= s.arg == kBadChunk;
  m = fmaxf(m, s.lmax);
  if (s.lmax > av || (s.lmax == av && s.arg < ai)) { av = s.lmax; ai = s.arg; }
}
__device__ __forceinline__ void row_norm(const ChunkStat* st, int nch, float c, float& lmax, double& S,
                                         int& arg, float& argval) {
  const int gl = threadIdx.x & (kRowGroup - 1);
  float m = -INFINITY;
  float av = -INFINITY;
  int ai = 0x7fffffff;
  bool bad = false;
  const bool in_regs = nch <= kRowRegs * kRowGroup;
  ChunkStat cs[kRowRegs];
  if (in_regs) {
#pragma unroll
    for (int k = 0; k < kRowRegs; ++k) {
      const int ch = gl + kRowGroup * k;
      if (ch < nch) cs[k] = st[ch];
      else cs[k] = ChunkStat{-INFINITY, 0x7fffffff, 0.0};
    }
#pragma unroll
    for (int k = 0; k < kRowRegs; ++k) row_norm_acc(cs[k], m, av, ai, bad);
  } else {
    for (int ch = gl; ch < nch; ch += kRowGroup) row_norm_acc(st[ch], m, av, ai, bad);
  }
#pragma unroll
  for (int o = kRowGroup / 2; o > 0; o >>= 1) {
    m = fmaxf(m, __shfl_xor(m, o));
    const float ov = __shfl_xor(av, o);
    const int oi = __shfl_xor(ai, o);
    if (ov > av || (ov == av && oi < ai)) { av = ov; ai = oi; }
  }
  if (group_any(bad)) {
    lmax = -INFINITY;
    S = 0.0;
    arg = kBadChunk;
    argval = -INFINITY;
    return;
  }
  // the chunks in the same order on both paths: lane gl sums gl, gl + 4, ...
  double acc = 0.0;
  if (m != -INFINITY) {
    if (in_regs) {
#pragma unroll
      for (int k = 0; k < kRowRegs; ++k)
        if (cs[k].lmax != -INFINITY) acc = fma(cs[k].s, exp2((double)(cs[k].lmax - m) * (double)c), acc);
    } else {
      for (int ch = gl; ch < nch; ch += kRowGroup) {
        const ChunkStat s = st[ch];
        if (s.lmax != -INFINITY) acc = fma(s.s, exp2((double)(s.lmax - m) * (double)c), acc);
      }
    }
  }
  S = group_sum(acc);
  lmax = m;
  arg = ai;
  argval = av;
}

// ---- split-K merge -----------------------------------------------------------
// Merge of the per-split partial attention of `item` (a packed (node, query
// head) row): partial rows are unnormalised outputs with their running max
// (log2 units) and sum; they are merged online in split order. lpr = D / 4
// lanes per row, lane dl holds one float4 of it. Headers and rows of eight
// splits are requested at once (a chunk past the last split re-reads the
// last one and is ignored). Used by the attention's merge kernel and, inside
// the step, by extra blocks of the row-statistics launch.
struct MergeArgs {
  int32_t NH, D, splits;
  int32_t blocks;          // 256-thread blocks needed (0: nothing to merge)
  const float* o_part;     // [splits, NH, D]
  const float2* ml_part;   // [splits, NH]
  float* out;              // [NH, D]
};
template <int NT = 256>
__device__ __forceinline__ void merge_split_rows(const MergeArgs& a, int block) {
  const int lpr = a.D >> 2;  // lanes per row
  const int item = block * (NT / lpr) + threadIdx.x / lpr;
  const int dl = threadIdx.x % lpr;
  if (item >= a.NH) return;
  const float4* o4 = (const float4*)a.o_part;
  float M = -INFINITY, den = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < a.splits; s0 += 8) {
    float2 ml[8];
    float4 ov[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = min(s0 + u, a.splits - 1);
      ml[u] = a.ml_part[(int64_t)s * a.NH + item];
      ov[u] = o4[((int64_t)s * a.NH + item) * lpr + dl];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (s0 + u >= a.splits || !(ml[u].y > 0.f)) continue;  // past the end, or the split saw no key of this row
      const float mn = fmaxf(M, ml[u].x);
      const float al = exp2f(M - mn), w = exp2f(ml[u].x - mn);  // M = -inf at first: al = 0
      acc.x = acc.x * al + w * ov[u].x;
      acc.y = acc.y * al + w * ov[u].y;
      acc.z = acc.z * al + w * ov[u].z;
      acc.w = acc.w * al + w * ov[u].w;
      den = den * al + w * ml[u].y;
      M = mn;
    }
  }
  const float inv = 1.0f / den;
  ((float4*)a.out)[(int64_t)item * lpr + dl] = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}
__host__ __device__ inline MergeArgs merge_args(int NH, int D, int splits, const float* o_part, const float2* ml_part,
                                                float* out) {
  MergeArgs a;
  a.NH = NH;
  a.D = D;
  a.splits = splits;
  a.blocks = splits > 1 ? (NH + 256 / (D / 4) - 1) / (256 / (D / 4)) : 0;
  a.o_part = o_part;
  a.ml_part = ml_part;
  a.out = out;
  return a;
}
// blocks of nt threads that merge_split_rows<nt> needs (0: nothing to merge)
__host__ __device__ inline int merge_blocks(const MergeArgs& a, int nt) {
  if (a.blocks == 0) return 0;
  const int rows = nt / (a.D / 4);
  return (a.NH + rows - 1) / rows;
}

}  // namespace sv
