// sv_sample.hip -- lossless rejection sampling over the vocabulary and the
// tree walk, for gfx950.
//
// Method: "Speculative Decoding: Accelerating Inference Speeds in Distributed
// LLMs", section "Mathematical Rejection Sampling Algorithm" (accept x_i iff
// r_i <= min(1, p_i(x_i)/q_i(x_i)); on rejection draw from the normalised
// residual max(0, p - q)) and "Proof of Lossless Distribution Equivalence";
// "Revisiting Lossy Verification in Speculative Decoding", section 2.1
// (h(x) = min(1, p/q)) and appendix F.1 (r(x), R = sum (p - q)+).
//
// Passes:
//  1. row_stats_kernel  -- one streaming read of every target-logit row:
//     per 4096-token chunk the max logit, its first index and
//     sum exp((logit - max)/T). That is all the walk needs to evaluate p at
//     any token and to draw from p at a leaf.
//  2. walk_kernel       -- one workgroup per request. It merges the chunk
//     statistics of its own rows into the per-row maximum, argmax and sum
//     (row_finalize_kernel does the same for all rows when the p rows are
//     requested as an output), then climbs down the tree
//     doing the accept tests on gathered p(x), q(x). A residual mass is only
//     computed when the walk actually rejects (a vocabulary pass over that
//     one row, logits and q), so rows that are never rejected are read once,
//     and q is read only where a residual is needed.
//
// Residual levels in closed form: after k rejections at one position the
// current distribution is P_k = max(0, p - c_k q) / M(c_k) with
// M(c) = sum_x max(0, p(x) - c q(x)), c_0 = 0 (P_0 = p, M(0) = 1) and
// c_{k+1} = c_k + M(c_k). (Induction: max(0, P_k - q) =
// max(0, p - (c_k + M(c_k)) q) / M(c_k), whose mass is M(c_{k+1}) / M(c_k).)
// So each level costs exactly one pass that evaluates M at the new c, and
// the same pass yields the per-chunk masses the inverse CDF needs.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Pass 1: per (row, chunk) statistics. One wave per chunk of 4096 logits; a
// lane holds 64 of them in registers, so the row is read from HBM once.
// ENT (the eta allowed set) also sums, per chunk and in fp64 with fp64
// weights, w64 = 2^y and w64 * y, y = (logit - max) * log2(e)/T formed in
// fp64: the row's entropy and the threshold come from these, within a few
// fp64 roundings of their exact values, so that the set is decided as its
// definition says (the fp32 weights of the sums for p would put the
// threshold up to ~1e-5 T off on flat rows).
//
// chunk_stat is that work for one chunk, by one wave (every lane calls it and
// gets the record): the row-statistics kernel runs it for every chunk of every
// row, and the walk, when it computes the statistics of the rows it reaches
// itself, runs the same code on those rows. A chunk holding a NaN or +inf
// gets arg = kBadChunk: the row has no distribution (row_norm), which the
// walk reports when it reaches the row.
// The arithmetic of chunk_stat on a chunk already in registers (tokens past
// the row's end hold -inf); the lazy walk loads its chunks its own way and
// reduces them with this same code.
template <bool GREEDY, bool VEC, bool ENT>
__device__ __forceinline__ void chunk_reduce(const float (&x)[64], int begin, float c, double c64, const double* tab,
                                             ChunkStat& st, double2& se) {
  const int lane = threadIdx.x & 63;
  // element (i) of this lane is token begin + 4*(lane + 64*(i/4)) + i%4 (VEC)
  // or begin + lane + 64*i (scalar); both visit a lane's tokens in increasing order
  float mx = -INFINITY;
  bool any_bad;
  if (GREEDY) {
    // the argmax (lowest index on ties) and an explicit NaN / +inf test
    int ai = 0x7fffffff;
    bool bad = false;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const float v = x[i];
      bad |= (v != v) || (v == INFINITY);
      if (v > mx) {
        mx = v;
        ai = VEC ? begin + 4 * (lane + 64 * (i >> 2)) + (i & 3) : begin + lane + 64 * i;
      }
    }
    any_bad = __any(bad);
    wave_argmax(mx, ai);
    st.lmax = mx;
    st.arg = any_bad ? kBadChunk : (mx == -INFINITY ? begin : ai);
    st.s = 0.0;
    se = make_double2(0.0, 0.0);
    return;
  }
  // sampling needs no argmax, and the NaN / +inf test comes from the sum:
  // with a finite maximum a NaN logit has a NaN weight; a +inf maximum gives
  // its own element a NaN weight (inf - inf); only a chunk whose maximum is
  // -inf (every logit -inf or NaN) is tested element by element. A lane
  // maximum that a signalling NaN turned into a NaN drops out of the wave
  // maximum, and that lane's NaN weight still flags the chunk.
#pragma unroll
  for (int i = 0; i < 64; ++i) mx = fmaxf(mx, x[i]);
  mx = wave_max(mx);
  double s = 0.0, s64 = 0.0, e64 = 0.0;
  if (mx != -INFINITY) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const float w = target_weight(x[i], mx, c);
      s += (double)w;
      if (ENT && x[i] != -INFINITY) {
        const double y = ((double)x[i] - (double)mx) * c64;
        const double w64 = exp2_neg_f64(y, tab);
        s64 += w64;
        e64 += w64 * y;
      }
    }
    s = wave_sum(s);
    if (ENT) {
      s64 = wave_sum(s64);
      e64 = wave_sum(e64);
    }
    any_bad = s != s;
  } else {
    bool nan = false;
#pragma unroll
    for (int i = 0; i < 64; ++i) nan |= x[i] != x[i];
    any_bad = __any(nan);
  }
  st.lmax = mx;
  st.arg = any_bad ? kBadChunk : begin;  // the argmax is read by greedy walks only
  st.s = s;
  se = make_double2(s64, e64);
}

// chunk_stat: the chunk's loads (tokens past the row's end as -inf), then
// chunk_reduce.
template <bool GREEDY, bool VEC, bool ENT>
__device__ __forceinline__ void chunk_stat(const float* __restrict__ base, int V, int ch, float c, double c64,
                                           const double* tab, ChunkStat& st, double2& se) {
  const int lane = threadIdx.x & 63;
  const int begin = ch * kChunk;
  const int end = min(V, begin + kChunk);
  float x[64];
  if (VEC) {
    const f32x4_t* b4 = (const f32x4_t*)(base + begin);
    const int n4 = (end - begin) >> 2;  // V % 4 == 0 on this path
    // streamed once: non-temporal loads (measured ~9 % faster on MI355X)
    if (n4 == kChunk / 4) {  // a whole chunk (uniform): no bounds tests
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const f32x4_t v = __builtin_nontemporal_load(b4 + lane + 64 * i);
        x[4 * i + 0] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int idx = lane + 64 * i;
        const f32x4_t v = idx < n4 ? __builtin_nontemporal_load(b4 + idx)
                                   : f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        x[4 * i + 0] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const int idx = begin + lane + 64 * i;
      x[i] = idx < end ? __builtin_nontemporal_load(base + idx) : -INFINITY;
    }
  }
  chunk_reduce<GREEDY, VEC, ENT>(x, begin, c, c64, tab, st, se);
}

template <bool GREEDY, bool VEC, bool ENT = false>
__global__ __launch_bounds__(256) void row_stats_kernel(const float* __restrict__ logits, int V,
                                                        int nch, float c, ChunkStat* __restrict__ stats,
                                                        int32_t* xcnt, int nsync, int64_t stat_items,
                                                        double2* __restrict__ ent = nullptr, double c64 = 0.0) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  // the sliced walk's per-request coordination words start at zero (the
  // grid has at least 64 threads per row, so more than nsync = 4 B)
  if (xcnt && (int64_t)blockIdx.x * 256 + threadIdx.x < nsync) xcnt[blockIdx.x * 256 + threadIdx.x] = 0;
  __shared__ double tab[ENT ? kExp2Tab : 1];  // 2^(j/256) for exp2_neg_f64
  if (ENT) {
    static_assert(kExp2Tab == 256, "one table entry per thread of the 256-thread workgroup");
    tab[threadIdx.x] = exp2((double)threadIdx.x / 256.0);
    __syncthreads();  // before any thread leaves
  }
  if (item >= stat_items) return;  // 0 when the walk computes its rows' statistics (then only the clearing)
  const int64_t row = item / nch;
  const int ch = (int)(item - row * nch);
  ChunkStat st;
  double2 se;
  chunk_stat<GREEDY, VEC, ENT>(logits + row * (int64_t)V, V, ch, c, c64, tab, st, se);
  if (lane == 0) {
    stats[item] = st;
    if (ENT) ent[item] = se;
  }
}

// Per-row normalisation merged from the chunk statistics, by one 4-lane
// group (row_norm); under truncation also the row's threshold on
// logit - row max (in fp64, with its fp32 guard band): min-p's constant, or
// for the eta set T (ln S + min(ln eps, ln delta - H)) with the entropy
// H = ln S - E / S, E = sum_x w_x z_x (z in nats relative to the row maximum)
// merged from the chunk accumulators like S. The walk runs it for its own
// rows; row_finalize_kernel runs it for every row when the p rows are an
// output, so both see bitwise the same values. st and ent point at the row's
// chunk records (in the workspace, or in LDS for a row the walk computed).
__device__ __forceinline__ void finalize_row_from(const SampleParams& p, const ChunkStat* st, const double2* ent,
                                                  RowStat& r, RowThr& thr) {
  const int gl = threadIdx.x & (kRowGroup - 1);
  const int nch = p.nch;
  float lmax, av;
  double S;
  int arg;
  row_norm(st, nch, p.c, lmax, S, arg, av);
  thr = p.mp_thr;
  if (p.eta && lmax != -INFINITY) {
    // the row's S and E = sum_x w_x y_x (y in log2 units relative to the row
    // maximum) from the chunks' fp64 sums, all in fp64
    double accS = 0.0, accE = 0.0;
    for (int ch = gl; ch < nch; ch += kRowGroup) {
      const ChunkStat cs = st[ch];
      if (cs.lmax != -INFINITY) {
        const double dl = ((double)cs.lmax - (double)lmax) * p.c64;  // chunk max relative to the row's
        const double2 se = ent[ch];
        const double sc = exp2(dl);
        accS = fma(sc, se.x, accS);
        accE = fma(sc, fma(dl, se.x, se.y), accE);
      }
    }
    const double S64 = group_sum(accS);
    const double E = group_sum(accE) * 0.69314718055994530942;  // log2 units -> nats
    const double lnS = log(S64);
    const double H = lnS - E / S64;
    thr = make_row_thr(p.temp * (lnS + fmin(p.ln_eps, p.ln_delta - H)));
  }
  r.lmax = lmax;
  r.arg = arg;
  r.S = S;
}
__device__ __forceinline__ void finalize_row(const SampleParams& p, int64_t row, RowStat& r, RowThr& thr) {
  finalize_row_from(p, p.stats + row * p.nch, p.ent ? p.ent + row * p.nch : nullptr, r, thr);
}

// finalize_row_from computed by a whole wave, for the row a lazy walk has
// just reduced: every lane takes chunks lane, lane + 64, ... for the maximum
// (and, greedy, the argmax) and then for the per-chunk fp64 factors (the
// exp2 of each chunk's offset from the row maximum, all in parallel), which
// it leaves in LDS (f0, f1: nch doubles each; fsc: the eta set's exp2). The
// first four lanes then run the fmas in exactly the order of the 4-lane
// group (lane gl takes chunks gl, gl + 4, ... in turn, then the group's
// butterfly), so every value is bitwise that of finalize_row_from (a chunk
// with no finite logit has factors 0 and 0, and fma(0, 0, acc) is acc). All
// 64 lanes of one wave call it; lanes 0..3 hold the results.
__device__ __forceinline__ void finalize_row_wave(const SampleParams& p, const ChunkStat* st, const double2* ent,
                                                  double* f0, double* f1, double* fsc, RowStat& r, RowThr& thr) {
  const int lane = threadIdx.x & (kWave - 1);
  const int gl = lane & (kRowGroup - 1);
  const int nch = p.nch;
  float m = -INFINITY, av = -INFINITY;
  int ai = 0x7fffffff;
  bool bad = false;
  for (int ch = lane; ch < nch; ch += kWave) row_norm_acc(st[ch], m, av, ai, bad);
  m = wave_max(m);
  if (p.greedy) {  // the argmax is read by greedy walks only
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
      const float ov = __shfl_xor(av, o);
      const int oi = __shfl_xor(ai, o);
      if (ov > av || (ov == av && oi < ai)) { av = ov; ai = oi; }
    }
  }
  thr = p.mp_thr;
  if (__any(bad)) {
    r.lmax = -INFINITY;
    r.arg = kBadChunk;
    r.S = 0.0;
    return;
  }
  const bool eta = p.eta && m != -INFINITY;
  if (m != -INFINITY) {
    for (int ch = lane; ch < nch; ch += kWave) {
      const ChunkStat cs = st[ch];
      const bool live = cs.lmax != -INFINITY;
      f0[ch] = live ? cs.s : 0.0;
      f1[ch] = live ? exp2((double)(cs.lmax - m) * (double)p.c) : 0.0;
      if (eta) fsc[ch] = live ? exp2(((double)cs.lmax - (double)m) * p.c64) : 0.0;
    }
  }
  // the wave's own LDS stores, read back by its first four lanes (one wave
  // executes its LDS operations in order; the fences keep the compiler's
  // order)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  double acc = 0.0, accS = 0.0, accE = 0.0;
  if (m != -INFINITY && lane < kRowGroup) {
    for (int ch = gl; ch < nch; ch += kRowGroup) acc = fma(f0[ch], f1[ch], acc);
    if (eta) {
      for (int ch = gl; ch < nch; ch += kRowGroup) {
        const ChunkStat cs = st[ch];
        if (cs.lmax != -INFINITY) {
          const double dl = ((double)cs.lmax - (double)m) * p.c64;
          const double2 se = ent[ch];
          accS = fma(fsc[ch], se.x, accS);
          accE = fma(fsc[ch], fma(dl, se.x, se.y), accE);
        }
      }
    }
  }
  r.lmax = m;
  r.arg = ai;
  r.S = group_sum(acc);
  if (eta) {
    const double S64 = group_sum(accS);
    const double E = group_sum(accE) * 0.69314718055994530942;  // log2 units -> nats
    const double lnS = log(S64);
    const double H = lnS - E / S64;
    thr = make_row_thr(p.temp * (lnS + fmin(p.ln_eps, p.ln_delta - H)));
  }
}

// Every row's normalisation, for the p-row output (64 rows per workgroup).
__global__ __launch_bounds__(256) void row_finalize_kernel(SampleParams p, int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * (256 / kRowGroup) + (threadIdx.x / kRowGroup);
  if (row >= rows) return;  // the whole 4-lane group leaves together
  RowStat r;
  RowThr thr;
  finalize_row(p, row, r, thr);
  if ((threadIdx.x & (kRowGroup - 1)) == 0) {
    p.rowstats[row] = r;
    if (p.trunc) p.rthr[row] = thr;
  }
}

// Optional output of the p rows (tests and diagnostics): one wave per
// (row, chunk), every element evaluated exactly as the walk evaluates it.
__global__ __launch_bounds__(256) void probs_kernel(const float* __restrict__ logits, int V, int64_t rows, int nch,
                                                    float c, const RowStat* __restrict__ rs,
                                                    float* __restrict__ probs) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= rows * nch) return;
  const int64_t row = item / nch;
  const int ch = (int)(item - row * nch);
  const RowStat r = rs[row];
  const float invS = (float)(1.0 / r.S);
  const float* src = logits + row * (int64_t)V;
  float* dst = probs + row * (int64_t)V;
  const int begin = ch * kChunk, end = min(V, begin + kChunk);
  for (int idx = begin + lane; idx < end; idx += 64) dst[idx] = target_prob(src[idx], r.lmax, c, invS);
}

// ---------------------------------------------------------------------------
// Pass 3: the walk. One workgroup per request. Everything a decision needs
// at the first level of a position (p and q at every drafted token, the row
// normalisations) is gathered into LDS up front, in one round trip; every
// thread then evaluates the same accept tests on the same LDS values and so
// follows the same path without broadcasts. The whole workgroup joins the
// vocabulary passes that rejections make (one per residual level) and the
// final draw.

constexpr int kHalf = kChunk / 2;      // vocabulary unit of one wave in a residual pass
constexpr int kSpinLimit = 1 << 16;    // polls of a slice barrier before it gives up (flagged)

// A request is served by S workgroups of NT threads: S = 1 with NT = 512, or
// S > 1 "slices" with NT = 256. Every slice gathers the same inputs and takes
// the same decisions; a residual pass is split over the waves of all slices,
// which exchange their half-chunk masses through global memory and a
// per-request arrival counter (agent-scope release / acquire), so every
// slice then holds the same masses in the same order. Slice 0 alone writes
// the request's outputs and draws.
//
// The slices of a request are ordinary workgroups, so nothing guarantees
// that all of them are resident at once. Before the first exchange they
// agree on a mode: each one counts itself in on arrival; once all S have
// arrived (all are then running, and none leaves before the walk ends) the
// request runs sliced, and if the window passes first, one slice claims the
// request and walks it alone while the others leave. A slice never waits on
// a workgroup that has not started.
template <int NT>
struct WalkShared {
  static constexpr int NW = NT / kWave;
  int32_t par[kMaxNodes];
  int32_t tok[kMaxNodes];
  double u[kMaxNodes];
  float lgx[kMaxNodes];       // target logit of node j's token at its parent's row
  float qx[kMaxNodes];        // draft probability of node j's token at its parent's row
  double wx[kMaxNodes];       // deterministic siblings: unnormalised target mass of node j's token
  RowStat rs[kMaxNodes + 1];  // the request's rows: r = 0 root, r = 1 + j after node j
  RowThr th[kMaxNodes + 1];   // their thresholds of the allowed set (truncation)
  double csum[kMaxChunks];    // chunk masses of the distribution being drawn from
  double hsum[2 * kMaxChunks];// half-chunk masses of a residual pass
  double wtot[NW];            // per-wave sums of the draw's scan
  int32_t wcand[NW];          // per-wave first crossing of the draw (-1: none)
  int32_t wlast[NW];          // per-wave last token with mass
  double total;
  int32_t bad;
  int32_t mode;               // slice mode agreed at start-up (sliced walks)
};

struct Slices {
  int n;           // workgroups serving the request
  int id;          // this one's index among them
  double* xs;      // [2][2 nch] half-chunk masses, alternating buffer per pass
  int32_t* cnt;    // arrivals at the request's pass barriers (zeroed before the walk)
  int32_t* status;
};

// Mass of half-chunk h (2048 tokens) under max(0, p - cc q), one wave. The
// vector path splits this into a load step (32 + 32 values per lane) and a
// reduce step, so that a wave can have the next half-chunk in flight while it
// reduces the current one. The loads are buffer loads whose resource covers
// exactly the row: a float4 past the row's end reads as zero without touching
// memory (the reduce masks it), so every step issues the same loads with no
// branch, and the compiler waits for exactly the half-chunk being reduced.
struct HalfRegs {
  f32x4_t l[8], q[8];
};

__device__ __forceinline__ void half_load(HalfRegs& r, __amdgpu_buffer_rsrc_t lrs, __amdgpu_buffer_rsrc_t qrs, int h,
                                          int lane) {
  const int off = h * (kHalf * 4) + 16 * lane;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    r.l[i] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(lrs, off + 1024 * i, 0, 0));
    r.q[i] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(qrs, off + 1024 * i, 0, 0));
  }
}

// Unnormalised mass S * sum max(0, p - cc q) of the half-chunk in r: the four
// tokens of a float4 are added in fp32 (in fp64 under truncation), the rest in
// fp64. MASK drops float4s past the row's end (only the row's last half-chunk
// needs it).
template <bool MASK, bool TR>
__device__ __forceinline__ double half_reduce(const HalfRegs& r, int V, int h, int lane, float lw, float lmax, float c,
                                              float ccS, const RowThr& theta) {
  const int n4 = V >> 2;
  const int b4 = h * (kHalf / 4) + lane;
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float w0 = allowed<TR>(residual_weight(r.l[i].x, r.q[i].x, lw, c, ccS), r.l[i].x, lmax, theta);
    const float w1 = allowed<TR>(residual_weight(r.l[i].y, r.q[i].y, lw, c, ccS), r.l[i].y, lmax, theta);
    const float w2 = allowed<TR>(residual_weight(r.l[i].z, r.q[i].z, lw, c, ccS), r.l[i].z, lmax, theta);
    const float w3 = allowed<TR>(residual_weight(r.l[i].w, r.q[i].w, lw, c, ccS), r.l[i].w, lmax, theta);
    if (TR) {
      // every token in fp64: a deterministic candidate's weight can then be
      // taken back out of these sums with no fp32 rounding left behind
      double t = ((double)w0 + (double)w1) + ((double)w2 + (double)w3);
      if (MASK) t = b4 + 64 * i < n4 ? t : 0.0;
      acc += t;
    } else {
      float t = (w0 + w1) + (w2 + w3);
      if (MASK) t = b4 + 64 * i < n4 ? t : 0.f;
      acc += (double)t;
    }
  }
  return wave_sum(acc);
}

template <bool VEC, bool TR>
__device__ __forceinline__ double half_mass(const HalfRegs& r, int V, int h, int lane, float lw, float lmax, float c,
                                            float ccS, const RowThr& theta) {
  // wave-uniform test: is the whole half-chunk inside the row?
  return (h + 1) * kHalf <= V ? half_reduce<false, TR>(r, V, h, lane, lw, lmax, c, ccS, theta)
                              : half_reduce<true, TR>(r, V, h, lane, lw, lmax, c, ccS, theta);
}

template <bool TR>
__device__ __forceinline__ double half_scalar(const float* lrow, const float* qrow, int V, int h, float lw, float lmax,
                                              float c, float ccS, const RowThr& theta, int lane) {
  const int begin = h * kHalf, end = min(V, begin + kHalf);
  float lv[32], qv[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int idx = begin + lane + 64 * i;
    lv[i] = idx < end ? lrow[idx] : -INFINITY;
    qv[i] = (idx < end && ccS != 0.f) ? qrow[idx] : 0.f;  // cc = 0: p itself, q not needed
  }
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < 32; ++i)
    acc += (double)allowed<TR>(residual_weight(lv[i], qv[i], lw, c, ccS), lv[i], lmax, theta);
  return wave_sum(acc);
}

// A row pointer the whole workgroup shares, in scalar registers: buffer
// resources built from it stay uniform (a resource the compiler must treat
// as per-lane costs a loop of scalar reads around every load).
__device__ __forceinline__ const float* uniform_ptr(const float* ptr) {
  const uint64_t v = (uint64_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const float*)(((uint64_t)hi << 32) | lo);
}

// A half-chunk mass for the other slices of the request: a device-coherent
// store (it reaches memory, not only this XCD's L2).
__device__ __forceinline__ void publish(double* dst, double v) {
  __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Barrier of a request's slices (the pass_no-th of the request): this
// workgroup's stores are complete before it counts itself in, so a slice that
// has seen every arrival reads every slice's device-coherent stores.
__device__ __forceinline__ void slice_barrier(const Slices& sl, int pass_no) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(sl.cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int target = sl.n * pass_no;
    for (int spin = 0; __hip_atomic_load(sl.cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target; ++spin) {
      if (spin >= kSpinLimit) {  // cannot happen while all slices are resident; never wait forever
        flag(sl.status, kStSync);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

// Vocabulary pass of the request's workgroups: csum[ch] = mass of chunk ch
// under max(0, p - cc q) (its two halves added in order); returns the total
// (bitwise the same in every thread of every slice). pass_no counts the
// request's passes from 1 (the barrier target and the buffer parity).
// lw is the reference maximum of the p weight (the row maximum lmax; +inf
// switches p off, so that with S = 1 and cc = -1 the masses are those of q);
// membership in the allowed set is always decided against lmax.
template <bool VEC, int NT, bool TR>
__device__ __forceinline__ double residual_pass(WalkShared<NT>& sh, const float* lrow, const float* qrow, int V, int nch,
                                                float lw, float lmax, float c, const RowThr& theta, double S,
                                                double cc,
                                                const Slices& sl, int pass_no, const ChunkStat* cst) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nh = 2 * nch;
  const int gw = sl.id * NW + wave, GW = sl.n * NW;  // this wave among all the request's waves
  double* xb = sl.xs + (pass_no & 1) * nh;
  const float ccS = (float)(cc * S);
  const double invS = 1.0 / S;
  // Under truncation a token outside the allowed set weighs 0, and the set
  // is an upper set of logits (l - l_max above a threshold), so a chunk whose
  // maximum (cst: the row's chunk records) is outside holds no allowed token:
  // its two half-chunks have mass exactly 0 and are not read. Bit k of lmask
  // tells whether the wave's k-th half-chunk (gw + k GW) is live; later ones
  // are looked up one by one.
  uint64_t lmask = ~0ull;
  if (TR) {
    const int hl = gw + lane * GW;
    lmask = __ballot(hl < nh && is_allowed<TR>(cst[hl >> 1].lmax, lmax, theta));
  }
  auto live = [&](int k, int h) -> bool {  // k and h are the same in every lane of the wave
    if (!TR) return true;
    if (k < 64) return (lmask >> k) & 1;
    const float cm = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(cst[h >> 1].lmax)));
    return is_allowed<TR>(cm, lmax, theta);
  };
  if (VEC) {
    // two half-chunks per wave in flight: the next one's loads are issued
    // before the current one is reduced (past the row's end they read zeros).
    if (gw < nh) {
      const __amdgpu_buffer_rsrc_t lrs =
          __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(lrow), (short)0, V * 4, 0x00020000);
      // cc == 0 (the min-p visit pass: mass of p itself) needs no q: an empty
      // resource makes every q load read zero without touching memory
      const __amdgpu_buffer_rsrc_t qrs =
          __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(qrow), (short)0,
                                            __builtin_amdgcn_readfirstlane(cc == 0.0 ? 0 : V * 4), 0x00020000);
      HalfRegs ra, rb;
      if constexpr (TR) {
        // the loads go to live half-chunks only; a dead one gets mass 0 here.
        // next_live(k): the wave's first live half-chunk from its k-th on
        auto next_live = [&](int k) -> int {
          for (int h = gw + k * GW; h < nh && !live(k, h); ++k, h += GW)
            if (lane == 0) {
              sh.hsum[h] = 0.0;
              if (sl.n > 1) publish(xb + h, 0.0);
            }
          return k;
        };
        int k = next_live(0), h = gw + k * GW;
        half_load(ra, lrs, qrs, h, lane);
        while (h < nh) {
          const int k1 = next_live(k + 1), h1 = gw + k1 * GW;
          half_load(rb, lrs, qrs, h1, lane);
          const double m0 = half_mass<VEC, TR>(ra, V, h, lane, lw, lmax, c, ccS, theta) * invS;
          if (lane == 0) {
            sh.hsum[h] = m0;
            if (sl.n > 1) publish(xb + h, m0);
          }
          const int k2 = h1 < nh ? next_live(k1 + 1) : k1, h2 = gw + k2 * GW;
          half_load(ra, lrs, qrs, h2, lane);
          if (h1 < nh) {
            const double m1 = half_mass<VEC, TR>(rb, V, h1, lane, lw, lmax, c, ccS, theta) * invS;
            if (lane == 0) {
              sh.hsum[h1] = m1;
              if (sl.n > 1) publish(xb + h1, m1);
            }
          }
          k = k2;
          h = h2;
        }
      } else {
        half_load(ra, lrs, qrs, gw, lane);
        for (int h = gw; h < nh; h += 2 * GW) {
          const int h1 = h + GW;
          half_load(rb, lrs, qrs, h1, lane);
          const double m0 = half_mass<VEC, TR>(ra, V, h, lane, lw, lmax, c, ccS, theta) * invS;
          if (lane == 0) {
            sh.hsum[h] = m0;
            if (sl.n > 1) publish(xb + h, m0);
          }
          half_load(ra, lrs, qrs, h1 + GW, lane);
          if (h1 < nh) {
            const double m1 = half_mass<VEC, TR>(rb, V, h1, lane, lw, lmax, c, ccS, theta) * invS;
            if (lane == 0) {
              sh.hsum[h1] = m1;
              if (sl.n > 1) publish(xb + h1, m1);
            }
          }
        }
      }
    }
  } else {
    for (int k = 0, h = gw; h < nh; ++k, h += GW) {
      const double m = live(k, h) ? half_scalar<TR>(lrow, qrow, V, h, lw, lmax, c, ccS, theta, lane) * invS : 0.0;
      if (lane == 0) {
        sh.hsum[h] = m;
        if (sl.n > 1) publish(xb + h, m);
      }
    }
  }
  if (sl.n > 1) {
    // every slice's masses are published, then read back by every slice.
    // The masses go to memory with device-coherent stores (past the XCD's
    // non-coherent L2, no write-back of the whole L2 as a release fence
    // would do) and come back with device-coherent loads (no invalidation of
    // the L2 either); the wait before the arrival makes sure this wave's
    // stores have completed, so a slice that sees every arrival reads every
    // slice's masses.
    slice_barrier(sl, pass_no);
    for (int h = threadIdx.x; h < nh; h += NT)
      sh.hsum[h] = __hip_atomic_load(xb + h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  for (int ch = threadIdx.x; ch < nch; ch += NT) sh.csum[ch] = sh.hsum[2 * ch] + sh.hsum[2 * ch + 1];
  __syncthreads();
  if (wave == 0) {
    double a = 0.0;
    for (int ch = lane; ch < nch; ch += 64) a += sh.csum[ch];
    a = wave_sum(a);
    if (lane == 0) sh.total = a;
  }
  __syncthreads();
  const double t = sh.total;
  __syncthreads();  // every thread has the total before sh.total is reused
  return t;
}

// Inverse CDF: the smallest token whose inclusive prefix mass exceeds
// u * total. The chunk is found by a sequential prefix over the chunk masses
// (every thread, same order, same result). Inside it, lane l of wave w owns
// the DPL = 4096 / NT tokens at 64 DPL w + DPL l: lane sums are scanned
// within each wave, the wave totals are added in wave order, and the first
// lane whose inclusive prefix crosses the remainder picks the token among its
// DPL.
// removed: nodes whose tokens are out of the distribution (deterministic
// siblings already tried); their weights count as zero.
template <bool VEC, int NT, bool TR>
__device__ __forceinline__ int draw_token(WalkShared<NT>& sh, const float* lrow, const float* qrow, int V, int nch,
                                          int level, float lw, float lmax, float c, const RowThr& theta, double S,
                                          double cc,
                                          double u, double total, uint64_t removed) {
  constexpr int NW = NT / kWave;
  constexpr int kDrawPerLane = kChunk / NT;
  static_assert(kDrawPerLane % 4 == 0, "the draw gives each lane whole float4 of a chunk");
  const float ccS = (float)(cc * S);
  const double invS = 1.0 / S;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const double target = u * total;
  double run = 0.0, rem = 0.0;
  int chosen = -1, last = -1;
  for (int ch = 0; ch < nch; ++ch) {
    const double m = sh.csum[ch];
    if (m > 0.0) {
      last = ch;
      if (chosen < 0) {
        if (run + m > target) {
          chosen = ch;
          rem = target - run;
        } else {
          run += m;
        }
      }
    }
  }
  if (chosen < 0 && last >= 0) {  // rounding: u*total beyond the sequential prefix
    chosen = last;
    rem = sh.csum[last];
  }
  chosen = __builtin_amdgcn_readfirstlane(chosen);
  if (chosen < 0) return -1;  // no mass anywhere (flagged by the caller's statistics)
  const int begin = chosen * kChunk, end = min(V, begin + kChunk);
  const int x0 = begin + kDrawPerLane * (kWave * wave + lane);
  float lv[kDrawPerLane], qv[kDrawPerLane];
  if (VEC) {  // V % 4 == 0 and begin % 4 == 0: a float4 is wholly in or out
#pragma unroll
    for (int h = 0; h < kDrawPerLane / 4; ++h) {
      const int x = x0 + 4 * h;
      const float4 l4 = x < end ? *(const float4*)(lrow + x) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      const float4 q4 = (level > 0 && x < end) ? *(const float4*)(qrow + x) : make_float4(0.f, 0.f, 0.f, 0.f);
      lv[4 * h] = l4.x; lv[4 * h + 1] = l4.y; lv[4 * h + 2] = l4.z; lv[4 * h + 3] = l4.w;
      qv[4 * h] = q4.x; qv[4 * h + 1] = q4.y; qv[4 * h + 2] = q4.z; qv[4 * h + 3] = q4.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kDrawPerLane; ++i) {
      lv[i] = x0 + i < end ? lrow[x0 + i] : -INFINITY;
      qv[i] = (level > 0 && x0 + i < end) ? qrow[x0 + i] : 0.f;
    }
  }
  double w[kDrawPerLane];
#pragma unroll
  for (int i = 0; i < kDrawPerLane; ++i) {
    // weights of the distribution being drawn from (level 0: unnormalised p;
    // above: max(0, p - cc q) as the residual passes compute it)
    w[i] = level == 0 ? (double)allowed<TR>(target_weight(lv[i], lmax, c), lv[i], lmax, theta)
                      : (double)allowed<TR>(residual_weight(lv[i], qv[i], lw, c, ccS), lv[i], lmax, theta) * invS;
  }
  if (removed) {  // the same in every thread
    uint32_t m = 0;
    for (uint64_t e = removed; e; e &= e - 1) {
      const int d = sh.tok[__ffsll((unsigned long long)e) - 1] - x0;
      if (d >= 0 && d < kDrawPerLane) m |= 1u << d;
    }
#pragma unroll
    for (int i = 0; i < kDrawPerLane; ++i) w[i] = ((m >> i) & 1u) ? 0.0 : w[i];
  }
  double seg = 0.0;
  int lastpos = -1;
#pragma unroll
  for (int i = 0; i < kDrawPerLane; ++i) {
    seg += w[i];
    lastpos = w[i] > 0.0 ? x0 + i : lastpos;
  }
  double incl = seg;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) sh.wtot[wave] = incl;
  int lp = lastpos;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) lp = max(lp, __shfl_xor(lp, o));
  if (lane == 0) sh.wlast[wave] = lp;
  __syncthreads();
  double base = 0.0;
  for (int wv = 0; wv < wave; ++wv) base += sh.wtot[wv];
  incl += base;
  const double excl = incl - seg;
  const uint64_t hit = __ballot(incl > rem && seg > 0.0);
  if (lane == 0) sh.wcand[wave] = -1;
  if (hit) {
    const int owner = __ffsll((unsigned long long)hit) - 1;
    double r = excl;
    int found = -1;
#pragma unroll
    for (int i = 0; i < kDrawPerLane; ++i) {  // branch-free: the first crossing wins
      r += w[i];
      found = (found < 0 && w[i] > 0.0 && r > rem) ? x0 + i : found;
    }
    if (found < 0) found = lastpos;  // rounding inside the owning lane
    found = __shfl(found, owner);
    if (lane == 0) sh.wcand[wave] = found;
  }
  __syncthreads();
  int y = -1, ylast = -1;
  for (int wv = 0; wv < NW; ++wv) {
    const int cnd = sh.wcand[wv];
    y = (y < 0 && cnd >= 0) ? cnd : y;
    ylast = max(ylast, sh.wlast[wv]);
  }
  if (y < 0) y = ylast;  // rounding: the chunk's last token with mass
  __syncthreads();       // the per-wave slots are free again
  return y;
}

// outputs of a request whose inputs are invalid: nothing accepted, no token
__device__ __forceinline__ void skip_request(const SampleParams& p, int b, int32_t* acc_nodes, int32_t* toks_out,
                                             int bits, bool clear) {
  if (clear) {
    for (int i = threadIdx.x; i < p.max_depth; i += blockDim.x) acc_nodes[i] = -1;
    for (int i = threadIdx.x; i <= p.max_depth; i += blockDim.x) toks_out[i] = -1;
  }
  if (threadIdx.x == 0) {
    flag(p.status, bits);
    p.accept_len[b] = 0;
    if (p.residual_passes) p.residual_passes[b] = 0;
  }
}

// The current row's chunk records when the walk computes the statistics of
// the rows it reaches (LAZY), and the eta sums' records and 2^(j/256) table
// (TR: truncation forms only).
template <bool ON, bool TR>
struct LazyRow {
  ChunkStat cst[ON ? kMaxChunks : 1];
  double2 cent[ON && TR ? kMaxChunks : 1];
  double tab[ON && TR ? kExp2Tab : 1];
};

// A chunk record of the row being reached, for the request's other slices:
// device-coherent 8-byte stores into the workspace's statistics, read back
// after the slice barrier with device-coherent loads.
__device__ __forceinline__ void publish_chunk(ChunkStat* dst, const ChunkStat& cs) {
  uint64_t w0;
  __builtin_memcpy(&w0, &cs, 8);
  __hip_atomic_store((uint64_t*)dst, w0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&dst->s, cs.s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ ChunkStat fetch_chunk(ChunkStat* src) {
  ChunkStat cs;
  const uint64_t w0 = __hip_atomic_load((uint64_t*)src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_memcpy(&cs, &w0, 8);
  cs.s = __hip_atomic_load(&src->s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return cs;
}

// LAZY (no p-row output): no row-statistics pass runs before the walk; the
// walk computes the statistics of each row when it reaches it, with the
// row-statistics kernel's per-chunk code, so the rows it never reaches (those
// after a rejected node) are not read at all and the results are bitwise
// those of the other form. A sliced request splits each row's chunks over
// all its slices' waves and exchanges the records at a slice barrier.
template <bool VEC, int NT, bool TR, bool LAZY = false>
__global__ __launch_bounds__(NT, 2) void walk_kernel(SampleParams p) {  // >= 2 waves per SIMD: 256 VGPRs at most
  __shared__ WalkShared<NT> sh;
  __shared__ LazyRow<LAZY, TR> lz;
  // blocks past the walk's merge the step's split-K attention partials: the
  // walk leaves most of HBM's bandwidth and most CUs idle, and the work is
  // independent of it (one launch fewer)
  const int nwalk = p.B * p.slices;
  if ((int)blockIdx.x >= nwalk) {
    merge_split_rows<NT>(p.merge, (int)blockIdx.x - nwalk);
    return;
  }
  const int b = blockIdx.x / p.slices, slice = blockIdx.x - b * p.slices;
  int32_t* sync = p.slices > 1 ? p.xcnt + (int64_t)b * kWalkSync : nullptr;  // [0] passes, [1] arrivals, [2] mode
  if (sync && threadIdx.x == 0) __hip_atomic_fetch_add(sync + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t t_join = sync ? wall_clock64() : 0;
  // slice 0 reports invalid requests and the uniforms (every slice computes
  // the same; slice 0 runs whatever the mode turns out to be)
  const bool first = slice == 0;
  const int tid = threadIdx.x, lane = tid & 63;
  const int md = p.max_depth;
  int32_t* acc_nodes = p.accepted_nodes + (int64_t)b * md;
  int32_t* toks_out = p.out_tokens + (int64_t)b * (md + 1);
  if (!sync) {  // a single workgroup: the outputs are its own from the start
    for (int i = tid; i < md; i += NT) acc_nodes[i] = -1;
    for (int i = tid; i <= md; i += NT) toks_out[i] = -1;
  }

  const int n0 = p.cu_nodes[b], n1 = p.cu_nodes[b + 1];
  const int T = n1 - n0;
  const bool pack_ok = n0 >= 0 && T >= 0 && T <= p.max_nodes && n1 <= p.N;
  if (b == 0 && first && tid == 0 && p.cu_nodes[p.B] != p.N) flag(p.status, kStPacking);
  if (!pack_ok) {
    if (first) skip_request(p, b, acc_nodes, toks_out, kStPacking, sync != nullptr);
    return;
  }
  const uint32_t rid = p.request_id ? p.request_id[b] : (uint32_t)b;
  if (tid < T) {
    sh.par[tid] = p.parent[n0 + tid];
    sh.tok[tid] = p.tokens[n0 + tid];
    const double u = uniform01(p.seed, rid, (uint32_t)tid, 0u, p.step);
    sh.u[tid] = u;
    if (first && p.uniforms_out) p.uniforms_out[n0 + tid] = u;
  }
  if (first && tid == 0 && p.uniforms_out) p.uniforms_out[p.N + b] = uniform01(p.seed, rid, 0u, 1u, p.step);
  // the normalisation of every row of the request (row r = 0 root, 1 + j after
  // node j), one 4-lane group per row; its loads need only the packing, so
  // they overlap those of the tree
  // (uniform by construction; said explicitly, so that the compiler keeps the
  // rows' buffer resources in scalar registers)
  const int64_t row0 = (int64_t)__builtin_amdgcn_readfirstlane(n0 + b);
  if constexpr (LAZY) {
    if (TR && p.eta)
      for (int i = tid; i < kExp2Tab; i += NT) lz.tab[i] = exp2((double)i / 256.0);
  } else {
    for (int r = tid / kRowGroup; r <= T; r += NT / kRowGroup) {
      RowStat rs;
      RowThr th;
      finalize_row(p, row0 + r, rs, th);
      if ((tid & (kRowGroup - 1)) == 0) {
        sh.rs[r] = rs;
        if (TR) sh.th[r] = th;
      }
    }
  }
  __syncthreads();
  if (tid < kWave) {
    bool bad_tree = false, bad_tok = false;
    if (lane < T) {
      bad_tree = sh.par[lane] < -1 || sh.par[lane] >= lane;
      bad_tok = sh.tok[lane] < 0 || sh.tok[lane] >= p.V;
    }
    const bool any_tree = __any(bad_tree), any_tok = __any(bad_tok);
    if (lane == 0) sh.bad = (any_tree ? kStTree : 0) | (any_tok ? kStToken : 0);
  }
  __syncthreads();
  const int bad = __builtin_amdgcn_readfirstlane(sh.bad);
  if (bad) {
    if (first) skip_request(p, b, acc_nodes, toks_out, bad, sync != nullptr);
    return;
  }

  const int64_t V = p.V;
  // gathers: p-logit and q of every drafted token at its parent's row
  if (tid < T) {
    const int64_t r = row0 + sh.par[tid] + 1;
    sh.lgx[tid] = p.logits[r * V + sh.tok[tid]];
    sh.qx[tid] = (p.greedy || p.det) ? 0.f : p.q[r * V + sh.tok[tid]];
  }
  __syncthreads();
  if (!LAZY && p.det && !p.greedy && tid < T) {
    // the token's unnormalised target mass, in the same terms as the sum it
    // will be taken out of: under truncation the visit pass's fp32 weight
    // relative to the row maximum; otherwise the row statistics' weight
    // relative to its chunk's maximum, scaled as row_norm scales chunk sums
    const int pr = sh.par[tid] + 1;
    const int64_t r = row0 + pr;
    const float lx = sh.lgx[tid];
    const RowStat rs = sh.rs[pr];
    double wx;
    if (TR) {
      wx = (double)allowed<TR>(target_weight(lx, rs.lmax, p.c), lx, rs.lmax, sh.th[pr]);
    } else {
      const ChunkStat cs = p.stats[r * p.nch + sh.tok[tid] / kChunk];
      wx = cs.lmax == -INFINITY ? 0.0
                                : (double)target_weight(lx, cs.lmax, p.c) *
                                      exp2((double)(cs.lmax - rs.lmax) * (double)p.c);
    }
    sh.wx[tid] = wx;
  }
  // the mode: sliced, or this slice alone, or another slice alone (leave)
  Slices sl{1, 0, nullptr, nullptr, p.status};
  if (sync) {
    if (tid == 0) {
      int mode;
      for (;;) {
        mode = __hip_atomic_load(sync + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (mode != 0) break;
        int want = 0;
        if (p.join_ticks > 0 &&
            __hip_atomic_load(sync + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= p.slices)
          want = 1;
        else if (wall_clock64() - t_join >= p.join_ticks) want = 2 + 4 * slice;
        if (want) {
          int expect = 0;
          mode = __hip_atomic_compare_exchange_strong(sync + 2, &expect, want, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT)
                     ? want
                     : expect;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      sh.mode = mode;
    }
    __syncthreads();
    const int mode = __builtin_amdgcn_readfirstlane(sh.mode);
    if (mode == 1) {
      sl = Slices{p.slices, slice, p.xs + (int64_t)b * 4 * p.nch, sync, p.status};
    } else if (mode != 2 + 4 * slice) {
      return;  // another slice walks this request alone
    }
    if (sl.id == 0) {
      for (int i = tid; i < md; i += NT) acc_nodes[i] = -1;
      for (int i = tid; i <= md; i += NT) toks_out[i] = -1;
    }
  }
  const bool lead = sl.id == 0;  // the slice that writes the request's outputs and draws
  __syncthreads();

  int pos = -1, depth = 0, passes = 0, bonus = -1;
  int npass = 0;  // slice barriers passed (every slice counts the same)
  for (;;) {
    const int r = pos + 1;
    const int64_t row = row0 + r;
    const float* lrow = p.logits + row * V;
    const float* qrow = (p.greedy || !p.q) ? nullptr : p.q + row * V;
    if constexpr (LAZY) {
      // this row's statistics (each wave takes chunks wave, wave + NW, ...),
      // then its normalisation, then the deterministic candidates' masses of
      // the children of this position: what the row-statistics pass and the
      // walk's start do for every row in the other form
      constexpr int NW = NT / kWave;
      const int wave = tid >> 6;
      const int gw = sl.id * NW + wave, GW = sl.n * NW;  // this wave among all the request's waves
      const float* base = uniform_ptr(lrow);
      ChunkStat* gst = p.stats + row * p.nch;
      double2* gent = TR && p.eta ? p.ent + row * p.nch : nullptr;
      for (int ch = gw; ch < p.nch; ch += GW) {
        ChunkStat cs;
        double2 se;
        if (p.greedy) chunk_stat<true, VEC, false>(base, p.V, ch, p.c, p.c64, lz.tab, cs, se);
        else if (TR && p.eta) chunk_stat<false, VEC, TR>(base, p.V, ch, p.c, p.c64, lz.tab, cs, se);
        else chunk_stat<false, VEC, false>(base, p.V, ch, p.c, p.c64, lz.tab, cs, se);
        if (lane == 0) {
          if (sl.n > 1) {
            publish_chunk(gst + ch, cs);
            if (gent) {
              publish(&gent[ch].x, se.x);
              publish(&gent[ch].y, se.y);
            }
          } else {
            lz.cst[ch] = cs;
            if (TR) lz.cent[ch] = se;
          }
        }
      }
      if (sl.n > 1) {
        slice_barrier(sl, ++npass);
        for (int ch = tid; ch < p.nch; ch += NT) {
          lz.cst[ch] = fetch_chunk(gst + ch);
          if (gent)
            lz.cent[ch] = make_double2(__hip_atomic_load(&gent[ch].x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                                       __hip_atomic_load(&gent[ch].y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        }
      }
      __syncthreads();
      if (tid < kWave) {
        RowStat rs;
        RowThr th;
        // (scratch: the residual pass's half-chunk masses and the draw's
        // chunk masses, both rewritten before their next use)
        finalize_row_wave(p, lz.cst, lz.cent, sh.hsum, sh.hsum + kMaxChunks, sh.csum, rs, th);
        if (tid == 0) {
          sh.rs[r] = rs;
          if (TR) sh.th[r] = th;
        }
      }
      __syncthreads();
      if (p.det && !p.greedy) {
        if (tid < T && sh.par[tid] == pos) {
          const float lx = sh.lgx[tid];
          const RowStat rs = sh.rs[r];
          double wx;
          if (TR) {
            wx = (double)allowed<TR>(target_weight(lx, rs.lmax, p.c), lx, rs.lmax, sh.th[r]);
          } else {
            const ChunkStat cs = lz.cst[sh.tok[tid] / kChunk];
            wx = cs.lmax == -INFINITY ? 0.0
                                      : (double)target_weight(lx, cs.lmax, p.c) *
                                            exp2((double)(cs.lmax - rs.lmax) * (double)p.c);
          }
          sh.wx[tid] = wx;
        }
        __syncthreads();
      }
    }
    const RowStat st = sh.rs[r];
    const RowThr th = TR ? sh.th[r] : RowThr{};  // this row's threshold of the allowed set
    // this row's chunk records (in LDS when the walk reduced the row itself)
    const ChunkStat* rowcs = LAZY ? (const ChunkStat*)lz.cst : p.stats + row * p.nch;
    // children of pos in increasing index: the same ballot in every wave
    const uint64_t kids = __ballot(lane < T && sh.par[lane] == pos);
    if (st.lmax == -INFINITY) {  // no finite logit: p is undefined here, stop without a token
      if (lead && tid == 0) flag(p.status, kStNonFinite);
      break;
    }

    if (p.greedy) {  // accept the first child carrying the argmax token
      int next = -1;
      for (uint64_t k = kids; k; k &= k - 1) {
        const int ch = __ffsll((unsigned long long)k) - 1;
        if (sh.tok[ch] == st.arg) { next = ch; break; }
      }
      next = __builtin_amdgcn_readfirstlane(next);
      if (next < 0) { bonus = st.arg; break; }
      if (lead && tid == 0) { acc_nodes[depth] = next; toks_out[depth] = sh.tok[next]; }
      ++depth;
      pos = next;
      continue;
    }

    if (TR && p.rule == 3) {
      // Truncation-based verification ([LOSSY] 3.2): the first child whose
      // token is in the allowed set is accepted (the fp32 membership test of
      // the truncation; no uniform). With every child rejected the token is
      // drawn from q restricted to the set: a pass with the p weight switched
      // off (reference maximum +inf) and cc S = -1 leaves q 1{x in A} masses.
      // At a leaf it is drawn from the truncated target.
      int accepted = -1;
      for (uint64_t k = kids; k; k &= k - 1) {
        const int ch = __ffsll((unsigned long long)k) - 1;
        if (is_allowed<TR>(sh.lgx[ch], st.lmax, th)) { accepted = ch; break; }
        ++passes;  // rejections
      }
      accepted = __builtin_amdgcn_readfirstlane(accepted);
      if (accepted >= 0) {
        if (lead && tid == 0) { acc_nodes[depth] = accepted; toks_out[depth] = sh.tok[accepted]; }
        ++depth;
        pos = accepted;
        continue;
      }
      int level = 0;
      float lw = st.lmax;
      double cc = 0.0, total = 0.0;
      if (kids) {
        total = residual_pass<VEC, NT, TR>(sh, lrow, qrow, p.V, p.nch, INFINITY, st.lmax, p.c, th, 1.0, -1.0, sl,
                                           ++npass, rowcs);
        if (__builtin_amdgcn_readfirstlane(total > 0.0 ? 1 : 0)) {
          level = 1;
          lw = INFINITY;
          cc = -1.0;
        } else if (lead && tid == 0) {
          flag(p.status, kStZeroResidual);
        }
      }
      if (level == 0)
        total = residual_pass<VEC, NT, TR>(sh, lrow, qrow, p.V, p.nch, st.lmax, st.lmax, p.c, th, 1.0, 0.0, sl,
                                           ++npass, rowcs);
      if (!lead) return;  // the draw needs no other slice
      const double uf = uniform01(p.seed, rid, 0u, 1u, p.step);
      bonus = draw_token<VEC, NT, TR>(sh, lrow, qrow, p.V, p.nch, level, lw, st.lmax, p.c, th, 1.0, cc, uf, total, 0);
      break;
    }

    // The target here: p, or under min-p truncation p_Theta = p on the allowed
    // set renormalised by its mass S_A (one vocabulary pass at this position,
    // which also leaves the chunk masses of p_Theta in csum for a draw).
    double Srow = st.S;
    bool csum_ok = false;      // csum holds the chunk masses of the current level
    if (TR) {
      Srow = residual_pass<VEC, NT, TR>(sh, lrow, qrow, p.V, p.nch, st.lmax, st.lmax, p.c, th, 1.0, 0.0, sl, ++npass, rowcs);
      csum_ok = true;
    }
    if (p.det) {
      // Deterministic candidates ([LOSSY] G.3): child i is accepted with
      // probability p~_i(x) = W(x) / M_i, M_i being the target's mass left
      // after the candidates rejected before it were taken out; a token
      // already taken out has p~ = 0. No vocabulary pass: W comes from the
      // gathers and M from the row's sum (under truncation, from this
      // position's pass). A remainder below 1e-12 of the row's mass is
      // rounding noise and counts as zero.
      double M = Srow;
      uint64_t removed = 0;  // children whose token is out of the target
      int accepted = -1;
      for (uint64_t k = kids; k; k &= k - 1) {
        const int ch = __ffsll((unsigned long long)k) - 1;
        const int x = sh.tok[ch];
        bool dup = false;
        for (uint64_t m = removed; m; m &= m - 1) dup |= sh.tok[__ffsll((unsigned long long)m) - 1] == x;
        const double W = sh.wx[ch];
        const double P = dup ? 0.0 : W / M;
        const int ok = __builtin_amdgcn_readfirstlane((P > 0.0 && sh.u[ch] <= P) ? 1 : 0);
        if (ok) { accepted = ch; break; }
        ++passes;
        if (!dup) {
          const double Mn = M - W;
          if (__builtin_amdgcn_readfirstlane(Mn > 1e-12 * Srow ? 1 : 0)) {
            M = Mn;
            removed |= 1ull << ch;
          } else if (lead && tid == 0) {
            flag(p.status, kStZeroResidual);
          }
        }
      }
      if (accepted >= 0) {
        if (lead && tid == 0) { acc_nodes[depth] = accepted; toks_out[depth] = sh.tok[accepted]; }
        ++depth;
        pos = accepted;
        continue;
      }
      if (!lead) return;  // the draw needs no other slice
      // draw from the target without the removed candidates: chunk masses
      // (from the row statistics, or this position's pass under truncation)
      // minus the removed weights
      if (!TR) {
        const ChunkStat* cs = rowcs;
        for (int ch = tid; ch < p.nch; ch += NT) {
          const ChunkStat s = cs[ch];
          sh.csum[ch] = s.lmax == -INFINITY ? 0.0 : s.s * exp2((double)(s.lmax - st.lmax) * (double)p.c);
        }
        __syncthreads();
      }
      if (removed) {
        if (tid == 0) {
          for (uint64_t m = removed; m; m &= m - 1) {
            const int j = __ffsll((unsigned long long)m) - 1;
            const int ch = sh.tok[j] / kChunk;
            const double before = sh.csum[ch], after = before - sh.wx[j];
            sh.csum[ch] = after > 1e-12 * before ? after : 0.0;
          }
        }
        __syncthreads();
      }
      const double uf = uniform01(p.seed, rid, 0u, 1u, p.step);
      bonus = draw_token<VEC, NT, TR>(sh, lrow, qrow, p.V, p.nch, 0, st.lmax, st.lmax, p.c, th, Srow, 0.0, uf, M,
                                      removed);
      break;
    }

    const float invS = (float)(1.0 / Srow);
    double cc = 0.0, M = 1.0;  // current distribution max(0, p - cc q) / M (cc = 0: p itself)
    int level = 0;
    int accepted = -1;
    for (uint64_t k = kids; k; k &= k - 1) {
      const int ch = __ffsll((unsigned long long)k) - 1;
      const float pf = allowed<TR>(target_prob(sh.lgx[ch], st.lmax, p.c, invS), sh.lgx[ch], st.lmax, th);
      const double qv = (double)sh.qx[ch];
      const double P = level == 0 ? (double)pf : fmax(0.0, (double)pf - cc * qv) / M;
      // accept test u * den <= num: lossless (P, q), lenience (P, l q) or
      // interpolation (lambda P + (1 - lambda) q, q)
      const double rp = (double)p.rule_param;
      const double num = p.rule == 2 ? rp * P + (1.0 - rp) * qv : P;
      const double den = p.rule == 1 ? rp * qv : qv;
      const int ok = __builtin_amdgcn_readfirstlane((num > 0.0 && sh.u[ch] * den <= num) ? 1 : 0);
      if (ok) { accepted = ch; break; }
      // rejected: the next sibling is tested against the next residual level
      const double cn = cc + M;
      const double Mn =
          residual_pass<VEC, NT, TR>(sh, lrow, qrow, p.V, p.nch, st.lmax, st.lmax, p.c, th, Srow, cn, sl, ++npass, rowcs);
      ++passes;
      if (__builtin_amdgcn_readfirstlane(Mn > 0.0 ? 1 : 0)) {
        cc = cn;
        M = Mn;
        ++level;
        csum_ok = true;
      } else {
        if (lead && tid == 0) flag(p.status, kStZeroResidual);
        csum_ok = false;
      }
    }
    if (accepted >= 0) {
      if (lead && tid == 0) { acc_nodes[depth] = accepted; toks_out[depth] = sh.tok[accepted]; }
      ++depth;
      pos = accepted;
      continue;
    }
    // final draw at this position from the current distribution
    double total;
    if (level == 0 && TR) {  // the chunk masses of p_Theta from this position's pass
      total = Srow;
    } else if (level == 0) {
      const ChunkStat* cs = rowcs;
      for (int ch = tid; ch < p.nch; ch += NT) {
        const ChunkStat s = cs[ch];
        sh.csum[ch] = s.lmax == -INFINITY ? 0.0 : s.s * exp2((double)(s.lmax - st.lmax) * (double)p.c);
      }
      __syncthreads();
      total = st.S;
    } else {
      if (!csum_ok) {
        residual_pass<VEC, NT, TR>(sh, lrow, qrow, p.V, p.nch, st.lmax, st.lmax, p.c, th, Srow, cc, sl, ++npass, rowcs);
        ++passes;
      }
      total = M;
    }
    if (!lead) return;  // the draw needs no other slice: the rest are done
    const double uf = uniform01(p.seed, rid, 0u, 1u, p.step);
    bonus = draw_token<VEC, NT, TR>(sh, lrow, qrow, p.V, p.nch, level, st.lmax, st.lmax, p.c, th, Srow, cc, uf, total,
                                    0);
    break;
  }
  if (lead && tid == 0) {
    toks_out[depth] = bonus;
    p.accept_len[b] = depth;
    if (p.residual_passes) p.residual_passes[b] = passes;
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_sampler(const SampleParams& p, bool vec4, hipStream_t stream, const SampleEvents& ev) {
  if (p.B <= 0) return hipSuccess;
  const int64_t rows = (int64_t)p.N + p.B;
  const int64_t items = rows * p.nch;
  // when the walk computes the statistics of the rows it reaches itself: no
  // statistics blocks, only the clearing of the sliced walk's coordination
  // words, if any
  const bool lazy = p.lazy != 0;
  const int ns = p.B * kWalkSync;
  int32_t* xc = p.slices > 1 ? p.xcnt : nullptr;
  const int64_t stat_items = lazy ? 0 : items;
  const int nsb = lazy ? ((xc && !p.coord_cleared) ? (ns + 255) / 256 : 0) : (int)((items + 3) / 4);
  const dim3 sgrid((unsigned)nsb);
  const dim3 pgrid((unsigned)((items + 3) / 4));     // the p-row output (one wave per (row, chunk) as well)
  if (ev.start) (void)hipEventRecord(ev.start, stream);
  if (sgrid.x > 0) {
    if (p.greedy) {
      if (vec4) row_stats_kernel<true, true><<<sgrid, 256, 0, stream>>>(p.logits, p.V, p.nch, p.c, p.stats, xc, ns, stat_items);
      else row_stats_kernel<true, false><<<sgrid, 256, 0, stream>>>(p.logits, p.V, p.nch, p.c, p.stats, xc, ns, stat_items);
    } else if (p.eta) {
      if (vec4)
        row_stats_kernel<false, true, true><<<sgrid, 256, 0, stream>>>(p.logits, p.V, p.nch, p.c, p.stats, xc,
                                                                      ns, stat_items, p.ent, p.c64);
      else
        row_stats_kernel<false, false, true><<<sgrid, 256, 0, stream>>>(p.logits, p.V, p.nch, p.c, p.stats, xc,
                                                                       ns, stat_items, p.ent, p.c64);
    } else {
      if (vec4) row_stats_kernel<false, true><<<sgrid, 256, 0, stream>>>(p.logits, p.V, p.nch, p.c, p.stats, xc, ns, stat_items);
      else row_stats_kernel<false, false><<<sgrid, 256, 0, stream>>>(p.logits, p.V, p.nch, p.c, p.stats, xc, ns, stat_items);
    }
  }
  if (ev.stats_stop) (void)hipEventRecord(ev.stats_stop, stream);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (p.probs_out && !p.greedy) {
    row_finalize_kernel<<<dim3((unsigned)((rows + 63) / 64)), 256, 0, stream>>>(p, rows);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    probs_kernel<<<pgrid, 256, 0, stream>>>(p.logits, p.V, rows, p.nch, p.c, p.rowstats, p.probs_out);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // the walk's grid: its workgroups, then the step's merge blocks, if any
  if (p.slices > 1) {
    const dim3 grid((unsigned)(p.B * p.slices + merge_blocks(p.merge, 256)));
    if (lazy) {
      if (p.trunc) {
        if (vec4) walk_kernel<true, 256, true, true><<<grid, dim3(256), 0, stream>>>(p);
        else walk_kernel<false, 256, true, true><<<grid, dim3(256), 0, stream>>>(p);
      } else {
        if (vec4) walk_kernel<true, 256, false, true><<<grid, dim3(256), 0, stream>>>(p);
        else walk_kernel<false, 256, false, true><<<grid, dim3(256), 0, stream>>>(p);
      }
    } else {
      if (p.trunc) {
        if (vec4) walk_kernel<true, 256, true><<<grid, dim3(256), 0, stream>>>(p);
        else walk_kernel<false, 256, true><<<grid, dim3(256), 0, stream>>>(p);
      } else {
        if (vec4) walk_kernel<true, 256, false><<<grid, dim3(256), 0, stream>>>(p);
        else walk_kernel<false, 256, false><<<grid, dim3(256), 0, stream>>>(p);
      }
    }
  } else {
    const dim3 grid((unsigned)(p.B + merge_blocks(p.merge, 512)));
    if (lazy) {
      if (p.trunc) {
        if (vec4) walk_kernel<true, 512, true, true><<<grid, dim3(512), 0, stream>>>(p);
        else walk_kernel<false, 512, true, true><<<grid, dim3(512), 0, stream>>>(p);
      } else {
        if (vec4) walk_kernel<true, 512, false, true><<<grid, dim3(512), 0, stream>>>(p);
        else walk_kernel<false, 512, false, true><<<grid, dim3(512), 0, stream>>>(p);
      }
    } else {
      if (p.trunc) {
        if (vec4) walk_kernel<true, 512, true><<<grid, dim3(512), 0, stream>>>(p);
        else walk_kernel<false, 512, true><<<grid, dim3(512), 0, stream>>>(p);
      } else {
        if (vec4) walk_kernel<true, 512, false><<<grid, dim3(512), 0, stream>>>(p);
        else walk_kernel<false, 512, false><<<grid, dim3(512), 0, stream>>>(p);
      }
    }
  }
  if (ev.stop) (void)hipEventRecord(ev.stop, stream);
  return hipGetLastError();
}

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

int walk_slices(int B, int nch, bool passes, int mode) {
  if (!passes || B <= 0 || mode == kWalkSingle) return 1;
  // every wave of the request gets at least one half-chunk; past 8 slices the
  // wider exchange costs more than the shorter passes save (measured: 16
  // slices were slower than 8 at batch 16 and 32, vocabulary 128256)
  const int64_t by_work = (2 * (int64_t)nch + 3) / 4;
  if (mode == kWalkSliced) return by_work >= 2 ? (int)(by_work < 8 ? by_work : 8) : 1;
  static int per_cu_cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  if (per_cu_cached[dev] == 0) {
    int a = 0, b = 0;
    int t = 0;
    // (the forms launched without the p-row output, the usual case: their
    // LDS holds a row's chunk records besides)
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, walk_kernel<true, 256, false, true>, 256, 0) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, walk_kernel<false, 256, false, true>, 256, 0) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&t, walk_kernel<true, 256, true, true>, 256, 0) != hipSuccess) {
      (void)hipGetLastError();
      a = b = t = 0;
    }
    per_cu_cached[dev] = max(1, min(min(a, b), t));  // 1 when unknown: then a batch of >= CUs requests gets 1 slice
  }
  const int64_t capacity = (int64_t)per_cu_cached[dev] * device_cus();
  int64_t s = capacity / B;
  if (s > by_work) s = by_work;
  if (s > 8) s = 8;
  // two slices would take the same CUs as one 512-thread workgroup per request
  return s >= 4 ? (int)s : 1;
}

}  // namespace sv
