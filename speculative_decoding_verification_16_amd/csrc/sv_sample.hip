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
//  2. walk_kernel       -- one workgroup per request. It climbs down the tree
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

// ---------------------------------------------------------------------------
// Pass 1: per (row, chunk) statistics. One wave per chunk of 4096 logits; a
// lane holds 64 of them in registers, so the row is read from HBM once.
template <bool GREEDY, bool VEC>
__global__ __launch_bounds__(256) void row_stats_kernel(const float* __restrict__ logits, int V, int64_t rows,
                                                        int nch, float c, ChunkStat* __restrict__ stats,
                                                        int32_t* status) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= rows * nch) return;
  const int64_t row = item / nch;
  const int ch = (int)(item - row * nch);
  const float* base = logits + row * (int64_t)V;
  const int begin = ch * kChunk;
  const int end = min(V, begin + kChunk);

  float x[64];
  if (VEC) {
    const float4* b4 = (const float4*)(base + begin);
    const int n4 = (end - begin) >> 2;  // V % 4 == 0 on this path
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int idx = lane + 64 * i;
      const float4 v = idx < n4 ? b4[idx] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      x[4 * i + 0] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const int idx = begin + lane + 64 * i;
      x[i] = idx < end ? base[idx] : -INFINITY;
    }
  }
  // element (i) of this lane is token begin + 4*(lane + 64*(i/4)) + i%4 (VEC)
  // or begin + lane + 64*i (scalar); both visit a lane's tokens in increasing order
  float mx = -INFINITY;
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
  if (__any(bad) && lane == 0) flag(status, kStNonFinite);
  wave_argmax(mx, ai);
  double s = 0.0;
  if (!GREEDY && mx != -INFINITY) {
#pragma unroll
    for (int i = 0; i < 64; ++i) s += (double)target_weight(x[i], mx, c);
    s = wave_sum(s);
  }
  if (lane == 0) {
    ChunkStat st;
    st.lmax = mx;
    st.arg = mx == -INFINITY ? begin : ai;
    st.s = s;
    stats[item] = st;
  }
}

// Optional output of the p rows (tests and diagnostics): same grid as pass 1.
template <bool VEC>
__global__ __launch_bounds__(256) void probs_kernel(const float* __restrict__ logits, int V, int64_t rows, int nch,
                                                    float c, const ChunkStat* __restrict__ stats,
                                                    float* __restrict__ probs) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= rows * nch) return;
  const int64_t row = item / nch;
  const int ch = (int)(item - row * nch);
  float lmax, av;
  double S;
  int arg;
  row_norm(stats + row * nch, nch, c, lmax, S, arg, av);
  const float invS = (float)(1.0 / S);
  const float* src = logits + row * (int64_t)V;
  float* dst = probs + row * (int64_t)V;
  const int begin = ch * kChunk, end = min(V, begin + kChunk);
  for (int idx = begin + lane; idx < end; idx += 64) dst[idx] = target_prob(src[idx], lmax, c, invS);
}

// ---------------------------------------------------------------------------
// Walk helpers (whole workgroup).

struct WalkShared {
  int32_t par[kMaxNodes];
  int32_t tok[kMaxNodes];
  double u[kMaxNodes];
  double csum[kMaxChunks];  // per-chunk masses of the distribution to draw from
  double part[32];          // wave partials
  float lmax;
  double S;
  int arg;
  uint64_t kids;
  int decision;
  double total;
  int ybest;
};

// mass of chunk ch under P(x) = max(0, p(x) - cc * q(x)) (unnormalised by M)
template <bool VEC>
__device__ __forceinline__ double residual_chunk(const float* lrow, const float* qrow, int V, int ch, float lmax,
                                                 float c, float invS, double cc, int lane) {
  const int begin = ch * kChunk, end = min(V, begin + kChunk);
  double acc = 0.0;
  if (VEC) {
    const float4* l4 = (const float4*)(lrow + begin);
    const float4* q4 = (const float4*)(qrow + begin);
    const int n4 = (end - begin) >> 2;
#pragma unroll 1
    for (int h = 0; h < 4; ++h) {
      float4 lv[4], qv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int idx = lane + 64 * (4 * h + i);
        lv[i] = idx < n4 ? l4[idx] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        qv[i] = idx < n4 ? q4[idx] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc += fmax(0.0, (double)target_prob(lv[i].x, lmax, c, invS) - cc * (double)qv[i].x);
        acc += fmax(0.0, (double)target_prob(lv[i].y, lmax, c, invS) - cc * (double)qv[i].y);
        acc += fmax(0.0, (double)target_prob(lv[i].z, lmax, c, invS) - cc * (double)qv[i].z);
        acc += fmax(0.0, (double)target_prob(lv[i].w, lmax, c, invS) - cc * (double)qv[i].w);
      }
    }
  } else {
    for (int idx = begin + lane; idx < end; idx += 64)
      acc += fmax(0.0, (double)target_prob(lrow[idx], lmax, c, invS) - cc * (double)qrow[idx]);
  }
  return wave_sum(acc);
}

// one element of the distribution being drawn from (level 0: unnormalised p)
__device__ __forceinline__ double draw_weight(const float* lrow, const float* qrow, int x, int level, float lmax,
                                              float c, float invS, double cc) {
  if (level == 0) return (double)target_weight(lrow[x], lmax, c);
  return fmax(0.0, (double)target_prob(lrow[x], lmax, c, invS) - cc * (double)qrow[x]);
}

// Vocabulary pass: csum[ch] = mass of chunk ch under max(0, p - cc q);
// returns the total (the same value in every thread).
template <bool VEC>
__device__ double residual_pass(WalkShared& sh, const float* lrow, const float* qrow, int V, int nch, float lmax,
                                float c, float invS, double cc) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int ch = wave; ch < nch; ch += nw) {
    const double m = residual_chunk<VEC>(lrow, qrow, V, ch, lmax, c, invS, cc, lane);
    if (lane == 0) sh.csum[ch] = m;
  }
  __syncthreads();
  if (wave == 0) {
    double a = 0.0;
    for (int ch = lane; ch < nch; ch += 64) a += sh.csum[ch];
    a = wave_sum(a);
    if (lane == 0) sh.total = a;
  }
  __syncthreads();
  const double t = sh.total;
  __syncthreads();  // everyone has the total before sh.total is reused
  return t;
}

// Inverse CDF over csum (masses per chunk, total = their sum): the smallest
// token whose inclusive prefix exceeds u * total. The chunk is found by a
// sequential prefix over chunk masses, the token by a wave scan inside it.
__device__ int draw_token(WalkShared& sh, const float* lrow, const float* qrow, int V, int nch, int level,
                          float lmax, float c, float invS, double cc, double u, double total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) {
    const double target = u * total;
    double run = 0.0;
    int chosen = -1;
    double rem = 0.0;
    for (int ch = 0; ch < nch; ++ch) {
      const double m = sh.csum[ch];
      if (m > 0.0) {
        if (run + m > target) { chosen = ch; rem = target - run; break; }
        run += m;
      }
    }
    if (chosen < 0) {  // rounding: u*total beyond the sequential prefix; take the last chunk with mass
      for (int ch = nch - 1; ch >= 0; --ch)
        if (sh.csum[ch] > 0.0) { chosen = ch; rem = sh.csum[ch]; break; }
    }
    sh.decision = chosen;
    sh.total = rem;
  }
  __syncthreads();
  const int ch = sh.decision;
  const double rem = sh.total;
  if (wave == 0) {
    int y = -1;
    if (ch >= 0) {
      // lane owns tokens [seg0, seg1) of the chunk
      const int begin = ch * kChunk, end = min(V, begin + kChunk);
      const int seg0 = begin + 64 * lane, seg1 = min(end, seg0 + 64);
      double seg = 0.0;
      int lastpos = -1;
      for (int x = seg0; x < seg1; ++x) {
        const double w = draw_weight(lrow, qrow, x, level, lmax, c, invS, cc);
        seg += w;
        if (w > 0.0) lastpos = x;
      }
      double incl = seg;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const double t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      const double excl = incl - seg;
      const uint64_t hit = __ballot(incl > rem && seg > 0.0);
      int found = -1;
      if (hit) {
        const int owner = __ffsll((unsigned long long)hit) - 1;
        if (lane == owner) {
          double run = excl;
          for (int x = seg0; x < seg1; ++x) {
            const double w = draw_weight(lrow, qrow, x, level, lmax, c, invS, cc);
            run += w;
            if (w > 0.0 && run > rem) { found = x; break; }
            if (w > 0.0) lastpos = x;
          }
          if (found < 0) found = lastpos;
        }
        found = __shfl(found, owner);
      } else {  // rounding: the chunk's last token with mass
        int lp = lastpos;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) lp = max(lp, __shfl_xor(lp, o));
        found = lp;
      }
      y = found;
    }
    if (lane == 0) sh.ybest = y;
  }
  __syncthreads();
  return sh.ybest;
}

// ---------------------------------------------------------------------------
// Pass 2: the walk. One workgroup per request; thread 0 takes the decisions,
// every thread joins the vocabulary passes. All control decisions are read
// back from LDS after a barrier, so the whole workgroup follows one path.
template <bool VEC>
__global__ __launch_bounds__(512) void walk_kernel(SampleParams p) {
  __shared__ WalkShared sh;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int md = p.max_depth;
  int32_t* acc_nodes = p.accepted_nodes + (int64_t)b * md;
  int32_t* toks_out = p.out_tokens + (int64_t)b * (md + 1);
  for (int i = tid; i < md; i += blockDim.x) acc_nodes[i] = -1;
  for (int i = tid; i <= md; i += blockDim.x) toks_out[i] = -1;

  const int n0 = p.cu_nodes[b], n1 = p.cu_nodes[b + 1];
  const int T = n1 - n0;
  const bool pack_ok = n0 >= 0 && T >= 0 && T <= p.max_nodes && n1 <= p.N;
  if (b == 0 && tid == 0 && p.cu_nodes[p.B] != p.N) flag(p.status, kStPacking);
  if (!pack_ok) {
    if (tid == 0) {
      flag(p.status, kStPacking);
      p.accept_len[b] = 0;
      if (p.residual_passes) p.residual_passes[b] = 0;
    }
    return;
  }
  const uint32_t rid = p.request_id ? p.request_id[b] : (uint32_t)b;
  if (tid < T) {
    sh.par[tid] = p.parent[n0 + tid];
    sh.tok[tid] = p.tokens[n0 + tid];
    const double u = uniform01(p.seed, rid, (uint32_t)tid, 0u, p.step);
    sh.u[tid] = u;
    if (p.uniforms_out) p.uniforms_out[n0 + tid] = u;
  }
  if (tid == 0 && p.uniforms_out) p.uniforms_out[p.N + b] = uniform01(p.seed, rid, 0u, 1u, p.step);
  __syncthreads();
  if (wave == 0) {
    bool bad_tree = false, bad_tok = false;
    if (lane < T) {
      bad_tree = sh.par[lane] < -1 || sh.par[lane] >= lane;
      bad_tok = sh.tok[lane] < 0 || sh.tok[lane] >= p.V;
    }
    const bool any_tree = __any(bad_tree), any_tok = __any(bad_tok);
    if (lane == 0) sh.decision = (any_tree ? kStTree : 0) | (any_tok ? kStToken : 0);
  }
  __syncthreads();
  if (sh.decision) {
    if (tid == 0) {
      flag(p.status, sh.decision);
      p.accept_len[b] = 0;
      if (p.residual_passes) p.residual_passes[b] = 0;
    }
    return;
  }

  const int64_t V = p.V;
  const int64_t row0 = (int64_t)n0 + b;
  int pos = -1, depth = 0, passes = 0, bonus = -1;
  for (;;) {
    __syncthreads();  // all reads of the previous position's shared values are done
    const int64_t row = row0 + pos + 1;
    const float* lrow = p.logits + row * V;
    const float* qrow = p.greedy ? nullptr : p.q + row * V;
    if (wave == 0) {
      float lmax, av;
      double S;
      int arg;
      row_norm(p.stats + row * p.nch, p.nch, p.c, lmax, S, arg, av);
      const uint64_t kids = __ballot(lane < T && sh.par[lane] == pos);
      if (lane == 0) {
        sh.lmax = lmax;
        sh.S = S;
        sh.arg = arg;
        sh.kids = kids;
        if (lmax == -INFINITY) flag(p.status, kStNonFinite);
      }
    }
    __syncthreads();
    const float lmax = sh.lmax;
    const double S = sh.S;
    const uint64_t kids = sh.kids;

    if (p.greedy) {
      // accept the first child carrying the argmax token
      const int a = sh.arg;
      int next = -1;
      for (uint64_t k = kids; k; k &= k - 1) {
        const int ch = __ffsll((unsigned long long)k) - 1;
        if (sh.tok[ch] == a) { next = ch; break; }
      }
      if (next < 0) { bonus = a; break; }
      if (tid == 0) { acc_nodes[depth] = next; toks_out[depth] = sh.tok[next]; }
      ++depth;
      pos = next;
      continue;
    }

    const float invS = (float)(1.0 / S);
    double cc = 0.0, M = 1.0;  // current distribution max(0, p - cc q) / M (cc = 0: p itself)
    int level = 0;
    bool csum_ok = false;      // csum holds the chunk masses of the current level
    int accepted = -1;
    for (uint64_t k = kids; k; k &= k - 1) {
      const int ch = __ffsll((unsigned long long)k) - 1;
      if (tid == 0) {
        const int x = sh.tok[ch];
        const float pf = target_prob(lrow[x], lmax, p.c, invS);
        const double qx = (double)qrow[x];
        const double P = level == 0 ? (double)pf : fmax(0.0, (double)pf - cc * qx) / M;
        sh.decision = (P > 0.0 && sh.u[ch] * qx <= P) ? 1 : 0;
      }
      __syncthreads();
      const bool acc = sh.decision != 0;
      __syncthreads();  // every thread has read the decision before it is reused
      if (acc) { accepted = ch; break; }
      // rejected: move to the next residual level
      const double cn = cc + M;
      const double Mn = residual_pass<VEC>(sh, lrow, qrow, p.V, p.nch, lmax, p.c, invS, cn);
      ++passes;
      if (Mn > 0.0) {
        cc = cn;
        M = Mn;
        ++level;
        csum_ok = true;
      } else {
        if (tid == 0) flag(p.status, kStZeroResidual);
        csum_ok = false;
      }
    }
    if (accepted >= 0) {
      if (tid == 0) { acc_nodes[depth] = accepted; toks_out[depth] = sh.tok[accepted]; }
      ++depth;
      pos = accepted;
      continue;
    }
    // final draw at this position from the current distribution
    double total;
    if (level == 0) {
      const ChunkStat* st = p.stats + row * p.nch;
      for (int ch = tid; ch < p.nch; ch += blockDim.x) {
        const ChunkStat s = st[ch];
        sh.csum[ch] = s.lmax == -INFINITY ? 0.0 : s.s * exp2((double)(s.lmax - lmax) * (double)p.c);
      }
      __syncthreads();
      if (wave == 0) {
        double a = 0.0;
        for (int ch = lane; ch < p.nch; ch += 64) a += sh.csum[ch];
        a = wave_sum(a);
        if (lane == 0) sh.total = a;
      }
      __syncthreads();
      total = sh.total;
      __syncthreads();
    } else {
      if (!csum_ok) {
        residual_pass<VEC>(sh, lrow, qrow, p.V, p.nch, lmax, p.c, invS, cc);
        ++passes;
      }
      total = M;
    }
    const double uf = uniform01(p.seed, rid, 0u, 1u, p.step);
    bonus = draw_token(sh, lrow, qrow, p.V, p.nch, level, lmax, p.c, invS, cc, uf, total);
    break;
  }
  if (tid == 0) {
    toks_out[depth] = bonus;
    p.accept_len[b] = depth;
    if (p.residual_passes) p.residual_passes[b] = passes;
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_sampler(const SampleParams& p, bool vec4, int walk_threads, hipStream_t stream,
                          hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (p.B <= 0) return hipSuccess;
  const int64_t rows = (int64_t)p.N + p.B;
  const int64_t items = rows * p.nch;
  const dim3 sgrid((unsigned)((items + 3) / 4));
  if (ev_start) (void)hipEventRecord(ev_start, stream);
  if (p.greedy) {
    if (vec4) row_stats_kernel<true, true><<<sgrid, 256, 0, stream>>>(p.logits, p.V, rows, p.nch, p.c, p.stats, p.status);
    else row_stats_kernel<true, false><<<sgrid, 256, 0, stream>>>(p.logits, p.V, rows, p.nch, p.c, p.stats, p.status);
  } else {
    if (vec4) row_stats_kernel<false, true><<<sgrid, 256, 0, stream>>>(p.logits, p.V, rows, p.nch, p.c, p.stats, p.status);
    else row_stats_kernel<false, false><<<sgrid, 256, 0, stream>>>(p.logits, p.V, rows, p.nch, p.c, p.stats, p.status);
  }
  if (ev_stop) (void)hipEventRecord(ev_stop, stream);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (p.probs_out && !p.greedy) {
    if (vec4) probs_kernel<true><<<sgrid, 256, 0, stream>>>(p.logits, p.V, rows, p.nch, p.c, p.stats, p.probs_out);
    else probs_kernel<false><<<sgrid, 256, 0, stream>>>(p.logits, p.V, rows, p.nch, p.c, p.stats, p.probs_out);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (vec4) walk_kernel<true><<<dim3(p.B), dim3(walk_threads), 0, stream>>>(p);
  else walk_kernel<false><<<dim3(p.B), dim3(walk_threads), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace sv
