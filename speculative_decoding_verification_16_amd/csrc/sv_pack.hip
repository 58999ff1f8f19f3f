// sv_pack.hip -- budgeted super-tree packing, for gfx950.
//
// Method: "ECHO: Elastic Speculative Decoding with Sparse Gating for
// High-Concurrency Scenarios", section 3.1 ("Super-Tree View": the batch's
// candidate trees are verified as one flattened union under the global cap
// sum_i K_i <= K_max) and Figure 3, step 3 (flatten and pack the ragged
// batch into one dense layout). Each candidate's effective score is the
// smallest score on its path; the K_max best candidates by (effective score
// descending, candidate index ascending) are kept -- a set that holds every
// kept node's ancestors -- and packed request by request in their original
// order with renumbered parents.
//
// One workgroup of 1024 threads (the work is B * 64 integers at most):
//  A. per request (one thread each): validate, walk the nodes in order with
//     e(j) = min(score(j), e(parent)), and write the unique 64-bit key
//     (order-preserving bits of e) << 32 | (~index) of every candidate;
//  B. radix select of the K-th largest key over the key array, eight 8-bit
//     digit passes with an LDS histogram;
//  C. per request: the 64-bit mask of kept nodes (key >= threshold), its
//     popcount, and an exclusive scan of the counts into cu_nodes;
//  D. per request: kept node j lands at cu_nodes[b] + popcount(mask below
//     j); its parent p at popcount(mask below p).
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

constexpr int kPackThreads = 1024;

// -0 counts as +0 and NaN as -inf; then an order-preserving map to uint32
__device__ __forceinline__ uint32_t score_key(float s) {
  if (s != s) s = -INFINITY;
  if (s == 0.f) s = 0.f;
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(kPackThreads) void pack_kernel(PackParams p) {
  __shared__ int32_t cnt[kPackMaxB + 1];  // kept per request, then the exclusive scan
  __shared__ uint32_t hist[256];
  __shared__ int32_t s_valid;
  __shared__ uint64_t s_prefix;
  __shared__ int64_t s_rank;
  __shared__ int32_t s_bad;
  const int tid = threadIdx.x;
  const int B = p.B;
  const int64_t M = p.M;
  if (tid == 0) {
    s_valid = 0;
    s_bad = (B > 0 && p.cu_cand[0] != 0) || (B > 0 && p.cu_cand[B] != M);
  }
  __syncthreads();
  for (int b = tid; b < B; b += kPackThreads)
    if (p.cu_cand[b + 1] < p.cu_cand[b]) s_bad = 1;  // benign race: every writer stores 1
  for (int64_t m = tid; m < M; m += kPackThreads) p.keys[m] = 0;
  __syncthreads();
  if (s_bad) {  // offsets not non-decreasing from 0 to M: nothing is kept
    for (int b = tid; b <= B; b += kPackThreads) p.cu_nodes[b] = 0;
    if (tid == 0) {
      *p.total = 0;
      flag(p.status, kStPacking);
    }
    return;
  }

  // A. effective scores and keys
  for (int b = tid; b < B; b += kPackThreads) {
    const int c0 = p.cu_cand[b], c1 = p.cu_cand[b + 1];
    const int T = c1 - c0;
    if (T > kMaxNodes) {
      flag(p.status, kStPacking);
      continue;
    }
    bool ok = true;
    for (int j = 0; j < T && ok; ++j) {
      const int pj = p.par[c0 + j];
      if (pj < -1 || pj >= j) {
        ok = false;
        break;
      }
      uint32_t e = score_key(p.score[c0 + j]);
      if (pj >= 0) e = min(e, (uint32_t)(p.keys[c0 + pj] >> 32));  // the parent's effective score
      p.keys[c0 + j] = ((uint64_t)e << 32) | (uint32_t)(0xffffffffu - (uint32_t)(c0 + j));
    }
    if (!ok) {
      for (int j = 0; j < T; ++j) p.keys[c0 + j] = 0;
      flag(p.status, kStTree);
      continue;
    }
    atomicAdd(&s_valid, T);
  }
  __syncthreads();

  // B. the K-th largest key (keys are unique; 0 marks a dropped candidate)
  const int64_t K = min((int64_t)p.budget, (int64_t)s_valid);
  uint64_t thr = ~0ull;
  if (K > 0) {
    if (tid == 0) {
      s_prefix = 0;
      s_rank = K;
    }
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int d = tid; d < 256; d += kPackThreads) hist[d] = 0;
      __syncthreads();
      const uint64_t pre = s_prefix;
      const uint64_t hi_mask = shift == 56 ? 0ull : (~0ull << (shift + 8));
      for (int64_t m = tid; m < M; m += kPackThreads) {
        const uint64_t k = p.keys[m];
        if (k != 0 && (k & hi_mask) == pre) atomicAdd(&hist[(k >> shift) & 255], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        int64_t r = s_rank, cum = 0;
        int d = 255;
        for (; d > 0; --d) {
          if (cum + hist[d] >= r) break;
          cum += hist[d];
        }
        s_rank = r - cum;
        s_prefix = pre | ((uint64_t)d << shift);
      }
      __syncthreads();
    }
    thr = s_prefix;
  }

  // C. kept counts per request and their exclusive scan
  for (int b = tid; b < B; b += kPackThreads) {
    const int c0 = p.cu_cand[b], c1 = p.cu_cand[b + 1];
    int c = 0;
    for (int m = c0; m < c1; ++m) {
      const uint64_t k = p.keys[m];
      c += (k != 0 && k >= thr);
    }
    cnt[b] = c;
  }
  __syncthreads();
  if (tid == 0) {  // B <= kPackMaxB: one sequential pass is a few microseconds at most
    int32_t run = 0;
    for (int b = 0; b < B; ++b) {
      const int32_t c = cnt[b];
      cnt[b] = run;
      run += c;
    }
    cnt[B] = run;
    *p.total = run;
  }
  __syncthreads();
  for (int b = tid; b <= B; b += kPackThreads) p.cu_nodes[b] = cnt[b];

  // D. the packed nodes
  for (int b = tid; b < B; b += kPackThreads) {
    const int c0 = p.cu_cand[b], c1 = p.cu_cand[b + 1];
    uint64_t mask = 0;
    for (int m = c0; m < c1; ++m) {
      const uint64_t k = p.keys[m];
      if (k != 0 && k >= thr) mask |= 1ull << (m - c0);
    }
    const int base = cnt[b];
    for (uint64_t r = mask; r; r &= r - 1) {
      const int j = __ffsll((unsigned long long)r) - 1;
      const int nj = base + __popcll(mask & ((1ull << j) - 1ull));
      const int pj = p.par[c0 + j];
      p.parent[nj] = pj < 0 ? -1 : __popcll(mask & ((1ull << pj) - 1ull));
      p.tokens[nj] = p.tok[c0 + j];
      p.src[nj] = c0 + j;
    }
  }
}

hipError_t launch_pack(const PackParams& p, hipStream_t stream) {
  pack_kernel<<<dim3(1), dim3(kPackThreads), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace sv
