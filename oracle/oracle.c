/*
 * oracle.c -- plain fp64 CPU oracle of the speculative-decoding verification
 * step. TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's
 * CPU-baseline leg call it to check and time the GPU library; the library
 * never calls it and shares no code with it.
 *
 * Every function follows the definition on the source pages step by step, in
 * fp64, with plain loops and no blocking, fusion or reordering:
 *   [SD]    "Speculative Decoding: Accelerating Inference Speeds in
 *           Distributed LLMs" (shyankdev.com blog)
 *   [LOSSY] "Revisiting Lossy Verification in Speculative Decoding:
 *           Mechanisms, Trade-offs, and Failure Modes"
 *   [ECHO]  "ECHO: Elastic Speculative Decoding with Sparse Gating for
 *           High-Concurrency Scenarios"
 * plus Philox4x32-10 from Salmon, Moraes, Dror, Shaw, "Parallel Random
 * Numbers: As Easy as 1, 2, 3" (SC'11).
 *
 * Readings of points the pages leave open are stated where they are used.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon et al., SC'11, section on the Philox family):
 * ten rounds of the 4x32 Philox S-box; each round multiplies words 0 and 2
 * by the two Philox multipliers, and the key is bumped by the two Weyl
 * constants between rounds.                                                */
#define ORC_PHILOX_M0 0xD2511F53u
#define ORC_PHILOX_M1 0xCD9E8D57u
#define ORC_PHILOX_W0 0x9E3779B9u
#define ORC_PHILOX_W1 0xBB67AE85u

void orc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += ORC_PHILOX_W0;
      k1 += ORC_PHILOX_W1;
    }
    uint64_t prod0 = (uint64_t)ORC_PHILOX_M0 * (uint64_t)c0;
    uint64_t prod1 = (uint64_t)ORC_PHILOX_M1 * (uint64_t)c2;
    uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
    uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The uniform variate r_i of [SD] "Mathematical Rejection Sampling
 * Algorithm": word 0 of Philox at counter (request id, node, purpose, step)
 * mapped into the open interval (0, 1) as (w0 + 1/2) / 2^32 (exact in fp64). */
double orc_uniform(uint64_t seed, uint32_t request_id, uint32_t j, uint32_t purpose, uint32_t step) {
  uint32_t ctr[4] = {request_id, j, purpose, step};
  uint32_t key[2] = {(uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32)};
  uint32_t w[4];
  orc_philox4x32_10(ctr, key, w);
  return ((double)w[0] + 0.5) * (1.0 / 4294967296.0);
}

/* ------------------------------------------------------------------------ */
/* Tree ([SD] "Tree Attention Mask Mechanics"): node j sees itself and every
 * ancestor, never a node of another branch. Ancestors are found by walking
 * parent pointers. Returns 0, or 1 + the first node whose parent is not in
 * [-1, j-1] (then anc/depth of later nodes are left unset).               */
int orc_ancestors(int T, const int32_t* parent, uint64_t* anc, int32_t* depth) {
  if (T < 0 || T > 64) return -1;
  for (int j = 0; j < T; ++j) {
    if (parent[j] < -1 || parent[j] >= j) return j + 1;
    uint64_t mask = 0;
    int d = 0;
    for (int x = j; x >= 0; x = parent[x]) {
      mask |= (uint64_t)1 << x;
      ++d;
    }
    anc[j] = mask;
    depth[j] = d; /* a child of the root has depth 1 */
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Work splitting for the slow loops: a plain parallel-for over an index
 * range with one contiguous slice per thread.                              */
typedef struct {
  void (*fn)(void* ctx, int64_t i);
  void* ctx;
  int64_t begin, end;
} orc_slice;

static void* orc_slice_run(void* arg) {
  orc_slice* s = (orc_slice*)arg;
  for (int64_t i = s->begin; i < s->end; ++i) s->fn(s->ctx, i);
  return NULL;
}

static void orc_parallel_for(int64_t n, int nthreads, void (*fn)(void*, int64_t), void* ctx) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > n) nthreads = (int)(n > 0 ? n : 1);
  if (nthreads == 1) {
    for (int64_t i = 0; i < n; ++i) fn(ctx, i);
    return;
  }
  pthread_t tids[256];
  orc_slice slices[256];
  int started[256];
  for (int t = 0; t < nthreads; ++t) {
    slices[t].fn = fn;
    slices[t].ctx = ctx;
    slices[t].begin = n * t / nthreads;
    slices[t].end = n * (t + 1) / nthreads;
    started[t] = pthread_create(&tids[t], NULL, orc_slice_run, &slices[t]) == 0;
    if (!started[t]) orc_slice_run(&slices[t]);
  }
  for (int t = 0; t < nthreads; ++t)
    if (started[t]) pthread_join(tids[t], NULL);
}

/* ------------------------------------------------------------------------ */
/* FP8 E4M3 in the OCP 8-bit floating point format (finite form, "E4M3FN"):
 * sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 holds the
 * subnormals m/8 * 2^-6; S.1111.111 is NaN and there is no infinity.      */
double orc_fp8_e4m3(uint8_t x) {
  int s = x >> 7, e = (x >> 3) & 15, m = x & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m / 8.0, -6);
  else v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* Element access: fp32 as is, bf16 by placing its 16 bits on top of an fp32
 * (exact), fp8 E4M3 decoded as above; all widened exactly to fp64.        */
static double orc_load(const void* base, int dtype, int64_t idx) {
  if (dtype == 0) return (double)((const float*)base)[idx];
  if (dtype == 2) return orc_fp8_e4m3(((const uint8_t*)base)[idx]);
  uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

typedef struct {
  int B, Hq, Hkv, D, dtype;
  int kv_dtype;            /* element type of the caches (2: fp8 E4M3)  */
  double k_scale, v_scale; /* cache element value = stored value * scale */
  const void *q, *k, *v;
  int64_t Lcap;
  const int32_t *ctx_len, *cu_nodes, *parent;
  double scale;
  const int64_t* items; /* pairs (packed node, q head) */
  double* out;
  int* err;
  /* paged caches (block_table != NULL): pools [num_blocks, Hkv, block_size, D] */
  const int32_t* block_table; /* [B, max_blocks] */
  int block_size, max_blocks;
  int64_t num_blocks;
} orc_attn_ctx;

/* Element index of dim 0 of cache slot t of request b, KV head g: the
 * contiguous layout [B, Hkv, Lcap, D], or through the block table, where slot
 * t of request b sits in block block_table[b, t / block_size] at row
 * t % block_size. -1 if the block id is out of range.                      */
static int64_t orc_slot_index(const orc_attn_ctx* c, int b, int64_t g, int64_t t) {
  if (!c->block_table) return (((int64_t)b * c->Hkv + g) * c->Lcap + t) * c->D;
  int64_t blk = c->block_table[(int64_t)b * c->max_blocks + t / c->block_size];
  if (blk < 0 || blk >= c->num_blocks) return -1;
  return ((blk * c->Hkv + g) * c->block_size + t % c->block_size) * c->D;
}

/* [SD] "Tree Attention Mask Mechanics" + "Interaction with Advanced
 * Attention Architectures (GQA & MLA)": one output vector of one query head
 * of one draft node. The query head h reads KV head h / (Hq / Hkv). Keys:
 * every committed context slot, then the draft slots of the node's own
 * ancestors and of itself. Softmax in fp64 with the maximum subtracted.    */
static void orc_attn_item(void* vctx, int64_t it) {
  orc_attn_ctx* c = (orc_attn_ctx*)vctx;
  int64_t n = c->items[2 * it], h = c->items[2 * it + 1];
  double* o = c->out + it * c->D;
  /* request owning packed node n: cu_nodes[b] <= n < cu_nodes[b+1] */
  int b = -1;
  for (int r = 0; r < c->B; ++r)
    if (c->cu_nodes[r] <= n && n < c->cu_nodes[r + 1]) { b = r; break; }
  if (b < 0) { *c->err = 1; return; }
  int j = (int)(n - c->cu_nodes[b]);
  int T = c->cu_nodes[b + 1] - c->cu_nodes[b];
  const int32_t* par = c->parent + c->cu_nodes[b];
  int64_t L = c->ctx_len[b];
  if (T > 64 || L < 0 || L + T > c->Lcap) { *c->err = 1; return; }
  /* visible draft nodes: j and its ancestors */
  int visible[64];
  int nvis = 0;
  for (int x = j; x >= 0; x = par[x]) {
    if (par[x] < -1 || par[x] >= x) { *c->err = 1; return; }
    visible[nvis++] = x;
  }
  int G = c->Hq / c->Hkv;
  int64_t g = h / G;
  int64_t nkeys = L + nvis;
  double* s = (double*)malloc(sizeof(double) * (size_t)nkeys);
  int64_t* slot = (int64_t*)malloc(sizeof(int64_t) * (size_t)nkeys);
  if (!s || !slot) { free(s); free(slot); *c->err = 1; return; }
  for (int64_t t = 0; t < L; ++t) slot[t] = t;
  for (int i = 0; i < nvis; ++i) slot[L + i] = L + visible[i];
  int64_t qbase = (n * c->Hq + h) * c->D;
  for (int64_t t = 0; t < nkeys; ++t) {
    slot[t] = orc_slot_index(c, b, g, slot[t]); /* slot -> element index */
    if (slot[t] < 0) { free(s); free(slot); *c->err = 1; return; }
  }
  double m = -INFINITY;
  for (int64_t t = 0; t < nkeys; ++t) {
    double acc = 0.0;
    for (int d = 0; d < c->D; ++d)
      acc += orc_load(c->q, c->dtype, qbase + d) * (c->k_scale * orc_load(c->k, c->kv_dtype, slot[t] + d));
    s[t] = c->scale * acc;
    if (s[t] > m) m = s[t];
  }
  double denom = 0.0;
  for (int64_t t = 0; t < nkeys; ++t) {
    s[t] = exp(s[t] - m);
    denom += s[t];
  }
  for (int d = 0; d < c->D; ++d) o[d] = 0.0;
  for (int64_t t = 0; t < nkeys; ++t) {
    double w = s[t] / denom;
    for (int d = 0; d < c->D; ++d) o[d] += w * (c->v_scale * orc_load(c->v, c->kv_dtype, slot[t] + d));
  }
  free(s);
  free(slot);
}

/* Attention for a list of (packed node, query head) pairs `items` [n_items,2]
 * (or, if items is NULL, for every node and head in order); out [n_items, D].
 * dtype 0 = fp32 inputs, 1 = bf16 inputs; kv_dtype the caches' type (the
 * same, or 2 = fp8 E4M3 whose elements are scaled by k_scale / v_scale).
 * block_table != NULL reads paged caches (see orc_slot_index; Lcap =
 * max_blocks * block_size). Returns 0, or 1 on bad packing or a block id
 * out of range.                                                           */
int orc_attention_ex(int B, int Hq, int Hkv, int D, int dtype, const void* q, const void* k, const void* v,
                     int64_t Lcap, const int32_t* ctx_len, const int32_t* cu_nodes, const int32_t* parent,
                     double scale, int64_t n_items, const int64_t* items, double* out, int nthreads,
                     const int32_t* block_table, int block_size, int max_blocks, int64_t num_blocks, int kv_dtype,
                     double k_scale, double v_scale) {
  if (Hkv <= 0 || Hq % Hkv != 0 || D <= 0) return 1;
  if (block_table && (block_size <= 0 || max_blocks <= 0 || Lcap != (int64_t)block_size * max_blocks)) return 1;
  int64_t* all = NULL;
  if (!items) {
    int64_t N = cu_nodes[B];
    n_items = N * Hq;
    all = (int64_t*)malloc(sizeof(int64_t) * 2 * (size_t)(n_items > 0 ? n_items : 1));
    if (!all) return 1;
    for (int64_t n = 0; n < N; ++n)
      for (int h = 0; h < Hq; ++h) {
        all[2 * (n * Hq + h)] = n;
        all[2 * (n * Hq + h) + 1] = h;
      }
    items = all;
  }
  int err = 0;
  orc_attn_ctx c = {B, Hq, Hkv, D, dtype, kv_dtype, k_scale, v_scale, q, k, v, Lcap, ctx_len, cu_nodes,
                    parent, scale, items, out, &err, block_table, block_size, max_blocks, num_blocks};
  orc_parallel_for(n_items, nthreads, orc_attn_item, &c);
  free(all);
  return err;
}

int orc_attention(int B, int Hq, int Hkv, int D, int dtype, const void* q, const void* k, const void* v,
                  int64_t Lcap, const int32_t* ctx_len, const int32_t* cu_nodes, const int32_t* parent,
                  double scale, int64_t n_items, const int64_t* items, double* out, int nthreads) {
  return orc_attention_ex(B, Hq, Hkv, D, dtype, q, k, v, Lcap, ctx_len, cu_nodes, parent, scale, n_items, items,
                          out, nthreads, NULL, 0, 0, 0, dtype, 1.0, 1.0);
}

/* ------------------------------------------------------------------------ */
/* Target distribution with temperature T > 0: p = softmax(logits / T), in
 * fp64 with the maximum subtracted. Returns 0, or 1 if a logit is NaN/+inf or
 * every logit is -inf.                                                     */
int orc_target_probs(int V, const float* logits, double T, double* p) {
  double m = -INFINITY;
  for (int x = 0; x < V; ++x) {
    double l = (double)logits[x];
    if (isnan(l) || l == INFINITY) return 1;
    double z = l / T;
    if (z > m) m = z;
  }
  if (m == -INFINITY) return 1;
  double S = 0.0;
  for (int x = 0; x < V; ++x) {
    p[x] = exp((double)logits[x] / T - m);
    S += p[x];
  }
  for (int x = 0; x < V; ++x) p[x] /= S;
  return 0;
}

/* Allowed sets of truncation sampling ([LOSSY] section 2.3). Both are
 * thresholds on the target probability relative to its maximum: with
 * z_x = (l_x - l_max) / T, p(x) / max p = exp(z_x), so p(x) >= tau is
 * l_x - l_max >= T (ln S + ln tau) (S = sum exp(z)) and p(x) >= p_base max p
 * is l_x - l_max >= T ln p_base. Membership is decided from that definition in
 * fp64: the difference of the two fp32 logits is formed in fp64 (exact for
 * any two logits within a factor 2^29 of each other) and compared with the
 * fp64 threshold.                                                          */
int orc_allowed(float lx, float lmax, double th) { return (double)lx - (double)lmax >= th; }

/* Largest logit of a row (fp32; -inf if none is above -inf; NaN ignored). */
static float orc_row_max(int V, const float* logits) {
  float m = -INFINITY;
  for (int x = 0; x < V; ++x)
    if (logits[x] > m) m = logits[x];
  return m;
}

/* Masks the normalised row p to {x : l_x - l_max >= th} and renormalises in
 * place; returns the mass kept.                                            */
double orc_truncate(int V, const float* logits, double th, double* p) {
  const float lmax = orc_row_max(V, logits);
  double Z = 0.0;
  for (int x = 0; x < V; ++x) {
    if (!orc_allowed(logits[x], lmax, th)) p[x] = 0.0;
    Z += p[x];
  }
  for (int x = 0; x < V; ++x) p[x] /= Z;
  return Z;
}

/* Min-p ([LOSSY] section 2.3: A = {x : p(x) >= p_base * max_v p(v)}, and the
 * truncated target p_Theta(x) = p(x) / Z on A, 0 elsewhere, which "truncation
 * sampling + SD" verifies against, appendix G.2/G.3): the threshold
 * T ln p_base on l_x - l_max. p (a normalised row) is masked and
 * renormalised in place.                                                    */
double orc_min_p_threshold(double T, double p_base) { return T * log(p_base); }

void orc_truncate_min_p(int V, const float* logits, double theta, double* p) { orc_truncate(V, logits, theta, p); }

/* eta-sampling ([LOSSY] section 2.3: A = {x : p(x) >= min(eps, delta exp(-H(p)))},
 * H the Shannon entropy of the target row in nats). With S = sum exp(z),
 * G = E_p[-z] (>= 0) and H = ln S + G, the threshold on l_x - l_max is
 * T (ln S + min(ln eps, ln delta - H)). Also returns G and the variance of z
 * under p (both in nats), from which a caller bounds how far a threshold
 * computed with fp32 weights can sit from this one.                       */
double orc_eta_threshold(int V, const float* logits, double T, double eps, double delta, double* gap, double* var) {
  const float lmax = orc_row_max(V, logits);
  double S = 0.0, E1 = 0.0, E2 = 0.0;
  for (int x = 0; x < V; ++x) {
    double z = ((double)logits[x] - (double)lmax) / T;
    double e = exp(z);
    S += e;
    if (e > 0.0) {
      E1 += e * z;
      E2 += e * z * z;
    }
  }
  double G = -E1 / S;
  double H = log(S) + G;
  if (gap) *gap = G;
  if (var) *var = fmax(0.0, E2 / S - G * G);
  return T * (log(S) + fmin(log(eps), log(delta) - H));
}

/* The eta truncation of a normalised row p in place; returns the threshold.
 * *margin (optional): the smallest distance of a token to it, in
 * log-probability units (|l_x - l_max - th| / T).                         */
double orc_truncate_eta(int V, const float* logits, double T, double eps, double delta, double* p, double* margin) {
  double th = orc_eta_threshold(V, logits, T, eps, delta, NULL, NULL);
  const float lmax = orc_row_max(V, logits);
  double mg = INFINITY;
  for (int x = 0; x < V; ++x) {
    double dist = fabs(((double)logits[x] - (double)lmax) - th) / T;
    if (dist < mg) mg = dist;
  }
  orc_truncate(V, logits, th, p);
  if (margin) *margin = mg;
  return th;
}

/* Entropy of the target row at temperature T, in nats (the H of the eta
 * allowed set above): H = -sum p ln p = ln S - sum p z.                    */
double orc_row_entropy(int V, const float* logits, double T) {
  const float lmax = orc_row_max(V, logits);
  double S = 0.0, E = 0.0;
  for (int x = 0; x < V; ++x) {
    double z = ((double)logits[x] - (double)lmax) / T;
    double e = exp(z);
    S += e;
    if (e > 0.0) E += e * z;
  }
  return log(S) - E / S;
}

/* Does the row define a target distribution? Not if a logit is NaN or +inf,
 * or if every logit is -inf (then softmax has no value).                   */
int orc_row_finite(int V, const float* logits) {
  int any = 0;
  for (int x = 0; x < V; ++x) {
    if (isnan(logits[x]) || logits[x] == INFINITY) return 0;
    if (logits[x] > -INFINITY) any = 1;
  }
  return any;
}

/* Greedy target token: argmax of the raw logits, lowest index on ties; NaN
 * entries are passed over (-1 if the row has no non-NaN entry).           */
int orc_argmax(int V, const float* logits) {
  int best = -1;
  for (int x = 0; x < V; ++x) {
    if (isnan(logits[x])) continue;
    if (best < 0 || logits[x] > logits[best]) best = x;
  }
  return best;
}

/* Residual after a rejection ([SD] R_i(x); [LOSSY] F.1 r(x)):
 * out = max(0, P - Q) / sum max(0, P - Q). Returns the mass sum; if it is 0
 * the distribution cannot be renormalised and out = P (kept unchanged).   */
double orc_residual(int V, const double* P, const double* Q, double* out) {
  double R = 0.0;
  for (int x = 0; x < V; ++x) {
    double d = P[x] - Q[x];
    if (d > 0.0) R += d;
  }
  for (int x = 0; x < V; ++x) {
    if (R > 0.0) {
      double d = P[x] - Q[x];
      out[x] = d > 0.0 ? d / R : 0.0;
    } else {
      out[x] = P[x];
    }
  }
  return R;
}

/* Removal of a tried deterministic candidate ([LOSSY] G.3: the target the
 * i-th candidate is tested against is p_Theta with the candidates tried
 * before it taken out and renormalised): out = P with P[x] set to 0, divided
 * by the mass left. Returns that mass; if it is 0 nothing is left to
 * renormalise and out = P (kept unchanged), as in orc_residual.           */
double orc_remove_candidate(int V, const double* P, int x, double* out) {
  double R = 0.0;
  for (int t = 0; t < V; ++t)
    if (t != x) R += P[t];
  for (int t = 0; t < V; ++t) out[t] = R > 0.0 ? (t == x ? 0.0 : P[t] / R) : P[t];
  return R;
}

/* Inverse-CDF draw from an (unnormalised) non-negative vector P:
 * y = min{ x : sum_{t<=x} P(t) > u * sum_t P(t) } in vocabulary order; the
 * strict '>' means a zero-mass token is never drawn. *margin (optional) is
 * the distance from u to the normalised CDF values on both sides of y.
 * Returns -1 if P has no mass.                                            */
int orc_inverse_cdf(int V, const double* P, double u, double* margin) {
  double total = 0.0;
  for (int x = 0; x < V; ++x) total += P[x];
  if (!(total > 0.0)) {
    if (margin) *margin = 0.0;
    return -1;
  }
  double target = u * total;
  double run = 0.0;
  for (int x = 0; x < V; ++x) {
    double before = run;
    run += P[x];
    if (run > target) {
      if (margin) {
        double lo = u - before / total, hi = run / total - u;
        *margin = lo < hi ? lo : hi;
      }
      return x;
    }
  }
  /* only reachable through rounding when u*total lands on the last step */
  for (int x = V - 1; x >= 0; --x)
    if (P[x] > 0.0) {
      if (margin) *margin = 0.0;
      return x;
    }
  return -1;
}

/* ------------------------------------------------------------------------ */
/* The verification walk of one request. */
typedef struct {
  int B, V;
  const int32_t *cu_nodes, *parent, *tokens;
  const float *logits, *q;
  double T;
  int trunc;     /* truncation of every target row: 0 none, 1 min-p, 2 eta */
  double p_base; /* min-p: its p_base                                        */
  double eta_eps, eta_delta; /* eta: its eps and delta                      */
  double set_tol; /* > 0: half-width of the allowed-set band in log-probability
                     units; 0: the band each set's own error bound gives   */
  int det;       /* siblings are deterministic candidates (q unused) */
  int rule;      /* accept rule: 0 lossless, 1 lenience, 2 interpolation,
                    3 truncation-based (accept iff the token is allowed)   */
  double rule_param; /* lenience l or interpolation lambda, in (0, 1]    */
  uint64_t seed;
  uint32_t step;
  const uint32_t* request_id;
  int max_depth;
  int32_t *accept_len, *accepted_nodes, *out_tokens;
  double* uniforms_out;
  int32_t *flag_depth, *flag_kind, *n_rejections, *status;
  double *min_accept_margin, *cdf_margin, *draw_mass;
  double accept_tol, cdf_tol;
} orc_walk_ctx;

/* What the decisions at one position observed. */
typedef struct {
  double min_accept_margin; /* smallest |u - h| over its accept tests      */
  double cdf_margin;        /* margin of its draw (INFINITY: no draw)      */
  double draw_mass;         /* probability of the drawn token (0: no draw) */
  int near_kind;            /* first near tie: 0 accept test, 1 draw,
                               3 deterministic remainder near 0; -1 none  */
  int rejections;
  int status;
} orc_rec;

/* A deterministic candidate's remainder at or below this fraction of the
 * row's mass is a near tie: a computation that subtracts fp32 weights from
 * their sum cannot tell it from zero.                                      */
#define ORC_REMAINDER_TOL 1e-11

/* The decisions at one position of request b: the children of pos (local
 * index, -1 = root) are tried in increasing index against the row's target
 * -- p, or with truncation p_Theta over {x : l_x - l_max >= th} -- and when
 * none is accepted one token is drawn from the current distribution.
 * Returns the accepted child, or -1 with *bonus = the drawn token (-1 when
 * the row defines no distribution). Scratch: P, Q, tmp of V doubles.      */
static int orc_position(const orc_walk_ctx* c, int b, int pos, double th, orc_rec* rec, int* bonus, double* P,
                        double* Q, double* tmp) {
  const int V = c->V;
  const int64_t n0 = c->cu_nodes[b];
  const int T = c->cu_nodes[b + 1] - c->cu_nodes[b];
  const int32_t* par = c->parent + n0;
  const int32_t* tok = c->tokens + n0;
  const uint32_t rid = c->request_id ? c->request_id[b] : (uint32_t)b;
  const int64_t row = n0 + b + pos + 1; /* root row n0 + b, node j's row n0 + b + 1 + j */
  const float* lrow = c->logits + row * (int64_t)V;
  rec->min_accept_margin = INFINITY;
  rec->cdf_margin = INFINITY;
  rec->draw_mass = 0.0;
  rec->near_kind = -1;
  rec->rejections = 0;
  rec->status = 0;
  *bonus = -1;
  /* target distribution at this position, and the draft distribution it is
   * checked against ([SD]: node j is checked against p_i and q_i of the
   * position it was drafted at, i.e. its parent's row)                     */
  if (orc_target_probs(V, lrow, c->T, P)) {
    rec->status |= 0x08;
    return -1;
  }
  const float lmax = orc_row_max(V, lrow);
  if (c->trunc) orc_truncate(V, lrow, th, P);
  if (!c->det)
    for (int x = 0; x < V; ++x) Q[x] = (double)c->q[row * (int64_t)V + x];
  int n_kids = 0;
  double remain = 1.0; /* deterministic candidates: fraction of the row's mass left */
  for (int ch = pos + 1; ch < T; ++ch) {
    if (par[ch] != pos) continue; /* children in increasing node index */
    ++n_kids;
    double u = orc_uniform(c->seed, rid, (uint32_t)ch, 0, c->step);
    int x = tok[ch];
    if (c->det) {
      /* [LOSSY] G.3, deterministic candidates: x^(i) is accepted with
       * probability p~_i(x^(i)), i.e. iff u <= P(x) with P the target after
       * the earlier candidates were taken out (a token tried before has
       * P = 0 and is rejected).                                             */
      double margin = fabs(u - P[x]);
      if (margin < rec->min_accept_margin) rec->min_accept_margin = margin;
      if (margin < c->accept_tol && rec->near_kind < 0) rec->near_kind = 0;
      if (P[x] > 0.0 && u <= P[x]) return ch;
      rec->rejections += 1;
      double R = orc_remove_candidate(V, P, x, tmp);
      if (!(R > 0.0)) rec->status |= 0x10;
      else remain *= R;
      if (remain <= ORC_REMAINDER_TOL && rec->near_kind < 0) rec->near_kind = 3;
      memcpy(P, tmp, sizeof(double) * (size_t)V);
      continue;
    }
    if (c->rule == 3) {
      /* [LOSSY] 3.2, truncation-based verification (SpecCascade with the
       * min-p set, typical acceptance with the eta set): h(x) = 1 if x is in
       * the allowed set, else 0. No uniform is involved.                    */
      if (orc_allowed(lrow[x], lmax, th)) return ch;
      rec->rejections += 1;
      continue;
    }
    /* [SD] acceptance rule r <= min(1, p/q), written as u*q <= p with p > 0
     * so that q(x) = 0 follows the formula (ratio +inf, accepted). The lossy
     * rules of [LOSSY] 3.1 change only this test: lenience h = min(1, p/(l q))
     * compares u*(l q) with p; interpolation (CoS) h = min(1, nu/q) with
     * nu = lambda p + (1 - lambda) q compares u*q with nu. Both keep the
     * residual max(0, P - q) of a rejection (A.3; A.1's r(x) is the same
     * distribution).                                                        */
    double num = P[x], den = Q[x];
    if (c->rule == 1) den = c->rule_param * Q[x];
    if (c->rule == 2) num = c->rule_param * P[x] + (1.0 - c->rule_param) * Q[x];
    double ratio = den > 0.0 ? num / den : (num > 0.0 ? INFINITY : 0.0);
    double margin = fabs(u - ratio);
    if (margin < rec->min_accept_margin) rec->min_accept_margin = margin;
    if (margin < c->accept_tol && rec->near_kind < 0) rec->near_kind = 0;
    if (num > 0.0 && u * den <= num) return ch;
    /* rejected: the next sibling (a fresh draw from the same q) is tested
     * against the renormalised residual of the current distribution       */
    rec->rejections += 1;
    double R = orc_residual(V, P, Q, tmp);
    if (!(R > 0.0)) rec->status |= 0x10;
    memcpy(P, tmp, sizeof(double) * (size_t)V);
  }
  if (c->rule == 3 && n_kids > 0) {
    /* every child rejected under truncation-based verification: the token
     * comes from the draft restricted to the allowed set,
     * r(x) = q(x) 1{x in A} / Z_A(q). Reading: [LOSSY] 3.2 gives the law the
     * rule generates, q(x) / Z_A(q) on A and 0 elsewhere, but no residual;
     * with P(generate x) = q(x) h(x) + (1 - Z_A(q)) r(x) this r is the only
     * one that yields it, at any number of i.i.d. siblings. A zero Z_A(q)
     * keeps the truncated target (flagged).                                 */
    double Z = 0.0;
    for (int x = 0; x < V; ++x) {
      tmp[x] = orc_allowed(lrow[x], lmax, th) ? Q[x] : 0.0;
      Z += tmp[x];
    }
    if (Z > 0.0) {
      for (int x = 0; x < V; ++x) P[x] = tmp[x] / Z;
    } else {
      rec->status |= 0x10;
    }
  }
  /* no child accepted (or none to try): one token from the current
   * distribution -- the residual after rejections (with deterministic
   * candidates: the target without the tried ones), p at a leaf          */
  double u = orc_uniform(c->seed, rid, 0, 1, c->step);
  double margin = 0.0;
  *bonus = orc_inverse_cdf(V, P, u, &margin);
  rec->cdf_margin = margin;
  if (*bonus >= 0) {
    double total = 0.0;
    for (int x = 0; x < V; ++x) total += P[x];
    rec->draw_mass = P[*bonus] / total;
  }
  if (margin < c->cdf_tol && rec->near_kind < 0) rec->near_kind = 1;
  return -1;
}

static int orc_cmp_desc(const void* a, const void* b) {
  double x = *(const double*)a, y = *(const double*)b;
  return x > y ? -1 : (x < y ? 1 : 0);
}

/* Does a threshold inside the band change the decisions at this position?
 * The sets {x : l_x - l_max >= t} for t in [th - band, th + band] differ
 * only in the tokens whose l_x - l_max lies in that interval; ordered by
 * that difference they enter one at a time, so the distinct sets are the
 * set without any of them and the sets with the top k of them. Each is
 * evaluated; 1 if one gives another outcome (accepted child, or bonus
 * token) than (acc, bonus).                                                */
static int orc_band_changes(const orc_walk_ctx* c, int b, int pos, double th, double band, int acc, int bonus,
                            double* P, double* Q, double* tmp) {
  const int V = c->V;
  const int64_t row = c->cu_nodes[b] + b + pos + 1;
  const float* lrow = c->logits + row * (int64_t)V;
  const float lmax = orc_row_max(V, lrow);
  int m = 0;
  for (int x = 0; x < V; ++x)
    if (fabs(((double)lrow[x] - (double)lmax) - th) <= band) ++m;
  if (m == 0) return 0;
  double* dv = (double*)malloc(sizeof(double) * (size_t)m);
  if (!dv) return 1;
  m = 0;
  for (int x = 0; x < V; ++x) {
    double d = (double)lrow[x] - (double)lmax;
    if (fabs(d - th) <= band) dv[m++] = d;
  }
  qsort(dv, (size_t)m, sizeof(double), orc_cmp_desc);
  int changed = 0;
  for (int k = -1; k < m && !changed; ++k) {
    if (k >= 1 && dv[k] == dv[k - 1]) continue; /* the same set as before */
    double t = k < 0 ? nextafter(dv[0], INFINITY) : dv[k];
    orc_rec r;
    int y = -1;
    int a = orc_position(c, b, pos, t, &r, &y, P, Q, tmp);
    changed = a != acc || (a < 0 && y != bonus);
  }
  free(dv);
  return changed;
}

static void orc_walk_one(void* vctx, int64_t bi) {
  orc_walk_ctx* c = (orc_walk_ctx*)vctx;
  int b = (int)bi, V = c->V;
  int64_t N = c->cu_nodes[c->B];
  int32_t* acc_nodes = c->accepted_nodes + (int64_t)b * c->max_depth;
  int32_t* toks_out = c->out_tokens + (int64_t)b * (c->max_depth + 1);
  for (int i = 0; i < c->max_depth; ++i) acc_nodes[i] = -1;
  for (int i = 0; i <= c->max_depth; ++i) toks_out[i] = -1;
  c->accept_len[b] = 0;
  c->flag_depth[b] = -1;
  c->flag_kind[b] = -1;
  c->n_rejections[b] = 0;
  c->status[b] = 0;
  c->min_accept_margin[b] = INFINITY;
  c->cdf_margin[b] = INFINITY;
  c->draw_mass[b] = 0.0;

  int64_t n0 = c->cu_nodes[b];
  int T = c->cu_nodes[b + 1] - c->cu_nodes[b];
  uint32_t rid = c->request_id ? c->request_id[b] : (uint32_t)b;
  if (c->uniforms_out) {
    for (int j = 0; j < T && j < 64; ++j) c->uniforms_out[n0 + j] = orc_uniform(c->seed, rid, (uint32_t)j, 0, c->step);
    c->uniforms_out[N + b] = orc_uniform(c->seed, rid, 0, 1, c->step);
  }
  /* validate packing, tree and tokens */
  if (T < 0 || T > 64 || T > c->max_depth) { c->status[b] |= 0x02; return; }
  const int32_t* par = c->parent + n0;
  const int32_t* tok = c->tokens + n0;
  for (int j = 0; j < T; ++j) {
    if (par[j] < -1 || par[j] >= j) { c->status[b] |= 0x01; return; }
    if (tok[j] < 0 || tok[j] >= V) { c->status[b] |= 0x04; return; }
  }
  int64_t row0 = n0 + b; /* row of the root position; node j's row is row0 + 1 + j */

  if (c->T == 0.0) {
    /* Greedy verification: accept the first child equal to the target's
     * argmax; the bonus token is the argmax at the final position. A row
     * with no distribution (NaN, +inf, all -inf) stops the walk without a
     * token, as in sampled verification.                                   */
    int pos = -1, d = 0;
    for (;;) {
      const float* lrow = c->logits + (row0 + pos + 1) * (int64_t)V;
      if (!orc_row_finite(V, lrow)) {
        c->status[b] |= 0x08;
        break;
      }
      int a = orc_argmax(V, lrow);
      int next = -1;
      for (int ch = pos + 1; ch < T; ++ch)
        if (par[ch] == pos && tok[ch] == a) { next = ch; break; }
      if (next < 0) {
        toks_out[d] = a;
        break;
      }
      acc_nodes[d] = next;
      toks_out[d] = tok[next];
      ++d;
      pos = next;
    }
    c->accept_len[b] = d;
    return;
  }

  double* P = (double*)malloc(sizeof(double) * (size_t)V);
  double* Q = (double*)malloc(sizeof(double) * (size_t)V);
  double* tmp = (double*)malloc(sizeof(double) * (size_t)V);
  if (!P || !Q || !tmp) { free(P); free(Q); free(tmp); c->status[b] |= 0x80; return; }

  int pos = -1, d = 0;
  for (;;) {
    const float* lrow = c->logits + (row0 + pos + 1) * (int64_t)V;
    /* this position's allowed-set threshold, and the band around it within
     * which another correct evaluation may place its own threshold        */
    double th = -INFINITY, band = 0.0;
    if (c->trunc == 1) {
      th = orc_min_p_threshold(c->T, c->p_base);
      /* T ln p_base in fp64 on either side: a few fp64 ulps apart at most */
      band = c->set_tol > 0.0 ? c->set_tol * c->T : 1e-12 * fmax(1.0, fabs(th));
    } else if (c->trunc == 2 && orc_row_finite(V, lrow)) {
      double G = 0.0, Var = 0.0;
      th = orc_eta_threshold(V, lrow, c->T, c->eta_eps, c->eta_delta, &G, &Var);
      /* Two evaluations of the threshold T (ln S + ln eps) or T (ln delta - G)
       * that weigh each token in fp64 (argument and exponential within a few
       * fp64 roundings) and sum V terms in fp64 in any order differ by at
       * most 2^-53 (V + 64) (8 + 8 G + 4 Var + 4 G^2) T (first order, every
       * rounding aligned): the band of the set's own error bound.           */
      band = c->set_tol > 0.0 ? c->set_tol * c->T
                              : c->T * ldexp((double)(V + 64) * (8.0 + 8.0 * G + 4.0 * Var + 4.0 * G * G), -53);
    }
    orc_rec rec;
    int bonus = -1;
    int acc = orc_position(c, b, pos, th, &rec, &bonus, P, Q, tmp);
    c->n_rejections[b] += rec.rejections;
    c->status[b] |= rec.status;
    if (rec.min_accept_margin < c->min_accept_margin[b]) c->min_accept_margin[b] = rec.min_accept_margin;
    if (rec.cdf_margin < INFINITY) c->cdf_margin[b] = rec.cdf_margin;
    c->draw_mass[b] = rec.draw_mass;
    if (c->flag_depth[b] < 0) {
      if (c->trunc && !(rec.status & 0x08) && orc_band_changes(c, b, pos, th, band, acc, bonus, P, Q, tmp)) {
        c->flag_depth[b] = d;
        c->flag_kind[b] = 2;
      } else if (rec.near_kind >= 0) {
        c->flag_depth[b] = d;
        c->flag_kind[b] = rec.near_kind;
      }
    }
    if (acc >= 0) {
      acc_nodes[d] = acc;
      toks_out[d] = tok[acc];
      ++d;
      pos = acc;
      continue;
    }
    toks_out[d] = bonus;
    break;
  }
  c->accept_len[b] = d;
  free(P);
  free(Q);
  free(tmp);
}

/* Verification of a packed batch (see the calling convention of the GPU
 * library: rows cu_nodes[b] + b + r, r = 0 root, r = 1 + j after node j).
 * T == 0 selects greedy verification; trunc = 1 verifies against the min-p
 * truncated target (p_base), trunc = 2 against the eta truncated target
 * (eta_eps, eta_delta); rule 3 is truncation-based verification
 * ([LOSSY] 3.2) over the allowed set of trunc 1 or 2; det != 0 treats the
 * siblings as deterministic candidates ([LOSSY] G.3; q unused and may be
 * NULL; a rejection takes the candidate out of the target); rule 1/2
 * selects the lossy lenience / interpolation accept test ([LOSSY] 3.1,
 * A.1, A.3) with rule_param = l / lambda in (0, 1] (not with det). Per
 * request it also reports
 *   flag_depth: accepted nodes before the first decision that is not fixed
 *               by the inputs to within the stated tolerances (-1: none);
 *   flag_kind:  0 = accept test with |u - h| < accept_tol, 1 = final draw
 *               with a CDF boundary within cdf_tol of u, 2 = allowed-set
 *               boundary: a threshold within the set's band (set_tol, or
 *               the set's own error bound when set_tol == 0: fp64 rounding
 *               of its evaluation) changes the position's outcome,
 *               3 = deterministic remainder at most 1e-11 of the row's mass;
 *   n_rejections: rejections (= residual renormalisations or removals);
 *   status: SV_STATUS-like bits (0x01 tree, 0x02 packing, 0x04 token,
 *           0x08 non-finite row reached, 0x10 zero residual, 0x80 out of
 *           memory);
 *   min_accept_margin, cdf_margin: the smallest |u - h| seen and the
 *           margin of the final draw;
 *   draw_mass: probability of the drawn token under the distribution it
 *           was drawn from (0: no draw). Given the token, u is uniform over
 *           its CDF interval, so the draw is a near tie (margin < cdf_tol)
 *           with probability min(1, 2 cdf_tol / draw_mass).              */
int orc_verify(int B, int V, const int32_t* cu_nodes, const int32_t* parent, const int32_t* tokens,
               const float* logits, const float* q, double T, int trunc, double p_base, double eta_eps,
               double eta_delta, double set_tol, int det, int rule, double rule_param, uint64_t seed, uint32_t step,
               const uint32_t* request_id, int max_depth, int32_t* accept_len, int32_t* accepted_nodes,
               int32_t* out_tokens, double* uniforms_out, int32_t* flag_depth, int32_t* flag_kind,
               int32_t* n_rejections, int32_t* status, double* min_accept_margin, double* cdf_margin,
               double* draw_mass, double accept_tol, double cdf_tol, int nthreads) {
  if (B < 0 || V < 1 || max_depth < 0 || T < 0.0) return 1;
  if (T > 0.0 && !det && !q) return 1;
  if (rule < 0 || rule > 3 || (rule && det)) return 1;
  if ((rule == 1 || rule == 2) && !(rule_param > 0.0 && rule_param <= 1.0)) return 1;
  if (rule == 3 && (!trunc || T == 0.0)) return 1; /* needs an allowed set */
  if (trunc < 0 || trunc > 2 || set_tol < 0.0) return 1;
  if (trunc == 1 && !(p_base > 0.0 && p_base < 1.0)) return 1;
  if (trunc == 2 && !(eta_eps > 0.0 && eta_eps < 1.0 && eta_delta > 0.0 && eta_delta <= 1.0)) return 1;
  if (T == 0.0) trunc = 0; /* greedy: the argmax is always allowed */
  orc_walk_ctx c = {B, V, cu_nodes, parent, tokens, logits, q, T, trunc, p_base, eta_eps, eta_delta, set_tol,
                    det, rule, rule_param, seed, step,
                    request_id, max_depth,
                    accept_len, accepted_nodes, out_tokens, uniforms_out, flag_depth, flag_kind,
                    n_rejections, status, min_accept_margin, cdf_margin, draw_mass, accept_tol, cdf_tol};
  orc_parallel_for(B, nthreads, orc_walk_one, &c);
  return 0;
}

/* p rows for a list of row indices (probability parity checks). */
int orc_target_rows(int V, const float* logits, double T, int64_t n_rows, const int64_t* rows, double* out) {
  int bad = 0;
  for (int64_t i = 0; i < n_rows; ++i)
    bad |= orc_target_probs(V, logits + rows[i] * (int64_t)V, T, out + i * (int64_t)V);
  return bad;
}

/* ------------------------------------------------------------------------ */
/* Budgeted super-tree packing ([ECHO] section 3.1: the batch's candidate
 * trees form one super-tree verified in one pass under the global cap
 * sum_i K_i <= K_max; Figure 3, step 3, flattens and packs the ragged
 * result into one dense layout). Reading: each candidate carries a score S
 * (ECHO's path score, the cumulative log q of its path: higher is better);
 * its effective score is the smallest score on its path,
 * S'(j) = min(S(j), S'(parent(j))), and the packer keeps the K_max best
 * candidates in the order (S' descending, request ascending, local index
 * ascending). S' never rises along a path and a parent precedes its child
 * at equal S', so a kept node's ancestors are kept; for path scores (which
 * never rise) this is the K_max best candidates. A NaN score counts as
 * -inf and -0 as +0. Kept nodes are packed request by request in their
 * original order, parents renumbered. A request with a parent outside
 * [-1, j-1] or more than 64 candidates keeps nothing (status bit 0x01 /
 * 0x02); offsets that are not non-decreasing from cu_cand[0] = 0 reject
 * the whole batch (0x02, nothing kept).                                   */
typedef struct {
  float s;   /* effective score */
  int64_t m; /* candidate index  */
} orc_pack_key;

static int orc_pack_cmp(const void* a, const void* b) {
  const orc_pack_key* x = (const orc_pack_key*)a;
  const orc_pack_key* y = (const orc_pack_key*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return x->m < y->m ? -1 : (x->m > y->m ? 1 : 0);
}

static float orc_canon_score(float s) {
  if (s != s) return -INFINITY;
  if (s == 0.0f) return 0.0f;
  return s;
}

int orc_pack(int B, const int32_t* cu_cand, const int32_t* cand_parent, const int32_t* cand_token,
             const float* cand_score, int64_t budget, int32_t* cu_nodes, int32_t* parent, int32_t* tokens,
             int32_t* src, int32_t* total_nodes, int32_t* status) {
  if (B < 0 || budget < 0) return 1;
  int64_t M = B > 0 ? cu_cand[B] : 0;
  orc_pack_key* keys = (orc_pack_key*)malloc(sizeof(orc_pack_key) * (size_t)(M > 0 ? M : 1));
  float* eff = (float*)malloc(sizeof(float) * (size_t)(M > 0 ? M : 1));
  char* keep = (char*)calloc((size_t)(M > 0 ? M : 1), 1);
  if (!keys || !eff || !keep) { free(keys); free(eff); free(keep); return 1; }
  *status = 0;
  int mono = B == 0 || cu_cand[0] == 0;
  for (int b = 0; b < B; ++b)
    if (cu_cand[b + 1] < cu_cand[b]) mono = 0;
  if (!mono) {
    for (int b = 0; b <= B; ++b) cu_nodes[b] = 0;
    *total_nodes = 0;
    *status = 0x02;
    free(keys); free(eff); free(keep);
    return 0;
  }
  int64_t n_valid = 0;
  for (int b = 0; b < B; ++b) {
    int64_t c0 = cu_cand[b], c1 = cu_cand[b + 1];
    int T = (int)(c1 - c0);
    int ok = T >= 0 && T <= 64 && c0 >= 0 && c1 <= M;
    if (!ok) { *status |= 0x02; continue; }
    for (int j = 0; j < T; ++j)
      if (cand_parent[c0 + j] < -1 || cand_parent[c0 + j] >= j) ok = 0;
    if (!ok) { *status |= 0x01; continue; }
    for (int j = 0; j < T; ++j) {
      /* smallest score on the path from j up to its top ancestor */
      float e = orc_canon_score(cand_score[c0 + j]);
      for (int x = cand_parent[c0 + j]; x >= 0; x = cand_parent[c0 + x]) {
        float sx = orc_canon_score(cand_score[c0 + x]);
        if (sx < e) e = sx;
      }
      eff[c0 + j] = e;
      keys[n_valid].s = e;
      keys[n_valid].m = c0 + j;
      ++n_valid;
    }
  }
  qsort(keys, (size_t)n_valid, sizeof(orc_pack_key), orc_pack_cmp);
  int64_t K = budget < n_valid ? budget : n_valid;
  for (int64_t i = 0; i < K; ++i) keep[keys[i].m] = 1;
  int64_t n = 0;
  cu_nodes[0] = 0;
  for (int b = 0; b < B; ++b) {
    int64_t c0 = cu_cand[b], c1 = cu_cand[b + 1];
    int T = (int)(c1 - c0);
    int newidx[64];
    int cnt = 0;
    if (T >= 0 && T <= 64 && c0 >= 0 && c1 <= M) {
      for (int j = 0; j < T; ++j) {
        newidx[j] = -1;
        if (!keep[c0 + j]) continue;
        int p = cand_parent[c0 + j];
        newidx[j] = cnt;
        parent[n] = p < 0 ? -1 : newidx[p];
        tokens[n] = cand_token[c0 + j];
        src[n] = (int32_t)(c0 + j);
        ++n;
        ++cnt;
      }
    }
    cu_nodes[b + 1] = (int32_t)n;
  }
  *total_nodes = (int32_t)n;
  free(keys);
  free(eff);
  free(keep);
  return 0;
}
