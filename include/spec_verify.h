/*
 * spec_verify.h -- C ABI of the speculative-decoding verification step on one
 * AMD Instinct MI355X (gfx950).
 *
 * One verification step for a batch of B requests, each carrying a draft tree
 * (a chain is the tree whose node j has parent j-1) of T_b candidate tokens:
 *
 *   1. tree-masked grouped-query attention of every draft node against its
 *      request's KV cache                          -> spec_verify_attn
 *   2. lossless rejection sampling over the whole vocabulary, walking the tree
 *      and emitting the accepted path plus one bonus token
 *                                                   -> spec_verify_sample
 *   3. both in one call (in order on one stream, or the two concurrently
 *      on two streams: sv_sample_args.step_overlap) -> spec_verify_step
 *
 * Sources (the method is defined there; section names are given per call):
 *   [SD]   "Speculative Decoding: Accelerating Inference Speeds in Distributed
 *          LLMs" (shyankdev.com blog).
 *   [LOSSY] "Revisiting Lossy Verification in Speculative Decoding: Mechanisms,
 *          Trade-offs, and Failure Modes" (arXiv 2607.26627).
 *   [ECHO] "ECHO: Elastic Speculative Decoding with Sparse Gating for
 *          High-Concurrency Scenarios" (arXiv 2604.09603).
 *   [SPEED] "SPEED-Bench: A Unified and Diverse Benchmark for Speculative
 *          Decoding" (arXiv 2604.09557).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every pointer in the argument structs is DEVICE memory owned by the
 *    caller, except where a field says otherwise. The library allocates no
 *    device memory; scratch lives in the caller's workspace (see
 *    spec_verify_workspace_size). It keeps no state between calls (apart
 *    from handles it creates once: spec_verify_step's second stream under
 *    SV_OVERLAP_ON, and the noalloc entry point's scratch address) and is
 *    reentrant; two calls may run concurrently on different streams if they
 *    use different workspaces and outputs.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream) and never synchronise with the host. The stream and every
 *    device pointer belong to the current HIP device of the calling thread
 *    (the library's own handles are kept per current device).
 *  - Argument errors are found on the host before anything is enqueued: the
 *    call then returns a non-SV_OK code, enqueues nothing and leaves a message
 *    for spec_verify_last_error(). SV_ERR_HIP means a launch failed.
 *  - Errors that depend on device data are OR-ed as SV_STATUS_* bits into the
 *    optional device word `status` (the library never clears it: zero it
 *    before the call for per-call status). Kernels stay in bounds whatever the
 *    data: offending requests are skipped or clamped as each bit documents.
 *  - Results are a pure function of the inputs (and of seed, step and
 *    request ids): every reduction runs in a fixed order, so two identical
 *    calls give bitwise identical outputs.
 *  - Packing ("Flatten & Pack", [ECHO] Figure 3 and the super-tree of its
 *    section 3.1): the nodes of all requests are concatenated; request b owns
 *    packed nodes [cu_nodes[b], cu_nodes[b+1]), T_b = cu_nodes[b+1]-cu_nodes[b],
 *    0 <= T_b <= 64, N = cu_nodes[B] = total_nodes. Local node j of request b
 *    is packed node cu_nodes[b] + j.
 *  - Trees are given as a parent array of LOCAL indices in topological order:
 *    parent[cu_nodes[b]+j] is in [-1, j-1]; -1 means the node hangs off the
 *    request's root (its last committed token).
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SV_OK = 0,
  SV_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size or value      */
  SV_ERR_TREE = 2,        /* reserved for host-visible tree errors            */
  SV_ERR_UNSUPPORTED = 3, /* valid but unsupported shape (e.g. D not 64/128)  */
  SV_ERR_WORKSPACE = 4,   /* workspace missing, misaligned or too small       */
  SV_ERR_HIP = 5          /* a HIP launch failed                              */
} sv_status;

typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

/* Data-error bits OR-ed into *status by the kernels. */
#define SV_STATUS_TREE_INVALID   0x01 /* parent outside [-1, j-1]: node treated as a root child (attn) / request skipped (sample) */
#define SV_STATUS_PACKING        0x02 /* cu_nodes not monotone, T_b > max_nodes, or cu_nodes[B] != total_nodes: request skipped */
#define SV_STATUS_TOKEN_RANGE    0x04 /* draft token outside [0, V): request skipped */
#define SV_STATUS_NONFINITE      0x08 /* the walk reached a row with a NaN or +inf logit, or whose logits are all
                                         -inf: it has no target distribution; the walk stops there, without a
                                         token at that position (out_tokens[b][accept_len[b]] = -1); rows the
                                         walk does not reach are not checked */
#define SV_STATUS_ZERO_RESIDUAL  0x10 /* residual mass rounded to 0 after a rejection: distribution kept unchanged */
#define SV_STATUS_CTX_RANGE      0x20 /* ctx_len[b] < 0 or ctx_len[b] + T_b > Lcap: request skipped */
#define SV_STATUS_SYNC           0x40 /* a sampler workgroup gave up waiting for the other workgroups of its request
                                         (not expected: they agree to cooperate only once all are running) */
#define SV_STATUS_BLOCK_RANGE    0x80 /* paged caches: a block id outside [0, num_blocks): its keys read as zeros,
                                         the request's outputs are undefined, nothing is read out of bounds */

/* ------------------------------------------------------------------------ */
/* Tree-masked GQA attention ([SD] "Tree Attention Mask Mechanics"; GQA as in
 * [SD] "Interaction with Advanced Attention Architectures (GQA & MLA)").
 *
 * For request b, query head h (KV head g = h / (Hq/Hkv)) and local node j:
 *   visible keys = context slots [0, ctx_len[b]) of the cache
 *                  + draft slot ctx_len[b] + i for every i that is j itself or
 *                    an ancestor of j (never a sibling branch);
 *   s_t = scale * <q, k_t>,  w = softmax(s) over the visible keys,
 *   out = sum_t w_t v_t.
 * The draft node i's key/value sit in cache slot ctx_len[b] + i (node order).
 * q and k are used as given (position encoding already applied).          */
typedef struct {
  int32_t B;           /* requests, >= 0                                      */
  int32_t total_nodes; /* N = cu_nodes[B]                                     */
  int32_t max_nodes;   /* upper bound on every T_b, 1..64; 0 means 64         */
  int32_t Hq, Hkv, D;  /* Hq % Hkv == 0; D is 64 or 128                       */
  int32_t dtype;       /* sv_dtype: element type of q, k_cache, v_cache      */
  const void* q;       /* [N, Hq, D], 16-byte aligned                         */
  const void* k_cache; /* [B, Hkv, Lcap, D], 16-byte aligned                  */
  const void* v_cache; /* [B, Hkv, Lcap, D], 16-byte aligned                  */
  int64_t Lcap;        /* slots per (request, KV head), >= 1                  */
  const int32_t* ctx_len;  /* [B] committed context length L_b             */
  const int32_t* cu_nodes; /* [B+1] packing offsets                        */
  const int32_t* parent;   /* [N] local parent (-1 = root); may be NULL if anc_mask given */
  const uint64_t* anc_mask;/* [N] optional: bit i set iff local node i is visible to the
                              node (itself or an ancestor); used instead of parent if non-NULL */
  float scale;         /* softmax scale; 0 means 1/sqrt(D)                    */
  int32_t num_splits;  /* KV-length splits; 0 = chosen by the library         */
  float* out;          /* [N, Hq, D] fp32, 16-byte aligned                    */
  int32_t* status;     /* optional device word for SV_STATUS_* bits           */
  /* Paged caches (optional; the layout of PagedAttention-style engines, which
   * [SD] "Tree Attention Mask Mechanics" names as the kernels a tree mask is
   * handed to). block_table == NULL: k_cache / v_cache are [B, Hkv, Lcap, D].
   * Otherwise they are pools [num_blocks, Hkv, block_size, D], and slot t of
   * request b (committed context and draft slots alike) sits in block
   * block_table[b * max_blocks + t / block_size] at row t % block_size;
   * Lcap must equal max_blocks * block_size. Blocks may be shared between
   * requests (a common prefix). block_size is a power of two, at least 64
   * (one 64-key tile never spans two blocks). An id outside [0, num_blocks)
   * sets SV_STATUS_BLOCK_RANGE.                                            */
  const int32_t* block_table; /* [B, max_blocks] device memory, or NULL     */
  int32_t block_size;
  int32_t max_blocks;
  int64_t num_blocks;
  /* FP8 caches (optional; with dtype SV_BF16 for q). kv_fp8 = 1: k_cache and
   * v_cache hold OCP FP8 E4M3 (finite form) bytes, contiguous or paged as
   * above, and the value of a key (value) element is its byte's value times
   * k_scale (v_scale), both finite and > 0. E4M3 values are exact in bf16;
   * k_scale is folded into the softmax scale and v_scale into the output.
   * The kernels are those of bf16 caches (16x16 or 32x32 MFMA tiles by the
   * rows per KV head); the bytes are widened to bf16 on their way to LDS.  */
  int32_t kv_fp8;
  float k_scale;
  float v_scale;
} sv_attn_args;

/* ------------------------------------------------------------------------ */
/* Lossless rejection sampling over the tree ([SD] "Mathematical Rejection
 * Sampling Algorithm" and "Proof of Lossless Distribution Equivalence";
 * [LOSSY] section 2.1 h(x) = min(1, p/q) and appendix F.1 residual r(x)).
 *
 * Rows: request b owns rows cu_nodes[b] + b + r, r = 0..T_b. Row r = 0 is the
 * root position (distribution of the first draft token); row r = 1 + j is the
 * position after local node j. Node j is tested against the p and q rows of
 * its parent's position. p = softmax(target_logits / temperature); q is used
 * exactly as given (already tempered by the caller, not renormalised).
 *
 * Walk (temperature > 0): at the current position, children are tried in
 * increasing node index; child c with token x is accepted iff
 *   P(x) > 0 and u_c * Q(x) <= P(x),   u_c = U(b, c, purpose 0),
 * where P is the current target distribution (p, then residuals). After a
 * rejection P <- max(0, P - Q) / sum max(0, P - Q) (kept unchanged, with
 * SV_STATUS_ZERO_RESIDUAL, if that sum is 0) and the next sibling is tried.
 * On acceptance the walk descends into the accepted node's row. When no child
 * is accepted (or there is none), the bonus token is
 *   y = min{ x : sum_{t<=x} P(t) > U(b, 0, purpose 1) * sum_t P(t) }.
 * Temperature 0 is greedy: accept the first child whose token equals the
 * argmax of the raw logits of the row (lowest index on ties); the bonus token
 * is the argmax of the final row.
 *
 * U(b, j, purpose) = (w0 + 0.5) * 2^-32 where w0 is word 0 of Philox4x32-10
 * (Salmon et al., SC'11) with key = (seed & 0xffffffff, seed >> 32) and
 * counter = (request_id[b], j, purpose, step).                            */
/* Sibling rule of the sampled walk ([LOSSY] appendix G.3).
 *   SV_SIBLINGS_SAMPLED: the children of a node are independent draws from q
 *     at its position; the rule above (q required).
 *   SV_SIBLINGS_DETERMINISTIC: the children are fixed candidates (say the
 *     drafter's top-k), tried in increasing node index. Candidate i with
 *     token x is accepted iff P_i(x) > 0 and u_c <= P_i(x), where P_i is the
 *     target with the tokens of the candidates rejected before it removed
 *     and renormalised (P_1 = p; a token already removed has P = 0). With no
 *     candidate accepted, the bonus token is drawn (inverse CDF as above)
 *     from the target without the rejected candidates. The emitted tokens
 *     follow p (p_Theta under min_p) exactly; q is not read (draft_probs may
 *     be NULL) and the walk needs no vocabulary pass without min_p. A
 *     remainder below 1e-12 of the row's mass counts as zero
 *     (SV_STATUS_ZERO_RESIDUAL, candidate kept).                            */
typedef enum { SV_SIBLINGS_SAMPLED = 0, SV_SIBLINGS_DETERMINISTIC = 1 } sv_siblings;

/* Accept test of the sampled walk with sampled siblings ([LOSSY] section 3.1,
 * collaborative verification; these change the emitted distribution).
 *   SV_RULE_LOSSLESS: u * Q(x) <= P(x), the rule above.
 *   SV_RULE_LENIENCE: u * (l Q(x)) <= P(x), h = min(1, P/(l Q)) with
 *     l = rule_param in (0, 1] (appendix A.3).
 *   SV_RULE_INTERPOLATION: u * Q(x) <= nu(x), nu = lambda P + (1 - lambda) Q,
 *     h = min(1, nu/Q) with lambda = rule_param in (0, 1] (CoS; appendix A.1).
 * Every other step is the lossless one: a rejection moves P to the residual
 * max(0, P - Q) normalised (the residual both appendices give), and the bonus
 * token is drawn from P. Products and sums are in fp64 from the fp32 rule_param. */
/*   SV_RULE_TRUNCATION: truncation-based verification ([LOSSY] section 3.2;
 *     SpecCascade with the min-p allowed set, typical acceptance with the eta
 *     set): h(x) = 1 if x is in the allowed set of min_p or eta_eps/eta_delta
 *     (one of them is required), else 0 -- the same fp32 membership test the
 *     truncation makes; no uniform is used. After every child of a position
 *     is rejected, the bonus token is drawn from q restricted to the set,
 *     q(x) 1{x in A} / sum_A q (the residual that gives the section's law
 *     q / Z_A(q); with no mass there the truncated target is used and
 *     SV_STATUS_ZERO_RESIDUAL set); at a leaf from the truncated target.
 *     rule_param is unused.                                                */
typedef enum { SV_RULE_LOSSLESS = 0, SV_RULE_LENIENCE = 1, SV_RULE_INTERPOLATION = 2,
               SV_RULE_TRUNCATION = 3 } sv_rule;

typedef struct {
  int32_t B, V;        /* requests (>= 0); vocabulary size (1 .. 1<<22)      */
  int32_t total_nodes; /* N = cu_nodes[B]                                     */
  int32_t max_nodes;   /* upper bound on every T_b, 1..64; 0 means 64         */
  const int32_t* cu_nodes;     /* [B+1] packing offsets                    */
  const int32_t* parent;       /* [N] local parent (-1 = root)             */
  const int32_t* draft_tokens; /* [N] token of each node                   */
  const float* target_logits;  /* [N+B, V] fp32 rows as described above    */
  const float* draft_probs;    /* [N+B, V] fp32; may be NULL if temperature == 0
                                  or the siblings are deterministic         */
  float temperature;   /* 0 = greedy; > 0 = sampled                           */
  float min_p;         /* 0 = off; in (0, 1) with temperature > 0: verify
                          against the min-p truncated target ([LOSSY] 2.3,
                          "truncation sampling + SD", G.2): p restricted to
                          A = {x : p(x) >= min_p * max p}, decided exactly as
                          l_x - l_max >= T ln min_p (the logit difference and
                          the threshold in fp64, from the fp32 T and min_p),
                          and renormalised; every rule below then applies
                          with p_Theta in place of p. Each visited position
                          costs one more vocabulary pass (the mass of A).
                          Not with probs_out.                                */
  float eta_eps;       /* 0 = off; in (0, 1) with temperature > 0 and min_p == 0:
                          verify against the eta truncated target ([LOSSY] 2.3):
                          A = {x : p(x) >= min(eta_eps, eta_delta exp(-H(p)))},
                          H the entropy of p in nats, decided as
                          l_x - l_max >= T (ln S + ln tau) with S the row's
                          sum of exp((l - l_max)/T); the threshold is formed
                          in fp64 per row from per-chunk fp64 sums of fp64
                          weights 2^y and 2^y y (y in log2 units, each
                          weight within a few fp64 ulps), gathered with the
                          row's statistics (by the statistics pass, or by the
                          walk for a row it reduces itself); membership is
                          then decided exactly as for min_p. Not with
                          probs_out.                                         */
  float eta_delta;     /* delta of the eta set, in (0, 1] when eta_eps > 0     */
  int32_t siblings;    /* sv_siblings: how the children of a node were drafted */
  int32_t rule;        /* sv_rule (SV_RULE_LOSSLESS unless sampled siblings)   */
  float rule_param;    /* l or lambda of the rule, in (0, 1]; unused when lossless */
  uint64_t seed;       /* Philox key                                          */
  uint32_t step;       /* Philox counter word 3 (replay / advance)            */
  const uint32_t* request_id; /* [B] Philox counter word 0; NULL means b    */
  int32_t max_depth;   /* row capacity of the outputs, >= max_nodes (0 -> 64) */
  int32_t* accept_len;      /* [B] accepted draft nodes (0..T_b); 0 for a skipped request */
  int32_t* accepted_nodes;  /* [B, max_depth] local ids along the accepted path, -1 padded */
  int32_t* out_tokens;      /* [B, max_depth+1] accepted tokens then the bonus token, -1 padded;
                               all -1 for a request skipped because of a data error */
  float* probs_out;         /* optional [N+B, V] fp32 p rows (temperature > 0 only) */
  double* uniforms_out;     /* optional [N+B]: [n] = U(b, j, 0) for packed node n = cu_nodes[b]+j,
                               [N+b] = U(b, 0, 1)                                   */
  int32_t* residual_passes; /* optional [B]: rejections during the walk (with sampled siblings, each
                               costs one vocabulary pass for the residual mass) */
  int32_t* status;          /* optional device word for SV_STATUS_* bits           */
  /* Layout of the walk (results are bitwise the same in every layout):
   *   SV_WALK_AUTO: one 512-thread workgroup per request, or, when the walk
   *     makes vocabulary passes and the batch leaves at least four workgroup
   *     slots per request on the device, up to 8 256-thread workgroups
   *     ("slices") per request that split every pass;
   *   SV_WALK_SINGLE: always one workgroup per request;
   *   SV_WALK_SLICED: slices whenever the walk makes vocabulary passes.
   * The slices of a request first agree to cooperate: once all have started
   * they walk it together; if join_ticks of the 100 MHz device clock pass
   * first, one of them walks it alone. join_ticks: 0 = 2000 (20 us);
   * > 0 = that many (at most 10^8); -1 = none (the first slice to look
   * walks alone).                                                          */
  int32_t walk_mode;
  int32_t join_ticks;
  /* Schedule of spec_verify_step (ignored by spec_verify_sample; results are
   * bitwise the same either way):
   *   SV_OVERLAP_OFF (0, the default): attention, then the sampler, all on
   *     the caller's stream;
   *   SV_OVERLAP_ON (1): the sampler on the caller's stream while the
   *     attention (with its split-K merge) runs on a second stream forked
   *     from the caller's at the call's start and joined back into it at the
   *     end (the caller's stream sees the whole step done, as with OFF). The
   *     attention leaves part of the HBM bandwidth unused and the sampler's
   *     logit reads stream through it. Faster for large batches (256
   *     requests of 152K-token rows: 0.68 -> 0.63 ms per step on one
   *     MI355X), slower for small ones (the fork and join cost a
   *     few microseconds); each kernel then takes longer than alone, as the
   *     two share the device. The second stream (non-blocking, default
   *     priority) and its two events are created by the library on first use,
   *     one set per host thread and device, and kept until the process ends.
   * spec_verify_step_noalloc always runs the OFF schedule.                 */
  int32_t step_overlap;
} sv_sample_args;

enum { SV_WALK_AUTO = 0, SV_WALK_SINGLE = 1, SV_WALK_SLICED = 2 };
enum { SV_OVERLAP_OFF = 0, SV_OVERLAP_ON = 1 };

/* ------------------------------------------------------------------------ */
/* Budgeted super-tree packing ([ECHO] section 3.1, "Super-Tree View": the
 * batch's candidate trees are verified as one flattened union under the
 * global cap sum_i K_i <= K_max; Figure 3, step 3: the ragged batch is
 * flattened and packed into one dense layout). The step before
 * spec_verify_step: its outputs are that call's cu_nodes, parent and
 * draft_tokens, and src tells the caller which candidate's q row, hidden
 * state and K/V each packed node carries.
 *
 * Candidate j of request b (local index, parents before children) has score
 * S (for instance ECHO's path score, the cumulative log q of its path:
 * higher is better; a NaN counts as -inf, -0 as +0). Its effective score is
 * the smallest score on its path, e(j) = min(S(j), e(parent(j))). The
 * min(budget, valid candidates) best candidates by (e descending, candidate
 * index ascending) are kept. That set holds every kept node's ancestors,
 * and for path scores, which never rise along a path, it is the K_max best
 * candidates. Kept nodes are packed request by request in their original
 * order with renumbered parents.
 *
 * Data errors: a request with more than 64 candidates (SV_STATUS_PACKING)
 * or a parent outside [-1, j-1] (SV_STATUS_TREE_INVALID) keeps nothing;
 * offsets that are not non-decreasing from cu_cand[0] = 0 to total_cand
 * keep nothing at all (SV_STATUS_PACKING).                                 */
typedef struct {
  int32_t B;                  /* requests, 0 .. 8192                          */
  int32_t total_cand;         /* M = cu_cand[B], 0 .. 2^24                    */
  const int32_t* cu_cand;     /* [B+1] candidate offsets                      */
  const int32_t* cand_parent; /* [M] local parent, -1 for a child of the root */
  const int32_t* cand_token;  /* [M] token of each candidate                  */
  const float* cand_score;    /* [M] score, higher is better                  */
  int32_t budget;             /* K_max >= 0                                   */
  int32_t* cu_nodes;          /* [B+1] out: packed offsets                    */
  int32_t* parent;            /* [min(budget, M)] out: packed local parents   */
  int32_t* draft_tokens;      /* [min(budget, M)] out: packed tokens          */
  int32_t* src;               /* [min(budget, M)] out: candidate index of each packed node */
  int32_t* total_nodes;       /* [1] out: N = cu_nodes[B]                     */
  int32_t* status;            /* optional device word for SV_STATUS_* bits    */
} sv_pack_args;

/* Workspace bytes of spec_verify_pack (8 per candidate; 0 on invalid
 * arguments, with the last error set, or when M == 0).                    */
size_t spec_verify_pack_workspace_size(const sv_pack_args* pack);

/* Budgeted packing; ws: 256-byte aligned device buffer of at least
 * spec_verify_pack_workspace_size(pack) bytes. All pointers are device
 * memory owned by the caller; asynchronous on stream.                      */
sv_status spec_verify_pack(const sv_pack_args* pack, void* ws, size_t ws_bytes, void* stream);

/* Bytes of workspace the calls need for these arguments (either pointer may be
 * NULL). Depends only on host-visible fields. Returns 0 on invalid arguments
 * (and sets the last error) or when no scratch is needed.                  */
size_t spec_verify_workspace_size(const sv_attn_args* attn, const sv_sample_args* sample);

/* Tree-masked GQA attention. ws: 256-byte aligned device buffer of at least
 * spec_verify_workspace_size(attn, NULL) bytes (may be NULL if that is 0).  */
sv_status spec_verify_attn(const sv_attn_args* attn, void* ws, size_t ws_bytes, void* stream);

/* Rejection-sampling walk. ws as above with spec_verify_workspace_size(NULL, sample). */
sv_status spec_verify_sample(const sv_sample_args* sample, void* ws, size_t ws_bytes, void* stream);

/* Layout of spec_verify_sample's walk for these arguments (host-visible
 * fields only; under SV_WALK_AUTO also the current device's CU count and
 * occupancy), for callers that account for the walk's memory traffic.
 *   *slices: workgroups per request, 1, or 2..8 for the sliced walk;
 *   *reached_rows_only: 1 when the walk computes the statistics of the logit
 *     rows it reaches by itself and reads no other row (no probs_out, and the
 *     N + B rows hold at least 128 MiB of logits), 0 when a statistics pass
 *     reads every row first. Results are bitwise the same either way.
 * Either pointer may be NULL. Returns SV_OK, or the error of invalid
 * arguments (with the last error set); nothing runs on the device.        */
sv_status spec_verify_walk_layout(const sv_sample_args* sample, int32_t* slices, int32_t* reached_rows_only);

/* Attention then sampling on one stream; the two argument sets must describe
 * the same batch (B, total_nodes, cu_nodes). ws: spec_verify_workspace_size(attn, sample). */
sv_status spec_verify_step(const sv_attn_args* attn, const sv_sample_args* sample,
                           void* ws, size_t ws_bytes, void* stream);

/* Timing events of spec_verify_step_timed (measurement): hipEvent_t handles
 * created by the caller, each recorded on the call's stream when non-NULL
 * (under SV_OVERLAP_ON, attn_start and attn_stop on the library's second
 * stream, where the attention runs; elapsed times between events of the two
 * streams then span concurrent work).                                      */
typedef struct {
  void* attn_start;   /* before the attention kernel (after tree preparation) */
  void* attn_stop;    /* after the attention kernel (before a split merge)    */
  void* sample_start; /* before the sampler's first kernel                    */
  void* stats_stop;   /* after the row-statistics kernel (which, when the walk
                         computes its rows' statistics itself, only clears the
                         sliced walk's coordination words, or does not run) */
  void* sample_stop;  /* after the walk (the sampler's last kernel; in the
                         step its launch also runs the attention's split-K
                         merge, if any, beside the walk)                      */
} sv_timing;

/* spec_verify_step that also records the events of *timing (may be NULL);
 * otherwise identical.                                                     */
sv_status spec_verify_step_timed(const sv_attn_args* attn, const sv_sample_args* sample, void* ws, size_t ws_bytes,
                                 void* stream, const sv_timing* timing);

/* spec_verify_step without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Its scratch is a 64 MiB (2^26-byte)
 * array owned by the library, one per GPU, held from the library's loading
 * on that GPU until the process ends; its address is looked up once per
 * device (the first call on it, with that device current). Every call on a
 * GPU shares that GPU's array and leaves its contents behind: calls that
 * overlap on one GPU (other streams or other host threads) race and must
 * not be issued. Arguments whose workspace (spec_verify_workspace_size)
 * exceeds 64 MiB are rejected with SV_ERR_UNSUPPORTED before anything is
 * enqueued. Allocates nothing; the results are bitwise those of
 * spec_verify_step.                                                        */
sv_status spec_verify_step_noalloc(const sv_attn_args* attn, const sv_sample_args* sample, void* stream);

/* Message of the last failed call on this thread ("" if none).             */
const char* spec_verify_last_error(void);

/* sizeof(sv_attn_args) for which == 0, sizeof(sv_sample_args) for which == 1,
 * sizeof(sv_pack_args) for which == 2, 0 otherwise: lets bindings check
 * their struct layout against this one.                                    */
size_t spec_verify_struct_size(int32_t which);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
