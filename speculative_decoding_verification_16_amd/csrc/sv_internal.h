// sv_internal.h -- parameter blocks and launchers shared between the host
// dispatch (sv_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sv_device.h"

namespace sv {

// ---- attention ---------------------------------------------------------------
struct AttnParams {
  int32_t B, N, Hq, Hkv, G, D;
  int32_t max_nodes;       // bound on T_b used for validation
  int64_t Lcap;
  const int32_t* ctx_len;
  const int32_t* cu_nodes;
  const uint64_t* anc;     // [N] ancestor-or-self masks, or nullptr: built per workgroup from parent
  const int32_t* parent;   // [N] parent array (when anc is nullptr)
  const void* q;           // [N, Hq, D]
  const void* k;           // [B, Hkv, Lcap, D]
  const void* v;
  float* out;              // [N, Hq, D] (used when splits == 1)
  float* o_part;           // [splits, N*Hq, D] unnormalised partial outputs
  float2* ml_part;         // [splits, N*Hq] (running max in log2 units, sum)
  int32_t splits;
  int32_t rows_per_wg;     // query rows (node, head-in-group) per workgroup
  int32_t n_rowgroups;     // workgroups along the rows of one (request, KV head, split)
  int32_t n_jobs;          // B * Hkv * splits
  // compacted work list (bf16 path with several row groups): entry 8 k + x is
  // the k-th live (job, row group) item of XCD class x, encoded as
  // job * n_rowgroups + row_group; item_tot[x] = live items of class x
  const int32_t* items;
  const int32_t* item_tot;
  float scale_log2;        // softmax scale * log2(e)
  int32_t* status;
  // paged caches: k / v are pools [num_blocks, Hkv, block_size, D] and slot t
  // of request b is row t % block_size of block block_table[b, t / block_size]
  const int32_t* block_table;  // [B, max_blocks], or null (contiguous caches)
  int32_t block_size, max_blocks;
  int32_t bs_shift;            // log2(block_size)
  int64_t num_blocks;
  // fp8 caches (OCP E4M3 bytes): k_scale is folded into scale_log2, v_scale
  // multiplies the output
  bool kv_fp8;
  float v_scale;
  // in the step: the sliced walk's coordination words, zeroed by the launch's
  // first workgroup (the walk follows on the same stream), or null
  int32_t* clear_words;
  int32_t nclear;
};

struct AttnPlan {
  bool mfma;        // bf16 MFMA path (else fp32 VALU path)
  int rows_per_wg;
  int n_rowgroups;  // workgroups per (request, KV head, split) along rows
  int splits;
  bool compact;     // live (job, row group) items are listed on the device first
};

// blocks of the 1-D bf16 attention grid: 8-job groups x row groups
inline int64_t attn_grid_blocks(int64_t n_jobs, int n_rowgroups) { return (n_jobs + 7) / 8 * 8 * n_rowgroups; }

// ancestor masks (when anc is given: written there from parent) and the
// compacted work list (when plan.compact), in one launch before the attention
hipError_t launch_attn_prep(const AttnParams& p, const AttnPlan& plan, const int32_t* parent, uint64_t* anc,
                            hipStream_t stream);
// (defer_merge: the split-K merge is not launched but described there, for
// the caller's next launch to run; nullptr: launched here)
hipError_t launch_attention(const AttnParams& p, const AttnPlan& plan, bool bf16, hipStream_t stream,
                            hipEvent_t ev_start, hipEvent_t ev_stop, MergeArgs* defer_merge = nullptr);

// ---- sampler -----------------------------------------------------------------
struct SampleParams {
  int32_t B, V, N, max_nodes, max_depth;
  int32_t nch;              // vocabulary chunks per row
  const int32_t* cu_nodes;
  const int32_t* parent;
  const int32_t* tokens;
  const float* logits;      // [N+B, V]
  const float* q;           // [N+B, V] (unused when greedy)
  float c;                  // log2(e) / temperature (0 when greedy)
  double c64;               // the same in fp64 (the eta set's fp64 sums)
  bool greedy;
  bool trunc;               // truncation of the target rows (min-p or eta)
  bool eta;                 // the eta allowed set (else min-p)
  RowThr mp_thr;            // min-p threshold on logit - row max: T ln min_p in fp64
  double temp, ln_eps, ln_delta; // eta: temperature, ln eps, ln delta
  double2* ent;             // [N+B, nch] eta: per-chunk fp64 sums of w and of w * log2-exponent
  RowThr* rthr;             // [N+B] per-row threshold of the allowed set (trunc)
  bool det;                 // siblings are deterministic candidates (q unused)
  int32_t rule;             // accept test: 0 lossless, 1 lenience, 2 interpolation, 3 truncation
  float rule_param;         // l or lambda of the rule
  uint64_t seed;
  uint32_t step;
  const uint32_t* request_id;
  int32_t* accept_len;
  int32_t* accepted_nodes;
  int32_t* out_tokens;
  float* probs_out;
  double* uniforms_out;
  int32_t* residual_passes;
  int32_t* status;
  ChunkStat* stats;         // [N+B, nch] workspace
  RowStat* rowstats;        // [N+B] workspace
  int32_t slices;           // workgroups per request in the walk (1: no exchange)
  int32_t lazy;             // the walk computes the statistics of the rows it reaches (no statistics pass)
  int32_t coord_cleared;    // the step's attention launch has already zeroed xcnt
  double* xs;               // [B, 2, 2 nch] workspace when slices > 1
  int32_t* xcnt;            // [B, kWalkSync] workspace when slices > 1 (zeroed by the sampler)
  uint32_t join_ticks;      // start-up window of a request's slices (100 MHz ticks; 0: none, the
                            // first slice to look walks its request alone)
  MergeArgs merge;          // the step's split-K merge, run by extra blocks of the walk's launch
                            // (blocks == 0: none)
};

// per-request words of the walk's slice coordination: pass-barrier arrivals,
// start-up arrivals, mode (0 undecided, 1 sliced, 2 + 4 s: slice s alone)
constexpr int kWalkSync = 4;

// compute units of the current device (cached per device; 256 if unknown)
int device_cus();

// walk layouts (sv_sample_args.walk_mode)
constexpr int kWalkAuto = 0, kWalkSingle = 1, kWalkSliced = 2;
constexpr uint32_t kJoinWindow = 2000;  // default start-up window of a request's slices, 100 MHz ticks (20 us)

// workgroups per request for the walk: 1 without vocabulary passes (passes)
// or in the single layout; min(8, work) "slices" of 256 threads in the sliced
// layout; automatically, slices when the batch leaves at least four
// workgroup slots per request on the current device, else 1
int walk_slices(int B, int nch, bool passes, int mode);

// optional timing events of the sampler (recorded on its stream when set)
struct SampleEvents {
  hipEvent_t start;       // before the row-statistics kernel
  hipEvent_t stats_stop;  // after it
  hipEvent_t stop;        // after the walk
};
hipError_t launch_sampler(const SampleParams& p, bool vec4, hipStream_t stream, const SampleEvents& ev);

// ---- budgeted super-tree packing ------------------------------------------------
constexpr int kPackMaxB = 8192;  // requests per packing call (one workgroup's LDS scan)
struct PackParams {
  int32_t B;
  int64_t M;                // candidates, cu_cand[B]
  const int32_t* cu_cand;   // [B+1]
  const int32_t* par;       // [M] local parents
  const int32_t* tok;       // [M]
  const float* score;       // [M]
  int32_t budget;           // K_max
  int32_t* cu_nodes;        // [B+1]
  int32_t* parent;          // [min(budget, M)]
  int32_t* tokens;
  int32_t* src;
  int32_t* total;           // [1]
  int32_t* status;
  uint64_t* keys;           // [M] workspace
};
hipError_t launch_pack(const PackParams& p, hipStream_t stream);

}  // namespace sv
