// sv_api.hip -- host side of the C ABI declared in include/spec_verify.h:
// argument validation, launch planning, workspace layout and dispatch.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "spec_verify.h"
#include "sv_device.h"
#include "sv_internal.h"

namespace {

thread_local char g_err[512] = "";

sv_status fail(sv_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int eff_max_nodes(int32_t m) { return m == 0 ? sv::kMaxNodes : m; }

// ---- attention -------------------------------------------------------------
sv_status check_attn(const sv_attn_args* a) {
  if (!a) return fail(SV_ERR_INVALID_ARG, "attn args is NULL");
  if (a->B < 0) return fail(SV_ERR_INVALID_ARG, "B < 0");
  if (a->total_nodes < 0) return fail(SV_ERR_INVALID_ARG, "total_nodes < 0");
  if (a->max_nodes < 0 || a->max_nodes > sv::kMaxNodes)
    return fail(SV_ERR_UNSUPPORTED, "max_nodes must be in [0, 64] (one 64-bit ancestor mask per node)");
  if (a->Hq <= 0 || a->Hkv <= 0 || a->Hq % a->Hkv != 0)
    return fail(SV_ERR_INVALID_ARG, "need Hq > 0, Hkv > 0 and Hq %% Hkv == 0");
  if (a->D != 64 && a->D != 128) return fail(SV_ERR_UNSUPPORTED, "head dim D must be 64 or 128");
  if (a->dtype != SV_F32 && a->dtype != SV_BF16) return fail(SV_ERR_INVALID_ARG, "dtype must be SV_F32 or SV_BF16");
  if (a->kv_fp8 != 0 && a->kv_fp8 != 1) return fail(SV_ERR_INVALID_ARG, "kv_fp8 must be 0 or 1");
  if (a->kv_fp8 && a->dtype != SV_BF16) return fail(SV_ERR_UNSUPPORTED, "fp8 caches need bf16 queries (dtype SV_BF16)");
  if (a->kv_fp8 && !(a->k_scale > 0.f && a->v_scale > 0.f && !isinf(a->k_scale) && !isinf(a->v_scale)))
    return fail(SV_ERR_INVALID_ARG, "k_scale and v_scale must be finite and > 0");
  if (a->Lcap < 1 || a->Lcap > (1ll << 24)) return fail(SV_ERR_INVALID_ARG, "Lcap must be in [1, 2^24]");
  if (a->block_table) {
    if (a->block_size < 64 || (a->block_size & (a->block_size - 1)) != 0)
      return fail(SV_ERR_UNSUPPORTED, "block_size must be a power of two, at least 64");
    if (a->max_blocks <= 0 || (int64_t)a->max_blocks * a->block_size != a->Lcap)
      return fail(SV_ERR_INVALID_ARG, "paged caches need max_blocks > 0 and Lcap == max_blocks * block_size");
    if (a->num_blocks <= 0) return fail(SV_ERR_INVALID_ARG, "num_blocks must be > 0");
    if (a->max_blocks > 192 * 256)
      return fail(SV_ERR_UNSUPPORTED, "max_blocks above 49152 (a split holds at most 256 block ids)");
    if (!aligned(a->block_table, 4)) return fail(SV_ERR_INVALID_ARG, "block_table must be 4-byte aligned");
  }
  if (!(a->scale >= 0.f) || isinf(a->scale)) return fail(SV_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if (a->num_splits < 0) return fail(SV_ERR_INVALID_ARG, "num_splits < 0");
  if ((int64_t)a->total_nodes * a->Hq * a->D >= (1ll << 31))
    return fail(SV_ERR_UNSUPPORTED, "N * Hq * D must stay below 2^31");
  // contiguous caches are addressed per (request, KV head) with 32-bit offsets;
  // paged ones per 64-key tile
  const int64_t kv_head_bytes = a->Lcap * a->D * (a->kv_fp8 ? 1 : (a->dtype == SV_BF16 ? 2 : 4));
  if (!a->block_table && kv_head_bytes >= (1ll << 31))
    return fail(SV_ERR_UNSUPPORTED, "Lcap * D * element size must stay below 2^31");
  if (a->B == 0) return SV_OK;
  if (!a->ctx_len || !a->cu_nodes) return fail(SV_ERR_INVALID_ARG, "ctx_len and cu_nodes are required");
  if (a->total_nodes == 0) return SV_OK;
  if (!a->q || !a->k_cache || !a->v_cache || !a->out)
    return fail(SV_ERR_INVALID_ARG, "q, k_cache, v_cache and out are required");
  if (!a->parent && !a->anc_mask) return fail(SV_ERR_INVALID_ARG, "one of parent / anc_mask is required");
  if (!aligned(a->q, 16) || !aligned(a->k_cache, 16) || !aligned(a->v_cache, 16) || !aligned(a->out, 16))
    return fail(SV_ERR_INVALID_ARG, "q, k_cache, v_cache and out must be 16-byte aligned");
  return SV_OK;
}

sv::AttnPlan plan_attn(const sv_attn_args* a) {
  sv::AttnPlan pl{};
  const int G = a->Hq / a->Hkv;
  const int rmax = G * eff_max_nodes(a->max_nodes);
  pl.mfma = a->dtype == SV_BF16;
  if (pl.mfma) {
    // 64 rows (16x16 MFMA) when every KV head has at most 64 query rows; else
    // 32x32 MFMA tiles, 256-row workgroups when every KV head fits in one,
    // otherwise 128-row workgroups
    pl.rows_per_wg = rmax <= 64 ? 64 : (rmax <= 128 || rmax > 256 ? 128 : 256);
  } else {
    pl.rows_per_wg = 8;
  }
  pl.n_rowgroups = (rmax + pl.rows_per_wg - 1) / pl.rows_per_wg;
  // with several row groups, requests with fewer rows would leave dead blocks
  // spread through the grid; they are listed out on the device instead
  pl.compact = pl.mfma && pl.n_rowgroups > 1;
  const int64_t max_splits_len = a->Lcap / 64 > 0 ? a->Lcap / 64 : 1;
  if (a->num_splits > 0) {
    pl.splits = (int)(a->num_splits < max_splits_len ? a->num_splits : max_splits_len);
  } else {
    // enough workgroups for 256 CUs, but each split keeps >= 256 keys and the
    // partial outputs it adds stay below half of the KV bytes (a quarter left
    // fp8 caches, whose KV bytes are half, one split on 128 workgroups for the
    // 60-node trees at batch 16)
    const int64_t items = (int64_t)a->B * a->Hkv * pl.n_rowgroups;
    const int64_t slots = pl.rows_per_wg > 128 ? 256 : 512;  // 8-wave workgroups: one per CU
    const int64_t want = (slots + items - 1) / (items > 0 ? items : 1);
    const int64_t by_len = a->Lcap / 256 > 0 ? a->Lcap / 256 : 1;
    const int64_t esz = a->kv_fp8 ? 1 : (a->dtype == SV_BF16 ? 2 : 4);
    const int64_t kv_bytes = 2 * (int64_t)a->B * a->Hkv * a->Lcap * a->D * esz;
    const int64_t part_bytes = 2 * (int64_t)a->total_nodes * a->Hq * (a->D + 2) * 4;
    const int64_t by_traffic = part_bytes > 0 ? kv_bytes / (2 * part_bytes) : 256;
    int64_t s = want;
    if (s > by_len) s = by_len;
    if (s > by_traffic) s = by_traffic;
    if (s > 256) s = 256;
    pl.splits = s < 1 ? 1 : (int)s;
  }
  if (a->block_table) {
    // paged caches: a split's key range spans at most 256 blocks (the block
    // ids a workgroup holds in registers); 192 per split leaves room for the
    // 64-key rounding of the range and an unaligned start
    const int64_t need = (a->max_blocks + 191) / 192;
    if (pl.splits < need) pl.splits = (int)need;
  }
  return pl;
}

struct WsLayout {
  size_t anc = 0, o_part = 0, ml_part = 0, items = 0, item_tot = 0, stats = 0, rowstats = 0, xs = 0, xcnt = 0,
         ent = 0, rtheta = 0, total = 0;
};

size_t attn_part_bytes(const sv_attn_args* a, const sv::AttnPlan& pl, size_t* ml) {
  if (pl.splits <= 1) {
    *ml = 0;
    return 0;
  }
  const size_t nh = (size_t)a->total_nodes * a->Hq;
  *ml = (size_t)pl.splits * nh * sizeof(float2);
  return (size_t)pl.splits * nh * a->D * sizeof(float);
}

int sample_nch(const sv_sample_args* s) { return (s->V + sv::kChunk - 1) / sv::kChunk; }

// does the walk make vocabulary passes (residual masses, the min-p visit pass)?
bool walk_passes(const sv_sample_args* s) {
  return s->temperature > 0.f && (s->siblings == SV_SIBLINGS_SAMPLED || s->min_p > 0.f || s->eta_eps > 0.f);
}

WsLayout layout(const sv_attn_args* a, const sv_sample_args* s) {
  WsLayout w;
  size_t off = 0;
  if (a && a->B > 0 && a->total_nodes > 0) {
    const sv::AttnPlan pl = plan_attn(a);
    if (!a->anc_mask) {
      w.anc = off;
      off += align_up((size_t)a->total_nodes * sizeof(uint64_t));
    }
    if (pl.compact) {
      w.items = off;
      off += align_up((size_t)sv::attn_grid_blocks(a->B * a->Hkv * pl.splits, pl.n_rowgroups) * sizeof(int32_t));
      w.item_tot = off;
      off += align_up(8 * sizeof(int32_t));
    }
    size_t ml = 0;
    const size_t op = attn_part_bytes(a, pl, &ml);
    if (op) {
      w.o_part = off;
      off += align_up(op);
      w.ml_part = off;
      off += align_up(ml);
    }
  }
  if (s && s->B > 0) {
    w.stats = off;
    off += align_up(((size_t)s->total_nodes + s->B) * sample_nch(s) * sizeof(sv::ChunkStat));
    w.rowstats = off;
    off += align_up(((size_t)s->total_nodes + s->B) * sizeof(sv::RowStat));
    if (s->temperature > 0.f && (s->min_p > 0.f || s->eta_eps > 0.f)) {
      w.rtheta = off;  // per-row threshold of the allowed set
      off += align_up(((size_t)s->total_nodes + s->B) * sizeof(sv::RowThr));
    }
    if (s->temperature > 0.f && s->eta_eps > 0.f) {
      w.ent = off;  // per-chunk entropy accumulators of the eta set
      off += align_up(((size_t)s->total_nodes + s->B) * sample_nch(s) * sizeof(double2));
    }
    if (walk_passes(s) && s->walk_mode != SV_WALK_SINGLE) {
      // the sliced walk's exchange buffers (reserved whenever the walk may be
      // sliced, so that the size does not depend on the device)
      w.xs = off;
      off += align_up((size_t)s->B * 4 * sample_nch(s) * sizeof(double));
      w.xcnt = off;
      off += align_up((size_t)s->B * sv::kWalkSync * sizeof(int32_t));
    }
  }
  w.total = off;
  return w;
}

// ---- sampler ---------------------------------------------------------------
sv_status check_sample(const sv_sample_args* s) {
  if (!s) return fail(SV_ERR_INVALID_ARG, "sample args is NULL");
  if (s->B < 0) return fail(SV_ERR_INVALID_ARG, "B < 0");
  if (s->V < 1 || s->V > sv::kMaxVocab) return fail(SV_ERR_UNSUPPORTED, "V must be in [1, 2^22]");
  if (s->total_nodes < 0) return fail(SV_ERR_INVALID_ARG, "total_nodes < 0");
  if (s->max_nodes < 0 || s->max_nodes > sv::kMaxNodes)
    return fail(SV_ERR_UNSUPPORTED, "max_nodes must be in [0, 64]");
  if (!(s->temperature >= 0.f) || isinf(s->temperature))
    return fail(SV_ERR_INVALID_ARG, "temperature must be finite and >= 0");
  if (s->temperature > 0.f && !isfinite(1.4426950408889634 / (double)s->temperature) )
    return fail(SV_ERR_INVALID_ARG, "temperature too small");
  if (!(s->min_p >= 0.f && s->min_p < 1.f)) return fail(SV_ERR_INVALID_ARG, "min_p must be in [0, 1)");
  if (s->siblings != SV_SIBLINGS_SAMPLED && s->siblings != SV_SIBLINGS_DETERMINISTIC)
    return fail(SV_ERR_INVALID_ARG, "siblings must be SV_SIBLINGS_SAMPLED or SV_SIBLINGS_DETERMINISTIC");
  if (!(s->eta_eps == 0.f || (s->eta_eps > 0.f && s->eta_eps < 1.f)))
    return fail(SV_ERR_INVALID_ARG, "eta_eps must be 0 or in (0, 1)");
  if (s->eta_eps > 0.f && !(s->eta_delta > 0.f && s->eta_delta <= 1.f))
    return fail(SV_ERR_INVALID_ARG, "eta_delta must be in (0, 1] when eta_eps > 0");
  if (s->eta_eps > 0.f && s->min_p > 0.f) return fail(SV_ERR_INVALID_ARG, "min_p and eta_eps are exclusive");
  if (s->rule != SV_RULE_LOSSLESS && s->rule != SV_RULE_LENIENCE && s->rule != SV_RULE_INTERPOLATION &&
      s->rule != SV_RULE_TRUNCATION)
    return fail(SV_ERR_INVALID_ARG,
                "rule must be SV_RULE_LOSSLESS, SV_RULE_LENIENCE, SV_RULE_INTERPOLATION or SV_RULE_TRUNCATION");
  if ((s->rule == SV_RULE_LENIENCE || s->rule == SV_RULE_INTERPOLATION) &&
      !(s->rule_param > 0.f && s->rule_param <= 1.f))
    return fail(SV_ERR_INVALID_ARG, "rule_param must be in (0, 1]");
  if (s->rule != SV_RULE_LOSSLESS && s->siblings == SV_SIBLINGS_DETERMINISTIC)
    return fail(SV_ERR_UNSUPPORTED, "the lossy rules need sampled siblings (they test or draw from q)");
  if (s->rule == SV_RULE_TRUNCATION && !(s->temperature > 0.f && (s->min_p > 0.f || s->eta_eps > 0.f)))
    return fail(SV_ERR_INVALID_ARG, "SV_RULE_TRUNCATION needs temperature > 0 and an allowed set (min_p or eta_eps)");
  if (s->walk_mode != SV_WALK_AUTO && s->walk_mode != SV_WALK_SINGLE && s->walk_mode != SV_WALK_SLICED)
    return fail(SV_ERR_INVALID_ARG, "walk_mode must be SV_WALK_AUTO, SV_WALK_SINGLE or SV_WALK_SLICED");
  if (s->join_ticks < -1 || s->join_ticks > 100000000)
    return fail(SV_ERR_INVALID_ARG, "join_ticks must be in [-1, 10^8]");
  if (s->step_overlap != SV_OVERLAP_OFF && s->step_overlap != SV_OVERLAP_ON)
    return fail(SV_ERR_INVALID_ARG, "step_overlap must be SV_OVERLAP_OFF or SV_OVERLAP_ON");
  const int md_needed = eff_max_nodes(s->max_nodes);
  if (s->max_depth < md_needed)
    return fail(SV_ERR_INVALID_ARG, "max_depth (%d) must be >= max_nodes (%d)", s->max_depth, md_needed);
  if (((int64_t)s->total_nodes + s->B) * (int64_t)s->V >= (1ll << 40))
    return fail(SV_ERR_UNSUPPORTED, "(N + B) * V too large");
  if (s->B == 0) return SV_OK;
  if (!s->cu_nodes || !s->target_logits || !s->accept_len || !s->accepted_nodes || !s->out_tokens)
    return fail(SV_ERR_INVALID_ARG, "cu_nodes, target_logits, accept_len, accepted_nodes, out_tokens are required");
  if (s->total_nodes > 0 && (!s->parent || !s->draft_tokens))
    return fail(SV_ERR_INVALID_ARG, "parent and draft_tokens are required when total_nodes > 0");
  if (s->temperature > 0.f && s->siblings == SV_SIBLINGS_SAMPLED && !s->draft_probs)
    return fail(SV_ERR_INVALID_ARG, "draft_probs is required when temperature > 0 with sampled siblings");
  if (s->probs_out && s->temperature == 0.f)
    return fail(SV_ERR_INVALID_ARG, "probs_out needs temperature > 0");
  if (s->probs_out && (s->min_p > 0.f || s->eta_eps > 0.f))
    return fail(SV_ERR_UNSUPPORTED, "probs_out is not available with truncation (the truncated rows are normalised "
                                    "only at the positions the walk visits)");
  if (!aligned(s->target_logits, 4) || (s->draft_probs && !aligned(s->draft_probs, 4)))
    return fail(SV_ERR_INVALID_ARG, "logit and probability rows must be 4-byte aligned");
  if (!aligned(s->uniforms_out, 8)) return fail(SV_ERR_INVALID_ARG, "uniforms_out must be 8-byte aligned");
  return SV_OK;
}

sv_status check_ws(const WsLayout& w, void* ws, size_t ws_bytes) {
  if (w.total == 0) return SV_OK;
  if (!ws) return fail(SV_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", w.total);
  if (!aligned(ws, kAlign)) return fail(SV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < w.total) return fail(SV_ERR_WORKSPACE, "workspace too small: %zu < %zu", ws_bytes, w.total);
  return SV_OK;
}

sv_status check_pack(const sv_pack_args* k) {
  if (!k) return fail(SV_ERR_INVALID_ARG, "pack args is NULL");
  if (k->B < 0 || k->B > sv::kPackMaxB) return fail(SV_ERR_UNSUPPORTED, "B must be in [0, %d]", sv::kPackMaxB);
  if (k->total_cand < 0 || k->total_cand > (1 << 24)) return fail(SV_ERR_INVALID_ARG, "total_cand must be in [0, 2^24]");
  if (k->budget < 0) return fail(SV_ERR_INVALID_ARG, "budget < 0");
  if (!k->cu_cand || !k->cu_nodes || !k->total_nodes)
    return fail(SV_ERR_INVALID_ARG, "cu_cand, cu_nodes and total_nodes are required");
  if (k->total_cand > 0 && (!k->cand_parent || !k->cand_token || !k->cand_score))
    return fail(SV_ERR_INVALID_ARG, "cand_parent, cand_token and cand_score are required when total_cand > 0");
  if (k->total_cand > 0 && k->budget > 0 && (!k->parent || !k->draft_tokens || !k->src))
    return fail(SV_ERR_INVALID_ARG, "parent, draft_tokens and src are required when something can be kept");
  return SV_OK;
}

sv_status hip_fail(hipError_t e, const char* what) {
  return fail(SV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// defer_merge: when set, the split-K merge is described there for the
// caller's next launch instead of being launched (the step runs it inside
// the walk's launch). clear_words: nclear words the launch's first workgroup
// zeroes (the step's sliced walk coordination words), or null.
sv_status run_attn(const sv_attn_args* a, char* ws, const WsLayout& w, hipStream_t st, hipEvent_t ev_start,
                   hipEvent_t ev_stop, sv::MergeArgs* defer_merge = nullptr, int32_t* clear_words = nullptr,
                   int nclear = 0) {
  if (a->B == 0 || a->total_nodes == 0) return SV_OK;
  const sv::AttnPlan pl = plan_attn(a);
  const int mn = eff_max_nodes(a->max_nodes);
  // masks built from parent when not given: by the prep kernel when the plan
  // needs it anyway (a work list), else by each attention workgroup in LDS
  const bool prep_masks = !a->anc_mask && pl.compact;
  uint64_t* w_anc = prep_masks ? (uint64_t*)(ws + w.anc) : nullptr;
  sv::AttnParams p{};
  p.B = a->B;
  p.N = a->total_nodes;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.G = a->Hq / a->Hkv;
  p.D = a->D;
  p.max_nodes = mn;
  p.Lcap = a->Lcap;
  p.ctx_len = a->ctx_len;
  p.cu_nodes = a->cu_nodes;
  p.anc = a->anc_mask ? a->anc_mask : w_anc;
  p.parent = a->parent;
  p.q = a->q;
  p.k = a->k_cache;
  p.v = a->v_cache;
  p.out = a->out;
  p.o_part = pl.splits > 1 ? (float*)(ws + w.o_part) : nullptr;
  p.ml_part = pl.splits > 1 ? (float2*)(ws + w.ml_part) : nullptr;
  p.splits = pl.splits;
  p.rows_per_wg = pl.rows_per_wg;
  p.n_rowgroups = pl.n_rowgroups;
  p.n_jobs = a->B * a->Hkv * pl.splits;
  p.items = pl.compact ? (const int32_t*)(ws + w.items) : nullptr;
  p.item_tot = pl.compact ? (const int32_t*)(ws + w.item_tot) : nullptr;
  const float scale = a->scale > 0.f ? a->scale : (float)(1.0 / sqrt((double)a->D));
  p.kv_fp8 = a->kv_fp8 != 0;
  p.v_scale = a->kv_fp8 ? a->v_scale : 1.f;
  p.scale_log2 = (float)((double)scale * (a->kv_fp8 ? (double)a->k_scale : 1.0) * 1.4426950408889634);
  p.status = a->status;
  p.clear_words = clear_words;
  p.nclear = nclear;
  p.block_table = a->block_table;
  p.block_size = a->block_table ? a->block_size : 0;
  p.max_blocks = a->block_table ? a->max_blocks : 0;
  p.num_blocks = a->block_table ? a->num_blocks : 0;
  p.bs_shift = 0;
  while (a->block_table && (1 << p.bs_shift) < a->block_size) ++p.bs_shift;
  hipError_t e = sv::launch_attn_prep(p, pl, a->parent, w_anc, st);
  if (e != hipSuccess) return hip_fail(e, "attention prep launch");
  e = sv::launch_attention(p, pl, a->dtype == SV_BF16, st, ev_start, ev_stop, defer_merge);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return SV_OK;
}

// workgroups per request of the walk (the sliced walk's coordination words
// exist in the workspace only when slicing can pay)
int walk_slices_for(const sv_sample_args* s, const WsLayout& w) {
  return w.xcnt ? sv::walk_slices(s->B, sample_nch(s), walk_passes(s), s->walk_mode) : 1;
}

// Whether the walk computes the statistics of only the rows it reaches: not
// with the p rows as an output (they need every row), and only when a
// statistics pass over every row would stream at least 128 MiB of logits.
// Below that the pass takes under 20 us at the measured 6.6 TB/s, while the
// walk's own per-row reduction adds a few microseconds of latency to every
// row a request reaches (a chain of 3-4 rows for the 8-request, 48-row
// batch: sampler 34 -> 54 us lazily; 16 requests of 61 rows: 119 -> 78 us).
constexpr double kLazyMinLogitBytes = 128.0 * 1024 * 1024;
bool walk_lazy(const sv_sample_args* s) {
  const double bytes = ((double)s->total_nodes + s->B) * (double)s->V * 4.0;
  return !s->probs_out && bytes >= kLazyMinLogitBytes;
}

sv_status run_sample(const sv_sample_args* s, char* ws, const WsLayout& w, hipStream_t st,
                     const sv::SampleEvents& ev, const sv::MergeArgs& merge = sv::MergeArgs{},
                     bool coord_cleared = false) {
  if (s->B == 0) return SV_OK;
  sv::SampleParams p{};
  p.merge = merge;
  p.B = s->B;
  p.V = s->V;
  p.N = s->total_nodes;
  p.max_nodes = eff_max_nodes(s->max_nodes);
  p.max_depth = s->max_depth;
  p.nch = sample_nch(s);
  p.cu_nodes = s->cu_nodes;
  p.parent = s->parent;
  p.tokens = s->draft_tokens;
  p.logits = s->target_logits;
  p.q = s->draft_probs;
  p.greedy = s->temperature == 0.f;
  p.c64 = p.greedy ? 0.0 : 1.4426950408889634 / (double)s->temperature;
  p.c = (float)p.c64;
  // min-p allowed set: logit - row max >= T ln min_p in fp64, from the fp32 T and min_p
  p.eta = !p.greedy && s->eta_eps > 0.f;
  p.trunc = !p.greedy && (s->min_p > 0.f || p.eta);
  p.mp_thr = sv::make_row_thr((p.trunc && !p.eta) ? (double)s->temperature * log((double)s->min_p) : 0.0);
  // eta allowed set: the per-row threshold T (ln S + min(ln eps, ln delta - H))
  // is formed by the row finalisation from these fp64 logs of the fp32 inputs
  p.temp = (double)s->temperature;
  p.ln_eps = p.eta ? log((double)s->eta_eps) : 0.0;
  p.ln_delta = p.eta ? log((double)s->eta_delta) : 0.0;
  p.ent = w.ent ? (double2*)(ws + w.ent) : nullptr;
  p.rthr = w.rtheta ? (sv::RowThr*)(ws + w.rtheta) : nullptr;
  p.seed = s->seed;
  p.step = s->step;
  p.request_id = s->request_id;
  p.accept_len = s->accept_len;
  p.accepted_nodes = s->accepted_nodes;
  p.out_tokens = s->out_tokens;
  p.probs_out = s->probs_out;
  p.uniforms_out = s->uniforms_out;
  p.residual_passes = s->residual_passes;
  p.status = s->status;
  p.stats = (sv::ChunkStat*)(ws + w.stats);
  p.rowstats = (sv::RowStat*)(ws + w.rowstats);
  p.det = s->siblings == SV_SIBLINGS_DETERMINISTIC;
  p.rule = s->rule;
  p.rule_param = s->rule_param;
  p.slices = walk_slices_for(s, w);
  p.lazy = walk_lazy(s) ? 1 : 0;
  p.coord_cleared = coord_cleared ? 1 : 0;
  p.xs = w.xcnt ? (double*)(ws + w.xs) : nullptr;
  p.xcnt = w.xcnt ? (int32_t*)(ws + w.xcnt) : nullptr;
  p.join_ticks = s->join_ticks == 0 ? sv::kJoinWindow : (s->join_ticks < 0 ? 0u : (uint32_t)s->join_ticks);
  const bool vec4 = (s->V % 4 == 0) && aligned(s->target_logits, 16) && (!s->draft_probs || aligned(s->draft_probs, 16));
  hipError_t e = sv::launch_sampler(p, vec4, st, ev);
  if (e != hipSuccess) return hip_fail(e, "sampler launch");
  return SV_OK;
}

// ---- library-owned scratch (spec_verify_step_noalloc) ----------------------
// A file-scope device array stands in for the caller's workspace. Each GPU
// holds its own copy (allocated when the code object is loaded on it, kept
// until the process ends); host code must use the address that
// hipGetSymbolAddress returns for the current device, never the array's
// name, which on the host is only a stand-in symbol.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

sv_status scratch_for_current_device(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(SV_ERR_UNSUPPORTED, "device index %d above 63", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || !aligned(ptr, kAlign)) return fail(SV_ERR_HIP, "scratch array has no usable device address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = (char*)g_scratch_ptr[dev];
  return SV_OK;
}

// ---- the step's second stream (SV_OVERLAP_ON) --------------------------------
// One non-blocking stream of default priority and two events (no timing) per
// host thread and device, created on first use and kept until the process
// ends. Per thread, so that two host threads' forks and joins never record
// into the same event.
struct ForkJoin {
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
thread_local ForkJoin g_fj[64];

sv_status fork_join_for_current_device(ForkJoin** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(SV_ERR_UNSUPPORTED, "device index %d above 63", dev);
  ForkJoin& f = g_fj[dev];
  if (!f.side) {
    hipStream_t s = nullptr;
    if ((e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking)) != hipSuccess) return hip_fail(e, "hipStreamCreate");
    hipEvent_t a = nullptr, b = nullptr;
    if ((e = hipEventCreateWithFlags(&a, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&b, hipEventDisableTiming)) != hipSuccess) {
      if (a) (void)hipEventDestroy(a);
      (void)hipStreamDestroy(s);
      return hip_fail(e, "hipEventCreate");
    }
    f.side = s;
    f.fork = a;
    f.join = b;
  }
  *out = &f;
  return SV_OK;
}

bool step_overlapped(const sv_attn_args* a, const sv_sample_args* s) {
  return s->step_overlap == SV_OVERLAP_ON && a->B > 0 && a->total_nodes > 0 && s->B > 0;
}

sv_status run_step(const sv_attn_args* attn, const sv_sample_args* sample, char* ws, const WsLayout& w,
                   hipStream_t stream, const sv_timing& t, bool allow_overlap) {
  const sv::SampleEvents sev{(hipEvent_t)t.sample_start, (hipEvent_t)t.stats_stop, (hipEvent_t)t.sample_stop};
  sv_status st;
  if (!allow_overlap || !step_overlapped(attn, sample)) {
    // the attention's split-K merge runs as extra blocks of the sampler's
    // walk launch (the sampler does not read the attention output); a sliced
    // walk without a statistics pass has its coordination words zeroed by the
    // attention launch, which always runs when there are nodes
    sv::MergeArgs merge{};
    int32_t* clear = nullptr;
    int nclear = 0;
    if (attn->B > 0 && attn->total_nodes > 0 && sample->B > 0 && w.xcnt && walk_lazy(sample) &&
        walk_slices_for(sample, w) > 1) {
      clear = (int32_t*)(ws + w.xcnt);
      nclear = sample->B * sv::kWalkSync;
    }
    if ((st = run_attn(attn, ws, w, stream, (hipEvent_t)t.attn_start, (hipEvent_t)t.attn_stop, &merge, clear,
                       nclear)) != SV_OK)
      return st;
    return run_sample(sample, ws, w, stream, sev, merge, clear != nullptr);
  }
  // the attention (with its own merge) on the side stream and the sampler on
  // the caller's, both from the call's start: they share only read-only
  // inputs and use disjoint parts of the workspace
  ForkJoin* fj = nullptr;
  if ((st = fork_join_for_current_device(&fj)) != SV_OK) return st;
  hipError_t e = hipEventRecord(fj->fork, stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord (fork)");
  if ((e = hipStreamWaitEvent(fj->side, fj->fork, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent (fork)");
  st = run_attn(attn, ws, w, fj->side, (hipEvent_t)t.attn_start, (hipEvent_t)t.attn_stop);
  if (st == SV_OK) st = run_sample(sample, ws, w, stream, sev);
  // joined even after a failed launch, so that the caller's stream never runs
  // ahead of work already on the side stream
  if ((e = hipEventRecord(fj->join, fj->side)) != hipSuccess) return hip_fail(e, "hipEventRecord (join)");
  if ((e = hipStreamWaitEvent(stream, fj->join, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent (join)");
  return st;
}

}  // namespace

extern "C" {

size_t spec_verify_workspace_size(const sv_attn_args* attn, const sv_sample_args* sample) {
  if (attn && check_attn(attn) != SV_OK) return 0;
  if (sample && check_sample(sample) != SV_OK) return 0;
  return layout(attn, sample).total;
}

sv_status spec_verify_attn(const sv_attn_args* attn, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  sv_status st = check_attn(attn);
  if (st != SV_OK) return st;
  const WsLayout w = layout(attn, nullptr);
  if ((st = check_ws(w, ws, ws_bytes)) != SV_OK) return st;
  return run_attn(attn, (char*)ws, w, (hipStream_t)stream, nullptr, nullptr);
}

sv_status spec_verify_sample(const sv_sample_args* sample, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  sv_status st = check_sample(sample);
  if (st != SV_OK) return st;
  const WsLayout w = layout(nullptr, sample);
  if ((st = check_ws(w, ws, ws_bytes)) != SV_OK) return st;
  return run_sample(sample, (char*)ws, w, (hipStream_t)stream, sv::SampleEvents{});
}

sv_status spec_verify_step_timed(const sv_attn_args* attn, const sv_sample_args* sample, void* ws, size_t ws_bytes,
                                 void* stream, const sv_timing* timing) {
  g_err[0] = 0;
  sv_status st = check_attn(attn);
  if (st != SV_OK) return st;
  if ((st = check_sample(sample)) != SV_OK) return st;
  if (attn->B != sample->B || attn->total_nodes != sample->total_nodes || attn->cu_nodes != sample->cu_nodes)
    return fail(SV_ERR_INVALID_ARG, "attn and sample args must describe the same batch (B, total_nodes, cu_nodes)");
  const WsLayout w = layout(attn, sample);
  if ((st = check_ws(w, ws, ws_bytes)) != SV_OK) return st;
  return run_step(attn, sample, (char*)ws, w, (hipStream_t)stream, timing ? *timing : sv_timing{}, true);
}

sv_status spec_verify_step(const sv_attn_args* attn, const sv_sample_args* sample, void* ws, size_t ws_bytes,
                           void* stream) {
  return spec_verify_step_timed(attn, sample, ws, ws_bytes, stream, nullptr);
}

sv_status spec_verify_step_noalloc(const sv_attn_args* attn, const sv_sample_args* sample, void* stream) {
  g_err[0] = 0;
  sv_status st = check_attn(attn);
  if (st != SV_OK) return st;
  if ((st = check_sample(sample)) != SV_OK) return st;
  const WsLayout w = layout(attn, sample);
  if (w.total > kScratchBytes)
    return fail(SV_ERR_UNSUPPORTED, "spec_verify_step_noalloc: these arguments need %zu bytes of scratch, above the "
                                    "library's %zu (64 MiB; use spec_verify_step with a caller workspace)",
                w.total, kScratchBytes);
  char* ws = nullptr;
  if ((st = scratch_for_current_device(&ws)) != SV_OK) return st;
  // the kernels write every scratch word they later read (the walk's slice
  // counters are cleared by an earlier kernel of the same call: the
  // attention launch, or the row-statistics launch), so
  // the previous call's contents need no clearing. One stream only: the
  // overlapped schedule's side stream would be created on first use.
  if (attn->B != sample->B || attn->total_nodes != sample->total_nodes || attn->cu_nodes != sample->cu_nodes)
    return fail(SV_ERR_INVALID_ARG, "attn and sample args must describe the same batch (B, total_nodes, cu_nodes)");
  return run_step(attn, sample, ws, w, (hipStream_t)stream, sv_timing{}, false);
}

sv_status spec_verify_walk_layout(const sv_sample_args* sample, int32_t* slices, int32_t* reached_rows_only) {
  g_err[0] = 0;
  sv_status st = check_sample(sample);
  if (st != SV_OK) return st;
  if (slices) *slices = walk_slices_for(sample, layout(nullptr, sample));
  if (reached_rows_only) *reached_rows_only = walk_lazy(sample) ? 1 : 0;
  return SV_OK;
}

const char* spec_verify_last_error(void) { return g_err; }

size_t spec_verify_struct_size(int32_t which) {
  if (which == 0) return sizeof(sv_attn_args);
  if (which == 1) return sizeof(sv_sample_args);
  if (which == 2) return sizeof(sv_pack_args);
  return 0;
}

size_t spec_verify_pack_workspace_size(const sv_pack_args* pk) {
  g_err[0] = 0;
  if (check_pack(pk) != SV_OK) return 0;
  return align_up((size_t)pk->total_cand * sizeof(uint64_t));
}

sv_status spec_verify_pack(const sv_pack_args* pk, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  sv_status st = check_pack(pk);
  if (st != SV_OK) return st;
  WsLayout w;
  w.total = align_up((size_t)pk->total_cand * sizeof(uint64_t));
  if ((st = check_ws(w, ws, ws_bytes)) != SV_OK) return st;
  if (pk->B == 0) return SV_OK;
  sv::PackParams p{};
  p.B = pk->B;
  p.M = pk->total_cand;
  p.cu_cand = pk->cu_cand;
  p.par = pk->cand_parent;
  p.tok = pk->cand_token;
  p.score = pk->cand_score;
  p.budget = pk->budget;
  p.cu_nodes = pk->cu_nodes;
  p.parent = pk->parent;
  p.tokens = pk->draft_tokens;
  p.src = pk->src;
  p.total = pk->total_nodes;
  p.status = pk->status;
  p.keys = (uint64_t*)ws;
  const hipError_t e = sv::launch_pack(p, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "packing launch");
  return SV_OK;
}

}  // extern "C"
