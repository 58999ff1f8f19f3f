// sv_attn.hip -- tree preprocessing and tree-masked GQA attention for gfx950.
//
// The mask follows "Speculative Decoding: Accelerating Inference Speeds in
// Distributed LLMs", section "Tree Attention Mask Mechanics": a draft node
// attends to the whole committed context, to its ancestors and to itself,
// never to another branch. GQA: query head h reads KV head h / (Hq/Hkv)
// (same page, "Interaction with Advanced Attention Architectures").
//
// Work decomposition: one workgroup per (request b, KV head g, row group,
// KV split). The rows of a workgroup are the (node j, head-in-group hh)
// pairs r = j*G + hh of one KV head, so every K/V byte fetched from HBM is
// shared by all G*T_b query rows that read it. Long contexts are cut into
// splits whose partial (max, sum, unnormalised output) are merged by a
// second kernel (flash-decoding style split-K).
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

// cache-policy operand of the buffer-load builtins for data read once: the
// non-temporal bit (streamed past the caches with low retention priority)
constexpr int kAuxNT = 2;

typedef short bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) uint16_t lds_u16_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// max over lanes l, l^16, l^32, l^48 (the four 16-lane rows of a wave) with
// the gfx950 row-swap permutes instead of LDS-routed shuffles
__device__ __forceinline__ float row_max4(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto r32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  v = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
  const uint32_t w = __float_as_uint(v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
}
__device__ __forceinline__ float row_sum4(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto r32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  v = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
  const uint32_t w = __float_as_uint(v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
}

// ---------------------------------------------------------------------------
// Tree preprocessing: ancestor-or-self bitmask of every node. One wave per
// request; lane j owns node j and climbs its parent chain with wave shuffles
// (each step must go to a strictly smaller index, so the climb ends within j
// steps). A chain that breaks that rule marks the node as a child of the root.
// Ancestor-or-self mask of node j (lane j of the wave; all 64 lanes call it)
// of a request of T nodes whose parents start at par; bad = a link that
// breaks the rule (the node is then treated as a child of the root: it sees
// the context and itself).
__device__ __forceinline__ uint64_t climb_mask(const int32_t* par, int T, int j, bool& bad) {
  const int pj = j < T ? par[j] : -1;
  uint64_t m = 1ull << j;
  int x = pj, prev = j;
  bad = false;
  for (int step = 0; step < kMaxNodes; ++step) {
    const bool act = j < T && !bad && x != -1;
    if (!__any(act)) break;
    if (act) {
      if (x < 0 || x >= prev) {
        bad = true;
      } else {
        m |= 1ull << x;
        prev = x;
      }
    }
    const bool go = act && !bad;
    const int nx = __shfl(pj, go ? x : 0);
    x = go ? nx : x;
  }
  return bad ? (1ull << j) : m;
}

__device__ __forceinline__ void tree_masks(const AttnParams& p, const int32_t* parent, uint64_t* anc, int b, int j) {
  if (b == 0 && j == 0 && p.cu_nodes[p.B] != p.N) flag(p.status, kStPacking);
  const int n0 = p.cu_nodes[b], n1 = p.cu_nodes[b + 1];
  const int T = n1 - n0;
  if (n0 < 0 || T < 0 || T > p.max_nodes || n1 > p.N) {
    if (j == 0) flag(p.status, kStPacking);
    return;
  }
  bool bad;
  const uint64_t m = climb_mask(parent + n0, T, j, bad);
  if (j < T) {
    if (bad) flag(p.status, kStTree);
    anc[n0 + j] = m;
  }
}

// The masks of one request inside an attention workgroup, when no mask
// array exists (p.anc == nullptr: the caller gave none and the plan needs
// no work list, so no prep launch ran): wave 0 climbs the parent array into
// LDS and the whole workgroup waits for it (every thread calls this). The
// request's first workgroup (report) raises the flags the prep kernel would.
__device__ __forceinline__ void masks_in_lds(const AttnParams& p, int b, int n0, int T, bool report, uint64_t* sm) {
  if (threadIdx.x < kWave) {
    const int j = threadIdx.x;
    bool bad;
    const uint64_t m = climb_mask(p.parent + n0, T, j, bad);
    if (j < T) sm[j] = m;
    if (report && __any(bad) && j == 0) flag(p.status, kStTree);
    if (report && b == 0 && j == 0 && p.cu_nodes[p.B] != p.N) flag(p.status, kStPacking);
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Work list of the bf16 grid. Blocks go to the XCDs round-robin by id, so the
// grid is decoded with the XCD class x = id % 8 fixed per job: all row groups
// of one (request, KV head, split) run on the same XCD back to back, and
// their repeated key reads are served by that XCD's L2. Without a list:
// id = ((job / 8) * n_rowgroups + rg) * 8 + job % 8. When requests differ in
// row count that grid holds blocks with no rows; they still take a turn in
// the hardware's round-robin placement over CUs, which leaves CUs idle
// (measured on MI355X: 448 of 512 workgroup slots busy for the batch-256
// super tree). attn_plan_kernel therefore lists the live items of each class
// first: block 8 k + x takes the k-th live item of class x.
__device__ __forceinline__ bool decode_block(const AttnParams& p, int lin, int& job, int& rg) {
  if (p.items) {
    const int x = lin & 7, k = lin >> 3;
    if (k >= p.item_tot[x]) return false;
    const int it = p.items[lin];
    job = it / p.n_rowgroups;
    rg = it - job * p.n_rowgroups;
  } else {
    const int qd = lin >> 3;
    rg = qd % p.n_rowgroups;
    job = (qd / p.n_rowgroups) * 8 + (lin & 7);
  }
  return job < p.n_jobs;
}

// Paged caches. Before its first tile a workgroup loads the block ids of its
// key range, up to 256 blocks (the planner splits longer ranges),
// into four VGPRs per lane (lane i of register k: block first + 64 k + i); a
// tile's id is then a v_readlane. No memory access and no wait sits on the
// path that issues a tile's loads: a table read there made every refill
// drain the loads in flight (measured on MI355X: 14-28 % slower attention
// with a scalar load per tile, 13-23 % with a window reloaded in the loop).
struct PagedIds {
  int first = 0;            // block index of lane 0 of ids[0] (uniform)
  int ids[4] = {-1, -1, -1, -1};
};

__device__ __forceinline__ void paged_load(const AttnParams& p, int b, int kb, PagedIds& pg) {
  pg.first = kb >> p.bs_shift;
  const int lane = (int)(threadIdx.x & 63);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = pg.first + 64 * k + lane;
    pg.ids[k] = idx < p.max_blocks ? p.block_table[(int64_t)b * p.max_blocks + idx] : -1;
  }
}

// element offset of logical slot t (uniform; its 64-key tile lies in one
// block) of request b, KV head g, in the pool; ok = false (flagged) for a
// block id out of range
__device__ __forceinline__ int64_t paged_slot(const AttnParams& p, int b, int g, int t, int D, bool& ok,
                                              const PagedIds& pg) {
  const int bi = (t >> p.bs_shift) - pg.first;
  const int l = bi & 63;
  const int r0 = __builtin_amdgcn_readlane(pg.ids[0], l), r1 = __builtin_amdgcn_readlane(pg.ids[1], l);
  const int r2 = __builtin_amdgcn_readlane(pg.ids[2], l), r3 = __builtin_amdgcn_readlane(pg.ids[3], l);
  const int k = bi >> 6;
  const int blk = (bi < 0 || k > 3) ? -1 : (k == 0 ? r0 : (k == 1 ? r1 : (k == 2 ? r2 : r3)));
  ok = blk >= 0 && (int64_t)blk < p.num_blocks;
  if (!ok) {
    if (threadIdx.x == 0) flag(p.status, kStBlock);
    return 0;
  }
  return ((((int64_t)blk * p.Hkv + g) << p.bs_shift) + (t & (p.block_size - 1))) * D;
}

// Buffer resource over the keys [t, min(t + 64, ke)) of a paged pool (pool:
// bf16 or fp32 elements of ESZ bytes): it reads zeros past ke, for a tile past
// the range and for a block id out of range, without touching memory.
template <int ESZ>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t paged_tile(const AttnParams& p, const void* pool, int b, int g,
                                                             int t, int ke, int D, const PagedIds& pg) {
  const int valid = min(64, ke - t);
  bool ok = false;
  const int64_t eo = valid > 0 ? paged_slot(p, b, g, t, D, ok, pg) : 0;
  return __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)pool + eo * ESZ), (short)0,
                                           ok ? valid * D * ESZ : 0, 0x00020000);
}

// Work list, built by one workgroup of 1024 threads: thread t handles XCD
// class x = t % 8 and,
// per round of 128 jobs of that class, the job 8 (m0 + t / 8) + x. A job of
// request b has ceil(G T_b / rows_per_wg) live row groups (none when the
// request's packing is invalid: every kernel skips those requests). The
// per-class exclusive prefix of those counts, in job order, places each
// job's row groups next to each other in its class list.
__device__ __forceinline__ void attn_plan(const AttnParams& p, int32_t* items, int32_t* item_tot) {
  __shared__ int32_t sc[1024];
  const int t = threadIdx.x, x = t & 7, k = t >> 3;
  const int groups = (p.n_jobs + 7) >> 3;
  const int per_req = p.Hkv * p.splits;
  int carry = 0;
  for (int m0 = 0; m0 < groups; m0 += 128) {
    const int j = 8 * (m0 + k) + x;
    int c = 0;
    if (j < p.n_jobs) {
      const int b = j / per_req;
      const int n0 = p.cu_nodes[b], n1 = p.cu_nodes[b + 1];
      const int T = n1 - n0;
      if (n0 >= 0 && T > 0 && T <= p.max_nodes && n1 <= p.N)
        c = min(p.n_rowgroups, (p.G * T + p.rows_per_wg - 1) / p.rows_per_wg);
    }
    // inclusive scan over the 128 jobs of each class (stride 8 in t)
    int v = c;
    sc[t] = v;
    __syncthreads();
    for (int s = 8; s < 1024; s <<= 1) {
      const int add = t >= s ? sc[t - s] : 0;
      __syncthreads();
      v += add;
      sc[t] = v;
      __syncthreads();
    }
    const int first = carry + v - c;
    for (int i = 0; i < c; ++i) items[8 * (first + i) + x] = j * p.n_rowgroups + i;
    carry += sc[1016 + x];  // class total of this round (thread k = 127)
    __syncthreads();        // sc is rewritten by the next round
  }
  if (k == 0) item_tot[x] = carry;
}

// Inside the step, the attention launch that precedes the walk on the stream
// also zeroes the sliced walk's per-request coordination words (its first
// workgroup, before anything else), which saves the sampler a launch.
__device__ __forceinline__ void clear_walk_words(const AttnParams& p, bool first) {
  if (p.clear_words && first)
    for (int i = threadIdx.x; i < p.nclear; i += blockDim.x) p.clear_words[i] = 0;
}

// One launch before the attention kernel: blocks [0, n_tree) build the
// ancestor masks (16 requests per block, a wave each); one more block, when
// the grid is compacted, builds the work list (it needs only the packing).
__global__ __launch_bounds__(1024) void attn_prep_kernel(AttnParams p, const int32_t* parent, uint64_t* anc,
                                                         int32_t* items, int32_t* item_tot, int n_tree) {
  if ((int)blockIdx.x < n_tree) {  // block-uniform: the tree part has no barrier
    const int b = blockIdx.x * 16 + (threadIdx.x >> 6);
    if (b < p.B) tree_masks(p, parent, anc, b, threadIdx.x & 63);
    return;
  }
  attn_plan(p, items, item_tot);
}

// ---------------------------------------------------------------------------
// bf16 path: MFMA 16x16x32 (gfx950).
//
// S^T = K Q^T is computed per 16-key x 16-row block with K as the A operand
// (keys x head-dim) and Q^T as the B operand, so the fp32 result leaves every
// lane holding 4 consecutive keys of one query row (row = lane % 16). After
// the online softmax those values are already laid out as the B operand of
// O^T = V^T P^T; V^T comes from LDS. Each lane therefore keeps the running
// max / sum of exactly one row and no transpose of P is needed.
//
// LDS tiles (64 keys), both row-major as they sit in the cache:
//   Ks [key][D]   16-byte unit u of row `key` stored at unit u ^ (key & 7);
//   Vs [key][D]   16-byte unit u of row `key` stored at unit u ^ 2 (key & 3).
// Tile writes are whole 16-byte units; the K operand is read as 16-byte
// units, the V^T operand with the gfx950 transposed reads. Both swizzles
// keep the writes and the operand reads free of bank conflicts.

// One workgroup = NW waves; wave w owns the RBW 16-row blocks
// r = row0 + 16 (w + NW i) + (lane % 16), i < RBW, of one (request, KV head,
// KV split): 16 NW RBW query rows. Every K / V fragment a wave reads from LDS
// feeds all of its row blocks. Trees with more rows than a workgroup holds
// take several row groups that stream the same keys (see decode_block).
//
// Memory pipeline: NBUF key tiles are in flight in registers (buffer loads
// issued NBUF tiles ahead); each tile is written to LDS, consumed by the
// MFMAs, and its registers are refilled with the tile NBUF positions later.
// Decode-shaped attention is bound by memory latency x bytes in flight per
// CU, and measured on MI355X several independent workgroups per CU (WPE
// waves per SIMD) hide it better than a deeper ring in fewer workgroups.
// FP8 caches (OCP E4M3, finite form): eight bytes per 16-byte LDS unit are
// loaded and widened to bf16 (every E4M3 value is exact in bf16) before the
// LDS write; k_scale is folded into the softmax scale by the host and
// v_scale multiplies the output. The rest of the kernel is unchanged.
__device__ __forceinline__ i32x4_t widen_fp8x8(i32x2_t x) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)x.x, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)x.x, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)x.y, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)x.y, 1.0f, true);
  return i32x4_t{(int)__builtin_bit_cast(uint32_t, a), (int)__builtin_bit_cast(uint32_t, b),
                 (int)__builtin_bit_cast(uint32_t, c), (int)__builtin_bit_cast(uint32_t, d)};
}

// Loads are non-temporal when the workgroup is the only reader of its key
// range (one row group per job); with several row groups (wide trees on fp8
// caches) they go through L2, where the job's other row groups, placed on the
// same XCD, find them.
template <bool FP8>
struct KvUnit {
  using T = i32x4_t;  // one 16-byte unit of bf16
  static __device__ __forceinline__ T load(__amdgpu_buffer_rsrc_t r, int off, int so, bool once) {
    return once ? __builtin_amdgcn_raw_buffer_load_b128(r, off, so, kAuxNT)
                : __builtin_amdgcn_raw_buffer_load_b128(r, off, so, 0);
  }
  static __device__ __forceinline__ i32x4_t bf16(T x) { return x; }
};
template <>
struct KvUnit<true> {
  using T = i32x2_t;  // the same unit as eight fp8 bytes
  static __device__ __forceinline__ T load(__amdgpu_buffer_rsrc_t r, int off, int so, bool once) {
    return __builtin_bit_cast(i32x2_t, once ? __builtin_amdgcn_raw_buffer_load_b64(r, off, so, kAuxNT)
                                            : __builtin_amdgcn_raw_buffer_load_b64(r, off, so, 0));
  }
  static __device__ __forceinline__ i32x4_t bf16(T x) { return widen_fp8x8(x); }
};

template <int D, int NBUF, int NW, int RBW, int WPE = 2, bool PAGED = false, bool FP8 = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPE)))
void attn_mfma_kernel(AttnParams p) {
  constexpr int ESZ = FP8 ? 1 : 2;   // bytes per cache element
  using KU = KvUnit<FP8>;
  constexpr int NT = 64 * NW;        // threads
  constexpr int KT = 64;             // keys per tile
  constexpr int KS = D / 32;         // k-steps of S^T (32 head dims each)
  constexpr int DB = D / 16;         // 16-wide blocks of the output head dim
  constexpr int UNITS = D / 8;       // 16-byte units per K row
  constexpr int ROWS = 16 * NW * RBW;
  constexpr int PER_THREAD = KT * D / 8 / NT; // K units / V items loaded per thread per tile
  static_assert(PER_THREAD >= 1 && KT * D / 8 == PER_THREAD * NT, "tile / thread split");
  __shared__ __attribute__((aligned(16))) uint16_t Ks[KT * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[KT * D];
  __shared__ uint64_t smask[kMaxNodes];  // the request's masks when no mask array exists

  int job, rg;
  clear_walk_words(p, blockIdx.x == 0);
  if (!decode_block(p, blockIdx.x, job, rg)) return;
  const int split = job % p.splits;
  const int bg = job / p.splits;
  const int g = bg % p.Hkv, b = bg / p.Hkv;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;

  const int n0 = p.cu_nodes[b], n1 = p.cu_nodes[b + 1];
  const int T = n1 - n0;
  const bool report = rg == 0 && split == 0 && g == 0;  // the request's first workgroup
  if (n0 < 0 || T < 0 || T > p.max_nodes || n1 > p.N) {  // flagged by tree prep, or here without it
    if (!p.anc && report && tid == 0) flag(p.status, kStPacking);
    return;
  }
  const int L = p.ctx_len[b];
  if (L < 0 || (int64_t)L + T > p.Lcap) {
    if (tid == 0 && rg == 0 && split == 0 && g == 0) flag(p.status, kStCtx);
    return;
  }
  const int R = p.G * T;
  const int row0 = rg * ROWS;
  if (row0 >= R) return;
  if (!p.anc) masks_in_lds(p, b, n0, T, report, smask);
  const int nkeys = L + T;
  const int kchunk = ((nkeys + p.splits - 1) / p.splits + KT - 1) / KT * KT;
  const int kb = split * kchunk;
  const int ke = min(nkeys, kb + kchunk);
  const int NH = p.N * p.Hq;

  // this wave's row blocks
  bool rb_any[RBW];
  bf16x8_t qf[RBW][KS];
  uint64_t amask[RBW];
  int orow[RBW];  // packed (node, q head) index, -1 if the row does not exist
  bool wave_any = false;
#pragma unroll
  for (int i = 0; i < RBW; ++i) {
    const int rbase = row0 + 16 * (wave + NW * i);
    rb_any[i] = rbase < R;
    wave_any |= rb_any[i];
    const int r = rbase + l16;
    amask[i] = 0;
    orow[i] = -1;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[i][ks] = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    if (r < R) {
      const int j = r / p.G, hh = r - j * p.G;
      orow[i] = (n0 + j) * p.Hq + g * p.G + hh;
      amask[i] = p.anc ? p.anc[n0 + j] : smask[j];
      const uint16_t* qp = (const uint16_t*)p.q + (int64_t)orow[i] * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[i][ks] = *(const bf16x8_t*)(qp + 32 * ks + 8 * g4);
    }
  }

  if (kb >= ke) {  // empty split: contributes nothing to the merge
#pragma unroll
    for (int i = 0; i < RBW; ++i)
      if (orow[i] >= 0 && g4 == 0) p.ml_part[(int64_t)split * NH + orow[i]] = make_float2(-INFINITY, 0.f);
    return;
  }

  const int64_t head_off = PAGED ? 0 : ((int64_t)b * p.Hkv + g) * p.Lcap * D;  // paged: per tile instead
  const char* kbase = (const char*)p.k + head_off * ESZ;
  const char* vbase = (const char*)p.v + head_off * ESZ;

  // K/V tiles come in through buffer loads: the resource covers exactly the
  // keys [0, ke) of this (request, KV head), so a key past the split end reads
  // as zero (never a stray cache slot), and the per-thread offsets are 32-bit
  // constants with the tile start in the scalar offset.
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, ke * D * ESZ, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, ke * D * ESZ, 0x00020000);
  int koff[PER_THREAD];  // K and V share the per-thread offsets (16-byte unit c of the tile)
#pragma unroll
  for (int i = 0; i < PER_THREAD; ++i) {
    const int c = tid + NT * i;
    koff[i] = ((c / UNITS) * D + 8 * (c % UNITS)) * ESZ;
  }
  typename KU::T kreg[NBUF][PER_THREAD];
  typename KU::T vreg[NBUF][PER_THREAD];
  // V^T operand addressing for the transposed LDS reads (see the PV step)
  const int vt_lane = (4 * g4 + (l16 >> 2)) * D + 4 * (l16 & 1) + 8 * ((l16 >> 1) & 1);
  const int vt_sw = l16 >> 2;

  f32x4_t o[RBW][DB];
  float m[RBW], l[RBW];
#pragma unroll
  for (int i = 0; i < RBW; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[i][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // prologue: the first NBUF tiles. Every load is non-temporal: this kernel
  // serves at most 64 rows per KV head, so each key range has one reader
  // (measured on MI355X: 11 % faster on 32k-token contexts). Paged caches:
  // one resource per tile, over that tile's block rows.
  PagedIds pg;
  if (PAGED) paged_load(p, b, kb, pg);
  const bool once = R <= ROWS;  // the only reader of this key range
#pragma unroll
  for (int s = 0; s < NBUF; ++s) {
    const int so = PAGED ? 0 : (kb + s * KT) * D * ESZ;
    const __amdgpu_buffer_rsrc_t kr = PAGED ? paged_tile<ESZ>(p, p.k, b, g, kb + s * KT, ke, D, pg) : krs;
    const __amdgpu_buffer_rsrc_t vr = PAGED ? paged_tile<ESZ>(p, p.v, b, g, kb + s * KT, ke, D, pg) : vrs;
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      kreg[s][i] = KU::load(kr, koff[i], so, once);
      vreg[s][i] = KU::load(vr, koff[i], so, once);
    }
    // keep the slots' loads in slot order, as the ring refills them: the
    // wait before writing slot s can then leave the later slots in flight
    __builtin_amdgcn_sched_barrier(0);
  }

  for (int tb = kb; tb < ke; tb += NBUF * KT) {
#pragma unroll
    for (int s = 0; s < NBUF; ++s) {
      const int t0 = tb + s * KT;
      __syncthreads();  // the previous tile's LDS reads are done
#pragma unroll
      for (int i = 0; i < PER_THREAD; ++i) {
        const int c = tid + NT * i;
        const int kk = c / UNITS, dc = c % UNITS;
        *(i32x4_t*)(Ks + kk * D + 8 * (dc ^ (kk & 7))) = KU::bf16(kreg[s][i]);
        *(i32x4_t*)(Vs + kk * D + 8 * (dc ^ (2 * (kk & 3)))) = KU::bf16(vreg[s][i]);
      }
      __syncthreads();
      // refill this ring slot with the tile NBUF positions ahead
      {
        const int so = PAGED ? 0 : (t0 + NBUF * KT) * D * ESZ;
        const __amdgpu_buffer_rsrc_t kr = PAGED ? paged_tile<ESZ>(p, p.k, b, g, t0 + NBUF * KT, ke, D, pg) : krs;
        const __amdgpu_buffer_rsrc_t vr = PAGED ? paged_tile<ESZ>(p, p.v, b, g, t0 + NBUF * KT, ke, D, pg) : vrs;
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
          kreg[s][i] = KU::load(kr, koff[i], so, once);
          vreg[s][i] = KU::load(vr, koff[i], so, once);
        }
      }
      // past the range (last ring round): the slot was only cycled; waves
      // without rows only help to stream the tiles
      if (t0 >= ke || !wave_any) continue;
      const bool full = (t0 + KT <= ke) && (t0 + KT <= L);

      // S^T for every row block of the wave; each K fragment is read once
      f32x4_t sc[RBW][4];
#pragma unroll
      for (int i = 0; i < RBW; ++i)
#pragma unroll
        for (int st = 0; st < 4; ++st) sc[i][st] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int key = 16 * st + l16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8_t a = *(const bf16x8_t*)(Ks + key * D + 8 * ((4 * ks + g4) ^ (key & 7)));
#pragma unroll
          for (int i = 0; i < RBW; ++i)
            if (rb_any[i]) sc[i][st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[i][ks], sc[i][st], 0, 0, 0);
        }
      }

      // online softmax in the log2 domain: p = 2^(s * scale_log2 - m), the
      // scale folded into one FMA, raw v_exp_f32 (arguments are <= 0, so only
      // denormal results flush, which softmax weights below 2^-126 afford)
      bf16x8_t pk[RBW][2];
#pragma unroll
      for (int i = 0; i < RBW; ++i) {
        if (!rb_any[i]) continue;
        float x[16];
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int e = 0; e < 4; ++e) x[4 * st + e] = sc[i][st][e];
        if (!full) {  // wave-uniform: only tiles that reach the draft slots or the split end
          // visibility of the tile's 64 keys for this lane's row, built
          // without branches: context keys, then the row's ancestor-or-self
          // draft slots, cut at the split end (the short-circuit form of this
          // test was miscompiled by the ROCm 7.2 compiler under some register
          // budgets)
          const int dl = L - t0;  // tile bit of the first draft slot
          const uint64_t ctx_bits = dl >= 64 ? ~0ull : (dl <= 0 ? 0ull : ((1ull << dl) - 1ull));
          const uint64_t drf_bits =
              dl >= 64 ? 0ull : (dl >= 0 ? (amask[i] << dl) : (-dl >= 64 ? 0ull : (amask[i] >> -dl)));
          const int dv = ke - t0;
          const uint64_t valid = dv >= 64 ? ~0ull : ((1ull << dv) - 1ull);
          const uint64_t lane_bits = ((ctx_bits | drf_bits) & valid) >> (4 * g4);
#pragma unroll
          for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const bool vis = (lane_bits >> (16 * st + e)) & 1ull;
              x[4 * st + e] = vis ? x[4 * st + e] : -INFINITY;
            }
        }
        float mx = x[0];
#pragma unroll
        for (int t = 1; t < 16; ++t) mx = fmaxf(mx, x[t]);
        // the row's 64 keys live in lanes l16, l16+16, l16+32, l16+48
        mx = row_max4(mx);
        // the reference maximum moves only by more than 8 (log2), as in the
        // 32x32 kernel: exponentials stay below 2^8 and most rescales go
        float mnew = fmaxf(m[i], mx * p.scale_log2);
        if (!__any(mnew > m[i] + 8.f)) mnew = m[i];
        const float msub = mnew == -INFINITY ? 0.f : mnew;
        float lsum = 0.f;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          x[t] = __builtin_amdgcn_exp2f(fmaf(x[t], p.scale_log2, -msub));
          lsum += x[t];
        }
        // rescale the running output only when some row's maximum moved
        if (__any(mnew != m[i])) {
          const float alpha = __builtin_amdgcn_exp2f(m[i] - msub);  // m = -inf (nothing seen yet) -> 0
          l[i] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) o[i][db] *= alpha;
        }
        l[i] += lsum;
        m[i] = mnew;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          // element 4h + e  <->  sub-tile st = 2 k2 + h, value e (RNE by v_cvt_pk_bf16_f32)
          const float* lo = x + 4 * (2 * k2);
          const float* hi = x + 4 * (2 * k2 + 1);
          const bf16x2_t p01 = {(__bf16)lo[0], (__bf16)lo[1]}, p23 = {(__bf16)lo[2], (__bf16)lo[3]};
          const bf16x2_t p45 = {(__bf16)hi[0], (__bf16)hi[1]}, p67 = {(__bf16)hi[2], (__bf16)hi[3]};
          const i32x4_t wv = {(int)__builtin_bit_cast(uint32_t, p01), (int)__builtin_bit_cast(uint32_t, p23),
                              (int)__builtin_bit_cast(uint32_t, p45), (int)__builtin_bit_cast(uint32_t, p67)};
          pk[i][k2] = __builtin_bit_cast(bf16x8_t, wv);
        }
      }

      // O^T += V^T P^T; each V fragment is read once for all row blocks.
      // The V^T operand (lane l: head dim 16 db + l % 16, keys 32 k2 + 16 h +
      // 4 (l / 16) + e for h = 0, 1 and e = 0..3, the key order of pk) comes
      // straight from the row-major V tile through two ds_read_b64_tr_b16:
      // in each 16-lane group, lane j points at the 4 head dims
      // 16 db + 4 (j % 4) .. + 3 of key base + j / 4, and lane i receives
      // element i % 4 of lanes i / 4, 4 + i / 4, 8 + i / 4, 12 + i / 4, i.e.
      // keys base .. base + 3 of head dim 16 db + i.
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int base = (32 * k2) * D + vt_lane + 16 * (db ^ vt_sw);
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds_u16_t*)(Vs + base));
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds_u16_t*)(Vs + base + 16 * D));
          const bf16x8_t a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int i = 0; i < RBW; ++i)
            if (rb_any[i]) o[i][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pk[i][k2], o[i][db], 0, 0, 0);
        }
      }
    }
  }

  // row sums across the four lane groups that share a row, then write
#pragma unroll
  for (int i = 0; i < RBW; ++i) {
    if (!rb_any[i]) continue;
    const float lt = row_sum4(l[i]);
    if (orow[i] < 0) continue;
    if (p.splits == 1) {
      const float inv = (FP8 ? p.v_scale : 1.0f) / lt;
      float* op = p.out + (int64_t)orow[i] * D + 4 * g4;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4_t v = o[i][db] * inv;
        *(float4*)(op + 16 * db) = make_float4(v[0], v[1], v[2], v[3]);
      }
    } else {
      float* op = p.o_part + ((int64_t)split * NH + orow[i]) * D + 4 * g4;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4_t v = FP8 ? o[i][db] * p.v_scale : o[i][db];
        *(float4*)(op + 16 * db) = make_float4(v[0], v[1], v[2], v[3]);
      }
      if (g4 == 0) p.ml_part[(int64_t)split * NH + orow[i]] = make_float2(m[i], lt);
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 path with 32x32 MFMA tiles (v_mfma_f32_32x32x16_bf16): every wave owns
// 32 query rows, so each K / V fragment read from LDS feeds twice as many rows
// as with 16x16 tiles at the same register cost per row.
//
// S^T = K Q^T per 32-key block: lane l holds keys 8 (v / 4) + 4 (l / 32) +
// v % 4 (v = 0..15) of row l % 32. For the PV contraction the 64 keys of a
// tile are taken in k-steps kk of 16: lane half h = l / 32 contributes keys
// 16 kk + 4 h + 0..3 and 16 kk + 8 + 4 h + 0..3, exactly elements
// 8 (kk % 2) .. + 7 of its score block kk / 2, so P^T needs no shuffle; the
// V^T operand is read in the same key order with transposed LDS reads.
// O^T per 32-dim block db: lane l holds dims 32 db + 8 (v / 4) + 4 h + v % 4
// of row l % 32.
template <int D, int NW, int WPE, bool PAGED = false, bool FP8 = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPE)))
void attn_mfma32_kernel(AttnParams p) {
  constexpr int NT = 64 * NW;        // threads
  constexpr int KT = 64;             // keys per tile
  constexpr int KS = D / 16;         // k-steps of S^T (16 head dims each)
  constexpr int DB = D / 32;         // 32-wide blocks of the output head dim
  constexpr int UNITS = D / 8;       // 16-byte units per K / V row
  constexpr int ROWS = 32 * NW;
  constexpr int PER_THREAD = KT * UNITS / NT;  // 16-byte units per thread per K or V tile
  static_assert(PER_THREAD >= 1 && KT * UNITS == PER_THREAD * NT, "tile / thread split");
  constexpr int ESZ = FP8 ? 1 : 2;   // bytes per cache element
  // two LDS buffers each for K and V, as four arrays so that the compiler can
  // tell the buffer being filled from the one being read
  __shared__ __attribute__((aligned(16))) uint16_t Ks0[KT * D];
  __shared__ __attribute__((aligned(16))) uint16_t Ks1[KT * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs0[KT * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs1[KT * D];
  __shared__ uint64_t smask[kMaxNodes];  // the request's masks when no mask array exists
  // LDS swizzles. K: 16-byte unit u of row `key` at u ^ (key & 15) for
  // D = 128 (u ^ (key & 7) for D = 64), so the 16 keys that one 256-byte read
  // pass serves hit 16 different units. V: 16-byte unit u at u ^ VSW (key & 3).
  // A transposed read spans four keys (key & 3) and, per 32-lane half, two
  // logical 32-byte chunks; with VSW = 4 for D = 128 those eight (key,
  // chunk) pairs sit in eight different chunks of the 256-byte bank row, so
  // the read is free of bank conflicts (u ^ 2 (key & 3) left two of them per
  // chunk: 2-way conflicts on every V read). D = 64 rows are 128 bytes and
  // alternate bank halves, so u ^ 2 (key & 3) suffices there.
  constexpr int KSWM = D >= 128 ? 15 : 7;
  constexpr int VSW = D >= 128 ? 4 : 2;

  int job, rg;
  clear_walk_words(p, blockIdx.x == 0);
  if (!decode_block(p, blockIdx.x, job, rg)) return;
  const int split = job % p.splits;
  const int bg = job / p.splits;
  const int g = bg % p.Hkv, b = bg / p.Hkv;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;

  const int n0 = p.cu_nodes[b], n1 = p.cu_nodes[b + 1];
  const int T = n1 - n0;
  const bool report = rg == 0 && split == 0 && g == 0;  // the request's first workgroup
  if (n0 < 0 || T < 0 || T > p.max_nodes || n1 > p.N) {  // flagged by tree prep, or here without it
    if (!p.anc && report && tid == 0) flag(p.status, kStPacking);
    return;
  }
  const int L = p.ctx_len[b];
  if (L < 0 || (int64_t)L + T > p.Lcap) {
    if (tid == 0 && rg == 0 && split == 0 && g == 0) flag(p.status, kStCtx);
    return;
  }
  const int R = p.G * T;
  const int row0 = rg * ROWS;
  if (row0 >= R) return;
  if (!p.anc) masks_in_lds(p, b, n0, T, report, smask);
  const int nkeys = L + T;
  const int kchunk = ((nkeys + p.splits - 1) / p.splits + KT - 1) / KT * KT;
  const int kb = split * kchunk;
  const int ke = min(nkeys, kb + kchunk);
  const int NH = p.N * p.Hq;

  // the 32 rows of this wave: r = row0 + 32 wave + l32
  const int rbase = row0 + 32 * wave;
  const bool wave_any = rbase < R;
  const int r = rbase + l32;
  bf16x8_t qf[KS];
  uint64_t amask = 0;
  int orow = -1;  // packed (node, q head) index, -1 if the row does not exist
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
  if (r < R) {
    const int j = r / p.G, hh = r - j * p.G;
    orow = (n0 + j) * p.Hq + g * p.G + hh;
    amask = p.anc ? p.anc[n0 + j] : smask[j];
    const uint16_t* qp = (const uint16_t*)p.q + (int64_t)orow * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const bf16x8_t*)(qp + 16 * ks + 8 * h);
  }

  if (kb >= ke) {  // empty split: contributes nothing to the merge
    if (orow >= 0 && h == 0) p.ml_part[(int64_t)split * NH + orow] = make_float2(-INFINITY, 0.f);
    return;
  }

  const int64_t head_off = PAGED ? 0 : ((int64_t)b * p.Hkv + g) * p.Lcap * D;  // paged: per tile instead
  const char* kbase = (const char*)p.k + head_off * ESZ;
  const char* vbase = (const char*)p.v + head_off * ESZ;
  // the resources cover exactly keys [0, ke): a key past the split end reads
  // as zero without touching memory, and so does a whole tile past the range
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, ke * D * ESZ, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, ke * D * ESZ, 0x00020000);
  // Tiles go from HBM straight into LDS (16-byte buffer loads with the LDS
  // flag: lane i of a wave instruction fills the 16 bytes at the instruction's
  // LDS base + 16 i). Thread c = tid + NT i fills unit c of a tile, row
  // kk = c / UNITS, slot u = c % UNITS, with the global unit the reads expect
  // in that slot: K unit u ^ (kk & KSWM), V unit u ^ VSW (kk & 3). The tile
  // start goes into the per-lane offset, so the bounds check covers it.
  int koff[PER_THREAD], voff[PER_THREAD];
#pragma unroll
  for (int i = 0; i < PER_THREAD; ++i) {
    const int c = tid + NT * i;
    const int kk = c / UNITS, u = c % UNITS;
    koff[i] = (kk * D + 8 * (u ^ (kk & KSWM))) * 2;
    voff[i] = (kk * D + 8 * (u ^ (VSW * (kk & 3)))) * 2;
  }
  const int wunit = 64 * wave;  // first tile unit this wave's instructions fill
  // When this workgroup is the only reader of its slab range (the job has a
  // single row group) the tiles are loaded non-temporally; otherwise the
  // other row groups' workgroups on the same XCD find them in L2. (Measured
  // on MI355X: non-temporal everywhere slowed the batch-256 super tree by
  // 6 %, whose larger trees have two to four row groups.)
  const bool stream_once = R <= ROWS;
  // (paged caches: a resource over the tile's block rows, built per tile)
  PagedIds pg;
  if (PAGED) paged_load(p, b, kb, pg);
  auto dma = [&](__amdgpu_buffer_rsrc_t rs, const void* pool, const int* off, uint16_t* dst, int t) {
    int tb = (kb + t * KT) * D * 2;
    if (PAGED) {
      rs = paged_tile<ESZ>(p, pool, b, g, kb + t * KT, ke, D, pg);
      tb = 0;
    }
    if (stream_once) {
#pragma unroll
      for (int i = 0; i < PER_THREAD; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + 8 * (wunit + NT * i)), 16,
                                                 (unsigned)(off[i] + tb), 0, 0, kAuxNT);
    } else {
#pragma unroll
      for (int i = 0; i < PER_THREAD; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + 8 * (wunit + NT * i)), 16,
                                                 (unsigned)(off[i] + tb), 0, 0, 0);
    }
  };
  // FP8 caches: no LDS DMA (it cannot widen). Thread c loads the eight fp8
  // bytes of unit c of a tile (row kk = c / UNITS, head dims 8 u .. 8 u + 7,
  // u = c % UNITS) into registers, widens them to bf16 (every E4M3 value is
  // exact in bf16) and writes them to the LDS slot the DMA would have filled
  // with that unit: u ^ (kk & KSWM) for K, u ^ VSW (kk & 3) for V (the XOR
  // swizzle is its own inverse). The reads and MFMAs are those of bf16.
  i32x2_t k8[FP8 ? PER_THREAD : 1], v8[FP8 ? PER_THREAD : 1];
  auto fetch8 = [&](__amdgpu_buffer_rsrc_t rs, const void* pool, i32x2_t* dst, int t) {
    int tb = (kb + t * KT) * D;
    if (PAGED) {
      rs = paged_tile<1>(p, pool, b, g, kb + t * KT, ke, D, pg);
      tb = 0;
    }
    if (stream_once) {
#pragma unroll
      for (int i = 0; i < PER_THREAD; ++i) {
        const int c = tid + NT * i;
        dst[i] = __builtin_bit_cast(
            i32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rs, (c / UNITS) * D + 8 * (c % UNITS), tb, kAuxNT));
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER_THREAD; ++i) {
        const int c = tid + NT * i;
        dst[i] = __builtin_bit_cast(i32x2_t,
                                    __builtin_amdgcn_raw_buffer_load_b64(rs, (c / UNITS) * D + 8 * (c % UNITS), tb, 0));
      }
    }
  };
  auto store8 = [&](const i32x2_t* src, uint16_t* lds, bool is_v) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int c = tid + NT * i;
      const int kk = c / UNITS, u = c % UNITS;
      const int slot = is_v ? (u ^ (VSW * (kk & 3))) : (u ^ (kk & KSWM));
      *(i32x4_t*)(lds + kk * D + 8 * slot) = widen_fp8x8(src[i]);
    }
  };
  // V^T operand addressing: lane l of 16-lane group G = l / 16 reads the head
  // dims 16 (G % 2) + 4 (l % 4) .. + 3 of key base + (l % 16) / 4
  const int lg = lane & 15, G = lane >> 4;
  const int vt_s = lg >> 2, vt_dg = G & 1;
  const int vt_lane = (4 * (G >> 1) + vt_s) * D + 4 * (lg & 1) + 8 * ((lg >> 1) & 1);

  f32x16_t o[DB];
  float m = -INFINITY, l = 0.f;
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16_t{};

  // S^T of one tile, two 32-key blocks
  auto s_tile = [&](const uint16_t* Kb, f32x16_t* sc) {
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
      sc[kq] = f32x16_t{};
      const int key = 32 * kq + l32;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t a = *(const bf16x8_t*)(Kb + key * D + 8 * ((2 * ks + h) ^ (key & KSWM)));
        sc[kq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sc[kq], 0, 0, 0);
      }
    }
  };

  // Tile t's online softmax (log2 domain, as in the 16x16 kernel) with
  // S_{t+1} = K_{t+1} Q^T issued in four groups of four MFMAs between its
  // steps, then O^T += V^T P^T in four 16-key steps. The S MFMAs do not
  // depend on the softmax, so the MFMA pipe works on them while the VALU
  // runs the max and the exponentials (the compiler keeps this order; an
  // explicit one-MFMA-then-VALU scheduling pattern measured ~1 % slower).
  auto softmax_s_pv = [&](f32x16_t* sc, f32x16_t* sn, const uint16_t* Knxt, const uint16_t* Vb, int t) {
    const int t0 = kb + t * KT;
    if (!((t0 + KT <= ke) && (t0 + KT <= L))) {  // wave-uniform: tiles that reach the draft slots or the split end
      const int dl = L - t0;
      const uint64_t ctx_bits = dl >= 64 ? ~0ull : (dl <= 0 ? 0ull : ((1ull << dl) - 1ull));
      const uint64_t drf_bits = dl >= 64 ? 0ull : (dl >= 0 ? (amask << dl) : (-dl >= 64 ? 0ull : (amask >> -dl)));
      const int dv = ke - t0;
      const uint64_t valid = dv >= 64 ? ~0ull : ((1ull << dv) - 1ull);
      const uint64_t lane_bits = ((ctx_bits | drf_bits) & valid) >> (4 * h);
#pragma unroll
      for (int kq = 0; kq < 2; ++kq)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const bool vis = (lane_bits >> (32 * kq + 8 * (v >> 2) + (v & 3))) & 1ull;
          sc[kq][v] = vis ? sc[kq][v] : -INFINITY;
        }
    }
    // K_{t+1} fragments (a tile past the range was filled with zeros)
    bf16x8_t ka[2][KS];
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
      const int key = 32 * kq + l32;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        ka[kq][ks] = *(const bf16x8_t*)(Knxt + key * D + 8 * ((2 * ks + h) ^ (key & KSWM)));
    }
    auto s_group = [&](int q) {  // MFMAs 4q .. 4q + 3 of S_{t+1} (each chain starts from zero)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int idx = 4 * q + j, kq = idx / KS, ks = idx % KS;
        sn[kq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kq][ks], qf[ks], ks == 0 ? f32x16_t{} : sn[kq], 0, 0,
                                                         0);
      }
    };
    static_assert(2 * KS % 4 == 0, "S MFMAs come in groups of four");
    constexpr int NG = 2 * KS / 4;  // groups: 4 for D = 128, 2 for D = 64
    s_group(0);
    float mx = sc[0][0];
#pragma unroll
    for (int kq = 0; kq < 2; ++kq)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[kq][v]);
    {
      // the row's other 32 keys are in lane l ^ 32
      const uint32_t u = __float_as_uint(mx);
      const auto r32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      mx = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
    }
    // The reference maximum moves only when some row's maximum exceeds it by
    // more than 8 (log2 units): until then the exponentials stay below 2^8,
    // exact to bf16's relative precision, and the rescale of O (64
    // multiplies per lane) is skipped. The result is the same softmax.
    // (Measured on MI355X: C3 attention 90 -> 84.5 us, C5 437 -> 419 us.)
    float mnew = fmaxf(m, mx * p.scale_log2);
    if (!__any(mnew > m + 8.f)) mnew = m;
    const float msub = mnew == -INFINITY ? 0.f : mnew;
    if (NG > 1) s_group(1 % NG);
    float lsum = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      sc[0][v] = __builtin_amdgcn_exp2f(fmaf(sc[0][v], p.scale_log2, -msub));
      lsum += sc[0][v];
    }
    if (NG > 2) s_group(2 % NG);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      sc[1][v] = __builtin_amdgcn_exp2f(fmaf(sc[1][v], p.scale_log2, -msub));
      lsum += sc[1][v];
    }
    if (NG > 3) s_group(3 % NG);
    if (__any(mnew != m)) {
      const float alpha = __builtin_amdgcn_exp2f(m - msub);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }
    l += lsum;
    m = mnew;
    // The wave issues its PV MFMAs at raised priority, so that the SIMD's
    // other wave, if it is in its softmax, runs its VALU work beside them
    // rather than in step with this wave. In eight-wave workgroups the two
    // waves of a SIMD are waves w and w + 4: only the upper one raises its
    // priority. (Measured on MI355X: C5 attention 432 -> 424 us, C3 even;
    // raising it during the softmax instead, or on both waves of an eight-wave
    // SIMD, was slower.)
    const bool pv_prio = NW == 4 || wave >= 4;
    if (pv_prio) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int kq = kk >> 1, v0 = 8 * (kk & 1);
      const bf16x2_t p01 = {(__bf16)sc[kq][v0 + 0], (__bf16)sc[kq][v0 + 1]};
      const bf16x2_t p23 = {(__bf16)sc[kq][v0 + 2], (__bf16)sc[kq][v0 + 3]};
      const bf16x2_t p45 = {(__bf16)sc[kq][v0 + 4], (__bf16)sc[kq][v0 + 5]};
      const bf16x2_t p67 = {(__bf16)sc[kq][v0 + 6], (__bf16)sc[kq][v0 + 7]};
      const i32x4_t wv = {(int)__builtin_bit_cast(uint32_t, p01), (int)__builtin_bit_cast(uint32_t, p23),
                          (int)__builtin_bit_cast(uint32_t, p45), (int)__builtin_bit_cast(uint32_t, p67)};
      const bf16x8_t pk = __builtin_bit_cast(bf16x8_t, wv);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int base = (16 * kk) * D + vt_lane + 16 * ((2 * db + vt_dg) ^ ((VSW / 2) * vt_s));
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds_u16_t*)(Vb + base));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds_u16_t*)(Vb + base + 8 * D));
        const bf16x8_t a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk, o[db], 0, 0, 0);
      }
    }
    if (pv_prio) __builtin_amdgcn_s_setprio(0);
  };

  // Pipeline: K runs one tile ahead of V. At the top of iteration t the loads
  // of K_{t+1} and V_t are in flight and S_t is in registers; after one wait
  // and one barrier, K_{t+2} and V_{t+1} are issued into the buffers freed by
  // K_t and V_{t-1}, then S_{t+1} is computed while tile t's softmax and PV
  // run (the S MFMAs do not depend on the softmax, so the two can co-issue).
  const int nt = (ke - kb + KT - 1) / KT;
  f32x16_t sc[2], sn[2];
  if constexpr (FP8) {
    fetch8(krs, p.k, k8, 0);
    store8(k8, Ks0, false);
    __syncthreads();
    fetch8(krs, p.k, k8, 1);
    fetch8(vrs, p.v, v8, 0);
    if (wave_any) s_tile(Ks0, sc);
    store8(k8, Ks1, false);
    store8(v8, Vs0, true);
  } else {
    dma(krs, p.k, koff, Ks0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    dma(krs, p.k, koff, Ks1, 1);
    dma(vrs, p.v, voff, Vs0, 0);
    if (wave_any) s_tile(Ks0, sc);
  }
  // one iteration; cur / nxt are the buffers of tiles t and t + 1 (S of the
  // tile after the last one is computed on the zeros the range check left in
  // its buffer and never used)
  // (scores of tile t in scur, tile t + 1 computed into snxt; the two sets
  // swap roles from one iteration to the next)
  auto step = [&](int t, uint16_t* Kcur, uint16_t* Knxt, uint16_t* Vcur, uint16_t* Vnxt, f32x16_t* scur,
                  f32x16_t* snxt) {
    if constexpr (FP8) {
      // K_{t+1} and V_t were written to LDS at the end of the last step; K_t
      // and V_{t-1} are no longer read once everyone is past the barrier, so
      // K_{t+2} and V_{t+1} go there after this step's work (their loads fly
      // meanwhile)
      __syncthreads();
      fetch8(krs, p.k, k8, t + 2);
      fetch8(vrs, p.v, v8, t + 1);
      if (wave_any) softmax_s_pv(scur, snxt, Knxt, Vcur, t);
      store8(k8, Kcur, false);
      store8(v8, Vnxt, true);
      return;
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of K_{t+1} and V_t have landed
    __syncthreads();                // everyone's have; K_t and V_{t-1} are no longer read
    dma(krs, p.k, koff, Kcur, t + 2);
    dma(vrs, p.v, voff, Vnxt, t + 1);
    if (!wave_any) return;          // waves without rows only help to stream the tiles
    softmax_s_pv(scur, snxt, Knxt, Vcur, t);
  };
  for (int t = 0; t < nt; t += 2) {
    step(t, Ks0, Ks1, Vs0, Vs1, sc, sn);
    if (t + 1 < nt) step(t + 1, Ks1, Ks0, Vs1, Vs0, sn, sc);
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load into LDS outlives the workgroup

  if (!wave_any) return;
  float lt;
  {
    const uint32_t u = __float_as_uint(l);
    const auto r32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    lt = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
  }
  if (orow < 0) return;
  if (p.splits == 1) {
    const float inv = (FP8 ? p.v_scale : 1.0f) / lt;
    float* op = p.out + (int64_t)orow * D + 4 * h;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g8 = 0; g8 < 4; ++g8)
        *(float4*)(op + 32 * db + 8 * g8) = make_float4(o[db][4 * g8] * inv, o[db][4 * g8 + 1] * inv,
                                                        o[db][4 * g8 + 2] * inv, o[db][4 * g8 + 3] * inv);
  } else {
    float* op = p.o_part + ((int64_t)split * NH + orow) * D + 4 * h;
    const float vs = FP8 ? p.v_scale : 1.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g8 = 0; g8 < 4; ++g8)
        *(float4*)(op + 32 * db + 8 * g8) = make_float4(o[db][4 * g8] * vs, o[db][4 * g8 + 1] * vs,
                                                        o[db][4 * g8 + 2] * vs, o[db][4 * g8 + 3] * vs);
    if (h == 0) p.ml_part[(int64_t)split * NH + orow] = make_float2(m, lt);
  }
}

// ---------------------------------------------------------------------------
// fp32 path (plain VALU): 8 query rows per workgroup, 32-key tiles in LDS.
// Thread t handles row t/32 and, per tile, key t%32 for the scores and head
// dims t%32 + 32k for the output.
template <int D, bool PAGED = false>
__global__ __launch_bounds__(256) void attn_valu_kernel(AttnParams p) {
  clear_walk_words(p, blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0);
  constexpr int KT = 32, RW = 8, DPT = D / 32;
  __shared__ float Qs[RW][D];
  __shared__ float Ks[KT][D + 1];
  __shared__ float Vs[KT][D];
  __shared__ float Ps[RW][KT];

  __shared__ uint64_t smask[kMaxNodes];  // the request's masks when no mask array exists
  const int b = blockIdx.z, g = blockIdx.y;
  const int rg = blockIdx.x / p.splits, split = blockIdx.x % p.splits;
  const int tid = threadIdx.x, rl = tid >> 5, kl = tid & 31;
  const int n0 = p.cu_nodes[b], n1 = p.cu_nodes[b + 1];
  const int T = n1 - n0;
  const bool report = blockIdx.x == 0 && g == 0;  // the request's first workgroup
  if (n0 < 0 || T < 0 || T > p.max_nodes || n1 > p.N) {
    if (!p.anc && report && tid == 0) flag(p.status, kStPacking);
    return;
  }
  const int L = p.ctx_len[b];
  if (L < 0 || (int64_t)L + T > p.Lcap) {
    if (tid == 0 && blockIdx.x == 0 && g == 0) flag(p.status, kStCtx);
    return;
  }
  const int R = p.G * T;
  const int row0 = rg * RW;
  if (row0 >= R) return;
  if (!p.anc) masks_in_lds(p, b, n0, T, report, smask);
  const int nkeys = L + T;
  const int kchunk = ((nkeys + p.splits - 1) / p.splits + KT - 1) / KT * KT;
  const int kb = split * kchunk;
  const int ke = min(nkeys, kb + kchunk);
  const int NH = p.N * p.Hq;
  const float* q = (const float*)p.q;

  for (int idx = tid; idx < RW * D; idx += 256) {
    const int r = row0 + idx / D, d = idx % D;
    float v = 0.f;
    if (r < R) {
      const int j = r / p.G, hh = r - j * p.G;
      v = q[((int64_t)(n0 + j) * p.Hq + g * p.G + hh) * D + d];
    }
    Qs[idx / D][d] = v;
  }
  const int r = row0 + rl;
  int orow = -1;
  uint64_t amask = 0;
  if (r < R) {
    const int j = r / p.G, hh = r - j * p.G;
    orow = (n0 + j) * p.Hq + g * p.G + hh;
    amask = p.anc ? p.anc[n0 + j] : smask[j];
  }
  if (kb >= ke) {
    if (orow >= 0 && kl == 0) p.ml_part[(int64_t)split * NH + orow] = make_float2(-INFINITY, 0.f);
    return;
  }
  const int64_t head_off = PAGED ? 0 : ((int64_t)b * p.Hkv + g) * p.Lcap * D;  // paged: per tile instead
  const float* kbase = (const float*)p.k + head_off;
  const float* vbase = (const float*)p.v + head_off;

  float m = -INFINITY, l = 0.f, o[DPT];
#pragma unroll
  for (int k2 = 0; k2 < DPT; ++k2) o[k2] = 0.f;

  PagedIds pg;
  if (PAGED) paged_load(p, b, kb, pg);
  for (int t0 = kb; t0 < ke; t0 += KT) {
    __syncthreads();
    // paged caches: the 32-key tile lies in one block (block_size % 64 == 0,
    // t0 % 32 == 0); a block id out of range reads as zeros (flagged)
    int64_t tile_off = (int64_t)t0 * D;
    bool tile_ok = true;
    if (PAGED) tile_off = paged_slot(p, b, g, t0, D, tile_ok, pg);
    for (int idx = tid; idx < KT * D; idx += 256) {
      const int kk = idx / D, d = idx % D, key = t0 + kk;
      const bool in = key < ke && tile_ok;
      Ks[kk][d] = in ? kbase[tile_off + (int64_t)kk * D + d] : 0.f;
      Vs[kk][d] = in ? vbase[tile_off + (int64_t)kk * D + d] : 0.f;
    }
    __syncthreads();
    float s = 0.f;
#pragma unroll 8
    for (int d = 0; d < D; ++d) s += Qs[rl][d] * Ks[kl][d];
    float x = s * p.scale_log2;
    const int key = t0 + kl;
    // branch-free visibility: context key, or an ancestor-or-self draft slot
    const int rel = key - L;
    const bool anc_bit = ((amask >> (rel & 63)) & 1ull) != 0;
    const bool vis = (key < ke) & ((key < L) | ((rel >= 0) & anc_bit));
    x = vis ? x : -INFINITY;
    float mx = x;
#pragma unroll
    for (int o2 = 16; o2 > 0; o2 >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o2));
    const float mnew = fmaxf(m, mx);
    const float msub = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = exp2f(m - msub);
    const float pv = exp2f(x - msub);
    float ls = pv;
#pragma unroll
    for (int o2 = 16; o2 > 0; o2 >>= 1) ls += __shfl_xor(ls, o2);
    l = l * alpha + ls;
    m = mnew;
    Ps[rl][kl] = pv;
    __syncthreads();
#pragma unroll
    for (int k2 = 0; k2 < DPT; ++k2) {
      const int d = kl + 32 * k2;
      float acc = o[k2] * alpha;
#pragma unroll 8
      for (int kk = 0; kk < KT; ++kk) acc += Ps[rl][kk] * Vs[kk][d];
      o[k2] = acc;
    }
  }
  if (orow < 0) return;
  if (p.splits == 1) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int k2 = 0; k2 < DPT; ++k2) p.out[(int64_t)orow * D + kl + 32 * k2] = o[k2] * inv;
  } else {
#pragma unroll
    for (int k2 = 0; k2 < DPT; ++k2) p.o_part[((int64_t)split * NH + orow) * D + kl + 32 * k2] = o[k2];
    if (kl == 0) p.ml_part[(int64_t)split * NH + orow] = make_float2(m, l);
  }
}

// ---------------------------------------------------------------------------
// Split-K merge: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s with
// M = max_s m_s over the splits that saw a key. A row of D head dims is
// spread over D / 4 lanes (one float4 each). Splits are taken eight at a
// time: every header and partial row of a chunk is requested at once (no
// load waits on another), then merged online in split order, rescaling the
// running sums whenever the maximum grows.
__global__ __launch_bounds__(256) void attn_combine_kernel(MergeArgs a) { merge_split_rows(a, blockIdx.x); }

// ---------------------------------------------------------------------------
hipError_t launch_attn_prep(const AttnParams& p, const AttnPlan& plan, const int32_t* parent, uint64_t* anc,
                            hipStream_t stream) {
  if (p.B <= 0) return hipSuccess;
  const int n_tree = anc ? (p.B + 15) / 16 : 0;
  const int blocks = n_tree + (plan.compact ? 1 : 0);
  if (blocks == 0) return hipSuccess;
  attn_prep_kernel<<<dim3(blocks), dim3(1024), 0, stream>>>(p, parent, anc, const_cast<int32_t*>(p.items),
                                                             const_cast<int32_t*>(p.item_tot), n_tree);
  return hipGetLastError();
}

// Up to 64 query rows per KV head (short chains, narrow trees): 4 waves x one
// 16-row block (16x16 MFMA), three workgroups per CU, key tiles staged
// through registers one tile ahead. Wider trees: waves of one 32-row block
// (32x32 MFMA, half the LDS operand bytes per row), key tiles loaded straight
// into double-buffered LDS with the next tile's S computed alongside the
// current tile's softmax; 8 waves (256 rows, one workgroup per CU) when every
// KV head's rows fit in 256, so that each slab is read by one workgroup, else
// 4 waves (128 rows, two workgroups per CU) with row groups (measured on
// MI355X: the 8-wave form is 6 % faster on 240-row trees, the 4-wave form
// faster on trees of up to 272 rows whose sizes vary). FP8 caches take the
// same kernels, the 32x32 one with its tiles staged through registers
// (measured on MI355X: 90 us against 137 us on the 64-row kernel for the
// 60-node trees at batch 16, 436 us against 481 us for the batch-256 super
// tree).
template <int D, bool PAGED>
static void launch_mfma_d(const AttnParams& p, int rows_per_wg, dim3 grid, hipStream_t stream) {
  if (p.kv_fp8) {
    if (rows_per_wg <= 64) attn_mfma_kernel<D, 1, 4, 1, 3, PAGED, true><<<grid, dim3(256), 0, stream>>>(p);
    else if (rows_per_wg <= 128) attn_mfma32_kernel<D, 4, 2, PAGED, true><<<grid, dim3(256), 0, stream>>>(p);
    else attn_mfma32_kernel<D, 8, 1, PAGED, true><<<grid, dim3(512), 0, stream>>>(p);
  } else if (rows_per_wg <= 64) attn_mfma_kernel<D, 1, 4, 1, 3, PAGED><<<grid, dim3(256), 0, stream>>>(p);
  else if (rows_per_wg <= 128) attn_mfma32_kernel<D, 4, 2, PAGED><<<grid, dim3(256), 0, stream>>>(p);
  else attn_mfma32_kernel<D, 8, 1, PAGED><<<grid, dim3(512), 0, stream>>>(p);
}

hipError_t launch_attention(const AttnParams& p, const AttnPlan& plan, bool bf16, hipStream_t stream,
                            hipEvent_t ev_start, hipEvent_t ev_stop, MergeArgs* defer_merge) {
  if (p.B <= 0 || p.N <= 0) return hipSuccess;
  if (ev_start) (void)hipEventRecord(ev_start, stream);
  if (bf16) {
    // 1-D grid, decoded XCD-aware inside the kernel (decode_block)
    const dim3 grid((unsigned)attn_grid_blocks(p.n_jobs, p.n_rowgroups));
    const bool paged = p.block_table != nullptr;
    if (p.D == 128) {
      if (paged) launch_mfma_d<128, true>(p, plan.rows_per_wg, grid, stream);
      else launch_mfma_d<128, false>(p, plan.rows_per_wg, grid, stream);
    } else {
      if (paged) launch_mfma_d<64, true>(p, plan.rows_per_wg, grid, stream);
      else launch_mfma_d<64, false>(p, plan.rows_per_wg, grid, stream);
    }
  } else {
    const dim3 grid(plan.n_rowgroups * plan.splits, p.Hkv, p.B);
    if (p.block_table) {
      if (p.D == 128) attn_valu_kernel<128, true><<<grid, dim3(256), 0, stream>>>(p);
      else attn_valu_kernel<64, true><<<grid, dim3(256), 0, stream>>>(p);
    } else {
      if (p.D == 128) attn_valu_kernel<128><<<grid, dim3(256), 0, stream>>>(p);
      else attn_valu_kernel<64><<<grid, dim3(256), 0, stream>>>(p);
    }
  }
  if (ev_stop) (void)hipEventRecord(ev_stop, stream);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const MergeArgs m = merge_args(p.N * p.Hq, p.D, plan.splits, p.o_part, p.ml_part, p.out);
  if (defer_merge) {
    *defer_merge = m;  // the caller's next launch merges the splits
  } else if (m.blocks > 0) {
    attn_combine_kernel<<<dim3((unsigned)m.blocks), dim3(256), 0, stream>>>(m);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace sv
