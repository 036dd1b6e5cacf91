// C ABI front end: argument validation (all of it before any side effect),
// the host FIFO block pool, the new block tables and lengths, workspace
// layout, and the stream-ordered launch sequence score -> select -> compact.

#include "../../include/kara.h"
#include "kara_internal.hpp"

#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <deque>
#include <mutex>
#include <string>
#include <vector>

struct kara_pool {
  int32_t n_blocks;
  std::deque<int32_t> fifo;
  std::vector<uint8_t> is_free;
};

namespace {

thread_local std::string g_err;

// A roctx range over a call that enqueues GPU work (shown by rocprofv3
// --marker-trace next to the kernels it launched); without a tool attached a
// push or pop is a call into an empty table.
struct TraceRange {
  explicit TraceRange(const char* name) { roctxRangePush(name); }
  ~TraceRange() { roctxRangePop(); }
  TraceRange(const TraceRange&) = delete;
  TraceRange& operator=(const TraceRange&) = delete;
};

kara_status fail(kara_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

kara_status hip_fail(hipError_t e, const char* what) {
  return fail(KARA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int log2_exact(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

kara_status check_shape(const kara_shape* sh) {
  if (!sh) return fail(KARA_E_INVAL, "shape is NULL");
  if (sh->n_layers < 1 || sh->n_q_heads < 1 || sh->n_kv_heads < 1 || sh->block_size < 1)
    return fail(KARA_E_INVAL, "shape: layers, heads and block size must be >= 1");
  if (sh->n_q_heads % sh->n_kv_heads != 0)
    return fail(KARA_E_INVAL, "shape: n_q_heads (%d) is not a multiple of n_kv_heads (%d)",
                sh->n_q_heads, sh->n_kv_heads);
  if (sh->dtype != KARA_F32 && sh->dtype != KARA_BF16)
    return fail(KARA_E_UNSUPPORTED, "shape: dtype %d not supported", sh->dtype);
  if (sh->block_size > 1024 || (sh->block_size & (sh->block_size - 1)) != 0)
    return fail(KARA_E_UNSUPPORTED, "shape: block_size %d is not a power of two <= 1024", sh->block_size);
  if (sh->head_dim != 64 && sh->head_dim != 128)
    return fail(KARA_E_UNSUPPORTED, "shape: head_dim %d not supported (64 or 128)", sh->head_dim);
  return KARA_OK;
}

kara_status check_params(const kara_params* p) {
  if (!p) return fail(KARA_E_INVAL, "params is NULL");
  if (p->window < 1 || p->window > kara::kMaxWindow)
    return fail(KARA_E_INVAL, "window %d outside [1, %d]", p->window, kara::kMaxWindow);
  if (p->protect < 0 || p->protect >= p->window)
    return fail(KARA_E_INVAL, "protect %d outside [0, window)", p->protect);
  const int C = p->window - p->protect;
  if (C > kara::kMaxRegion)
    return fail(KARA_E_INVAL, "compressible region %d exceeds %d", C, kara::kMaxRegion);
  if (p->top_k < 1 || p->top_k > C) return fail(KARA_E_INVAL, "top_k %d outside [1, %d]", p->top_k, C);
  if (p->budget < 1 || p->budget > C) return fail(KARA_E_INVAL, "budget %d outside [1, %d]", p->budget, C);
  if (p->flags & ~(KARA_UNIDIRECTIONAL | KARA_NO_CHUNKS))
    return fail(KARA_E_INVAL, "flags 0x%x hold unknown bits", (unsigned)p->flags);
  return KARA_OK;
}

size_t elt_size(const kara_shape* sh) { return sh->dtype == KARA_BF16 ? 2 : 4; }

// Sequence-level checks shared by every entry point that reads the pool.
kara_status check_sequences(const kara_shape* sh, const kara_params* p, int32_t n_seqs,
                            int32_t n_blocks, const int32_t* table_h, int32_t max_blocks,
                            const int32_t* lens_h, const kara_pool* pool) {
  if (n_seqs < 0) return fail(KARA_E_INVAL, "n_seqs < 0");
  if (n_seqs == 0) return KARA_OK;
  if (!table_h || !lens_h) return fail(KARA_E_INVAL, "host block table or lengths NULL");
  if (n_blocks < 1 || max_blocks < 1) return fail(KARA_E_INVAL, "n_blocks and max_blocks must be >= 1");
  const int bs = sh->block_size;
  std::vector<uint8_t> seen((size_t)n_blocks, 0);
  for (int32_t b = 0; b < n_seqs; ++b) {
    const int64_t L = lens_h[b];
    if (L < p->window) return fail(KARA_E_INVAL, "sequence %d: length %lld < window %d", b, (long long)L, p->window);
    if (ceil_div(L, bs) > max_blocks)
      return fail(KARA_E_INVAL, "sequence %d: length %lld needs more than max_blocks=%d blocks", b,
                  (long long)L, max_blocks);
    const int64_t f0 = (L - p->window) / bs;
    const int64_t f1 = ceil_div(L, bs);
    if (f0 + ceil_div((L - p->window) % bs + p->budget + p->protect, bs) > max_blocks)
      return fail(KARA_E_INVAL, "sequence %d: compacted tail does not fit max_blocks", b);
    for (int64_t e = f0; e < f1; ++e) {
      const int32_t id = table_h[(size_t)b * max_blocks + e];
      if (id < 0 || id >= n_blocks)
        return fail(KARA_E_INVAL, "sequence %d: block table entry %lld = %d out of range [0, %d)", b,
                    (long long)e, id, n_blocks);
      if (seen[id]) return fail(KARA_E_INVAL, "block %d appears twice in the compressed tails", id);
      seen[id] = 1;
      if (pool && pool->n_blocks == n_blocks && pool->is_free[id])
        return fail(KARA_E_INVAL, "block %d is in use by sequence %d but also free in the pool", id, b);
    }
  }
  return KARA_OK;
}

struct Plan {
  std::vector<int32_t> fresh;   // all fresh ids, sequences in call order
  std::vector<int32_t> freed;   // old tail ids, sequences in call order, positions ascending
};

// One sequence's compaction plan: the boundary block's table position, the
// fresh blocks its compacted tail takes, and its new length L - C + R.
struct SeqPlan {
  int64_t f0, n_fresh, new_len;
};

SeqPlan plan_sequence(int64_t L, const kara_params* p, int bs) {
  SeqPlan q;
  q.f0 = (L - p->window) / bs;
  q.n_fresh = ceil_div((L - p->window) % bs + p->budget + p->protect, bs);
  q.new_len = L - (p->window - p->protect) + p->budget;
  return q;
}

// Fills the new tables and lengths from the front of the pool without popping.
kara_status make_plan(const kara_shape* sh, const kara_params* p, int32_t n_seqs,
                      const int32_t* table_h, int32_t max_blocks, const int32_t* lens_h,
                      const kara_pool* pool, int32_t* new_table_h, int32_t* new_lens_h, Plan* plan) {
  const int bs = sh->block_size;
  int64_t need = 0;
  for (int32_t b = 0; b < n_seqs; ++b) need += plan_sequence(lens_h[b], p, bs).n_fresh;
  if (need > (int64_t)pool->fifo.size())
    return fail(KARA_E_NOBLOCKS, "need %lld fresh blocks, pool has %zu", (long long)need, pool->fifo.size());
  if (!new_table_h || !new_lens_h) return fail(KARA_E_INVAL, "host outputs NULL");
  plan->fresh.assign(pool->fifo.begin(), pool->fifo.begin() + need);
  plan->freed.clear();
  size_t cur = 0;
  for (int32_t b = 0; b < n_seqs; ++b) {
    const SeqPlan q = plan_sequence(lens_h[b], p, bs);
    const int32_t* row = table_h + (size_t)b * max_blocks;
    int32_t* out = new_table_h + (size_t)b * max_blocks;
    for (int64_t e = 0; e < q.f0; ++e) out[e] = row[e];
    for (int64_t e = 0; e < q.n_fresh; ++e) out[q.f0 + e] = plan->fresh[cur++];
    for (int64_t e = q.f0 + q.n_fresh; e < max_blocks; ++e) out[e] = -1;
    new_lens_h[b] = (int32_t)q.new_len;
  }
  for (int32_t b = 0; b < n_seqs; ++b) {
    const int64_t L = lens_h[b];
    const int64_t f0 = (L - p->window) / bs;
    for (int64_t e = f0; e < ceil_div(L, bs); ++e) plan->freed.push_back(table_h[(size_t)b * max_blocks + e]);
  }
  return KARA_OK;
}

void commit_plan(kara_pool* pool, const Plan& plan) {
  for (size_t i = 0; i < plan.fresh.size(); ++i) {
    pool->is_free[pool->fifo.front()] = 0;
    pool->fifo.pop_front();
  }
  for (int32_t id : plan.freed) {
    pool->fifo.push_back(id);
    pool->is_free[id] = 1;
  }
}

// Workspace: [partial column sums of every 512-row chunk (one row per unit
// for the resident-key scorer)][resident scorer over two key blocks: per-row
// normaliser inputs, per-unit exact-route flags][retained positions]
struct Workspace {
  size_t partials, zrow, flags, retained, total;
};

Workspace layout(const kara_shape* sh, const kara_params* p, int32_t n_seqs) {
  const size_t U = (size_t)n_seqs * sh->n_layers * sh->n_kv_heads;
  const int C = p->window - p->protect;
  const int G = sh->n_q_heads / sh->n_kv_heads;
  const int uni = (p->flags & KARA_UNIDIRECTIONAL) ? 1 : 0;
  const size_t n_split = (size_t)kara::score_splits(sh->dtype, sh->head_dim, p->window, G, uni);
  const bool two = kara::resident_two_blocks(sh->dtype, sh->head_dim, p->window, G, uni);
  Workspace w;
  w.partials = 0;
  w.zrow = align_up(U * n_split * C * sizeof(float));
  w.flags = w.zrow + (two ? align_up(U * (size_t)G * p->window * sizeof(float)) : 0);
  w.retained = w.flags + (two ? align_up(U * sizeof(int32_t)) : 0);
  w.total = w.retained + align_up(U * p->budget * sizeof(int32_t));
  return w;
}

// Points the scorer's per-row and per-unit buffers into the workspace.
void attach_resident(kara::ScoreArgs* a, const kara_shape* sh, const kara_params* p, const Workspace& w,
                     void* workspace) {
  if (kara::resident_two_blocks(sh->dtype, sh->head_dim, p->window, a->G, a->unidirectional)) {
    a->zrow = (float*)((char*)workspace + w.zrow);
    a->uflags = (int32_t*)((char*)workspace + w.flags);
  }
}

kara::ScoreArgs score_args(const kara_shape* sh, const kara_params* p, int32_t n_seqs,
                           const void* q, const void* kv, int32_t n_blocks, const int32_t* table_d,
                           int32_t max_blocks, const int32_t* lens_d, float* out) {
  kara::ScoreArgs a;
  a.q = q;
  a.pool = kv;
  a.table = table_d;
  a.lens = lens_d;
  a.out = out;
  a.S = n_seqs;
  a.Lyr = sh->n_layers;
  a.Hq = sh->n_q_heads;
  a.Hkv = sh->n_kv_heads;
  a.G = sh->n_q_heads / sh->n_kv_heads;
  a.D = sh->head_dim;
  a.bs = sh->block_size;
  a.bs_shift = log2_exact(sh->block_size);
  a.NB = n_blocks;
  a.MB = max_blocks;
  a.W = p->window;
  a.C = p->window - p->protect;
  a.n_split = kara::score_splits(sh->dtype, a.D, a.W, a.G, (p->flags & KARA_UNIDIRECTIONAL) ? 1 : 0);
  a.n_units = n_seqs * sh->n_layers * sh->n_kv_heads;
  a.c = (float)(1.4426950408889634 / std::sqrt((double)sh->head_dim));
  a.unidirectional = (p->flags & KARA_UNIDIRECTIONAL) ? 1 : 0;
  a.q_slots = nullptr;
  a.q_counts = nullptr;
  a.q_n_slots = 0;
  a.zrow = nullptr;
  a.uflags = nullptr;
  a.key_lo = 0;
  a.key_hi = 0;
  return a;
}

kara::CompactArgs compact_args(const kara_shape* sh, const kara_params* p, int32_t n_seqs,
                               void* kv, int32_t n_blocks, const int32_t* old_d, const int32_t* new_d,
                               int32_t max_blocks, const int32_t* lens_d, const int32_t* retained_d) {
  kara::CompactArgs a;
  a.pool = kv;
  a.old_table = old_d;
  a.new_table = new_d;
  a.lens = lens_d;
  a.retained = retained_d;
  a.S = n_seqs;
  a.Lyr = sh->n_layers;
  a.Hkv = sh->n_kv_heads;
  a.row_bytes = (int)(sh->head_dim * elt_size(sh));
  a.bs = sh->block_size;
  a.NB = n_blocks;
  a.MB = max_blocks;
  a.W = p->window;
  a.B = p->protect;
  a.R = p->budget;
  return a;
}

bool is_aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

// Validation and launch arguments shared by decode attention and its
// paged-read probe (everything but the query states, outputs and workspace).
kara_status attention_args(const kara_shape* shape, int32_t n_seqs, int32_t layer, const void* kv_pool,
                           int32_t n_blocks, const int32_t* block_table_d, int32_t max_blocks,
                           const int32_t* seq_lens_h, const int32_t* seq_lens_d, kara::AttnArgs* a,
                           int32_t* max_len_out) {
  kara_status st;
  if ((st = check_shape(shape)) != KARA_OK) return st;
  if (shape->n_q_heads / shape->n_kv_heads > 8)
    return fail(KARA_E_UNSUPPORTED, "decode attention supports at most 8 query heads per KV head");
  if (n_seqs < 0) return fail(KARA_E_INVAL, "n_seqs < 0");
  if (layer < 0 || layer >= shape->n_layers)
    return fail(KARA_E_INVAL, "layer %d outside [0, %d)", layer, shape->n_layers);
  if (n_blocks < 1 || max_blocks < 1) return fail(KARA_E_INVAL, "n_blocks and max_blocks must be >= 1");
  // the kernels index a layer's K rows with 32-bit row numbers
  if ((uint64_t)n_blocks * shape->n_kv_heads * shape->block_size >= ((uint64_t)1 << 32))
    return fail(KARA_E_UNSUPPORTED, "n_blocks * n_kv_heads * block_size = %llu rows per layer exceed 2^32",
                (unsigned long long)n_blocks * shape->n_kv_heads * shape->block_size);
  *max_len_out = 0;
  if (n_seqs == 0) return KARA_OK;
  if (!seq_lens_h) return fail(KARA_E_INVAL, "host lengths NULL");
  int32_t max_len = 0;
  for (int32_t b = 0; b < n_seqs; ++b) {
    const int64_t L = seq_lens_h[b];
    if (L < 1 || L > (int64_t)max_blocks * shape->block_size)
      return fail(KARA_E_INVAL, "sequence %d: length %lld outside [1, max_blocks * block_size]", b, (long long)L);
    max_len = L > max_len ? (int32_t)L : max_len;
  }
  if (!kv_pool || !block_table_d || !seq_lens_d) return fail(KARA_E_INVAL, "device pointer NULL");
  if (!is_aligned(kv_pool, 16)) return fail(KARA_E_INVAL, "q and kv_pool must be 16-byte aligned");
  a->q = nullptr;
  a->pool = kv_pool;
  a->table = block_table_d;
  a->lens = seq_lens_d;
  a->part_o = a->part_ml = a->out = nullptr;
  a->S = n_seqs;
  a->layer = layer;
  a->Hq = shape->n_q_heads;
  a->Hkv = shape->n_kv_heads;
  a->D = shape->head_dim;
  a->bs = shape->block_size;
  a->bs_shift = log2_exact(shape->block_size);
  a->NB = n_blocks;
  a->MB = max_blocks;
  // 1024-token splits when they alone give the launch enough workgroups
  long big_grid = 0;
  for (int32_t b = 0; b < n_seqs; ++b) big_grid += ceil_div(seq_lens_h[b], kara::kAttnChunkMax);
  big_grid *= shape->n_kv_heads;
  a->chunk = big_grid >= kara::kAttnBigGrid ? kara::kAttnChunkMax : kara::kAttnChunkMin;
  a->n_split = ceil_div(max_len, a->chunk);
  a->c = (float)(1.4426950408889634 / std::sqrt((double)shape->head_dim));
  *max_len_out = max_len;
  return KARA_OK;
}

}  // namespace

extern "C" {

const char* kara_last_error(void) { return g_err.c_str(); }

const char* kara_version(void) { return "kara-mi355x 0.1 (gfx950)"; }

kara_status kara_pool_create(int32_t n_blocks, const int32_t* free_ids, int32_t n_free, kara_pool** out) {
  if (!out) return fail(KARA_E_INVAL, "out is NULL");
  if (n_blocks < 1) return fail(KARA_E_INVAL, "n_blocks must be >= 1");
  if (n_free < 0 || n_free > n_blocks || (n_free > 0 && !free_ids))
    return fail(KARA_E_INVAL, "bad free list");
  std::vector<uint8_t> is_free((size_t)n_blocks, 0);
  for (int32_t i = 0; i < n_free; ++i) {
    const int32_t id = free_ids[i];
    if (id < 0 || id >= n_blocks) return fail(KARA_E_INVAL, "free id %d out of range", id);
    if (is_free[id]) return fail(KARA_E_INVAL, "free id %d repeated", id);
    is_free[id] = 1;
  }
  kara_pool* pl = new (std::nothrow) kara_pool;
  if (!pl) return fail(KARA_E_INVAL, "out of host memory");
  pl->n_blocks = n_blocks;
  pl->fifo.assign(free_ids, free_ids + n_free);
  pl->is_free.swap(is_free);
  *out = pl;
  return KARA_OK;
}

kara_status kara_pool_alloc(kara_pool* pool, int32_t n, int32_t* ids_out) {
  if (!pool || n < 0 || (n > 0 && !ids_out)) return fail(KARA_E_INVAL, "bad arguments");
  if ((size_t)n > pool->fifo.size())
    return fail(KARA_E_NOBLOCKS, "need %d blocks, pool has %zu", n, pool->fifo.size());
  for (int32_t i = 0; i < n; ++i) {
    ids_out[i] = pool->fifo.front();
    pool->is_free[ids_out[i]] = 0;
    pool->fifo.pop_front();
  }
  return KARA_OK;
}

kara_status kara_pool_free(kara_pool* pool, const int32_t* ids, int32_t n) {
  if (!pool || n < 0 || (n > 0 && !ids)) return fail(KARA_E_INVAL, "bad arguments");
  std::vector<int32_t> seen;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || id >= pool->n_blocks) return fail(KARA_E_INVAL, "id %d out of range", id);
    if (pool->is_free[id]) return fail(KARA_E_INVAL, "id %d is already free", id);
    for (int32_t x : seen)
      if (x == id) return fail(KARA_E_INVAL, "id %d repeated", id);
    seen.push_back(id);
  }
  for (int32_t i = 0; i < n; ++i) {
    pool->fifo.push_back(ids[i]);
    pool->is_free[ids[i]] = 1;
  }
  return KARA_OK;
}

int32_t kara_pool_num_free(const kara_pool* pool) { return pool ? (int32_t)pool->fifo.size() : 0; }

int32_t kara_pool_snapshot(const kara_pool* pool, int32_t* ids_out, int32_t cap) {
  if (!pool || !ids_out || cap <= 0) return 0;
  int32_t n = 0;
  for (int32_t id : pool->fifo) {
    if (n >= cap) break;
    ids_out[n++] = id;
  }
  return n;
}

void kara_pool_destroy(kara_pool* pool) { delete pool; }

size_t kara_workspace_bytes(const kara_shape* shape, const kara_params* params, int32_t n_seqs) {
  if (check_shape(shape) != KARA_OK || check_params(params) != KARA_OK || n_seqs < 0) return 0;
  return layout(shape, params, n_seqs).total;
}

}  // extern "C"

namespace {

// Where the window query states come from: one [S][Lyr][W][Hq][D] array, or
// a ring of each sequence's last W query states.
struct QuerySource {
  const void* q;
  const kara_query_ring* ring;  // null for the plain array
};

kara_status compress_impl(const kara_shape* shape, const kara_params* params, int32_t n_seqs,
                          QuerySource qs, void* kv_pool, int32_t n_blocks,
                          const int32_t* block_table_h, const int32_t* block_table_d,
                          int32_t max_blocks, const int32_t* seq_lens_h, const int32_t* seq_lens_d,
                          kara_pool* pool, int32_t* new_block_table_h, int32_t* new_block_table_d,
                          int32_t* new_seq_lens_h, void* workspace, size_t workspace_bytes,
                          void* stream, float* scores_out_d, int32_t* cand_out_d,
                          int32_t* retained_out_d, void* const* stage_events) {
  const void* q_window = qs.q;
  kara_status st;
  if ((st = check_shape(shape)) != KARA_OK) return st;
  if ((st = check_params(params)) != KARA_OK) return st;
  if (!pool) return fail(KARA_E_INVAL, "pool is NULL");
  if (pool->n_blocks != n_blocks) return fail(KARA_E_INVAL, "pool covers %d blocks, cache has %d", pool->n_blocks, n_blocks);
  if ((st = check_sequences(shape, params, n_seqs, n_blocks, block_table_h, max_blocks, seq_lens_h, pool)) != KARA_OK)
    return st;
  if (n_seqs == 0) return KARA_OK;
  if (qs.ring && (qs.ring->n_slots < 1 || !qs.ring->slots_d || !qs.ring->counts_d))
    return fail(KARA_E_INVAL, "query ring: n_slots < 1 or slot/count arrays NULL");
  if (qs.ring && qs.ring->window != params->window)
    return fail(KARA_E_INVAL, "query ring holds windows of %d, the call compresses windows of %d",
                qs.ring->window, params->window);
  if (!q_window || !kv_pool || !block_table_d || !seq_lens_d || !new_block_table_d)
    return fail(KARA_E_INVAL, "device pointer NULL");
  if (!is_aligned(q_window, 16) || !is_aligned(kv_pool, 16))
    return fail(KARA_E_INVAL, "query states and kv_pool must be 16-byte aligned");
  const Workspace ws = layout(shape, params, n_seqs);
  if (!workspace || workspace_bytes < ws.total || !is_aligned(workspace, kAlign))
    return fail(KARA_E_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", ws.total);
  Plan plan;
  if ((st = make_plan(shape, params, n_seqs, block_table_h, max_blocks, seq_lens_h, pool,
                      new_block_table_h, new_seq_lens_h, &plan)) != KARA_OK)
    return st;

  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)workspace;
  float* partials = (float*)(w + ws.partials);
  float* scores = scores_out_d;
  int32_t* retained = retained_out_d ? retained_out_d : (int32_t*)(w + ws.retained);
  hipError_t e = hipMemcpyAsync(new_block_table_d, new_block_table_h,
                                (size_t)n_seqs * max_blocks * sizeof(int32_t), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "block table upload");
  auto mark = [&](int i) -> hipError_t {
    return stage_events ? hipEventRecord((hipEvent_t)stage_events[i], s) : hipSuccess;
  };
  if ((e = mark(0)) != hipSuccess) return hip_fail(e, "stage event");
  kara::ScoreArgs sa = score_args(shape, params, n_seqs, q_window, kv_pool, n_blocks, block_table_d,
                                  max_blocks, seq_lens_d, partials);
  attach_resident(&sa, shape, params, ws, workspace);
  if (qs.ring) {
    sa.q_slots = qs.ring->slots_d;
    sa.q_counts = qs.ring->counts_d;
    sa.q_n_slots = qs.ring->n_slots;
  }
  {
    TraceRange range("score");
    if ((e = kara::launch_score(sa, shape->dtype, s)) != hipSuccess) return hip_fail(e, "score launch");
  }
  if ((e = mark(1)) != hipSuccess) return hip_fail(e, "stage event");
  kara::SelectArgs se;
  se.partials = partials;
  se.n_split = sa.n_split;
  se.cand_in = nullptr;
  se.scores_out = scores;
  se.cand_out = cand_out_d;
  se.retained_out = retained;
  se.n_units = sa.n_units;
  se.C = sa.C;
  se.K = params->top_k;
  se.R = params->budget;
  se.mode = kara::kSelectFull;
  se.no_chunks = (params->flags & KARA_NO_CHUNKS) ? 1 : 0;
  {
    TraceRange range("select");
    if ((e = kara::launch_select(se, s)) != hipSuccess) return hip_fail(e, "select launch");
  }
  if ((e = mark(2)) != hipSuccess) return hip_fail(e, "stage event");
  kara::CompactArgs ca = compact_args(shape, params, n_seqs, kv_pool, n_blocks, block_table_d,
                                      new_block_table_d, max_blocks, seq_lens_d, retained);
  {
    TraceRange range("compact");
    if ((e = kara::launch_compact(ca, s)) != hipSuccess) return hip_fail(e, "compact launch");
  }
  if ((e = mark(3)) != hipSuccess) return hip_fail(e, "stage event");
  commit_plan(pool, plan);
  return KARA_OK;
}

}  // namespace

extern "C" {

kara_status kara_compress(const kara_shape* shape, const kara_params* params, int32_t n_seqs,
                          const void* q_window, void* kv_pool, int32_t n_blocks,
                          const int32_t* block_table_h, const int32_t* block_table_d,
                          int32_t max_blocks, const int32_t* seq_lens_h, const int32_t* seq_lens_d,
                          kara_pool* pool, int32_t* new_block_table_h, int32_t* new_block_table_d,
                          int32_t* new_seq_lens_h, void* workspace, size_t workspace_bytes,
                          void* stream, float* scores_out_d, int32_t* cand_out_d,
                          int32_t* retained_out_d, void* const* stage_events) {
  TraceRange range("kara_compress");
  return compress_impl(shape, params, n_seqs, QuerySource{q_window, nullptr}, kv_pool, n_blocks,
                       block_table_h, block_table_d, max_blocks, seq_lens_h, seq_lens_d, pool,
                       new_block_table_h, new_block_table_d, new_seq_lens_h, workspace,
                       workspace_bytes, stream, scores_out_d, cand_out_d, retained_out_d,
                       stage_events);
}

kara_status kara_compress_ring(const kara_shape* shape, const kara_params* params, int32_t n_seqs,
                               const kara_query_ring* ring, void* kv_pool, int32_t n_blocks,
                               const int32_t* block_table_h, const int32_t* block_table_d,
                               int32_t max_blocks, const int32_t* seq_lens_h,
                               const int32_t* seq_lens_d, kara_pool* pool,
                               int32_t* new_block_table_h, int32_t* new_block_table_d,
                               int32_t* new_seq_lens_h, void* workspace, size_t workspace_bytes,
                               void* stream, float* scores_out_d, int32_t* cand_out_d,
                               int32_t* retained_out_d, void* const* stage_events) {
  TraceRange range("kara_compress_ring");
  if (!ring) return fail(KARA_E_INVAL, "query ring is NULL");
  return compress_impl(shape, params, n_seqs, QuerySource{ring->q_ring, ring}, kv_pool, n_blocks,
                       block_table_h, block_table_d, max_blocks, seq_lens_h, seq_lens_d, pool,
                       new_block_table_h, new_block_table_d, new_seq_lens_h, workspace,
                       workspace_bytes, stream, scores_out_d, cand_out_d, retained_out_d,
                       stage_events);
}

kara_status kara_append(const kara_shape* shape, int32_t window, int32_t n_seqs, int32_t layer,
                        const void* q_d, const void* k_d, const void* v_d, void* kv_pool,
                        int32_t n_blocks, const int32_t* block_table_d, int32_t max_blocks,
                        const int32_t* positions_d, const kara_query_ring* ring, void* stream) {
  TraceRange range("kara_append");
  kara_status st;
  if ((st = check_shape(shape)) != KARA_OK) return st;
  if (window < 1 || window > kara::kMaxWindow)
    return fail(KARA_E_INVAL, "window %d outside [1, %d]", window, kara::kMaxWindow);
  if (n_seqs < 0) return fail(KARA_E_INVAL, "n_seqs < 0");
  if (layer < -1 || layer >= shape->n_layers)
    return fail(KARA_E_INVAL, "layer %d outside [-1, %d)", layer, shape->n_layers);
  if (n_blocks < 1 || max_blocks < 1) return fail(KARA_E_INVAL, "n_blocks and max_blocks must be >= 1");
  if (!ring || ring->n_slots < 1) return fail(KARA_E_INVAL, "query ring NULL or without slots");
  if (ring->window != window)
    return fail(KARA_E_INVAL, "query ring holds windows of %d, the call appends with window %d", ring->window,
                window);
  if (n_seqs == 0) return KARA_OK;
  if (!q_d || !k_d || !v_d || !kv_pool || !block_table_d || !positions_d || !ring->q_ring ||
      !ring->slots_d || !ring->counts_d)
    return fail(KARA_E_INVAL, "device pointer NULL");
  if (!is_aligned(q_d, 16) || !is_aligned(k_d, 16) || !is_aligned(v_d, 16) || !is_aligned(kv_pool, 16) ||
      !is_aligned(ring->q_ring, 16))
    return fail(KARA_E_INVAL, "state arrays, kv_pool and the ring must be 16-byte aligned");
  kara::AppendArgs a;
  a.q = q_d;
  a.k = k_d;
  a.v = v_d;
  a.pool = kv_pool;
  a.ring = ring->q_ring;
  a.table = block_table_d;
  a.positions = positions_d;
  a.slots = ring->slots_d;
  a.counts = ring->counts_d;
  a.S = n_seqs;
  a.Lyr = shape->n_layers;
  a.n_lyr_in = layer >= 0 ? 1 : shape->n_layers;
  a.layer = layer;
  a.Hq = shape->n_q_heads;
  a.Hkv = shape->n_kv_heads;
  a.row_bytes = (int)(shape->head_dim * elt_size(shape));
  a.bs = shape->block_size;
  a.NB = n_blocks;
  a.MB = max_blocks;
  a.W = window;
  a.n_slots = ring->n_slots;
  const hipError_t e = kara::launch_append(a, (hipStream_t)stream);
  return e == hipSuccess ? KARA_OK : hip_fail(e, "append launch");
}

size_t kara_attention_workspace_bytes(const kara_shape* shape, int32_t n_seqs, int32_t max_len) {
  if (check_shape(shape) != KARA_OK || n_seqs < 0 || max_len < 1) return 0;
  // sized for the finer split, whichever the launch picks
  const size_t n_split = (size_t)ceil_div(max_len, kara::kAttnChunkMin);
  const size_t parts = (size_t)n_seqs * shape->n_q_heads * n_split;
  return align_up(parts * shape->head_dim * sizeof(float)) + align_up(parts * 2 * sizeof(float));
}

kara_status kara_decode_attention(const kara_shape* shape, int32_t n_seqs, int32_t layer,
                                  const void* q_d, const void* kv_pool, int32_t n_blocks,
                                  const int32_t* block_table_d, int32_t max_blocks,
                                  const int32_t* seq_lens_h, const int32_t* seq_lens_d,
                                  float* out_d, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  TraceRange range("kara_decode_attention");
  kara::AttnArgs a;
  int32_t max_len = 0;
  kara_status st = attention_args(shape, n_seqs, layer, kv_pool, n_blocks, block_table_d, max_blocks, seq_lens_h,
                                  seq_lens_d, &a, &max_len);
  if (st != KARA_OK || n_seqs == 0) return st;
  if (!q_d || !out_d) return fail(KARA_E_INVAL, "device pointer NULL");
  if (!is_aligned(q_d, 16)) return fail(KARA_E_INVAL, "q and kv_pool must be 16-byte aligned");
  const size_t need = kara_attention_workspace_bytes(shape, n_seqs, max_len);
  if (!workspace || workspace_bytes < need || !is_aligned(workspace, kAlign))
    return fail(KARA_E_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need);
  a.q = q_d;
  const size_t parts = (size_t)n_seqs * a.Hq * a.n_split;
  a.part_o = (float*)workspace;
  a.part_ml = (float*)((char*)workspace + align_up(parts * a.D * sizeof(float)));
  a.out = out_d;
  const hipError_t e = kara::launch_attention(a, shape->dtype, (hipStream_t)stream);
  return e == hipSuccess ? KARA_OK : hip_fail(e, "attention launch");
}

kara_status kara_probe_paged_read(const kara_shape* shape, int32_t n_seqs, int32_t layer, const void* kv_pool,
                                  int32_t n_blocks, const int32_t* block_table_d, int32_t max_blocks,
                                  const int32_t* seq_lens_h, const int32_t* seq_lens_d, void* dst_d,
                                  void* stream, double* bytes_out) {
  TraceRange range("kara_probe_paged_read");
  if (!bytes_out) return fail(KARA_E_INVAL, "bytes_out is NULL");
  if (shape && shape->dtype != KARA_BF16)
    return fail(KARA_E_UNSUPPORTED, "the paged-read probe mirrors the bf16 attention kernel only");
  kara::AttnArgs a;
  int32_t max_len = 0;
  kara_status st = attention_args(shape, n_seqs, layer, kv_pool, n_blocks, block_table_d, max_blocks, seq_lens_h,
                                  seq_lens_d, &a, &max_len);
  if (st != KARA_OK) return st;
  double bytes = 0.0;
  for (int32_t b = 0; b < n_seqs; ++b) bytes += (double)seq_lens_h[b];
  *bytes_out = bytes * a.Hkv * 2.0 * a.D * 2.0;
  if (n_seqs == 0) return KARA_OK;
  if (!dst_d || !is_aligned(dst_d, 4)) return fail(KARA_E_INVAL, "dst NULL or not 4-byte aligned");
  const hipError_t e = kara::launch_paged_read_probe(a, (uint32_t*)dst_d, (hipStream_t)stream);
  return e == hipSuccess ? KARA_OK : hip_fail(e, "probe launch");
}

kara_status kara_score(const kara_shape* shape, const kara_params* params, int32_t n_seqs,
                       const void* q_window, const void* kv_pool, int32_t n_blocks,
                       const int32_t* block_table_h, const int32_t* block_table_d, int32_t max_blocks,
                       const int32_t* seq_lens_h, const int32_t* seq_lens_d, float* scores_d,
                       void* workspace, size_t workspace_bytes, void* stream) {
  TraceRange range("kara_score");
  kara_status st;
  if ((st = check_shape(shape)) != KARA_OK) return st;
  if ((st = check_params(params)) != KARA_OK) return st;
  if ((st = check_sequences(shape, params, n_seqs, n_blocks, block_table_h, max_blocks, seq_lens_h, nullptr)) != KARA_OK)
    return st;
  if (n_seqs == 0) return KARA_OK;
  if (!q_window || !kv_pool || !block_table_d || !seq_lens_d || !scores_d)
    return fail(KARA_E_INVAL, "device pointer NULL");
  if (!is_aligned(q_window, 16) || !is_aligned(kv_pool, 16))
    return fail(KARA_E_INVAL, "q_window and kv_pool must be 16-byte aligned");
  const Workspace ws = layout(shape, params, n_seqs);
  const int G = shape->n_q_heads / shape->n_kv_heads;
  const int uni = (params->flags & KARA_UNIDIRECTIONAL) ? 1 : 0;
  const bool direct = kara::score_splits(shape->dtype, shape->head_dim, params->window, G, uni) == 1;
  if ((!direct || kara::resident_two_blocks(shape->dtype, shape->head_dim, params->window, G, uni)) &&
      (!workspace || workspace_bytes < ws.retained || !is_aligned(workspace, kAlign)))
    return fail(KARA_E_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", ws.retained);
  hipStream_t s = (hipStream_t)stream;
  float* partials = direct ? scores_d : (float*)((char*)workspace + ws.partials);
  kara::ScoreArgs sa = score_args(shape, params, n_seqs, q_window, kv_pool, n_blocks, block_table_d,
                                  max_blocks, seq_lens_d, partials);
  attach_resident(&sa, shape, params, ws, workspace);
  hipError_t e = kara::launch_score(sa, shape->dtype, s);
  if (e != hipSuccess) return hip_fail(e, "score launch");
  if (!direct && (e = kara::launch_reduce(partials, scores_d, sa.n_units, sa.n_split, sa.C, s)) != hipSuccess)
    return hip_fail(e, "reduce launch");
  return KARA_OK;
}

kara_status kara_topk(int32_t n_units, int32_t region, int32_t top_k, const float* scores_d,
                      int32_t* cand_d, void* stream) {
  TraceRange range("kara_topk");
  if (n_units < 0) return fail(KARA_E_INVAL, "n_units < 0");
  if (region < 1 || region > kara::kMaxRegion) return fail(KARA_E_INVAL, "region %d outside [1, %d]", region, kara::kMaxRegion);
  if (top_k < 1 || top_k > region) return fail(KARA_E_INVAL, "top_k %d outside [1, %d]", top_k, region);
  if (n_units == 0) return KARA_OK;
  if (!scores_d || !cand_d) return fail(KARA_E_INVAL, "device pointer NULL");
  kara::SelectArgs se;
  se.partials = scores_d;
  se.n_split = 1;
  se.cand_in = nullptr;
  se.scores_out = nullptr;
  se.cand_out = cand_d;
  se.retained_out = nullptr;
  se.n_units = n_units;
  se.C = region;
  se.K = top_k;
  se.R = top_k;
  se.mode = kara::kSelectTopK;
  se.no_chunks = 0;
  hipError_t e = kara::launch_select(se, (hipStream_t)stream);
  return e == hipSuccess ? KARA_OK : hip_fail(e, "topk launch");
}

kara_status kara_token2chunk(int32_t n_units, int32_t region, int32_t top_k, int32_t budget,
                             const float* scores_d, const int32_t* cand_d, int32_t* retained_d,
                             void* stream) {
  TraceRange range("kara_token2chunk");
  if (n_units < 0) return fail(KARA_E_INVAL, "n_units < 0");
  if (region < 1 || region > kara::kMaxRegion) return fail(KARA_E_INVAL, "region %d outside [1, %d]", region, kara::kMaxRegion);
  if (top_k < 1 || top_k > region) return fail(KARA_E_INVAL, "top_k %d outside [1, %d]", top_k, region);
  if (budget < 1 || budget > region) return fail(KARA_E_INVAL, "budget %d outside [1, %d]", budget, region);
  if (n_units == 0) return KARA_OK;
  if (!scores_d || !cand_d || !retained_d) return fail(KARA_E_INVAL, "device pointer NULL");
  kara::SelectArgs se;
  se.partials = scores_d;
  se.n_split = 1;
  se.cand_in = cand_d;
  se.scores_out = nullptr;
  se.cand_out = nullptr;
  se.retained_out = retained_d;
  se.n_units = n_units;
  se.C = region;
  se.K = top_k;
  se.R = budget;
  se.mode = kara::kSelectT2C;
  se.no_chunks = 0;
  hipError_t e = kara::launch_select(se, (hipStream_t)stream);
  return e == hipSuccess ? KARA_OK : hip_fail(e, "token2chunk launch");
}

kara_status kara_paged_compact(const kara_shape* shape, const kara_params* params, int32_t n_seqs,
                               void* kv_pool, int32_t n_blocks, const int32_t* block_table_h,
                               const int32_t* block_table_d, int32_t max_blocks,
                               const int32_t* seq_lens_h, const int32_t* seq_lens_d,
                               const int32_t* retained_d, kara_pool* pool, int32_t* new_block_table_h,
                               int32_t* new_block_table_d, int32_t* new_seq_lens_h, void* stream) {
  TraceRange range("kara_paged_compact");
  kara_status st;
  if ((st = check_shape(shape)) != KARA_OK) return st;
  if ((st = check_params(params)) != KARA_OK) return st;
  if (!pool) return fail(KARA_E_INVAL, "pool is NULL");
  if (pool->n_blocks != n_blocks) return fail(KARA_E_INVAL, "pool covers %d blocks, cache has %d", pool->n_blocks, n_blocks);
  if ((st = check_sequences(shape, params, n_seqs, n_blocks, block_table_h, max_blocks, seq_lens_h, pool)) != KARA_OK)
    return st;
  if (n_seqs == 0) return KARA_OK;
  if (!kv_pool || !block_table_d || !seq_lens_d || !retained_d || !new_block_table_d)
    return fail(KARA_E_INVAL, "device pointer NULL");
  if (!is_aligned(kv_pool, 16)) return fail(KARA_E_INVAL, "kv_pool must be 16-byte aligned");
  Plan plan;
  if ((st = make_plan(shape, params, n_seqs, block_table_h, max_blocks, seq_lens_h, pool,
                      new_block_table_h, new_seq_lens_h, &plan)) != KARA_OK)
    return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(new_block_table_d, new_block_table_h,
                                (size_t)n_seqs * max_blocks * sizeof(int32_t), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "block table upload");
  kara::CompactArgs ca = compact_args(shape, params, n_seqs, kv_pool, n_blocks, block_table_d,
                                      new_block_table_d, max_blocks, seq_lens_d, retained_d);
  if ((e = kara::launch_compact(ca, s)) != hipSuccess) return hip_fail(e, "compact launch");
  commit_plan(pool, plan);
  return KARA_OK;
}

kara_status kara_plan_lengths(const kara_params* params, int32_t block_size, int32_t n_seqs,
                              const int32_t* seq_lens_h, int32_t* new_lens_out, int32_t* fresh_blocks_out) {
  kara_status st;
  if ((st = check_params(params)) != KARA_OK) return st;
  if (block_size < 1 || block_size > 1024 || (block_size & (block_size - 1)) != 0)
    return fail(KARA_E_UNSUPPORTED, "block_size %d is not a power of two <= 1024", block_size);
  if (n_seqs < 0) return fail(KARA_E_INVAL, "n_seqs < 0");
  if (n_seqs > 0 && (!seq_lens_h || !new_lens_out || !fresh_blocks_out))
    return fail(KARA_E_INVAL, "plan arrays NULL");
  for (int32_t b = 0; b < n_seqs; ++b)
    if (seq_lens_h[b] < params->window)
      return fail(KARA_E_INVAL, "sequence %d: length %d < window %d", b, seq_lens_h[b], params->window);
  for (int32_t b = 0; b < n_seqs; ++b) {
    const SeqPlan q = plan_sequence(seq_lens_h[b], params, block_size);
    new_lens_out[b] = (int32_t)q.new_len;
    fresh_blocks_out[b] = (int32_t)q.n_fresh;
  }
  return KARA_OK;
}

kara_status kara_schedule_step(int64_t step, int32_t period, int32_t window, int32_t n_seqs,
                               const int32_t* seq_lens, const int32_t* watermarks,
                               const uint8_t* selected, int32_t* batch_out, int32_t* n_batch) {
  if (period < 1 || window < 1 || n_seqs < 0 || step < 0 || !n_batch)
    return fail(KARA_E_INVAL, "bad schedule arguments");
  if (n_seqs > 0 && (!seq_lens || !watermarks || !selected || !batch_out))
    return fail(KARA_E_INVAL, "schedule arrays NULL");
  for (int32_t b = 0; b < n_seqs; ++b)
    if (watermarks[b] < 0 || watermarks[b] > seq_lens[b])
      return fail(KARA_E_INVAL, "sequence %d: watermark %d outside [0, %d]", b, watermarks[b], seq_lens[b]);
  int32_t n = 0;
  if (step > 0 && step % period == 0) {
    for (int32_t b = 0; b < n_seqs; ++b)
      if (selected[b] && (int64_t)seq_lens[b] - watermarks[b] >= window) batch_out[n++] = b;
  }
  *n_batch = n;
  return KARA_OK;
}

static int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

size_t kara_probe_scratch_bytes(void) {
  const int n_cu = device_cus();
  return n_cu > 0 ? (size_t)kara::probe_grid(n_cu) * 256 * sizeof(float) : 0;
}

kara_status kara_probe(int32_t kind, int64_t iters, void* dst_d, const void* src_d, size_t n_bytes, void* stream,
                       double* work_out) {
  TraceRange range("kara_probe");
  if (!work_out) return fail(KARA_E_INVAL, "work_out is NULL");
  if (kind < KARA_PROBE_MFMA || kind > KARA_PROBE_WRITE) return fail(KARA_E_INVAL, "probe kind %d unknown", kind);
  const int n_cu = device_cus();
  if (n_cu < 1) return fail(KARA_E_HIP, "no current HIP device");
  if (!dst_d) return fail(KARA_E_INVAL, "dst is NULL");
  if (kind == KARA_PROBE_COPY) {
    if (!src_d) return fail(KARA_E_INVAL, "src is NULL");
    if (n_bytes % 16 != 0 || !is_aligned(dst_d, 16) || !is_aligned(src_d, 16))
      return fail(KARA_E_INVAL, "copy probe: size and both addresses must be multiples of 16");
  } else if (kind == KARA_PROBE_READ) {
    if (!src_d) return fail(KARA_E_INVAL, "src is NULL");
    if (n_bytes % 16 != 0 || !is_aligned(src_d, 16) || !is_aligned(dst_d, 4))
      return fail(KARA_E_INVAL, "read probe: size and src must be multiples of 16, dst of 4");
  } else if (kind == KARA_PROBE_WRITE) {
    if (n_bytes % 16 != 0 || !is_aligned(dst_d, 16))
      return fail(KARA_E_INVAL, "write probe: size and dst must be multiples of 16");
  } else {
    if (iters < 1) return fail(KARA_E_INVAL, "iters must be >= 1");
    if (n_bytes < (size_t)kara::probe_grid(n_cu) * 256 * sizeof(float))
      return fail(KARA_E_INVAL, "dst holds %zu bytes, the probe writes %zu", n_bytes,
                  (size_t)kara::probe_grid(n_cu) * 256 * sizeof(float));
  }
  hipError_t e = kara::launch_probe(kind, iters, dst_d, src_d, n_bytes, n_cu, (hipStream_t)stream, work_out);
  return e == hipSuccess ? KARA_OK : hip_fail(e, "probe launch");
}

}  // extern "C"

// ---------------------------------------------------------------------------
// kara_compress_static: kara_compress for callers that cannot allocate device
// memory.  Its scratch (the scoring kernel's partial column sums and the kept
// positions) lives in one file-scope device array per GPU, loaded with the
// library's code object; host code reaches it only through the address
// hipGetSymbolAddress returns for the current device.

static __device__ __align__(256) char scratch[KARA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The array's device address on the current device, looked up on the first
// call on that device (with the device current) and kept.
kara_status static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(KARA_E_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "static scratch address");
    if (!ptr) return fail(KARA_E_HIP, "static scratch address is NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KARA_OK;
}

}  // namespace

extern "C" {

size_t kara_static_scratch_bytes(void) { return (size_t)KARA_STATIC_SCRATCH_BYTES; }

kara_status kara_compress_static(const kara_shape* shape, const kara_params* params, int32_t n_seqs,
                                 const void* q_window, void* kv_pool, int32_t n_blocks,
                                 const int32_t* block_table_h, const int32_t* block_table_d,
                                 int32_t max_blocks, const int32_t* seq_lens_h, const int32_t* seq_lens_d,
                                 kara_pool* pool, int32_t* new_block_table_h, int32_t* new_block_table_d,
                                 int32_t* new_seq_lens_h, void* stream, float* scores_out_d,
                                 int32_t* cand_out_d, int32_t* retained_out_d, void* const* stage_events) {
  TraceRange range("kara_compress_static");
  kara_status st;
  if ((st = check_shape(shape)) != KARA_OK) return st;
  if ((st = check_params(params)) != KARA_OK) return st;
  if (n_seqs < 0) return fail(KARA_E_INVAL, "n_seqs < 0");
  const size_t need = layout(shape, params, n_seqs).total;
  if (need > (size_t)KARA_STATIC_SCRATCH_BYTES)
    return fail(KARA_E_WORKSPACE,
                "kara_compress_static: %d sequences need %zu bytes of scratch, the static scratch holds %zu; "
                "compress fewer sequences per call or use kara_compress with a workspace",
                n_seqs, need, (size_t)KARA_STATIC_SCRATCH_BYTES);
  if (n_seqs == 0)
    return compress_impl(shape, params, 0, QuerySource{q_window, nullptr}, kv_pool, n_blocks, block_table_h,
                         block_table_d, max_blocks, seq_lens_h, seq_lens_d, pool, new_block_table_h,
                         new_block_table_d, new_seq_lens_h, nullptr, 0, stream, scores_out_d, cand_out_d,
                         retained_out_d, stage_events);
  void* ptr = nullptr;
  if ((st = static_scratch(&ptr)) != KARA_OK) return st;
  return compress_impl(shape, params, n_seqs, QuerySource{q_window, nullptr}, kv_pool, n_blocks, block_table_h,
                       block_table_d, max_blocks, seq_lens_h, seq_lens_d, pool, new_block_table_h,
                       new_block_table_d, new_seq_lens_h, ptr, (size_t)KARA_STATIC_SCRATCH_BYTES, stream,
                       scores_out_d, cand_out_d, retained_out_d, stage_events);
}

}  // extern "C"
