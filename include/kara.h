/*
 * kara.h - C ABI of the Kara decode-time KV-cache compression step on AMD
 * Instinct MI355X (gfx950).
 *
 * The step, per sequence b, layer l and KV head h ("unit"), over the trailing
 * window of W tokens of the sequence:
 *   1. score   every key j < C = W - B of the window by the softmax attention
 *              that ALL W window queries of the head's query group give it,
 *              each softmax over all W window keys with no causal mask;
 *   2. top-K   keep the K best-scored keys as candidates;
 *   3. chunks  expand gaps between consecutive candidates into chunks, filling
 *              a budget of R kept tokens of the region;
 *   4. compact copy the kept K/V rows into fresh blocks of the paged cache and
 *              return the sequence's old trailing blocks to the free pool.
 * Sources: "Technical Summary: Kara - Sliding-Window KV Cache Compression for
 * Efficient Serving of Reasoning LLMs" (gist.science), Methodology 1
 * (Mechanism, Rationale, Selection), 2 (Process, Outcome) and 3 (Periodic
 * Compression Policy); the paper's Abstract (decoding-time compression of the
 * recently generated context; expanding a subset of the selected pairs into
 * chunks; adaptation to PagedAttention).
 *
 * Readings this library fixes where the pages are silent: softmax scale
 * 1/sqrt(D); query head q belongs to KV head q / G (G = Hq / Hkv); Top-K ties
 * go to the lower position; chunk score (s[a] + s[b]) / (g + 2) for
 * consecutive candidates a < b with g = b - a - 1 > 0, computed in float32
 * (round-to-nearest add, then divide); chunks accepted as the longest prefix of
 * the (score desc, left endpoint asc) order whose gaps fit in R - K; the
 * highest-scored remaining positions (ties to the lower position) top the set
 * up to exactly R; if R < K the kept set is the top-R set.  Every (layer, head)
 * thus keeps exactly R tokens, so one block table and one length per sequence
 * stay valid and the new lengths are known on the host before any kernel runs.
 *
 * Memory layouts (row-major, innermost last):
 *   q_window  [n_seqs][n_layers][W][n_q_heads][head_dim]            (dtype)
 *   kv_pool   [n_layers][2][n_blocks][n_kv_heads][block_size][head_dim]
 *             index 1 of the second axis: 0 = K, 1 = V                 (dtype)
 *   tables    [n_seqs][max_blocks] int32 block ids
 *   scores    [n_seqs][n_layers][n_kv_heads][C] float32
 *   cand      [n_seqs][n_layers][n_kv_heads][K] int32, ascending
 *   retained  [n_seqs][n_layers][n_kv_heads][R] int32, ascending, in [0, C)
 * Window-local position i of sequence b is token lens[b] - W + i.
 * q_window, kv_pool and a query ring must be 16-byte aligned (the kernels move
 * 16-byte pieces, the scorer straight from global memory into LDS); other
 * base addresses return KARA_E_INVAL.
 *
 * Ownership: the caller owns every buffer and the stream.  The library never
 * allocates device memory; kara_compress and kara_score use a caller-provided
 * device workspace of kara_workspace_bytes() bytes.  A kara_pool is host
 * memory owned by the library between kara_pool_create and kara_pool_destroy.
 * "dev" pointers are device memory, "host" pointers host memory.
 *
 * Errors: every entry point validates all of its arguments before any side
 * effect.  A non-OK status from validation means nothing changed (pool, host
 * outputs and device memory are untouched).  KARA_E_HIP means a HIP call
 * failed after validation; work already enqueued may have run and the stream
 * should be treated as poisoned.  A kara_pool is changed only by a call that
 * returns KARA_OK (on KARA_E_HIP the fresh blocks stay free and the old ones
 * stay with their sequences), but the host outputs of kara_compress may
 * already hold the planned tables and lengths.  kara_last_error() returns a
 * message for the last non-OK status of the calling thread.
 *
 * Ordering: kernels are enqueued on `stream` (a hipStream_t; NULL is the null
 * stream) and the calls return without waiting for them.  Host outputs are
 * valid on return; device outputs are valid once the stream reaches the call.
 * Entry points are not thread-safe with respect to the same kara_pool.
 */
#ifndef KARA_H
#define KARA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KARA_OK = 0,
  KARA_E_INVAL = 1,        /* invalid argument; nothing changed */
  KARA_E_NOBLOCKS = 2,     /* the free pool holds too few blocks; nothing changed */
  KARA_E_HIP = 3,          /* a HIP runtime call failed after validation */
  KARA_E_UNSUPPORTED = 4,  /* shape or dtype the kernels are not built for; nothing changed */
  KARA_E_WORKSPACE = 5     /* workspace NULL or smaller than kara_workspace_bytes(); nothing changed */
} kara_status;

typedef enum { KARA_F32 = 0, KARA_BF16 = 1 } kara_dtype;

/* Model and cache geometry.  Supported: head_dim 64 or 128; n_q_heads a
 * multiple of n_kv_heads; block_size >= 1; dtype KARA_F32 or KARA_BF16. */
typedef struct {
  int32_t n_layers;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t dtype;           /* kara_dtype */
} kara_shape;

/* Ablation flags for kara_params.flags ("Technical Summary: Kara",
 * Experimental Results, Ablation Studies: the bidirectional scoring and the
 * Token2Chunk module are each removed in turn).  0 is the method itself. */
enum {
  /* Unidirectional scoring: window query i takes its softmax over window keys
   * j <= i only (causal attention), so key j is scored by the queries at and
   * after it. */
  KARA_UNIDIRECTIONAL = 1,
  /* Token2Chunk off: the kept set is the top-R set of the region (ties to the
   * lower position); candidates are never expanded into chunks. */
  KARA_NO_CHUNKS = 2
};

/* Method parameters: window W, protected buffer B, candidates K, budget R,
 * ablation flags.  Valid: 1 <= W <= 4096, 0 <= B < W, C = W - B <= 2048,
 * 1 <= K <= C, 1 <= R <= C, flags a combination of the KARA_UNIDIRECTIONAL
 * and KARA_NO_CHUNKS bits. */
typedef struct {
  int32_t window;
  int32_t protect;
  int32_t top_k;
  int32_t budget;
  int32_t flags;
} kara_params;

/* Host free list of the paged cache's block ids (the paper's Abstract adapts
 * the method to PagedAttention; "Technical Summary: Kara", Methodology 3:
 * compression rewrites the trailing blocks of a sequence and frees what they
 * held).  Allocation pops the front, freeing pushes the back (first in, first
 * out), so block assignment is deterministic.  The pool object is host memory
 * owned by the library (create / destroy); ids refer to blocks of the
 * caller's device cache. */
typedef struct kara_pool kara_pool;

/* Message for the calling thread's last non-OK status ("" if none); the
 * string is owned by the library and valid until the thread's next call. */
const char* kara_last_error(void);

/* Library version string. */
const char* kara_version(void);

/* Creates a pool over ids [0, n_blocks) whose free list is free_ids[0..n_free)
 * in that order (front first).  Ids must be in range and distinct.
 * KARA_E_INVAL on bad arguments (*out untouched). */
kara_status kara_pool_create(int32_t n_blocks, const int32_t* free_ids, int32_t n_free,
                             kara_pool** out);

/* Pops n ids from the front into ids_out[0..n).  KARA_E_NOBLOCKS if fewer than
 * n are free (nothing popped). */
kara_status kara_pool_alloc(kara_pool* pool, int32_t n, int32_t* ids_out);

/* Pushes ids[0..n) to the back, in order.  KARA_E_INVAL if an id is out of
 * range, already free or repeated (nothing pushed). */
kara_status kara_pool_free(kara_pool* pool, const int32_t* ids, int32_t n);

/* Number of free ids. */
int32_t kara_pool_num_free(const kara_pool* pool);

/* Copies up to cap free ids, front first, into ids_out; returns how many. */
int32_t kara_pool_snapshot(const kara_pool* pool, int32_t* ids_out, int32_t cap);

void kara_pool_destroy(kara_pool* pool);

/* Device workspace bytes that kara_compress and kara_score need for n_seqs
 * sequences of this shape (0 on invalid arguments): the scorer's column sums
 * of every unit ("Technical Summary: Kara", Methodology 1: scores accumulated
 * over all window queries), for windows of more than 1024 keys one float per
 * (unit, query row) and one flag per unit, and the kept positions of every
 * unit (Methodology 2).  The caller allocates it (256-byte aligned) and owns
 * it; the library keeps no pointer past the call's stream order. */
size_t kara_workspace_bytes(const kara_shape* shape, const kara_params* params, int32_t n_seqs);

/* Whole step for n_seqs sequences (the selected ones, in call order).
 *
 * q_window       dev   window query states (layout above), dtype of shape.
 * kv_pool        dev   K/V pool; the kept rows are written into fresh blocks.
 *                      Rows of all other blocks are not written.
 * n_blocks             blocks in the pool.
 * block_table_h  host  [n_seqs][max_blocks]; entries of positions
 *                      (lens[b]-W)/bs .. ceil(lens[b]/bs)-1 must be distinct
 *                      valid ids not in the free list; earlier entries are
 *                      copied unchanged and never read.
 * block_table_d  dev   device copy of block_table_h (same contents).
 * seq_lens_h     host  [n_seqs] lengths, each >= W and <= max_blocks * bs.
 * seq_lens_d     dev   device copy of seq_lens_h.
 * pool                 free list; on success the fresh blocks (sum over b of
 *                      ceil((p_b + R + B) / bs), p_b = (lens[b] - W) mod bs)
 *                      are popped, sequences in call order, and then the old
 *                      blocks of positions (lens[b]-W)/bs .. ceil(lens[b]/bs)-1
 *                      are pushed, sequences in call order and positions
 *                      ascending.  Reuse of a pushed block is safe for work
 *                      enqueued later on the same stream.
 * new_block_table_h host out [n_seqs][max_blocks]: positions before the
 *                      boundary block unchanged, then the fresh ids, then -1.
 * new_block_table_d dev out, filled by a stream-ordered copy of
 *                      new_block_table_h (pinned host memory must stay
 *                      unchanged until the stream passes the call).
 * new_seq_lens_h host out [n_seqs]: lens[b] - C + R.
 * workspace      dev   kara_workspace_bytes() bytes, 256-byte aligned.
 * stream               hipStream_t.
 * scores_out_d, cand_out_d, retained_out_d   optional dev outputs (NULL: not
 *                      written) in the layouts above.
 * params->flags        ablations: KARA_UNIDIRECTIONAL scores with causal
 *                      window attention, KARA_NO_CHUNKS keeps the top-R set
 *                      (the candidates in cand_out_d are still the top-K).
 * stage_events         optional (NULL: none) array of 4 hipEvent_t, recorded
 *                      on `stream` before the scoring kernel, after it, after
 *                      the selection kernel and after the compaction kernel,
 *                      for callers that time the stages.
 * Errors: KARA_E_INVAL, KARA_E_UNSUPPORTED, KARA_E_WORKSPACE, KARA_E_NOBLOCKS
 * (all with nothing changed), KARA_E_HIP. */
kara_status kara_compress(const kara_shape* shape, const kara_params* params, int32_t n_seqs,
                          const void* q_window, void* kv_pool, int32_t n_blocks,
                          const int32_t* block_table_h, const int32_t* block_table_d,
                          int32_t max_blocks, const int32_t* seq_lens_h,
                          const int32_t* seq_lens_d, kara_pool* pool,
                          int32_t* new_block_table_h, int32_t* new_block_table_d,
                          int32_t* new_seq_lens_h, void* workspace, size_t workspace_bytes,
                          void* stream, float* scores_out_d, int32_t* cand_out_d,
                          int32_t* retained_out_d, void* const* stage_events);

/* Stage 1 alone: window scores of every unit into scores_d (dev, [n_seqs]
 * [n_layers][n_kv_heads][C] float32).  Arguments as for kara_compress;
 * top_k and budget are validated but unused; the KARA_UNIDIRECTIONAL flag
 * selects the unidirectional ablation.  Summary, Methodology 1 (Mechanism,
 * Rationale). */
kara_status kara_score(const kara_shape* shape, const kara_params* params, int32_t n_seqs,
                       const void* q_window, const void* kv_pool, int32_t n_blocks,
                       const int32_t* block_table_h, const int32_t* block_table_d,
                       int32_t max_blocks, const int32_t* seq_lens_h, const int32_t* seq_lens_d,
                       float* scores_d, void* workspace, size_t workspace_bytes, void* stream);

/* Stage 2 alone (with top_k = R it is also the whole selection of the
 * KARA_NO_CHUNKS ablation): for each of n_units rows of `region` float32 scores (dev,
 * finite), the top_k positions with the largest score (ties to the lower
 * position, -0 equal to +0), ascending, into cand_d (dev [n_units][top_k]).
 * Summary, Methodology 1 (Selection).  1 <= top_k <= region <= 2048. */
kara_status kara_topk(int32_t n_units, int32_t region, int32_t top_k, const float* scores_d,
                      int32_t* cand_d, void* stream);

/* Stage 3 alone: Token2Chunk of each unit from its scores (dev [n_units]
 * [region]) and ascending candidates (dev [n_units][top_k], strictly
 * increasing, in [0, region)), into retained_d (dev [n_units][budget]).
 * Summary, Methodology 2 (Process, Outcome).  1 <= budget <= region.
 * Candidates that break the stated form give an unspecified (but in-range,
 * fault-free) result. */
kara_status kara_token2chunk(int32_t n_units, int32_t region, int32_t top_k, int32_t budget,
                             const float* scores_d, const int32_t* cand_d, int32_t* retained_d,
                             void* stream);

/* Stage 4 alone: the bookkeeping and copy of kara_compress for given kept
 * positions retained_d (dev [n_seqs][n_layers][n_kv_heads][R], ascending in
 * [0, C); out-of-range entries are clamped, never dereferenced out of
 * bounds).  Pool, tables and lengths as for kara_compress.  Summary,
 * Methodology 3 (Periodic Compression Policy: trailing blocks). */
kara_status kara_paged_compact(const kara_shape* shape, const kara_params* params, int32_t n_seqs,
                               void* kv_pool, int32_t n_blocks, const int32_t* block_table_h,
                               const int32_t* block_table_d, int32_t max_blocks,
                               const int32_t* seq_lens_h, const int32_t* seq_lens_d,
                               const int32_t* retained_d, kara_pool* pool,
                               int32_t* new_block_table_h, int32_t* new_block_table_d,
                               int32_t* new_seq_lens_h, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the whole
 * step exactly as kara_compress, with the same arguments minus the
 * workspace, and the same kernels and results.  Its scratch (the partial
 * column sums and the kept positions, kara_workspace_bytes() bytes) is a
 * device array of KARA_STATIC_SCRATCH_BYTES (256 MiB) inside the library,
 * one per GPU, held until the process ends; its address is looked up on the
 * first call on each device (make that call outside graph capture).  The call
 * allocates no device memory.  Calls whose scratch need exceeds the array
 * fail with KARA_E_WORKSPACE and change nothing (at W=1024, C=896 the array
 * holds about 9,000 units of (sequence, layer, KV head); at W=2048, C=1792
 * about 1,800).  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (other host threads, other streams) race and
 * must be serialised by the caller; nothing in it needs clearing between
 * calls (every byte a call reads was written earlier in the same call). */
#define KARA_STATIC_SCRATCH_BYTES ((size_t)256 << 20)
size_t kara_static_scratch_bytes(void);
kara_status kara_compress_static(const kara_shape* shape, const kara_params* params, int32_t n_seqs,
                                 const void* q_window, void* kv_pool, int32_t n_blocks,
                                 const int32_t* block_table_h, const int32_t* block_table_d,
                                 int32_t max_blocks, const int32_t* seq_lens_h,
                                 const int32_t* seq_lens_d, kara_pool* pool,
                                 int32_t* new_block_table_h, int32_t* new_block_table_d,
                                 int32_t* new_seq_lens_h, void* stream, float* scores_out_d,
                                 int32_t* cand_out_d, int32_t* retained_out_d,
                                 void* const* stage_events);

/* ------------------------------------------------------------------------
 * Around the step: keeping the window's query states, and decode attention
 * over the (compressed) paged cache.
 * ------------------------------------------------------------------------ */

/* Window query states kept on the device ("Technical Summary: Kara",
 * Methodology 1, Mechanism: the query states of all window tokens score the
 * region, so they must still exist when the window is scored).  Each sequence
 * slot holds the query states of its last W produced tokens: token n (counted
 * over everything the sequence has produced, whether or not it was later
 * compacted away) sits at ring position n mod W.
 *   q_ring    dev [n_slots][n_layers][W][n_q_heads][head_dim] (dtype)
 *   n_slots   ring rows
 *   window    W the ring was built with; kara_compress_ring and kara_append
 *             reject a call whose window differs (KARA_E_INVAL)
 *   slots_d   dev [n_seqs] ring row of each sequence of the call
 *   counts_d  dev [n_seqs] tokens produced so far: for kara_compress_ring the
 *             count N, so the window is tokens N - W .. N - 1; for
 *             kara_append the index of the token being appended.
 * Under the periodic schedule's watermark a window never reaches back into a
 * compacted region, so its W tokens are the last W produced and the trailing
 * W physical tokens of the cache.  Device indices are clamped (slots to
 * [0, n_slots)), never dereferenced out of bounds. */
typedef struct {
  void* q_ring;
  int32_t n_slots;
  int32_t window;
  const int32_t* slots_d;
  const int32_t* counts_d;
} kara_query_ring;

/* One decode step's states of n_seqs sequences, at one layer (layer in
 * [0, n_layers): q_d [n_seqs][Hq][D], k_d and v_d [n_seqs][Hkv][D]) or at
 * every layer (layer = -1: q_d [n_seqs][n_layers][Hq][D], k_d and v_d
 * [n_seqs][n_layers][Hkv][D]), all dev and of the shape's dtype.  K and V go
 * to physical position positions_d[b] (dev) of sequence b through
 * block_table_d (dev [n_seqs][max_blocks]; the caller has allocated the
 * block); the query states go to ring position counts_d[b] mod W of ring row
 * slots_d[b].  Positions are clamped to the table and block ids to the pool.
 * Errors: KARA_E_INVAL, KARA_E_UNSUPPORTED (nothing written), KARA_E_HIP. */
kara_status kara_append(const kara_shape* shape, int32_t window, int32_t n_seqs, int32_t layer,
                        const void* q_d, const void* k_d, const void* v_d, void* kv_pool,
                        int32_t n_blocks, const int32_t* block_table_d, int32_t max_blocks,
                        const int32_t* positions_d, const kara_query_ring* ring, void* stream);

/* kara_compress with the window query states read from a ring (above)
 * instead of a [n_seqs][n_layers][W][Hq][D] array: row i of sequence b's
 * window is ring position (counts_d[b] - W + i) mod W of ring row
 * slots_d[b].  Every other argument, output and error as for kara_compress. */
kara_status kara_compress_ring(const kara_shape* shape, const kara_params* params, int32_t n_seqs,
                               const kara_query_ring* ring, void* kv_pool, int32_t n_blocks,
                               const int32_t* block_table_h, const int32_t* block_table_d,
                               int32_t max_blocks, const int32_t* seq_lens_h,
                               const int32_t* seq_lens_d, kara_pool* pool,
                               int32_t* new_block_table_h, int32_t* new_block_table_d,
                               int32_t* new_seq_lens_h, void* workspace, size_t workspace_bytes,
                               void* stream, float* scores_out_d, int32_t* cand_out_d,
                               int32_t* retained_out_d, void* const* stage_events);

/* Device workspace bytes kara_decode_attention needs for n_seqs sequences of
 * at most max_len tokens (0 on invalid arguments). */
size_t kara_attention_workspace_bytes(const kara_shape* shape, int32_t n_seqs, int32_t max_len);

/* Decode attention at one layer over every sequence's cached tokens, read
 * through its block table (Paper, Abstract: the compressed cache is served
 * through PagedAttention; this is how the compacted tables are consumed).
 *   q_d          dev [n_seqs][Hq][D] query states (dtype)
 *   out_d        dev [n_seqs][Hq][D] float32:
 *                out[b][g] = sum_t softmax_t(q[b][g] . k_t / sqrt(D)) v_t
 *                over tokens t < lens[b] of KV head g / G at `layer`
 *   seq_lens_h   host [n_seqs] lengths in [1, max_blocks * bs] (sizes the
 *                launch); seq_lens_d the device copy (read by the kernels,
 *                clamped to the same range)
 *   workspace    dev, kara_attention_workspace_bytes(shape, n_seqs,
 *                max(seq_lens_h)) bytes, 256-byte aligned.
 * Supported: n_q_heads / n_kv_heads <= 8, and n_blocks * n_kv_heads *
 * block_size < 2^32 (a layer's K rows are numbered in 32 bits).  Block ids
 * are clamped to the pool.
 * Errors: KARA_E_INVAL, KARA_E_UNSUPPORTED, KARA_E_WORKSPACE (nothing
 * written), KARA_E_HIP. */
kara_status kara_decode_attention(const kara_shape* shape, int32_t n_seqs, int32_t layer,
                                  const void* q_d, const void* kv_pool, int32_t n_blocks,
                                  const int32_t* block_table_d, int32_t max_blocks,
                                  const int32_t* seq_lens_h, const int32_t* seq_lens_d,
                                  float* out_d, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* Periodic compression schedule ("Technical Summary: Kara", Methodology 3,
 * Periodic Compression Policy: every fixed number of decode steps the
 * trailing blocks of selected sequences are compressed; Summary, Methodology
 * intro and Paper, Abstract: compression acts only on recently generated
 * context).
 *
 * At a decode step `step` that is a positive multiple of `period`, a sequence
 * b is compressed when the caller selected it (selected[b] != 0; the random
 * draw that picks the subset is the caller's) and its whole trailing window
 * lies after its watermark: seq_lens[b] - watermarks[b] >= window.  The
 * watermark is the length below which tokens have already been through a
 * compressed region; after a compression the caller sets it to
 * new_len - protect, so the protected tokens are scored again next time and
 * no token is compressed twice.  A fresh sequence has watermark 0.
 * Writes the eligible sequence indices, ascending, to batch_out[0..*n_batch)
 * (batch_out holds n_seqs entries).  At other steps *n_batch = 0.
 * KARA_E_INVAL on bad arguments (nothing written). */
kara_status kara_schedule_step(int64_t step, int32_t period, int32_t window, int32_t n_seqs,
                               const int32_t* seq_lens, const int32_t* watermarks,
                               const uint8_t* selected, int32_t* batch_out, int32_t* n_batch);

/* Host-only plan of a compression step for callers that size pools or
 * simulate schedules ("Technical Summary: Kara", Methodology 3: the trailing
 * blocks of a compressed sequence are replaced, the rest of its table is
 * kept).  For each sequence b (seq_lens_h[b] >= W): new_lens_out[b] =
 * seq_lens_h[b] - C + R, the length kara_compress returns, and
 * fresh_blocks_out[b] = ceil((p_b + R + B) / block_size) with
 * p_b = (seq_lens_h[b] - W) mod block_size, the fresh blocks it pops for b.
 * The same arithmetic as kara_compress's own plan; touches no pool.
 * KARA_E_INVAL / KARA_E_UNSUPPORTED on bad arguments (nothing written). */
kara_status kara_plan_lengths(const kara_params* params, int32_t block_size, int32_t n_seqs,
                              const int32_t* seq_lens_h, int32_t* new_lens_out, int32_t* fresh_blocks_out);

/* ------------------------------------------------------------------------
 * Serving-policy simulator (host only).  Periodic window compression against
 * threshold-triggered whole-cache compression under a KV memory cap and a
 * concurrency limit ("Technical Summary: Kara", Problem Statement 1:
 * threshold triggering lowers throughput as concurrency grows; Methodology
 * 3: the periodic policy; paper, Fig. 1 caption: compression frees memory so
 * more sequences decode at once).  Per-step costs are inputs (measured kernel
 * timings); the rules of a step are, in order:
 *   1. admission: waiting requests enter in order while fewer than max_batch
 *      run and the pool holds the prompt's blocks plus one spare block;
 *   2. decode: each running sequence, in admission order, appends one token,
 *      taking a new block when its length is a multiple of block_size (with
 *      no free block it stalls for the step); if all of them stalled, the
 *      most recently admitted one is preempted: its blocks are freed and it
 *      returns to the front of the queue to restart from its prompt;
 *   3. sequences that generated all their tokens leave and free their blocks;
 *   4. compression: periodic - at multiples of `period`, every running
 *      sequence with length - watermark >= window goes from L to
 *      L - (window - protect) + budget tokens, its tail from block
 *      (L - window) / bs on rewritten into ceil(((L - window) mod bs + budget
 *      + protect) / bs) blocks, watermark = new length - protect;
 *      threshold - every running sequence with length >= threshold keeps
 *      `keep` tokens (ceil(keep / bs) blocks);
 *   5. step time = decode_ms_fixed + decode_ms_per_token * (cached tokens of
 *      the sequences running at the start of step 2) + compression cost
 *      (periodic: compress_ms_per_seq per sequence; threshold:
 *      compress_ms_per_key times the sequence's length).
 * Request i generates kara_sim_gen_length(config, i) tokens: gen_min +
 * SplitMix64(seed + i) mod (gen_max - gen_min + 1).
 * ------------------------------------------------------------------------ */

enum { KARA_POLICY_PERIODIC = 0, KARA_POLICY_THRESHOLD = 1, KARA_POLICY_NONE = 2 /* no compression */ };

typedef struct {
  int32_t policy;              /* KARA_POLICY_* */
  int32_t n_requests, max_batch, cap_blocks, block_size;
  int32_t prompt_len, gen_min, gen_max;
  uint64_t seed;
  int32_t window, protect, budget, period;   /* periodic */
  int32_t threshold, keep;                    /* threshold */
  double decode_ms_fixed, decode_ms_per_token;
  double compress_ms_per_seq, compress_ms_per_key;
  int32_t max_steps;
} kara_sim_config;

typedef struct {
  int64_t steps, tokens, compressions, stalls, peak_blocks;
  int64_t preemptions, wasted;  /* restarts, and tokens generated before them */
  int32_t finished;            /* requests that generated all their tokens */
  double total_ms, compress_ms, mean_active;
} kara_sim_result;

/* Tokens request `request` generates (see above). */
int32_t kara_sim_gen_length(const kara_sim_config* config, int32_t request);

/* Runs the simulation until every request finished or max_steps steps.
 * Optional per-step outputs (NULL: not written), max_steps entries each:
 * running sequences after the step, compressions in the step, step time.
 * KARA_E_INVAL on inconsistent settings (nothing written). */
kara_status kara_policy_sim(const kara_sim_config* config, kara_sim_result* result,
                            int32_t* active_per_step, int32_t* compressions_per_step,
                            double* ms_per_step);

/* ---- Measurement aid: the chip's own ceilings ----------------------------
 * Not part of the compression step.  A fully loaded MI355X runs below the
 * clock its nominal peaks assume, so the benchmark sets each kernel's rate
 * against what this device reaches for the same kind of work:
 *   KARA_PROBE_MFMA  matrix cores alone: independent chains of 32x32x16 bf16
 *                    MFMAs, operands in registers; work in flops.
 *   KARA_PROBE_VALU  the scoring kernel's per-logit VALU work alone (one
 *                    multiply-add, one exp2, one add per element); work in
 *                    elements.
 *   KARA_PROBE_COPY  a streaming copy of n_bytes from src_d to dst_d with
 *                    16-byte nontemporal loads and stores; work in bytes read
 *                    plus bytes written.
 *   KARA_PROBE_MIX   the resident-key scoring kernel's tile loop without its
 *                    per-tile work: per logit 2 * 128 bf16 MFMA flops
 *                    (16x16x32, keys resident) and a multiply, exp2, row-sum
 *                    add and column FMA, interleaved as in that kernel, with
 *                    the query fragments read from LDS; work in logits.
 *   KARA_PROBE_READ  a streaming read of n_bytes from src_d with the copy's
 *                    loads and launch shape; dst_d is a 4-byte sink (written
 *                    only if the loaded words fold to a fixed value, in
 *                    practice never); work in bytes read.
 *   KARA_PROBE_WRITE a streaming write of n_bytes to dst_d with the copy's
 *                    stores and launch shape (src_d unused); work in bytes
 *                    written.
 * MFMA, VALU and MIX run `iters` loop iterations in each of two waves per
 * SIMD and write one float per thread to dst_d, which must hold
 * kara_probe_scratch_bytes() bytes (n_bytes gives its size).  COPY, READ and
 * WRITE ignore iters; n_bytes and their buffer addresses must be multiples
 * of 16 (READ's sink: of 4).  The launch is
 * enqueued on `stream` (the caller times it, e.g. with events); *work_out
 * receives the launch's work in the unit above.  dst_d and src_d are
 * caller-owned device buffers; src_d must hold n_bytes.  KARA_E_INVAL on bad
 * arguments (nothing launched); KARA_E_HIP when there is no current device or
 * the launch fails.  kara_probe_scratch_bytes() returns 0 when there is no
 * current device. */
enum { KARA_PROBE_MFMA = 0, KARA_PROBE_VALU = 1, KARA_PROBE_COPY = 2, KARA_PROBE_MIX = 3, KARA_PROBE_READ = 4,
       KARA_PROBE_WRITE = 5 };
size_t kara_probe_scratch_bytes(void);
kara_status kara_probe(int32_t kind, int64_t iters, void* dst_d, const void* src_d, size_t n_bytes, void* stream,
                       double* work_out);

/* Measurement aid, not part of the compression step: the memory traffic of
 * kara_decode_attention (bf16) alone, to set that kernel's rate against what
 * the same access pattern reaches on this device.  Takes the arguments of
 * kara_decode_attention except the query states, output and workspace, with
 * the same meaning, layout, validation and errors (KARA_E_UNSUPPORTED also for
 * a float32 shape), and launches a kernel with the same workgroup
 * decomposition (one split of 512 or 1024 tokens of one sequence and KV head
 * per workgroup, chosen by the same rule), the same block-id staging and the
 * same 16-byte loads of every cached token's K and V rows of `layer`, with no
 * arithmetic.  dst_d: 4 bytes of device memory, 4-byte aligned (written only
 * if the loaded words fold to a fixed value, in practice never).
 * *bytes_out receives the bytes the launch reads by definition:
 * sum(seq_lens_h) * n_kv_heads * 2 * head_dim * 2.  Enqueued on `stream`;
 * the caller times it. */
kara_status kara_probe_paged_read(const kara_shape* shape, int32_t n_seqs, int32_t layer, const void* kv_pool,
                                  int32_t n_blocks, const int32_t* block_table_d, int32_t max_blocks,
                                  const int32_t* seq_lens_h, const int32_t* seq_lens_d, void* dst_d,
                                  void* stream, double* bytes_out);

#ifdef __cplusplus
}
#endif

#endif /* KARA_H */
