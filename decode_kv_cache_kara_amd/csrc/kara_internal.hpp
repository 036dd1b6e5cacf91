// Internal launch interface between the C ABI front end (kara_api.cpp) and the
// gfx950 kernels.  Not installed; the public surface is include/kara.h.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace kara {

constexpr int kMaxWindow = 4096;
constexpr int kMaxRegion = 2048;

// Rows (query-head x window-position pairs) scored by one workgroup of the
// score kernel (16 waves x 32 rows).
constexpr int kScoreRowsPerChunk = 512;

struct ScoreArgs {
  const void* q;          // [S][Lyr][W][Hq][D]
  const void* pool;       // [Lyr][2][NB][Hkv][bs][D]
  const int32_t* table;   // [S][MB]
  const int32_t* lens;    // [S]
  float* out;             // [U][n_split][C]: partial column sums of each row chunk
  int S, Lyr, Hq, Hkv, G, D, bs, bs_shift, NB, MB, W, C;
  int n_split;            // row chunks per unit = ceil(G*W / kScoreRowsPerChunk)
  int n_units;            // S * Lyr * Hkv
  float c;                // log2(e) / sqrt(D)
  int unidirectional;     // 1: query i sees window keys j <= i only
  // Query states from a ring instead of q: sequence b's window row i is ring
  // position (q_counts[b] - W + i) mod W of ring row q_slots[b].
  const int32_t* q_slots; // null: q is [S][Lyr][W][Hq][D]
  const int32_t* q_counts;
  int q_n_slots;
  // Resident-key scoring of windows longer than one key block: per-row
  // normaliser inputs [U][G*W] and per-unit exact-route flags [U] (workspace).
  float* zrow;
  int32_t* uflags;
  int key_lo, key_hi;     // resident key range of one launch (set by the launcher)
};

inline int score_chunks(int G, int W) {
  return (G * W + kScoreRowsPerChunk - 1) / kScoreRowsPerChunk;
}

// Scoring with the window's keys resident in registers
// (kara_score_resident.hip): bf16 states, head size 128, windows of at most
// 2048 keys (one pass up to 1024 keys, three launches over two key blocks
// beyond), at most 16384 rows per unit, the method's bidirectional scoring.
// It writes each unit's scores directly (one "chunk" per unit).
constexpr int kResidentBlock = 1024;
constexpr int kResidentMaxWindow = 2 * kResidentBlock;
constexpr int kResidentMaxRows = 16384;

inline bool use_resident(int dtype, int D, int W, int G, int unidirectional) {
  return dtype == 1 && D == 128 && W <= kResidentMaxWindow && G * W <= kResidentMaxRows && !unidirectional;
}

// Whether the resident scorer needs the per-row and per-unit workspace.
inline bool resident_two_blocks(int dtype, int D, int W, int G, int unidirectional) {
  return use_resident(dtype, D, W, G, unidirectional) && W > kResidentBlock;
}

// N-tiles of 16 keys per wave (2, 4, 6 or 8) that hold n_keys keys.
int resident_tiles(int n_keys);

// Partial column-sum rows per unit that the scorer writes.
inline int score_splits(int dtype, int D, int W, int G, int unidirectional) {
  return use_resident(dtype, D, W, G, unidirectional) ? 1 : score_chunks(G, W);
}

hipError_t launch_score(const ScoreArgs& a, int dtype, hipStream_t stream);
hipError_t launch_score_resident(const ScoreArgs& a, hipStream_t stream);

// Sums the n_split partial rows of every unit (in chunk order) into scores.
hipError_t launch_reduce(const float* partials, float* scores, int n_units, int n_split, int C,
                         hipStream_t stream);

enum SelectMode { kSelectTopK = 0, kSelectT2C = 1, kSelectFull = 2 };

struct SelectArgs {
  const float* partials;  // [U][n_split][C]; unit scores are the chunk-ordered sums
  int n_split;
  const int32_t* cand_in; // [U][K] (kSelectT2C only)
  float* scores_out;      // optional [U][C]
  int32_t* cand_out;      // optional [U][K]
  int32_t* retained_out;  // [U][R] (kSelectT2C / kSelectFull)
  int n_units, C, K, R;
  int mode;
  int no_chunks;          // 1: the kept set is the top-R set (no Token2Chunk)
};

hipError_t launch_select(const SelectArgs& a, hipStream_t stream);

struct AppendArgs {
  const void* q;              // [S][n_lyr_in][Hq][D]
  const void* k;              // [S][n_lyr_in][Hkv][D]
  const void* v;
  void* pool;                 // [Lyr][2][NB][Hkv][bs][D]
  void* ring;                 // [n_slots][Lyr][W][Hq][D]
  const int32_t* table;       // [S][MB]
  const int32_t* positions;   // [S] physical position of the new token
  const int32_t* slots;       // [S]
  const int32_t* counts;      // [S] index of the new token among those produced
  int S, Lyr, n_lyr_in, layer, Hq, Hkv, row_bytes, bs, NB, MB, W, n_slots;
};

hipError_t launch_append(const AppendArgs& a, hipStream_t stream);

// Tokens of one (sequence, KV head) per decode-attention workgroup: 1024 when
// a launch has at least kAttnBigGrid workgroups of that size, else 512
// (measured: 1024 is 6 % faster on one-layer caches of the Qwen3-14B-shaped
// batch at its compacted lengths, 25 % slower on the Qwen3-4B-shaped batch's
// compacted cache, whose launch then has about 2.3k workgroups).
constexpr int kAttnChunkMin = 512;
constexpr int kAttnChunkMax = 1024;
constexpr long kAttnBigGrid = 8192;

struct AttnArgs {
  const void* q;              // [S][Hq][D]
  const void* pool;           // [Lyr][2][NB][Hkv][bs][D]
  const int32_t* table;       // [S][MB]
  const int32_t* lens;        // [S]
  float* part_o;              // [S][Hq][n_split][D]
  float* part_ml;             // [S][Hq][n_split][2]: max (log2 units), sum
  float* out;                 // [S][Hq][D]
  int S, layer, Hq, Hkv, D, bs, bs_shift, NB, MB, n_split;
  int chunk;                  // tokens per split: kAttnChunkMin or kAttnChunkMax
  float c;                    // log2(e) / sqrt(D)
};

hipError_t launch_attention(const AttnArgs& a, int dtype, hipStream_t stream);
// The bf16 attention kernel's loads alone (a measurement aid; dst: 4 bytes).
hipError_t launch_paged_read_probe(const AttnArgs& a, uint32_t* dst, hipStream_t stream);

struct CompactArgs {
  void* pool;                 // [Lyr][2][NB][Hkv][bs][D]
  const int32_t* old_table;   // [S][MB]
  const int32_t* new_table;   // [S][MB]
  const int32_t* lens;        // [S] (old lengths)
  const int32_t* retained;    // [S][Lyr][Hkv][R]
  int S, Lyr, Hkv, row_bytes, bs, NB, MB, W, B, R;
};

hipError_t launch_compact(const CompactArgs& a, hipStream_t stream);

// Measurement probes (kara_probe.hip): workgroups per launch of kinds 0, 1, 3
// on a device with n_cu compute units, and the launch; *work receives the
// launch's work in the kind's unit (flops, elements, bytes, logits).
int probe_grid(int n_cu);
hipError_t launch_probe(int kind, int64_t iters, void* dst, const void* src, size_t n_bytes, int n_cu,
                        hipStream_t stream, double* work);

}  // namespace kara
