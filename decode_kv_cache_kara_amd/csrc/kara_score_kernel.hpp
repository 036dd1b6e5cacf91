// Window scoring on gfx950 matrix cores.
//
// Per unit (sequence, layer, KV head) the rows are the G*W (window position,
// query head of the group) pairs and the columns are the W window keys.  The
// score of key j < C is the column sum of the row-softmaxed logits
// q.k/sqrt(D), every softmax running over all W keys with no mask
// ("Technical Summary: Kara", Methodology 1, Mechanism and Rationale).
//
// A column sum needs each row's softmax normaliser before that row's
// probabilities can be added, so every block of rows makes two passes over the
// keys, both on MFMA:
//   pass 1  S^T = K Q^T (keys on the MFMA M axis, queries on N): each lane owns
//           one query and 16 keys of a 32x32 tile, so the running row maximum
//           and exp-sum stay in the lane; the two lane halves merge at the end.
//   pass 2  S = Q K^T (queries on M, keys on N): each lane owns one key and 16
//           queries, so p = exp2(x*c - bias_row) is added into a per-lane
//           column accumulator; lane halves and waves merge through LDS.
// The same Q register fragments serve as the B operand of pass 1 and the A
// operand of pass 2 (for 32x32 MFMA both operands map lane l to matrix index
// l%32 and K-chunk l/32).  Key tiles of 64 rows are staged through LDS, double
// buffered, with a 16-byte row pad so the per-lane 16-byte reads do not
// collide on banks.
//
// Per logit, pass 1 needs an FMA, an exp2 and an add (its row maximum is
// taken once, from the first keys, see below) and pass 2 an FMA, an exp2 and
// an add, against 2*D MFMA flops.  On gfx950 v_exp_f32 occupies the VALU
// issue for about three FMAs and does not co-issue with other VALU work, so
// the VALU stream (about 11-13 ms at the Qwen3-4B 36-layer batch of 32) is
// longer than the MFMA stream (about 8 ms); the schedule keeps the VALU
// stream dense and hides the MFMAs under it:
//   * each wave owns 64 rows (two 32-row query tiles sharing every K
//     fragment read from LDS; at most 256 VGPRs, two waves per SIMD) and
//     software-pipelines over 32-key subtiles: the MFMAs of the next subtile
//     are issued between the exponentials of the current one (scheduling
//     groups below), so no wave waits for its own matrix results;
//   * LDS holds three 64-key tiles (two being multiplied, one being filled),
//     so there is one barrier per tile; the window's block ids are staged in
//     LDS once; sums use independent partial chains.

// Unidirectional ablation ("Technical Summary: Kara", Experimental Results,
// Ablation Studies): window query i sees keys j <= i only.  A workgroup then
// stops at the key tile that holds its last row's position, subtiles that
// cross a wave's diagonal are masked element by element, and the partial
// column sums of keys past the last tile are written as zeros.
//
// The window's query states come either as one array per call or from a ring
// that keeps each sequence's last W query states (row i of the window is then
// ring position (count - W + i) mod W); only the row addresses differ.
//
// One workgroup scores 512 rows of one unit.  The workgroups of a unit are
// dispatched back to back onto the same XCD (block ids are interleaved across
// the 8 XCDs) so that unit's K rows are fetched from HBM once and then served
// from that XCD's L2.  Each workgroup writes its 512-row partial column sums;
// the selection kernel adds the partials of a unit in chunk order, so results
// do not depend on scheduling.

// This header holds the kernel template; each dtype and head size is
// instantiated in a translation unit of its own (kara_score_<type>_d<D>.hip)
// so that the library builds in parallel.

#pragma once

#include "kara_internal.hpp"

#include <cmath>
#include <type_traits>

namespace kara {
namespace {


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// 32-row query tiles per wave.  For bf16 two tiles let every K fragment
// read from LDS feed two MFMAs and leave room in 256 VGPRs (two waves per
// SIMD) for the compiler to keep fragment reads ahead of their MFMAs
// (measured 3% faster than one tile at four waves per SIMD).  fp32 states
// (small workloads only) have twice the operand registers and keep one tile.
template <typename T>
struct ScoreCfg {
  static constexpr int kRT = sizeof(T) == 2 ? 2 : 1;
  static constexpr int kRowsPerWave = 32 * kRT;
  static constexpr int kWaves = kScoreRowsPerChunk / kRowsPerWave;
  static constexpr int kThreads = kWaves * 64;
  // one row tile: at most 128 VGPRs (four waves per SIMD); two: at most 256
  static constexpr int kMinWavesPerEU = kRT == 1 ? 4 : 2;
  // Keys per LDS tile (one barrier each).  128-key tiles halve the barriers
  // and fit in LDS for bf16 but measured within 1 % of 64-key tiles.
  static constexpr int kKeyTile = 64;
};


template <typename T>
struct Mma;

template <>
struct Mma<__bf16> {
  static constexpr int kStep = 16;    // reduction length per instruction
  static constexpr int kPerLane = 8;  // operand elements per lane
  typedef bf16x8 Frag;
  static __device__ __forceinline__ f32x16 run(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ Frag zero() {
    Frag z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
    return z;
  }
};

template <>
struct Mma<float> {
  static constexpr int kStep = 2;
  static constexpr int kPerLane = 1;
  typedef float Frag;
  static __device__ __forceinline__ f32x16 run(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ Frag zero() { return 0.0f; }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }


// Row (M index) of accumulator element r of lane `lane` in a 32x32 MFMA tile.
__device__ __forceinline__ int acc_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

template <typename T, int D, bool kUni>
__global__ __launch_bounds__(ScoreCfg<T>::kThreads, ScoreCfg<T>::kMinWavesPerEU) void score_kernel(ScoreArgs a) {
  constexpr int kRT = ScoreCfg<T>::kRT;
  constexpr int kRowsPerWave = ScoreCfg<T>::kRowsPerWave;
  constexpr int kWaves = ScoreCfg<T>::kWaves;
  constexpr int kThreads = ScoreCfg<T>::kThreads;
  constexpr int kKeyTile = ScoreCfg<T>::kKeyTile;
  constexpr int kSub = kKeyTile / 32;               // 32-key subtiles per tile
  using M = Mma<T>;
  typedef typename M::Frag Frag;
  constexpr int NK = D / M::kStep;
  constexpr int kRowBytes = D * (int)sizeof(T);
  constexpr int kStride = kRowBytes + 16;
  constexpr int kPiecesPerRow = kRowBytes / 16;
  constexpr int kTilePieces = kKeyTile * kPiecesPerRow;
  constexpr int kPerThread = (kTilePieces + kThreads - 1) / kThreads;

  __shared__ __attribute__((aligned(16))) char kbuf[3][kKeyTile * kStride];
  __shared__ float bias_lds[kWaves * kRowsPerWave];
  __shared__ float col_ring[2][kWaves][kKeyTile];
  __shared__ int32_t s_blk[kMaxWindow + 1];        // the window's block ids
  __shared__ int s_redo;                            // pass 1 must run again exactly

  // Block -> (unit, chunk).  Consecutive block ids go to different XCDs, so
  // unit = slot-group * 8 + xcd keeps all chunks of a unit on one XCD.
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int slot = bid >> 3;
  const int unit = (slot / a.n_split) * 8 + xcd;
  const int chunk = slot % a.n_split;
  if (unit >= a.n_units) return;  // uniform for the whole block

  const int h = unit % a.Hkv;
  const int bl = unit / a.Hkv;   // b * Lyr + l
  const int l = bl % a.Lyr;
  const int b = bl / a.Lyr;
  const int W = a.W, C = a.C, G = a.G;
  const int rows = G * W;
  const float c = a.c;

  // Device copies of lengths and tables are trusted only up to clamping: every
  // address stays inside the buffers whatever they hold.
  int L = a.lens[b];
  const int max_tok = a.MB * a.bs;
  L = L < W ? W : (L > max_tok ? max_tok : L);
  const int start = L - W;
  const int32_t* trow = a.table + (size_t)b * a.MB;
  // Window query rows: row i of the window is q[b][l][i], or, from a ring,
  // ring position (count - W + i) mod W of the sequence's ring row.
  size_t q_row0 = (size_t)bl * W;
  int ring_off = 0;
  if (a.q_slots) {
    int slot = a.q_slots[b];
    slot = slot < 0 ? 0 : (slot >= a.q_n_slots ? a.q_n_slots - 1 : slot);
    const int n = a.q_counts[b];
    q_row0 = ((size_t)slot * a.Lyr + l) * W;
    ring_off = (n < 0 ? 0 : n) % W;               // (n - W + i) mod W = (n + i) mod W
  }
  const T* qbase = (const T*)a.q + q_row0 * a.Hq * D + (size_t)h * G * D;
  const char* kbase = (const char*)a.pool +
      ((size_t)l * 2 * a.NB * a.Hkv * a.bs + (size_t)h * a.bs) * D * sizeof(T);
  const size_t blk_bytes = (size_t)a.Hkv * a.bs * D * sizeof(T);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row0 = chunk * kScoreRowsPerChunk + wave * kRowsPerWave;

  // Query fragments of this wave's rows, kept in registers for both passes.
  // Row r is window position r / G, head r % G of the group.
  Frag qf[kRT][NK];
#pragma unroll
  for (int qt = 0; qt < kRT; ++qt) {
    const int row = row0 + qt * 32 + (lane & 31);
    if (row < rows) {
      const int i = row / G, g = row - (row / G) * G;
      const int slot_i = i + ring_off < W ? i + ring_off : i + ring_off - W;
      const T* p = qbase + ((size_t)slot_i * a.Hq + g) * D + (lane >> 5) * M::kPerLane;
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) qf[qt][ks] = *(const Frag*)(p + ks * M::kStep);
    } else {
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) qf[qt][ks] = M::zero();
    }
  }

  // Global -> register staging of key tiles: a tile is fetched one tile ahead
  // of its LDS store.  Block sizes are powers of two (bs = 1 << bs_shift).
  // The window's block ids are staged in LDS first, so a tile's row
  // addresses need no global loads; a thread always moves the same row piece
  // of a tile, so only the tile offset changes between tiles.
  const int e0 = start >> a.bs_shift;
  const int n_e = ((start + W - 1) >> a.bs_shift) - e0 + 1;
  if (tid == 0) s_redo = 0;
  for (int i = tid; i < n_e; i += kThreads) {
    const int blk = trow[e0 + i];
    s_blk[i] = blk < 0 ? 0 : (blk >= a.NB ? a.NB - 1 : blk);
  }
  __syncthreads();
  typedef uint4 Stage[kPerThread];
  Stage stage0;
  const int bs_mask = (1 << a.bs_shift) - 1;
  auto load_tile = [&](Stage& st, int tile0) {
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int p = tid + u * kThreads;
      const int r = p / kPiecesPerRow, pc = p % kPiecesPerRow;
      const int j = tile0 + r;
      if (p < kTilePieces && j < W) {
        const int t = start + j;
        const char* src = kbase + (size_t)s_blk[(t >> a.bs_shift) - e0] * blk_bytes +
                          (size_t)(t & bs_mask) * kRowBytes + pc * 16;
        st[u] = *(const uint4*)src;
      } else {
        st[u] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  auto store_tile = [&](const Stage& st, int buf) {
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int p = tid + u * kThreads;
      if (p < kTilePieces) {
        const int r = p / kPiecesPerRow, pc = p % kPiecesPerRow;
        *(uint4*)(&kbuf[buf][r * kStride + pc * 16]) = st[u];
      }
    }
  };
  auto kfrag = [&](int buf, int kt, int ks) -> Frag {
    const char* p = &kbuf[buf][(kt * 32 + (lane & 31)) * kStride +
                               (ks * M::kStep + (lane >> 5) * M::kPerLane) * (int)sizeof(T)];
    return *(const Frag*)p;
  };

  // ---- software-pipelined schedule -----------------------------------------
  // Within each wave the MFMAs of the next 32-key subtile are issued between
  // the exponentials of the current one (scheduling groups below), so the
  // matrix core and the VALU of every SIMD work at the same time.  Each key
  // fragment read from LDS feeds the MFMAs of all kRT row tiles of the wave.
  // LDS holds three key tiles: the two being multiplied and the one being
  // filled.
  typedef f32x16 Acc[kRT];
  Acc acc[2];   // subtile s is multiplied into acc[s & 1]
  auto mma_sub = [&](Acc& acc, int buf, int kt, auto keys_on_m) {
#pragma unroll
    for (int qt = 0; qt < kRT; ++qt) {
      f32x16 z = {};
      acc[qt] = z;
    }
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const Frag kf = kfrag(buf, kt, ks);
#pragma unroll
      for (int qt = 0; qt < kRT; ++qt) {
        if constexpr (decltype(keys_on_m)::value) acc[qt] = M::run(kf, qf[qt][ks], acc[qt]);
        else acc[qt] = M::run(qf[qt][ks], kf, acc[qt]);
      }
    }
  };
  auto interleave = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, kRT, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 6 * kRT, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  auto prologue = [&](int n_tiles) {
    load_tile(stage0, 0);
    store_tile(stage0, 0);
    load_tile(stage0, (n_tiles > 1 ? 1 : 0) * kKeyTile);
    store_tile(stage0, 1);
    __syncthreads();
    load_tile(stage0, (n_tiles > 2 ? 2 : n_tiles - 1) * kKeyTile);
  };

  // ---------------- pass 1: row max and exp-sum over all W keys -------------
  float m_run[kRT], l_run[kRT];
  // Unidirectional: each lane's query positions, and the first position of
  // the wave (subtiles whose last key is past it cross the diagonal).
  int i_lane[kRT];
#pragma unroll
  for (int qt = 0; qt < kRT; ++qt) i_lane[qt] = (row0 + qt * 32 + (lane & 31)) / G;
  const int i_wave = row0 / G;
  // Keeps a step's VALU results ahead of the point that follows (the compiler
  // would otherwise sink the exponentials past the next barrier, away from the
  // MFMAs they are meant to overlap).
  auto pin = [&]() {
#pragma unroll
    for (int qt = 0; qt < kRT; ++qt) asm volatile("" ::"v"(m_run[qt]), "v"(l_run[qt]));
  };
  // Two ways to accumulate the row statistics.  Exact: a running maximum,
  // updated every subtile, with the sum rescaled when it moves.  Fixed
  // reference (the method's scoring, not the unidirectional ablation): the
  // maximum of the lane's first 16 keys is the reference for the whole row, so
  // every later subtile costs one multiply-add, one exp2 and one add per
  // logit.  The sum is then exact in the same way (it is scaled by a power of
  // two fixed per row) unless a later logit exceeds the reference by more
  // than the float range allows (about 88 nats) or the lane saw no key in its
  // first subtile; then the whole workgroup runs pass 1 again exactly.
  float mc_fix[kRT];
  auto stats_sub = [&](Acc& accs, int key0, auto masked, auto exact, bool first) {
#pragma unroll
    for (int qt = 0; qt < kRT; ++qt) {
      f32x16& acc = accs[qt];
      if constexpr (kUni) {
        if (key0 + 31 > i_wave) {
          // key = key0 + acc_row(r, lane) is seen iff key <= i_lane
          const int lim = i_lane[qt] - key0 - 4 * (lane >> 5);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (8 * (r >> 2) + (r & 3) > lim) acc[r] = -INFINITY;
        }
      } else if constexpr (decltype(masked)::value) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key0 + acc_row(r, lane) >= W) acc[r] = -INFINITY;
      }
      float mc;
      if (decltype(exact)::value || first) {
        float m0 = fmaxf(acc[0], acc[1]), m1 = fmaxf(acc[8], acc[9]);
#pragma unroll
        for (int r = 2; r < 8; ++r) {
          m0 = fmaxf(m0, acc[r]);
          m1 = fmaxf(m1, acc[8 + r]);
        }
        const float mx = fmaxf(fmaxf(m0, m1), m_run[qt]);
        // Only a masked subtile can leave a lane with no key seen so far.
        mc = mx * c;
        if (kUni || decltype(masked)::value) mc = (mx == -INFINITY) ? 0.0f : mc;
        if (!decltype(exact)::value) mc_fix[qt] = mc;
        l_run[qt] *= fast_exp2(m_run[qt] * c - mc);
        m_run[qt] = mx;
      } else {
        mc = mc_fix[qt];
      }
      float sp[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sp[r] = fast_exp2(fmaf(acc[r], c, -mc));
#pragma unroll
      for (int r = 4; r < 16; ++r) sp[r & 3] += fast_exp2(fmaf(acc[r], c, -mc));
      l_run[qt] += (sp[0] + sp[1]) + (sp[2] + sp[3]);
    }
  };
  // Key tiles: all of the window, or (unidirectional) up to the tile holding
  // the position of the workgroup's last row.  Uniform over the workgroup.
  int T1 = (W + kKeyTile - 1) / kKeyTile;
  int T2 = (C + kKeyTile - 1) / kKeyTile;
  if constexpr (kUni) {
    const int last_row = min(rows, (chunk + 1) * kScoreRowsPerChunk) - 1;
    const int i_last = last_row / G;
    T1 = i_last / kKeyTile + 1;
    T2 = min(C - 1, i_last) / kKeyTile + 1;
  }
  auto pass1 = [&](auto exact) {
#pragma unroll
    for (int qt = 0; qt < kRT; ++qt) {
      m_run[qt] = -INFINITY;
      l_run[qt] = 0.0f;
    }
    prologue(T1);
    mma_sub(acc[0], 0, 0, std::true_type());
    for (int t = 0; t + 1 < T1; ++t) {
      const int bt = t % 3, bn = (t + 1) % 3;
#pragma unroll
      for (int k = 0; k < kSub; ++k) {
        if (k + 1 < kSub) mma_sub(acc[(k + 1) & 1], bt, k + 1, std::true_type());
        else mma_sub(acc[0], bn, 0, std::true_type());
        stats_sub(acc[k & 1], t * kKeyTile + 32 * k, std::false_type(), exact, t == 0 && k == 0);
        interleave();
        pin();
      }
      store_tile(stage0, (t + 2) % 3);
      __syncthreads();
      load_tile(stage0, (t + 3 < T1 ? t + 3 : T1 - 1) * kKeyTile);
    }
    {
      const int t = T1 - 1, bt = t % 3;
#pragma unroll
      for (int k = 0; k < kSub; ++k) {
        if (k + 1 < kSub) mma_sub(acc[(k + 1) & 1], bt, k + 1, std::true_type());
        stats_sub(acc[k & 1], t * kKeyTile + 32 * k, std::true_type(), exact, t == 0 && k == 0);
      }
    }
  };
  if constexpr (kUni) {
    pass1(std::true_type());
    __syncthreads();
  } else {
    pass1(std::false_type());
    bool bad = false;
#pragma unroll
    for (int qt = 0; qt < kRT; ++qt) bad = bad || !(l_run[qt] < INFINITY) || m_run[qt] == -INFINITY;
    if (__ballot(bad) && lane == 0) s_redo = 1;
    __syncthreads();
    if (s_redo) {                                   // uniform over the workgroup
      pass1(std::true_type());
      __syncthreads();
    }
  }

  // Merge the two lane halves (same query, disjoint keys) and publish the row
  // bias  m*c + log2(sum)  so that  p = exp2(x*c - bias).
#pragma unroll
  for (int qt = 0; qt < kRT; ++qt) {
    const float mo = __shfl_xor(m_run[qt], 32);
    const float lo = __shfl_xor(l_run[qt], 32);
    const float mm = fmaxf(m_run[qt], mo);
    const float mc = mm * c;
    const float sum = l_run[qt] * fast_exp2(m_run[qt] * c - mc) + lo * fast_exp2(mo * c - mc);
    const int row = row0 + qt * 32 + (lane & 31);
    const float bias = (row < rows) ? mc + log2f(sum) : INFINITY;
    if (lane < 32) bias_lds[wave * kRowsPerWave + qt * 32 + lane] = bias;
  }
  __syncthreads();

  // ---------------- pass 2: column sums over keys j < C ---------------------
  float nbias[kRT][16];
#pragma unroll
  for (int qt = 0; qt < kRT; ++qt)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      nbias[qt][r] = -bias_lds[wave * kRowsPerWave + qt * 32 + acc_row(r, lane)];
  float* out = a.out + ((size_t)unit * a.n_split + chunk) * C;
  auto col_sub = [&](const Acc& accs, int t, int kt) {
    float sp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    bool plain = true;
    if constexpr (kUni) {
      const int key0 = t * kKeyTile + kt * 32;
      if (key0 + 31 > i_wave) {
        // row = row0 + qt*32 + acc_row(r, lane) sees key = key0 + lane%32
        // iff key*G <= row
        plain = false;
#pragma unroll
        for (int qt = 0; qt < kRT; ++qt) {
          const int lim = (key0 + (lane & 31)) * G - row0 - qt * 32 - 4 * (lane >> 5);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = fast_exp2(fmaf(accs[qt][r], c, nbias[qt][r]));
            sp[r & 3] += (8 * (r >> 2) + (r & 3) >= lim) ? e : 0.0f;
          }
        }
      }
    }
    if (plain) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sp[r] = fast_exp2(fmaf(accs[0][r], c, nbias[0][r]));
#pragma unroll
      for (int r = 4; r < 16; ++r) sp[r & 3] += fast_exp2(fmaf(accs[0][r], c, nbias[0][r]));
#pragma unroll
      for (int qt = 1; qt < kRT; ++qt)
#pragma unroll
        for (int r = 0; r < 16; ++r) sp[r & 3] += fast_exp2(fmaf(accs[qt][r], c, nbias[qt][r]));
    }
    float col = (sp[0] + sp[1]) + (sp[2] + sp[3]);
    col += __shfl_xor(col, 32);
    if (lane < 32) col_ring[t & 1][wave][kt * 32 + lane] = col;
  };
  auto flush_cols = [&](int t) {
    // waves 0 .. kKeyTile/64 - 1 each add up 64 keys' per-wave partials
    const int key = t * kKeyTile + wave * 64 + lane;
    if (wave < kKeyTile / 64 && key < C) {
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) sum += col_ring[t & 1][w][wave * 64 + lane];
      out[key] = sum;
    }
  };
  prologue(T2);
  mma_sub(acc[0], 0, 0, std::false_type());
  for (int t = 0; t + 1 < T2; ++t) {
    const int bt = t % 3, bn = (t + 1) % 3;
    if (t > 0) flush_cols(t - 1);
#pragma unroll
    for (int k = 0; k < kSub; ++k) {
      if (k + 1 < kSub) mma_sub(acc[(k + 1) & 1], bt, k + 1, std::false_type());
      else mma_sub(acc[0], bn, 0, std::false_type());
      col_sub(acc[k & 1], t, k);
      interleave();
    }
    store_tile(stage0, (t + 2) % 3);
    __syncthreads();
    load_tile(stage0, (t + 3 < T2 ? t + 3 : T2 - 1) * kKeyTile);
  }
  {
    const int t = T2 - 1, bt = t % 3;
    if (t > 0) flush_cols(t - 1);
#pragma unroll
    for (int k = 0; k < kSub; ++k) {
      if (k + 1 < kSub) mma_sub(acc[(k + 1) & 1], bt, k + 1, std::false_type());
      col_sub(acc[k & 1], t, k);
    }
    __syncthreads();
    flush_cols(t);
  }
  if constexpr (kUni) {
    // keys past the last tile get nothing from this chunk's rows
    for (int key = T2 * kKeyTile + tid; key < C; key += kThreads) out[key] = 0.0f;
  }
}

}  // namespace

template <typename T, int D>
hipError_t launch_score_typed(const ScoreArgs& a, hipStream_t stream) {
  const int units_pad = (a.n_units + 7) / 8 * 8;
  const unsigned grid = (unsigned)units_pad * (unsigned)a.n_split;
  if (a.unidirectional)
    hipLaunchKernelGGL((score_kernel<T, D, true>), dim3(grid), dim3(ScoreCfg<T>::kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((score_kernel<T, D, false>), dim3(grid), dim3(ScoreCfg<T>::kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kara
