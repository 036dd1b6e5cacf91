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
// l%32 and K-chunk l/32).  Key tiles of 64 rows are staged through LDS with a
// 16-byte row pad, so the per-lane 16-byte fragment reads do not collide on
// banks.
//
// Per logit, pass 1 needs an FMA, an exp2 and an add (its row maximum is
// taken once, from the first keys, see below) and pass 2 an FMA, an exp2 and
// an add, against 2*D MFMA flops.  On gfx950 v_exp_f32 holds the VALU for
// about 2.5 FMAs, so the VALU stream is longer than the MFMA stream; MFMA and
// VALU work overlap well when one wave interleaves them and poorly when they
// come from different waves of a SIMD, so every wave interleaves its own:
//   * each wave owns 64 rows (two 32-row query tiles sharing every K
//     fragment read from LDS; at most 256 VGPRs, two waves per SIMD) and
//     software-pipelines over 32-key subtiles: the MFMAs of the next subtile
//     are issued between the exponentials of the current one, in regions
//     fenced against reordering, and K fragments are read from LDS a few
//     regions before their MFMAs (the pipeline section below);
//   * LDS holds three 64-key tiles (two being multiplied, one being filled),
//     so there is one barrier per tile; the byte offsets of the window's K
//     rows are staged in LDS once; sums use independent partial chains.
// Under this load the chip runs below its nominal clock, limited by power,
// so work that moves data without need (extra LDS reads, extra
// instructions) costs time even where it fits in idle issue slots.

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
  // Consecutive 512-row chunks of one unit scored by one workgroup: the unit's
  // K row offsets are staged once, and each next chunk's query fragments are
  // loaded while the previous chunk finishes.
  static constexpr int kChunksPerWG = sizeof(T) == 2 ? 2 : 1;
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
  constexpr int kChunksPerWG = kUni ? 1 : ScoreCfg<T>::kChunksPerWG;
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
  __shared__ float col_ring[2][kWaves][2][kKeyTile];
  __shared__ uint64_t s_off[kMaxWindow];           // byte offsets of the window's K rows
  __shared__ int s_redo;                            // pass 1 must run again exactly

  // Block -> (unit, first chunk).  Consecutive block ids go to different
  // XCDs, so unit = slot-group * 8 + xcd keeps all chunks of a unit on one
  // XCD; a block scores kChunksPerWG consecutive chunks.
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int slot = bid >> 3;
  const int groups = (a.n_split + kChunksPerWG - 1) / kChunksPerWG;
  const int unit = (slot / groups) * 8 + xcd;
  int chunk = (slot % groups) * kChunksPerWG;
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
  int row0 = chunk * kScoreRowsPerChunk + wave * kRowsPerWave;

  // Start-up order: the block table reads are issued first and the query
  // fragment loads after them, so the K row offsets (which need only the
  // table) are staged in LDS while the query fragments are still in flight;
  // memory reads of a wave complete in issue order.
  if (tid == 0) s_redo = 0;
  constexpr int kFill = (kMaxWindow + kThreads - 1) / kThreads;
  int blk[kFill];
#pragma unroll
  for (int u = 0; u < kFill; ++u) {
    const int j = tid + u * kThreads;
    blk[u] = j < W ? trow[(start + j) >> a.bs_shift] : 0;
  }

  // Query fragments of this wave's rows (from row r0 on), kept in registers
  // for both passes.  Row r is window position r / G, head r % G of the group.
  Frag qf[kRT][NK];
  auto load_q = [&](int r0) {
#pragma unroll
    for (int qt = 0; qt < kRT; ++qt) {
      const int row = r0 + qt * 32 + (lane & 31);
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
  };
  load_q(row0);

  // Global -> register staging of key tiles: a tile is fetched one tile ahead
  // of its LDS store.  The byte offset of every window row's K row (its
  // block's place in the pool plus its place in the block) is staged in LDS
  // once, so a row address costs one LDS read and one add; a thread always
  // moves the same row piece of a tile.
  {
    const int bs_mask = (1 << a.bs_shift) - 1;
#pragma unroll
    for (int u = 0; u < kFill; ++u) {
      const int j = tid + u * kThreads;
      const int bk = blk[u] < 0 ? 0 : (blk[u] >= a.NB ? a.NB - 1 : blk[u]);
      if (j < W) s_off[j] = (uint64_t)(uint32_t)bk * blk_bytes + (uint64_t)(((start + j) & bs_mask) * kRowBytes);
    }
  }
  __syncthreads();
  constexpr int kRowsPerPass = kThreads / kPiecesPerRow;
  const int my_r = tid / kPiecesPerRow;
  const int my_pc = tid - my_r * kPiecesPerRow;
  const char* kpiece = kbase + my_pc * 16;
  typedef uint4 Stage[kPerThread];
  Stage stage0;
  auto load_tile = [&](Stage& st, int tile0) {
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int r = my_r + u * kRowsPerPass;
      const int j = tile0 + r;
      if (r < kKeyTile && j < W) st[u] = *(const uint4*)(kpiece + s_off[j]);
      else st[u] = make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store_tile = [&](const Stage& st, int buf) {
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int r = my_r + u * kRowsPerPass;
      if (r < kKeyTile) *(uint4*)(&kbuf[buf][r * kStride + my_pc * 16]) = st[u];
    }
  };
  auto kfrag = [&](int buf, int kt, int ks) -> Frag {
    const char* p = &kbuf[buf][(kt * 32 + (lane & 31)) * kStride +
                               (ks * M::kStep + (lane >> 5) * M::kPerLane) * (int)sizeof(T)];
    return *(const Frag*)p;
  };
  // Stages the first two key tiles (both fetched before either is stored)
  // and starts fetching the third.
  auto prologue = [&](int n_tiles) {
    Stage stage1;
    load_tile(stage0, 0);
    load_tile(stage1, (n_tiles > 1 ? 1 : 0) * kKeyTile);
    store_tile(stage0, 0);
    store_tile(stage1, 1);
    __syncthreads();
    load_tile(stage0, (n_tiles > 2 ? 2 : n_tiles - 1) * kKeyTile);
  };

  // ---- software pipeline ---------------------------------------------------
  // Subtile q of a pass is 32 keys: slice q % kSub of key tile q / kSub, which
  // sits in LDS buffer (q / kSub) % 3.  Step q multiplies subtile q+1 into one
  // register tile while the VALU turns the logits of subtile q, in the other
  // register tile, into exponentials and sums.  A step is kRegions regions
  // fenced against reordering; region i issues the MFMAs of K fragment group
  // i (kPer fragments, each shared by the kRT query tiles of the wave), 1 /
  // kRegions of the VALU work, and the LDS reads of the group kDist regions
  // ahead, which therefore has kDist regions of work in which to arrive.
  // Groups rotate through a ring of kRing register sets.  Reads reach at most
  // two subtiles ahead, so they touch only the current key tile and the next,
  // both resident (three LDS buffers: two read, one being filled; one barrier
  // per tile).
  constexpr int kRegions = NK < 8 ? NK : 8;
  constexpr int kPer = NK / kRegions;
  constexpr int kRing = kPer == 1 ? kRegions : 2;
  constexpr int kDist = kRing / 2;
  constexpr int kElems = kRT * 16;                  // logits per lane per subtile
  static_assert(kSub >= 2 && kSub % 2 == 0 && kRegions % kRing == 0, "pipeline shape");
  Frag kf[kRing][kPer];
  typedef f32x16 Acc[kRT];
  Acc acc[2];   // subtile q is multiplied into acc[q & 1]
  auto fetch = [&](int g, int buf, int kt) {
#pragma unroll
    for (int p = 0; p < kPer; ++p) kf[g % kRing][p] = kfrag(buf, kt, g * kPer + p);
  };
  // One step: MFMAs of the subtile in (mbuf, mkt) into nxt when do_m, reads
  // that run into the subtile after it (fbuf, fkt) when do_f, VALU chunk i
  // by valu(i).
  auto step = [&](Acc& nxt, int mbuf, int mkt, int fbuf, int fkt, bool do_m, bool do_f, auto keys_on_m,
                  auto&& valu) {
    if (do_m) {
#pragma unroll
      for (int qt = 0; qt < kRT; ++qt) {
        f32x16 z = {};
        nxt[qt] = z;
      }
    }
#pragma unroll
    for (int i = 0; i < kRegions; ++i) {
      if (do_m && i + kDist < kRegions) fetch(i + kDist, mbuf, mkt);
      if (do_f && i + kDist >= kRegions) fetch(i + kDist - kRegions, fbuf, fkt);
      if (do_m) {
#pragma unroll
        for (int p = 0; p < kPer; ++p) {
          const Frag f = kf[i % kRing][p];
#pragma unroll
          for (int qt = 0; qt < kRT; ++qt) {
            if constexpr (decltype(keys_on_m)::value) nxt[qt] = M::run(f, qf[qt][i * kPer + p], nxt[qt]);
            else nxt[qt] = M::run(qf[qt][i * kPer + p], f, nxt[qt]);
          }
        }
      }
      valu(i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Starts a pass: subtile 0 multiplied into acc[0], the first reads of
  // subtile 1 issued.
  auto start_pass = [&](auto keys_on_m) {
#pragma unroll
    for (int g = 0; g < kDist; ++g) fetch(g, 0, 0);
    step(acc[0], 0, 0, 0, 1, true, true, keys_on_m, [](int) {});
  };

  // ---------------- the workgroup's chunks, one after another ---------------
  for (int ci = 0;; ++ci) {
    // another chunk follows: its query fragments are loaded during this
    // chunk's last VALU-only step, once these are no longer read
    const bool more = ci + 1 < kChunksPerWG && chunk + 1 < a.n_split;
    // ---------------- pass 1: row max and exp-sum over all W keys -------------
    float m_run[kRT], l_run[kRT];
    // Unidirectional: each lane's query positions, and the first position of
    // the wave (subtiles whose last key is past it cross the diagonal).
    int i_lane[kRT];
  #pragma unroll
    for (int qt = 0; qt < kRT; ++qt) i_lane[qt] = (row0 + qt * 32 + (lane & 31)) / G;
    const int i_wave = row0 / G;
    // Keeps a step's VALU results ahead of the point that follows.
    auto pin = [&]() {
  #pragma unroll
      for (int qt = 0; qt < kRT; ++qt) asm volatile("" ::"v"(m_run[qt]), "v"(l_run[qt]));
    };
    // Two ways to accumulate the row statistics.  Exact: a running maximum,
    // updated every subtile, with the sum rescaled when it moves.  Fixed
    // reference (the first run of pass 1): the maximum of the lane's first 16
    // visible keys is the reference for the whole row, so
    // every subtile costs one multiply-add, one exp2 and one add per logit.  The
    // sum is then exact in the same way (it is scaled by a power of two fixed
    // per row) unless a later logit exceeds the reference by more than the
    // float range allows (about 88 nats) or the lane saw no key in its first
    // subtile; then the whole workgroup runs pass 1 again exactly.
    float mc_fix[kRT], mcur[kRT], sp1[kRT][4];
    auto mask_sub = [&](Acc& accs, int key0, bool tail) {
  #pragma unroll
      for (int qt = 0; qt < kRT; ++qt) {
        f32x16& v = accs[qt];
        if constexpr (kUni) {
          if (key0 + 31 > i_wave) {
            // key = key0 + acc_row(r, lane) is seen iff key <= i_lane
            const int lim = i_lane[qt] - key0 - 4 * (lane >> 5);
  #pragma unroll
            for (int r = 0; r < 16; ++r)
              if (8 * (r >> 2) + (r & 3) > lim) v[r] = -INFINITY;
          }
        } else if (tail) {
  #pragma unroll
          for (int r = 0; r < 16; ++r)
            if (key0 + acc_row(r, lane) >= W) v[r] = -INFINITY;
        }
      }
    };
    auto lane_max = [&](const f32x16& v) {
      float m0 = fmaxf(v[0], v[1]), m1 = fmaxf(v[8], v[9]);
  #pragma unroll
      for (int r = 2; r < 8; ++r) {
        m0 = fmaxf(m0, v[r]);
        m1 = fmaxf(m1, v[8 + r]);
      }
      return fmaxf(m0, m1);
    };
    // VALU chunk i of pass 1 on the subtile starting at key0.
    auto stats_valu = [&](Acc& accs, int key0, bool tail, auto exact, int i) {
      if (i == 0) {
        mask_sub(accs, key0, tail);
  #pragma unroll
        for (int qt = 0; qt < kRT; ++qt) {
          if constexpr (decltype(exact)::value) {
            const float mx = fmaxf(lane_max(accs[qt]), m_run[qt]);
            const float mc = (mx == -INFINITY) ? 0.0f : mx * c;
            l_run[qt] *= fast_exp2(m_run[qt] * c - mc);
            m_run[qt] = mx;
            mcur[qt] = mc;
          } else {
            mcur[qt] = mc_fix[qt];
          }
        }
      }
  #pragma unroll
      for (int e = i * kElems / kRegions; e < (i + 1) * kElems / kRegions; ++e) {
        const int qt = e / 16, r = e % 16;
        const float x = fast_exp2(fmaf(accs[qt][r], c, -mcur[qt]));
        if (r < 4) sp1[qt][r] = x;
        else sp1[qt][r & 3] += x;
        if (r == 15) l_run[qt] += (sp1[qt][0] + sp1[qt][1]) + (sp1[qt][2] + sp1[qt][3]);
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
      start_pass(std::true_type());
      if constexpr (!decltype(exact)::value) {
        // the reference: the maximum of the lane's first 16 keys
        mask_sub(acc[0], 0, true);
  #pragma unroll
        for (int qt = 0; qt < kRT; ++qt) {
          m_run[qt] = lane_max(acc[0][qt]);
          mc_fix[qt] = (m_run[qt] == -INFINITY) ? 0.0f : m_run[qt] * c;
        }
      }
      for (int t = 0; t + 1 < T1; ++t) {
        const int bt = t % 3, bn = (t + 1) % 3;
  #pragma unroll
        for (int k = 0; k < kSub; ++k) {
          step(acc[(k + 1) & 1], k + 1 < kSub ? bt : bn, (k + 1) % kSub, k + 2 < kSub ? bt : bn, (k + 2) % kSub,
               true, true, std::true_type(),
               [&](int i) { stats_valu(acc[k & 1], t * kKeyTile + 32 * k, false, exact, i); });
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
          step(acc[(k + 1) & 1], bt, (k + 1) % kSub, bt, (k + 2) % kSub, k + 1 < kSub, k + 2 < kSub,
               std::true_type(), [&](int i) { stats_valu(acc[k & 1], t * kKeyTile + 32 * k, true, exact, i); });
        }
      }
    };
    // The first two key tiles of pass 2 are fetched now, to arrive while
    // pass 1 is checked and the row biases are published; they are stored once
    // every wave is past pass 1 (its LDS tiles are then free).
    // The unidirectional ablation takes the same fixed reference: a causal
    // row whose lane half sees none of its first keys (window positions 0-3)
    // makes the workgroup rerun pass 1 exactly, which happens only in a
    // unit's first chunk.
    Stage p2_t0, p2_t1;
    {
      pass1(std::false_type());
      load_tile(p2_t0, 0);
      load_tile(p2_t1, (T2 > 1 ? 1 : 0) * kKeyTile);
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
    store_tile(p2_t0, 0);
    store_tile(p2_t1, 1);
    __syncthreads();
    if (tid == 0) s_redo = 0;                       // every wave has read it
    load_tile(stage0, (T2 > 2 ? 2 : T2 - 1) * kKeyTile);

    // ---------------- pass 2: column sums over keys j < C ---------------------
    float nbias[kRT][16];
  #pragma unroll
    for (int qt = 0; qt < kRT; ++qt)
  #pragma unroll
      for (int r = 0; r < 16; ++r)
        nbias[qt][r] = -bias_lds[wave * kRowsPerWave + qt * 32 + acc_row(r, lane)];
    float* out = a.out + ((size_t)unit * a.n_split + chunk) * C;
    float sp2[4];
    bool plain = true;
    int lim2[kRT];
    // VALU chunk i of pass 2 on slice kt of key tile t: each lane adds the
    // probabilities of its key over its 16 rows of every query tile; the two
    // lane halves (disjoint rows) go to LDS separately.
    auto col_valu = [&](const Acc& accs, int t, int kt, int i) {
      if constexpr (kUni) {
        if (i == 0) {
          const int key0 = t * kKeyTile + kt * 32;
          // row = row0 + qt*32 + acc_row(r, lane) sees key = key0 + lane%32
          // iff key*G <= row
          plain = !(key0 + 31 > i_wave);
  #pragma unroll
          for (int qt = 0; qt < kRT; ++qt)
            lim2[qt] = (key0 + (lane & 31)) * G - row0 - qt * 32 - 4 * (lane >> 5);
        }
      }
  #pragma unroll
      for (int e = i * kElems / kRegions; e < (i + 1) * kElems / kRegions; ++e) {
        const int qt = e / 16, r = e % 16;
        float x = fast_exp2(fmaf(accs[qt][r], c, nbias[qt][r]));
        if constexpr (kUni) x = (plain || 8 * (r >> 2) + (r & 3) >= lim2[qt]) ? x : 0.0f;
        if (e < 4) sp2[e] = x;
        else sp2[e & 3] += x;
      }
      if (i == kRegions - 1)
        col_ring[t & 1][wave][lane >> 5][kt * 32 + (lane & 31)] = (sp2[0] + sp2[1]) + (sp2[2] + sp2[3]);
    };
    auto flush_cols = [&](int t) {
      // waves 0 .. kKeyTile/64 - 1 each add up 64 keys' per-wave partials
      const int key = t * kKeyTile + wave * 64 + lane;
      if (wave < kKeyTile / 64 && key < C) {
        float sum = 0.0f;
  #pragma unroll
        for (int w = 0; w < kWaves; ++w)
          sum += col_ring[t & 1][w][0][wave * 64 + lane] + col_ring[t & 1][w][1][wave * 64 + lane];
        out[key] = sum;
      }
    };
    start_pass(std::false_type());
    for (int t = 0; t + 1 < T2; ++t) {
      const int bt = t % 3, bn = (t + 1) % 3;
      if (t > 0) flush_cols(t - 1);
      __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
      for (int k = 0; k < kSub; ++k) {
        step(acc[(k + 1) & 1], k + 1 < kSub ? bt : bn, (k + 1) % kSub, k + 2 < kSub ? bt : bn, (k + 2) % kSub, true,
             true, std::false_type(), [&](int i) { col_valu(acc[k & 1], t, k, i); });
      }
      store_tile(stage0, (t + 2) % 3);
      __syncthreads();
      load_tile(stage0, (t + 3 < T2 ? t + 3 : T2 - 1) * kKeyTile);
    }
    {
      const int t = T2 - 1, bt = t % 3;
      if (t > 0) flush_cols(t - 1);
      __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
      for (int k = 0; k < kSub; ++k) {
        if (k == kSub - 1 && more) load_q(row0 + kScoreRowsPerChunk);
        step(acc[(k + 1) & 1], bt, (k + 1) % kSub, bt, (k + 2) % kSub, k + 1 < kSub, k + 2 < kSub, std::false_type(),
             [&](int i) { col_valu(acc[k & 1], t, k, i); });
      }
      __syncthreads();
      flush_cols(t);
    }
    if constexpr (kUni) {
      // keys past the last tile get nothing from this chunk's rows
      for (int key = T2 * kKeyTile + tid; key < C; key += kThreads) out[key] = 0.0f;
    }
    if (!more) break;
    ++chunk;
    row0 += kScoreRowsPerChunk;
  }
}

}  // namespace

template <typename T, int D>
hipError_t launch_score_typed(const ScoreArgs& a, hipStream_t stream) {
  const int units_pad = (a.n_units + 7) / 8 * 8;
  const int per_wg = a.unidirectional ? 1 : ScoreCfg<T>::kChunksPerWG;
  const unsigned groups = (unsigned)((a.n_split + per_wg - 1) / per_wg);
  const unsigned grid = (unsigned)units_pad * groups;
  if (a.unidirectional)
    hipLaunchKernelGGL((score_kernel<T, D, true>), dim3(grid), dim3(ScoreCfg<T>::kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((score_kernel<T, D, false>), dim3(grid), dim3(ScoreCfg<T>::kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kara
