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
// The exponentials, not the MFMAs, bound this kernel: per logit pass 1 needs a
// max, an FMA, an exp2 (half-rate on gfx950) and an add, pass 2 an FMA, an
// exp2 and an add, against 2*D MFMA flops.  So the schedule is built to keep
// the VALU busy and hide the matrix work under it:
//   * ping-pong: waves are split in two groups that share every SIMD; in each
//     barrier-separated phase one group issues MFMAs while the other runs the
//     exponentials of the tile it multiplied in the previous phase;
//   * each wave owns kRT x 32 rows so that several waves of each group sit on
//     every SIMD and the VALU stream of one wave hides the latency of
//     another's; sums and maxima are split into independent partial chains;
//   * key tiles are fetched two phases ahead of their LDS store.
//
// One workgroup scores 512 rows of one unit.  The workgroups of a unit are
// dispatched back to back onto the same XCD (block ids are interleaved across
// the 8 XCDs) so that unit's K rows are fetched from HBM once and then served
// from that XCD's L2.  Each workgroup writes its 512-row partial column sums;
// the selection kernel adds the partials of a unit in chunk order, so results
// do not depend on scheduling.

#include "kara_internal.hpp"

#include <cmath>
#include <type_traits>

namespace kara {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kRT = kScoreRowTiles;              // 32-row query tiles per wave
constexpr int kWaves = kScoreRowsPerChunk / (32 * kRT);
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 32 * kRT;
constexpr int kKeyTile = 64;

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

// With 32-row waves (at most 128 VGPRs) four waves share each SIMD; ask for
// enough co-resident workgroups to reach that.
constexpr int kMinBlocks = kRT == 1 ? (16 / kWaves > 0 ? 16 / kWaves : 1) : 1;

template <typename T, int D>
__global__ __launch_bounds__(kThreads, kMinBlocks) void score_kernel(ScoreArgs a) {
  using M = Mma<T>;
  typedef typename M::Frag Frag;
  constexpr int NK = D / M::kStep;
  constexpr int kRowBytes = D * (int)sizeof(T);
  constexpr int kStride = kRowBytes + 16;
  constexpr int kPiecesPerRow = kRowBytes / 16;
  constexpr int kTilePieces = kKeyTile * kPiecesPerRow;
  constexpr int kPerThread = (kTilePieces + kThreads - 1) / kThreads;

  __shared__ __attribute__((aligned(16))) char kbuf[2][kKeyTile * kStride];
  __shared__ float bias_lds[kWaves * kRowsPerWave];
  __shared__ float col_ring[2][kWaves][kKeyTile];

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
  const T* qbase = (const T*)a.q + (size_t)bl * W * a.Hq * D + (size_t)h * G * D;
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
      const T* p = qbase + ((size_t)i * a.Hq + g) * D + (lane >> 5) * M::kPerLane;
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) qf[qt][ks] = *(const Frag*)(p + ks * M::kStep);
    } else {
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) qf[qt][ks] = M::zero();
    }
  }

  // Global -> register staging of key tiles, two register sets so that a
  // tile's loads are in flight for three phases before they are written to
  // LDS.  Block sizes are powers of two (bs = 1 << bs_shift).
  typedef uint4 Stage[kPerThread];
  Stage stage0, stage1;
  const int bs_mask = (1 << a.bs_shift) - 1;
  auto load_tile = [&](Stage& st, int tile0) {
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int p = tid + u * kThreads;
      const int r = p / kPiecesPerRow, pc = p % kPiecesPerRow;
      const int j = tile0 + r;
      if (p < kTilePieces && j < W) {
        const int t = start + j;
        int blk = trow[t >> a.bs_shift];
        blk = blk < 0 ? 0 : (blk >= a.NB ? a.NB - 1 : blk);
        const char* src = kbase + (size_t)blk * blk_bytes + (size_t)(t & bs_mask) * kRowBytes + pc * 16;
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

  // MFMA of the 64-key tile held in LDS buffer `buf` against this wave's
  // query tiles: acc[kt][qt].  Pass 1 computes S^T (keys on the M axis), pass
  // 2 computes S (queries on M).
  f32x16 acc[2][kRT];
  auto mma_tile = [&](int buf, auto keys_on_m) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x16 z = {};
#pragma unroll
      for (int qt = 0; qt < kRT; ++qt) acc[kt][qt] = z;
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        const Frag kf = kfrag(buf, kt, ks);
#pragma unroll
        for (int qt = 0; qt < kRT; ++qt) {
          if constexpr (decltype(keys_on_m)::value) acc[kt][qt] = M::run(kf, qf[qt][ks], acc[kt][qt]);
          else acc[kt][qt] = M::run(qf[qt][ks], kf, acc[kt][qt]);
        }
      }
    }
  };

  // Ping-pong schedule.  Group A (waves 0..kWaves/2-1) and group B share the
  // SIMDs evenly (wave w runs on the SIMD of wave w mod 4).  Time runs in
  // barrier-separated phases, two per key tile; a wave multiplies tile t in
  // one phase and runs the exponentials of that tile in the next, and group B
  // runs one phase behind group A:
  //   phase    2t        2t+1       2t+2
  //   group A  MFMA(t)   VALU(t)    MFMA(t+1)
  //   group B  VALU(t-1) MFMA(t)    VALU(t)
  // Tile t+2 is fetched from global memory in phase 2t and written to LDS in
  // phase 2t+3.
#ifndef KARA_PINGPONG
#define KARA_PINGPONG 1
#endif
  const int lag = (KARA_PINGPONG && wave >= kWaves / 2) ? 1 : 0;
  auto pipeline = [&](int n_tiles, auto work) {
    load_tile(stage0, 0);
    store_tile(stage0, 0);
    if (n_tiles > 1) load_tile(stage1, kKeyTile);
    __syncthreads();
    auto phase_pair = [&](int t, Stage& ld, const Stage& st) {
      if (t > n_tiles) return;
      if (t + 2 < n_tiles) load_tile(ld, (t + 2) * kKeyTile);   // same parity as t
      {
        const int q = 2 * t - lag;
        if (q >= 0 && q < 2 * n_tiles) work(q, 2 * t);
      }
      __syncthreads();
      if (t == n_tiles) return;
      {
        const int q = 2 * t + 1 - lag;
        if (q < 2 * n_tiles) work(q, 2 * t + 1);
      }
      if (t + 1 < n_tiles) store_tile(st, (t + 1) & 1);         // loaded two phases ago
      __syncthreads();
    };
    for (int t = 0; t <= n_tiles; t += 2) {
      phase_pair(t, stage0, stage1);
      phase_pair(t + 1, stage1, stage0);
    }
  };

  // ---------------- pass 1: row max and exp-sum over all W keys -------------
  float m_run[kRT], l_run[kRT];
#pragma unroll
  for (int qt = 0; qt < kRT; ++qt) {
    m_run[qt] = -INFINITY;
    l_run[qt] = 0.0f;
  }
  auto row_stats = [&](int tile0, auto masked) {
#pragma unroll
    for (int qt = 0; qt < kRT; ++qt) {
      // keys past the window (ragged last tile) are masked in place
      if constexpr (decltype(masked)::value) {
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          const int kt = e >> 4, r = e & 15;
          if (tile0 + kt * 32 + acc_row(r, lane) >= W) acc[kt][qt][r] = -INFINITY;
        }
      }
      auto v = [&](int e) -> float { return acc[e >> 4][qt][e & 15]; };
      float mp[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        mp[k] = fmaxf(v(8 * k), v(8 * k + 1));
#pragma unroll
        for (int e = 2; e < 8; ++e) mp[k] = fmaxf(mp[k], v(8 * k + e));
      }
      const float mx = fmaxf(fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3])), m_run[qt]);
      const float mc = (mx == -INFINITY) ? 0.0f : mx * c;
      float sp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int e = 0; e < 32; ++e) sp[e & 3] += fast_exp2(fmaf(v(e), c, -mc));
      l_run[qt] = l_run[qt] * fast_exp2(m_run[qt] * c - mc) + ((sp[0] + sp[1]) + (sp[2] + sp[3]));
      m_run[qt] = mx;
    }
  };

  const int T1 = (W + kKeyTile - 1) / kKeyTile;
  pipeline(T1, [&](int q, int) {
    const int tq = q >> 1;
    if (!(q & 1)) {
      mma_tile(tq & 1, std::true_type());
    } else if (tq + 1 < T1) {
      row_stats(tq * kKeyTile, std::false_type());
    } else {
      row_stats(tq * kKeyTile, std::true_type());
    }
  });

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
  const int T2 = (C + kKeyTile - 1) / kKeyTile;
  float nbias[kRT][16];
#pragma unroll
  for (int qt = 0; qt < kRT; ++qt)
#pragma unroll
    for (int r = 0; r < 16; ++r) nbias[qt][r] = -bias_lds[wave * kRowsPerWave + qt * 32 + acc_row(r, lane)];

  // Per-wave column sums of a tile go to a two-tile ring in LDS; once both
  // groups have added theirs, wave 0 sums the waves in order and writes out.
  float* out = a.out + ((size_t)unit * a.n_split + chunk) * C;
  auto col_sums = [&](int t) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      float sp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int qt = 0; qt < kRT; ++qt)
#pragma unroll
        for (int r = 0; r < 16; ++r) sp[r & 3] += fast_exp2(fmaf(acc[kt][qt][r], c, nbias[qt][r]));
      float col = (sp[0] + sp[1]) + (sp[2] + sp[3]);
      col += __shfl_xor(col, 32);
      if (lane < 32) col_ring[t & 1][wave][kt * 32 + lane] = col;
    }
  };
  auto flush_cols = [&](int t) {
    const int key = t * kKeyTile + lane;
    if (wave == 0 && key < C) {
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) sum += col_ring[t & 1][w][lane];
      out[key] = sum;
    }
  };

  pipeline(T2, [&](int q, int p) {
    // tile t's column partials are complete after phase 2t+2; flush them in 2t+3
    if ((p & 1) && p >= 3) flush_cols((p - 3) >> 1);
    const int tq = q >> 1;
    if (!(q & 1)) mma_tile(tq & 1, std::false_type());
    else col_sums(tq);
  });
  flush_cols(T2 - 1);
}

__global__ __launch_bounds__(256) void reduce_kernel(const float* __restrict__ partials,
                                                     float* __restrict__ scores, int n_units,
                                                     int n_split, int C) {
  const size_t n = (size_t)n_units * C;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t u = i / C, j = i - (i / C) * C;
    const float* p = partials + u * n_split * C + j;
    float s = 0.0f;
    for (int k = 0; k < n_split; ++k) s += p[(size_t)k * C];
    scores[i] = s;
  }
}

template <typename T, int D>
hipError_t launch_typed(const ScoreArgs& a, hipStream_t stream) {
  const int units_pad = (a.n_units + 7) / 8 * 8;
  const unsigned grid = (unsigned)units_pad * (unsigned)a.n_split;
  hipLaunchKernelGGL((score_kernel<T, D>), dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score(const ScoreArgs& a, int dtype, hipStream_t stream) {
  if (a.n_units == 0) return hipSuccess;
  if (dtype == 1) {
    if (a.D == 128) return launch_typed<__bf16, 128>(a, stream);
    if (a.D == 64) return launch_typed<__bf16, 64>(a, stream);
  } else {
    if (a.D == 128) return launch_typed<float, 128>(a, stream);
    if (a.D == 64) return launch_typed<float, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_reduce(const float* partials, float* scores, int n_units, int n_split, int C,
                         hipStream_t stream) {
  if (n_units == 0) return hipSuccess;
  const size_t n = (size_t)n_units * C;
  unsigned grid = (unsigned)((n + 255) / 256);
  if (grid > 65536u) grid = 65536u;
  hipLaunchKernelGGL(reduce_kernel, dim3(grid), dim3(256), 0, stream, partials, scores, n_units,
                     n_split, C);
  return hipGetLastError();
}

}  // namespace kara
