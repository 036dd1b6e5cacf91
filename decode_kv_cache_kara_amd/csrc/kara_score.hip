// Window scoring on gfx950 matrix cores.
//
// Per unit (sequence, layer, KV head) the rows are the G*W (window position,
// query head of the group) pairs and the columns are the W window keys.  The
// score of key j < C is the column sum of the row-softmaxed logits
// q.k/sqrt(D), every softmax running over all W keys with no mask
// ("Technical Summary: Kara", Methodology 1, Mechanism and Rationale).
//
// A column sum needs each row's softmax normaliser before that row's
// probabilities can be added, so the work runs in two passes over the keys for
// every block of rows, both on MFMA:
//   pass 1  S^T = K Q^T (keys on the MFMA M axis, queries on N): each lane owns
//           one query and 16 keys of a 32x32 tile, so the running row maximum
//           and exp-sum stay in the lane; the two lane halves merge at the end.
//   pass 2  S = Q K^T (queries on M, keys on N): each lane owns one key and 16
//           queries, so p = exp2(x*c - bias_row) is added into a per-lane
//           column accumulator; the two halves and the 8 waves merge in LDS.
// The same Q register fragments serve as the B operand of pass 1 and the A
// operand of pass 2 (for 32x32 MFMA both operands map lane l to matrix index
// l%32 and K-chunk l/32).  Key tiles of 64 rows are staged through LDS, double
// buffered, with a 16-byte row pad so the per-lane 16-byte reads do not
// collide on banks.
//
// One workgroup = 8 waves x 64 rows = 512 rows of one unit.  The workgroups of
// a unit are dispatched back to back onto the same XCD (block ids are
// interleaved across the 8 XCDs) so that unit's K rows are fetched from HBM
// once and then served from that XCD's L2.  Each workgroup writes its 512-row
// partial column sums; the selection kernel adds the partials of a unit in
// chunk order, so results do not depend on scheduling.

#include "kara_internal.hpp"

#include <cmath>

namespace kara {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 64;
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

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void score_kernel(ScoreArgs a) {
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
  extern __shared__ float col_lds[];  // [kWaves][C]

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

  // Query fragments of this wave's 64 rows (two 32-row tiles), kept in
  // registers for both passes.  Row r is window position r / G, head r % G.
  Frag qf[2][NK];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
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

  uint4 stage[kPerThread];
  auto load_tile = [&](int tile0) {
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int p = tid + u * kThreads;
      const int r = p / kPiecesPerRow, pc = p - (p / kPiecesPerRow) * kPiecesPerRow;
      const int j = tile0 + r;
      if (p < kTilePieces && j < W) {
        const int t = start + j;
        int blk = trow[t / a.bs];
        blk = blk < 0 ? 0 : (blk >= a.NB ? a.NB - 1 : blk);
        const char* src = kbase + (size_t)blk * blk_bytes + (size_t)(t % a.bs) * kRowBytes + pc * 16;
        stage[u] = *(const uint4*)src;
      } else {
        stage[u] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int p = tid + u * kThreads;
      if (p < kTilePieces) {
        const int r = p / kPiecesPerRow, pc = p - (p / kPiecesPerRow) * kPiecesPerRow;
        *(uint4*)(&kbuf[buf][r * kStride + pc * 16]) = stage[u];
      }
    }
  };
  auto kfrag = [&](int buf, int kt, int ks) -> Frag {
    const char* p = &kbuf[buf][(kt * 32 + (lane & 31)) * kStride +
                               (ks * M::kStep + (lane >> 5) * M::kPerLane) * (int)sizeof(T)];
    return *(const Frag*)p;
  };

  // ---------------- pass 1: row max and exp-sum over all W keys -------------
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.0f, 0.0f};
  const int n_tiles1 = (W + kKeyTile - 1) / kKeyTile;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int t = 0; t < n_tiles1; ++t) {
    const int buf = t & 1;
    const int tile0 = t * kKeyTile;
    if (t + 1 < n_tiles1) load_tile(tile0 + kKeyTile);
    f32x16 acc[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        f32x16 z = {};
        acc[kt][qt] = z;
      }
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const Frag k0 = kfrag(buf, 0, ks);
      const Frag k1 = kfrag(buf, 1, ks);
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        acc[0][qt] = M::run(k0, qf[qt][ks], acc[0][qt]);
        acc[1][qt] = M::run(k1, qf[qt][ks], acc[1][qt]);
      }
    }
    if (tile0 + kKeyTile > W) {  // ragged last tile: keys >= W do not exist
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (tile0 + kt * 32 + acc_row(r, lane) >= W) {
            acc[kt][0][r] = -INFINITY;
            acc[kt][1][r] = -INFINITY;
          }
    }
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float mx = m_run[qt];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[kt][qt][r]);
      const float mc = (mx == -INFINITY) ? 0.0f : mx * c;
      float s = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += fast_exp2(fmaf(acc[kt][qt][r], c, -mc));
      l_run[qt] = l_run[qt] * fast_exp2(m_run[qt] * c - mc) + s;
      m_run[qt] = mx;
    }
    if (t + 1 < n_tiles1) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Merge the two lane halves (same query, disjoint keys) and publish the row
  // bias  m*c + log2(sum)  so that  p = exp2(x*c - bias).
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float mo = __shfl_xor(m_run[qt], 32);
    const float lo = __shfl_xor(l_run[qt], 32);
    const float mm = fmaxf(m_run[qt], mo);
    const float mc = mm * c;
    const float sum = l_run[qt] * fast_exp2(m_run[qt] * c - mc) + lo * fast_exp2(mo * c - mc);
    const int row = row0 + qt * 32 + (lane & 31);
    const float bias = (row < rows) ? mc + log2f(sum) : INFINITY;
    if (lane < 32) bias_lds[wave * kRowsPerWave + qt * 32 + lane] = bias;
  }

  // ---------------- pass 2: column sums over keys j < C ---------------------
  const int n_tiles2 = (C + kKeyTile - 1) / kKeyTile;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  float nbias[2][16];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int r = 0; r < 16; ++r) nbias[qt][r] = -bias_lds[wave * kRowsPerWave + qt * 32 + acc_row(r, lane)];

  for (int t = 0; t < n_tiles2; ++t) {
    const int buf = t & 1;
    const int tile0 = t * kKeyTile;
    if (t + 1 < n_tiles2) load_tile(tile0 + kKeyTile);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x16 acc[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        f32x16 z = {};
        acc[qt] = z;
      }
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        const Frag kf = kfrag(buf, kt, ks);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) acc[qt] = M::run(qf[qt][ks], kf, acc[qt]);
      }
      float col = 0.0f;
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int r = 0; r < 16; ++r) col += fast_exp2(fmaf(acc[qt][r], c, nbias[qt][r]));
      col += __shfl_xor(col, 32);
      const int key = tile0 + kt * 32 + (lane & 31);
      if (lane < 32 && key < C) col_lds[wave * C + key] = col;
    }
    if (t + 1 < n_tiles2) store_tile(buf ^ 1);
    __syncthreads();
  }

  float* out = a.out + ((size_t)unit * a.n_split + chunk) * C;
  for (int j = tid; j < C; j += kThreads) {
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += col_lds[w * C + j];
    out[j] = s;
  }
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
  const size_t dyn = (size_t)kWaves * a.C * sizeof(float);
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)score_kernel<T, D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       kWaves * kMaxRegion * (int)sizeof(float));
    if (e != hipSuccess) return e;
    configured = true;
  }
  const int units_pad = (a.n_units + 7) / 8 * 8;
  const unsigned grid = (unsigned)units_pad * (unsigned)a.n_split;
  hipLaunchKernelGGL((score_kernel<T, D>), dim3(grid), dim3(kThreads), dyn, stream, a);
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
