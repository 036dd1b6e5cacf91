// Paged K/V compaction ("Technical Summary: Kara", Methodology 3: the trailing
// blocks of a selected sequence are compressed, freeing blocks for more
// sequences).
//
// For every (sequence, layer, K/V, KV head) the kept rows are written, in
// order, into the sequence's fresh blocks: first the p tokens of the boundary
// block that precede the window (so the boundary block can be dropped), then
// the R kept window positions, then the B protected tokens.  Source blocks are
// never written, so the copy is hazard-free and can run again on the same
// inputs.  A row is head_dim elements (256 B for bf16 x 128); each lane moves
// 16 B, a wave moves rows in groups, and every lane issues all its loads (8)
// before its stores.  The unit's kept positions and the sequence's tail block
// ids are staged in LDS first, so a row's source and destination addresses
// need no global loads.

#include "kara_internal.hpp"

namespace kara {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Table entries a unit can touch: the tail from the boundary block, at most
// ceil((W + bs - 1) / bs) blocks, old or new.
__host__ __device__ inline int tail_blocks(int W, int bs) { return (W + bs - 1) / bs + 1; }

__global__ __launch_bounds__(kThreads) void compact_kernel(CompactArgs a) {
  extern __shared__ int32_t sh[];         // [R] kept positions, old tail ids, new tail ids
  const int cu = blockIdx.x;              // ((b * Lyr + l) * 2 + kv) * Hkv + h
  const int h = cu % a.Hkv;
  const int t1 = cu / a.Hkv;
  const int kv = t1 & 1;
  const int bl = t1 >> 1;                 // b * Lyr + l
  const int l = bl % a.Lyr;
  const int b = bl / a.Lyr;
  const int tid = threadIdx.x;

  const int W = a.W, B = a.B, R = a.R, bs = a.bs;
  const int max_tok = a.MB * bs;
  int L = a.lens[b];
  L = L < W ? W : (L > max_tok ? max_tok : L);
  const int start = L - W;
  const int f0 = start / bs;
  const int p = start - f0 * bs;
  const int n_rows = p + R + B;
  const int C = W - B;
  const int n_tail = tail_blocks(W, bs);

  // Stage the unit's kept positions and the sequence's old and new tail block
  // ids in LDS, so that every row copy below is one dependent global load.
  int32_t* s_ret = sh;
  int32_t* s_old = sh + R;
  int32_t* s_new = s_old + n_tail;
  auto clampb = [&](int blk) { return blk < 0 ? 0 : (blk >= a.NB ? a.NB - 1 : blk); };
  const int32_t* ret = a.retained + (size_t)bl * a.Hkv * R + (size_t)h * R;
  for (int i = tid; i < R; i += kThreads) {
    const int j = ret[i];
    s_ret[i] = j < 0 ? 0 : (j >= C ? C - 1 : j);
  }
  for (int i = tid; i < n_tail; i += kThreads) {
    const int e = f0 + i < a.MB ? f0 + i : a.MB - 1;
    s_old[i] = clampb(a.old_table[(size_t)b * a.MB + e]);
    s_new[i] = clampb(a.new_table[(size_t)b * a.MB + e]);
  }
  __syncthreads();

  const size_t row_bytes = (size_t)a.row_bytes;
  const size_t blk_bytes = (size_t)a.Hkv * bs * row_bytes;
  char* base = (char*)a.pool + ((size_t)(l * 2 + kv) * a.NB * a.Hkv + h) * bs * row_bytes;
  const int pieces = a.row_bytes / 16;            // 16-B pieces per row
  const int rows_per_pass = kThreads / pieces;    // rows moved per pass of the block
  const int my_row = tid / pieces;
  const int pc = tid - my_row * pieces;
  if (my_row >= rows_per_pass) return;            // lanes beyond whole rows idle (no barriers below)

  // Row n of the new tail: the boundary block's leading tokens, the kept
  // window positions, the protected tokens.  Token t of the old sequence lies
  // in old tail block t / bs - f0; new row n in new tail block n / bs.
  auto src_of = [&](int n) -> const u32x4* {
    const int t = n < p ? f0 * bs + n : (n < p + R ? start + s_ret[n - p] : L - B + (n - p - R));
    return (const u32x4*)(base + (size_t)s_old[t / bs - f0] * blk_bytes + (size_t)(t % bs) * row_bytes) + pc;
  };
  auto dst_of = [&](int n) -> u32x4* {
    return (u32x4*)(base + (size_t)s_new[n / bs] * blk_bytes + (size_t)(n % bs) * row_bytes) + pc;
  };

  for (int n0 = my_row; n0 < n_rows; n0 += rows_per_pass * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int n = n0 + u * rows_per_pass;
      if (n < n_rows) v[u] = __builtin_nontemporal_load(src_of(n));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int n = n0 + u * rows_per_pass;
      if (n < n_rows) __builtin_nontemporal_store(v[u], dst_of(n));
    }
  }
}

}  // namespace

hipError_t launch_compact(const CompactArgs& a, hipStream_t stream) {
  const long long n = (long long)a.S * a.Lyr * 2 * a.Hkv;
  if (n == 0) return hipSuccess;
  const size_t lds = ((size_t)a.R + 2 * (size_t)tail_blocks(a.W, a.bs)) * sizeof(int32_t);
  hipLaunchKernelGGL(compact_kernel, dim3((unsigned)n), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace kara
