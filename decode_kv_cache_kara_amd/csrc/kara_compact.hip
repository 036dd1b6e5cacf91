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
// 16 B, a wave moves rows in groups, and every lane issues all its loads before
// its stores so that several 16-B loads per lane are in flight.

#include "kara_internal.hpp"

namespace kara {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void compact_kernel(CompactArgs a) {
  const int cu = blockIdx.x;              // ((b * Lyr + l) * 2 + kv) * Hkv + h
  const int h = cu % a.Hkv;
  const int t1 = cu / a.Hkv;
  const int kv = t1 & 1;
  const int bl = t1 >> 1;                 // b * Lyr + l
  const int l = bl % a.Lyr;
  const int b = bl / a.Lyr;

  const int W = a.W, B = a.B, R = a.R, bs = a.bs;
  const int max_tok = a.MB * bs;
  int L = a.lens[b];
  L = L < W ? W : (L > max_tok ? max_tok : L);
  const int start = L - W;
  const int f0 = start / bs;
  const int p = start - f0 * bs;
  const int n_rows = p + R + B;
  const int C = W - B;

  const int32_t* ret = a.retained + (size_t)bl * a.Hkv * R + (size_t)h * R;
  const int32_t* otab = a.old_table + (size_t)b * a.MB;
  const int32_t* ntab = a.new_table + (size_t)b * a.MB;
  const size_t row_bytes = (size_t)a.row_bytes;
  const size_t blk_bytes = (size_t)a.Hkv * bs * row_bytes;
  char* base = (char*)a.pool + ((size_t)(l * 2 + kv) * a.NB * a.Hkv + h) * bs * row_bytes;

  const int pieces = a.row_bytes / 16;            // 16-B pieces per row
  const int rows_per_pass = kThreads / pieces;    // rows moved per pass of the block
  const int my_row = threadIdx.x / pieces;
  const int pc = threadIdx.x - my_row * pieces;
  if (my_row >= rows_per_pass) return;            // lanes beyond whole rows idle (no barriers below)

  auto clampb = [&](int blk) { return blk < 0 ? 0 : (blk >= a.NB ? a.NB - 1 : blk); };
  auto src_of = [&](int n) -> const u32x4* {
    int t;
    if (n < p) {
      t = f0 * bs + n;
    } else if (n < p + R) {
      int j = ret[n - p];
      j = j < 0 ? 0 : (j >= C ? C - 1 : j);
      t = start + j;
    } else {
      t = L - B + (n - p - R);
    }
    return (const u32x4*)(base + (size_t)clampb(otab[t / bs]) * blk_bytes + (size_t)(t % bs) * row_bytes) + pc;
  };
  auto dst_of = [&](int n) -> u32x4* {
    const int pos = f0 * bs + n;                  // token position in the new sequence
    int e = pos / bs;
    e = e >= a.MB ? a.MB - 1 : e;
    return (u32x4*)(base + (size_t)clampb(ntab[e]) * blk_bytes + (size_t)(pos % bs) * row_bytes) + pc;
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
  hipLaunchKernelGGL(compact_kernel, dim3((unsigned)n), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kara
