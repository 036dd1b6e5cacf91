// Top-K candidate selection and Token2Chunk, one workgroup per unit.
//
// Scores live in LDS as float32 and as order-preserving 32-bit keys.  Both
// selections (the K candidates; the top-up of the budget) are exact radix
// selects over the keys (four 8-bit digit passes with an LDS histogram), with
// ties at the threshold resolved by position through a block-wide prefix count,
// so the results are the "largest score, lower position first" sets bit for bit
// ("Technical Summary: Kara", Methodology 1, Selection).
//
// Token2Chunk ("Technical Summary: Kara", Methodology 2, Process and Outcome;
// paper Abstract: a subset of the selected pairs is expanded): consecutive
// candidates a < b with g = b - a - 1 > 0 interior positions form a span with
// score sigma = (s[a] + s[b]) / (g + 2) in float32 (one rounded add, one
// correctly rounded divide).  Spans are ranked by (sigma desc, a asc), the gaps
// are prefix-summed in that order, and every span whose inclusive prefix fits
// in R - K is accepted: the longest fitting prefix of the order.  The
// highest-scored positions outside candidates and accepted spans then top the
// set up to exactly R.  All decisions are integer or exactly specified float32
// operations, so this kernel and the CPU checker agree bit for bit on the same
// float32 scores.
//
// With Token2Chunk switched off (the ablation of "Technical Summary: Kara",
// Experimental Results, Ablation Studies) the kept set is the top-R set.

#include "kara_internal.hpp"

namespace kara {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

enum : uint8_t { kFree = 0, kCand = 1, kSpan = 2, kTopUp = 3 };

// LDS of one workgroup, carved from dynamic shared memory sized by the call:
// per position of the region its score, order key and state; per candidate
// (or span between consecutive candidates) the candidate position, chunk
// score, gap, rank and ranked gap; and small scratch.
struct SelectShared {
  float* s;           // [C]
  uint32_t* key;      // [C]
  uint8_t* state;     // [C]
  int* cand;          // [K]
  float* sigma;       // [K]
  int* gap;           // [K]
  int* ordgap;        // [K] gaps in rank order, then their inclusive prefix sums
  int* rank;          // [K]
  int* hist;          // [256]
  int* scan_tmp;      // [kWaves]
  int* misc;          // [4]
};

__host__ __device__ inline size_t select_lds_bytes(int C, int K) {
  const size_t c4 = (size_t)C * 4, k4 = (size_t)K * 4;
  return 2 * c4 + ((size_t)C + 3) / 4 * 4 + 5 * k4 + (256 + kWaves + 4) * 4;
}

__device__ inline SelectShared carve(char* base, int C, int K) {
  SelectShared sh;
  char* p = base;
  auto take = [&](size_t n) { char* q = p; p += (n + 3) / 4 * 4; return q; };
  sh.s = (float*)take((size_t)C * 4);
  sh.key = (uint32_t*)take((size_t)C * 4);
  sh.state = (uint8_t*)take((size_t)C);
  sh.cand = (int*)take((size_t)K * 4);
  sh.sigma = (float*)take((size_t)K * 4);
  sh.gap = (int*)take((size_t)K * 4);
  sh.ordgap = (int*)take((size_t)K * 4);
  sh.rank = (int*)take((size_t)K * 4);
  sh.hist = (int*)take(256 * 4);
  sh.scan_tmp = (int*)take(kWaves * 4);
  sh.misc = (int*)take(4 * 4);
  return sh;
}

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive prefix of v over threads in index order; *total = sum over all.
__device__ int block_excl_scan(int v, SelectShared& sh, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v);
  if (lane == 63) sh.scan_tmp[w] = inc;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int x = sh.scan_tmp[i];
    if (i < w) off += x;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return off + inc - v;
}

// Contiguous segment of [0, n) owned by this thread (prefix scans run in
// position order).
__device__ __forceinline__ void segment(int n, int* j0, int* j1) {
  const int per = (n + kThreads - 1) / kThreads;
  int a = threadIdx.x * per;
  int b = a + per;
  *j0 = a < n ? a : n;
  *j1 = b < n ? b : n;
}

// Marks with `tag` the n largest-key positions among those in state kFree
// (ties to the lower position).  Requires 1 <= n <= number of free positions.
__device__ void select_largest(SelectShared& sh, int C, int n, uint8_t tag) {
  const int tid = threadIdx.x;
  // The keys of the free positions agree on every bit above the highest bit in
  // which their largest and smallest differ, so the digit passes start at the
  // digit that holds that bit: a pass above it would put every key in one bin
  // (and spend its time on one contended LDS counter).
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (int j = tid; j < C; j += kThreads) {
    if (sh.state[j] == kFree) {
      const uint32_t k = sh.key[j];
      kmin = k < kmin ? k : kmin;
      kmax = k > kmax ? k : kmax;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t a = __shfl_xor(kmin, o), b = __shfl_xor(kmax, o);
    kmin = a < kmin ? a : kmin;
    kmax = b > kmax ? b : kmax;
  }
  uint32_t* scratch = (uint32_t*)sh.hist;
  if ((tid & 63) == 0) {
    scratch[2 * (tid >> 6)] = kmin;
    scratch[2 * (tid >> 6) + 1] = kmax;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t a = scratch[2 * w], b = scratch[2 * w + 1];
    kmin = a < kmin ? a : kmin;
    kmax = b > kmax ? b : kmax;
  }
  __syncthreads();
  const uint32_t diff = kmin ^ kmax;
  const int top = diff == 0u ? -8 : (31 - __clz(diff)) / 8 * 8;   // -8: all free keys are equal
  uint32_t mask = top >= 24 ? 0u : ~((1u << (top + 8)) - 1u);
  uint32_t prefix = kmax & mask;
  int remaining = n;
  for (int shift = top; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int j = tid; j < C; j += kThreads) {
      if (sh.state[j] == kFree) {
        const uint32_t k = sh.key[j];
        if ((k & mask) == prefix) atomicAdd(&sh.hist[(k >> shift) & 255u], 1);
      }
    }
    __syncthreads();
    if (tid < 64) {
      // lane l holds digits 255-4l .. 252-4l; counts accumulate from the top digit down
      const int d0 = 255 - 4 * tid;
      const int c0 = sh.hist[d0], c1 = sh.hist[d0 - 1], c2 = sh.hist[d0 - 2], c3 = sh.hist[d0 - 3];
      const int s = c0 + c1 + c2 + c3;
      const int inc = wave_incl_scan(s);
      const int before = inc - s;
      if (before < remaining && remaining <= inc) {
        int acc = before, d;
        if (acc + c0 >= remaining) {
          d = d0;
        } else if ((acc += c0) + c1 >= remaining) {
          d = d0 - 1;
        } else if ((acc += c1) + c2 >= remaining) {
          d = d0 - 2;
        } else {
          acc += c2;
          d = d0 - 3;
        }
        sh.misc[0] = d;
        sh.misc[1] = acc;
      }
    }
    __syncthreads();
    remaining -= sh.misc[1];
    prefix |= (uint32_t)sh.misc[0] << shift;
    mask |= 255u << shift;
    __syncthreads();
  }
  // prefix is the key of the n-th largest; take `remaining` of the keys equal
  // to it, lowest positions first.
  const uint32_t T = prefix;
  int j0, j1;
  segment(C, &j0, &j1);
  int eq = 0;
  for (int j = j0; j < j1; ++j) eq += (sh.state[j] == kFree && sh.key[j] == T);
  int tot;
  int before = block_excl_scan(eq, sh, &tot);
  for (int j = j0; j < j1; ++j) {
    if (sh.state[j] != kFree) continue;
    const uint32_t k = sh.key[j];
    if (k > T) {
      sh.state[j] = tag;
    } else if (k == T) {
      if (before < remaining) sh.state[j] = tag;
      ++before;
    }
  }
  __syncthreads();
}

// Writes the ascending positions whose state satisfies `pred` to out[0..cap).
template <typename P>
__device__ int write_positions(SelectShared& sh, int C, P pred, int32_t* out, int cap) {
  int j0, j1;
  segment(C, &j0, &j1);
  int cnt = 0;
  for (int j = j0; j < j1; ++j) cnt += pred(sh.state[j]) ? 1 : 0;
  int tot;
  int off = block_excl_scan(cnt, sh, &tot);
  for (int j = j0; j < j1; ++j)
    if (pred(sh.state[j])) {
      if (off < cap) out[off] = j;
      ++off;
    }
  __syncthreads();
  return tot;
}

__device__ void clear_state(SelectShared& sh, int C) {
  for (int j = threadIdx.x; j < C; j += kThreads) sh.state[j] = kFree;
  __syncthreads();
}

// Token2Chunk from candidates marked kCand; leaves kCand/kSpan/kTopUp marks on
// exactly R positions.
__device__ void token2chunk(SelectShared& sh, int C, int R) {
  const int tid = threadIdx.x;
  // ascending candidate list, and each thread's count of candidates before its segment
  int j0, j1;
  segment(C, &j0, &j1);
  int cnt = 0;
  for (int j = j0; j < j1; ++j) cnt += (sh.state[j] == kCand);
  int K;
  const int cbefore = block_excl_scan(cnt, sh, &K);
  {
    int o = cbefore;
    for (int j = j0; j < j1; ++j)
      if (sh.state[j] == kCand) sh.cand[o++] = j;
  }
  __syncthreads();
  if (R <= K) return;  // budget already met by the candidates

  // spans between consecutive candidates
  const int nspan = K - 1;
  for (int m = tid; m < nspan; m += kThreads) {
    const int a = sh.cand[m], b = sh.cand[m + 1];
    const int g = b - a - 1;
    sh.gap[m] = g;
    sh.sigma[m] = g > 0 ? __fdiv_rn(__fadd_rn(sh.s[a], sh.s[b]), (float)(g + 2)) : 0.0f;
  }
  __syncthreads();
  // rank among spans with a gap: (sigma desc, left endpoint asc)
  for (int m = tid; m < nspan; m += kThreads) {
    if (sh.gap[m] == 0) {
      sh.rank[m] = -1;
      continue;
    }
    const float sm = sh.sigma[m];
    int r = 0;
    for (int o = 0; o < nspan; ++o) {
      if (sh.gap[o] == 0) continue;
      const float so = sh.sigma[o];
      r += (so > sm || (so == sm && o < m)) ? 1 : 0;
    }
    sh.rank[m] = r;
  }
  __syncthreads();
  int nvalid_local = 0;
  for (int m = tid; m < nspan; m += kThreads) {
    if (sh.rank[m] >= 0) {
      sh.ordgap[sh.rank[m]] = sh.gap[m];
      ++nvalid_local;
    }
  }
  __syncthreads();
  int nvalid;
  {
    int dummy = block_excl_scan(nvalid_local, sh, &nvalid);
    (void)dummy;
  }
  // inclusive prefix of the gaps in rank order
  {
    int a0, a1;
    segment(nvalid, &a0, &a1);
    int sum = 0;
    for (int r = a0; r < a1; ++r) sum += sh.ordgap[r];
    int tot;
    int run = block_excl_scan(sum, sh, &tot);
    for (int r = a0; r < a1; ++r) {
      run += sh.ordgap[r];
      sh.ordgap[r] = run;
    }
  }
  __syncthreads();
  const int room = R - K;
  // accepted spans mark their interiors; span m holds the non-candidates whose
  // candidate count so far is m + 1
  {
    int seen = cbefore;
    for (int j = j0; j < j1; ++j) {
      if (sh.state[j] == kCand) {
        ++seen;
      } else if (seen >= 1 && seen <= nspan) {
        const int r = sh.rank[seen - 1];
        if (r >= 0 && sh.ordgap[r] <= room) sh.state[j] = kSpan;
      }
    }
  }
  // tokens added by the accepted spans = the largest accepted prefix sum
  int used_local = 0;
  for (int m = tid; m < nspan; m += kThreads) {
    const int r = sh.rank[m];
    if (r >= 0 && sh.ordgap[r] <= room && sh.ordgap[r] > used_local) used_local = sh.ordgap[r];
  }
  // block max through the histogram scratch
  if (tid == 0) sh.misc[2] = 0;
  __syncthreads();
  atomicMax(&sh.misc[2], used_local);
  __syncthreads();
  const int need = room - sh.misc[2];
  __syncthreads();
  if (need > 0) select_largest(sh, C, need, kTopUp);
}

__global__ __launch_bounds__(kThreads) void select_kernel(SelectArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  SelectShared sh = carve(smem, a.C, a.K);
  const int unit = blockIdx.x;
  const int C = a.C, K = a.K, R = a.R;
  const int tid = threadIdx.x;

  const float* p = a.partials + (size_t)unit * a.n_split * C;
  for (int j = tid; j < C; j += kThreads) {
    float s = 0.0f;
    for (int k = 0; k < a.n_split; ++k) s += p[(size_t)k * C + j];
    sh.s[j] = s;
    sh.key[j] = order_key(s);
    sh.state[j] = kFree;
    if (a.scores_out) a.scores_out[(size_t)unit * C + j] = s;
  }
  __syncthreads();

  if (a.mode == kSelectT2C) {
    const int32_t* ci = a.cand_in + (size_t)unit * K;
    for (int m = tid; m < K; m += kThreads) {
      int j = ci[m];
      j = j < 0 ? 0 : (j >= C ? C - 1 : j);
      sh.state[j] = kCand;
    }
    __syncthreads();
  } else {
    select_largest(sh, C, K, kCand);
    if (a.cand_out) write_positions(sh, C, [](uint8_t st) { return st == kCand; }, a.cand_out + (size_t)unit * K, K);
    if (a.mode == kSelectTopK) return;
  }

  if (R < K) {
    clear_state(sh, C);
    select_largest(sh, C, R, kCand);
  } else if (a.no_chunks) {
    // Token2Chunk off: the top-R set is the top-K set plus the R - K best of
    // the rest (one total order: score desc, position asc).
    if (R > K) select_largest(sh, C, R - K, kTopUp);
  } else {
    token2chunk(sh, C, R);
  }
  write_positions(sh, C, [](uint8_t st) { return st != kFree; }, a.retained_out + (size_t)unit * R, R);
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  if (a.n_units == 0) return hipSuccess;
  // at most 2 * 8 KiB + 2 KiB + 5 * 8 KiB + 1 KiB (C = K = 2048): within the
  // default 64 KiB of dynamic LDS
  const size_t bytes = select_lds_bytes(a.C, a.K);
  hipLaunchKernelGGL(select_kernel, dim3(a.n_units), dim3(kThreads), bytes, stream, a);
  return hipGetLastError();
}

}  // namespace kara
