// Top-K candidate selection and Token2Chunk, one wave per unit.
//
// The unit's scores are the chunk-ordered sums of the scoring kernel's partial
// column sums.  Both selections (the K candidates; the top-up of the budget)
// are exact radix selects over order-preserving 32-bit keys: from the highest
// bit in which the eligible keys differ down, the threshold key is fixed one
// bit at a time by counting matching keys with wave ballots, and keys equal to
// the threshold are taken in position order through a wave prefix count, so
// the results are the "largest score, lower position first" sets bit for bit
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

#include <type_traits>

namespace kara {
namespace {

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

// ---------------------------------------------------------------------------
// One wave per unit.  Lane l owns the contiguous positions [l*P, l*P + P) of
// the region (P = ceil(C / 64)), so position order is (lane, slot) order and
// prefix counts are wave scans.  The order keys of a lane's positions stay in
// registers and the marks of its positions in bit masks (bit i = slot i);
// the scores, a flag per position, and per candidate or span the position,
// chunk score, gap, rank and ranked gap live in the wave's part of LDS.
// There is no workgroup barrier: the waves of a workgroup score different
// units, and a wave orders its own LDS accesses with a wavefront fence.
// ---------------------------------------------------------------------------

constexpr int kSelWaves = 4;   // units per workgroup when LDS allows

struct WaveShared {
  float* s;         // [C]
  uint8_t* flag;    // [C]
  int* cand;        // [K]
  float* sigma;     // [K]
  int* gap;         // [K]
  int* rank;        // [K]
  int* ordgap;      // [K]
};

__host__ __device__ inline size_t wave_lds_bytes(int C, int K) {
  return (size_t)C * 4 + ((size_t)C + 3) / 4 * 4 + (size_t)K * 20;
}

__device__ inline WaveShared carve_wave(char* base, int C, int K) {
  WaveShared sh;
  char* p = base;
  auto take = [&](size_t n) { char* q = p; p += (n + 3) / 4 * 4; return q; };
  sh.s = (float*)take((size_t)C * 4);
  sh.flag = (uint8_t*)take((size_t)C);
  sh.cand = (int*)take((size_t)K * 4);
  sh.sigma = (float*)take((size_t)K * 4);
  sh.gap = (int*)take((size_t)K * 4);
  sh.rank = (int*)take((size_t)K * 4);
  sh.ordgap = (int*)take((size_t)K * 4);
  return sh;
}

// Makes this wave's earlier LDS writes visible to its later LDS reads.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int t = __shfl_xor(v, o);
    v = t > v ? t : v;
  }
  return v;
}

// Exclusive prefix over lanes; *total = sum over the wave.
__device__ __forceinline__ int wave_excl(int v, int* total) {
  const int inc = wave_incl_scan(v);
  *total = __shfl(inc, 63);
  return inc - v;
}

// Sum of v over the wave (every lane gets it): DPP sums within each row of 16
// lanes, then the four row sums.
__device__ __forceinline__ int wave_sum(int v) {
  auto add_dpp = [](int x, auto ctrl) {
    return x + __builtin_amdgcn_update_dpp(0, x, decltype(ctrl)::value, 0xF, 0xF, false);
  };
  v = add_dpp(v, std::integral_constant<int, 0xB1>());    // quad_perm [1,0,3,2]
  v = add_dpp(v, std::integral_constant<int, 0x4E>());    // quad_perm [2,3,0,1]
  v = add_dpp(v, std::integral_constant<int, 0x141>());   // row_half_mirror
  v = add_dpp(v, std::integral_constant<int, 0x140>());   // row_mirror
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
         __builtin_amdgcn_readlane(v, 48);
}

// Marks (returned bit mask) of the n largest keys among the lane slots in
// `elig` over the wave, ties to the lower position.  Requires 1 <= n <= the
// number of eligible slots.  Bitwise radix select: from the highest bit in
// which the eligible keys differ down, the n-th largest key T is fixed one bit
// at a time.  `live` marks the eligible slots whose key matches T on the bits
// fixed so far; at each bit the live keys with the bit set are counted over the
// wave: if there are at least as many as still wanted, T has the bit set and
// the others leave; otherwise they are all above T, are taken, and leave.
// The live slots left at the end hold keys equal to T and are taken in
// position order up to n.
template <int kP>
__device__ uint32_t wave_select(const uint32_t* key, uint32_t elig, int n) {
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < kP; ++i) {
    if ((elig >> i) & 1u) {
      kmin = key[i] < kmin ? key[i] : kmin;
      kmax = key[i] > kmax ? key[i] : kmax;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t a = __shfl_xor(kmin, o), b = __shfl_xor(kmax, o);
    kmin = a < kmin ? a : kmin;
    kmax = b > kmax ? b : kmax;
  }
  const uint32_t diff = kmin ^ kmax;
  uint32_t live = elig, above = 0u;
  int remaining = n;
  if (diff != 0u) {
    for (int b = 31 - __clz((int)diff); b >= 0; --b) {
      uint32_t ones = 0u;                        // slots whose key has bit b set
#pragma unroll
      for (int i = 0; i < kP; ++i) ones |= ((key[i] >> b) & 1u) << i;
      const uint32_t hi = live & ones;
      const int cnt = wave_sum(__popc(hi));
      if (cnt >= remaining) {
        live = hi;
      } else {
        above |= hi;
        live &= ~ones;
        remaining -= cnt;
      }
    }
  }
  int tot;
  int before = wave_excl(__popc(live), &tot);
  uint32_t sel = above;
#pragma unroll
  for (int i = 0; i < kP; ++i) {
    if ((live >> i) & 1u) {
      if (before < remaining) sel |= 1u << i;
      ++before;
    }
  }
  return sel;
}

// Writes the ascending positions marked in `m` to out[0..cap).
template <int kP>
__device__ void wave_write(uint32_t m, int j0, int32_t* out, int cap) {
  int tot;
  int off = wave_excl(__popc(m), &tot);
#pragma unroll
  for (int i = 0; i < kP; ++i) {
    if ((m >> i) & 1u) {
      if (off < cap) out[off] = j0 + i;
      ++off;
    }
  }
}

template <int kP>
__global__ __launch_bounds__(64 * kSelWaves) void select_wave_kernel(SelectArgs a, size_t wave_bytes) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int unit = blockIdx.x * (int)(blockDim.x >> 6) + wave;
  if (unit >= a.n_units) return;                  // per wave: no workgroup barriers below
  const int C = a.C, K = a.K, R = a.R;
  WaveShared sh = carve_wave(smem + (size_t)wave * wave_bytes, C, K);
  const int P = (C + 63) / 64;
  const int j0 = lane * P;
  const int nmine = C - j0 < 0 ? 0 : (C - j0 > P ? P : C - j0);
  const uint32_t valid = nmine >= 32 ? 0xffffffffu : ((1u << nmine) - 1u);

  // unit scores: the partial sums of the row chunks added in chunk order.
  // Four positions and eight chunks are loaded at a time (32 loads in flight
  // per lane) before any is added, so the wave waits once per batch rather
  // than once per load.
  const float* pp = a.partials + (size_t)unit * a.n_split * C;
  constexpr int kJ = 4, kKb = 8;
  for (int jb = 0; jb < C; jb += 64 * kJ) {
    float acc[kJ];
#pragma unroll
    for (int u = 0; u < kJ; ++u) acc[u] = 0.0f;
    for (int k0 = 0; k0 < a.n_split; k0 += kKb) {
      float v[kJ][kKb];
#pragma unroll
      for (int u = 0; u < kJ; ++u) {
        const int j = jb + lane + 64 * u;
#pragma unroll
        for (int kk = 0; kk < kKb; ++kk)
          v[u][kk] = (j < C && k0 + kk < a.n_split) ? pp[(size_t)(k0 + kk) * C + j] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kJ; ++u)
#pragma unroll
        for (int kk = 0; kk < kKb; ++kk)
          if (k0 + kk < a.n_split) acc[u] += v[u][kk];
    }
#pragma unroll
    for (int u = 0; u < kJ; ++u) {
      const int j = jb + lane + 64 * u;
      if (j < C) {
        sh.s[j] = acc[u];
        sh.flag[j] = 0;
        if (a.scores_out) a.scores_out[(size_t)unit * C + j] = acc[u];
      }
    }
  }
  wave_sync();
  uint32_t key[kP];
#pragma unroll
  for (int i = 0; i < kP; ++i) key[i] = i < nmine ? order_key(sh.s[j0 + i]) : 0u;

  uint32_t cand;
  if (a.mode == kSelectT2C) {
    const int32_t* ci = a.cand_in + (size_t)unit * K;
    for (int m = lane; m < K; m += 64) {
      int j = ci[m];
      j = j < 0 ? 0 : (j >= C ? C - 1 : j);
      sh.flag[j] = 1;
    }
    wave_sync();
    cand = 0u;
#pragma unroll
    for (int i = 0; i < kP; ++i)
      if (i < nmine && sh.flag[j0 + i]) cand |= 1u << i;
  } else {
    cand = wave_select<kP>(key, valid, K);
    if (a.cand_out) wave_write<kP>(cand, j0, a.cand_out + (size_t)unit * K, K);
    if (a.mode == kSelectTopK) return;
  }

  uint32_t keep;
  if (R < K) {
    keep = wave_select<kP>(key, valid, R);
  } else if (a.no_chunks) {
    // Token2Chunk off: the top-K set plus the R - K best of the rest
    keep = cand | (R > K ? wave_select<kP>(key, valid & ~cand, R - K) : 0u);
  } else {
    // Token2Chunk: candidates in ascending order
    int nc;
    const int cb = wave_excl(__popc(cand), &nc);
    {
      int o = cb;
#pragma unroll
      for (int i = 0; i < kP; ++i)
        if ((cand >> i) & 1u) sh.cand[o++] = j0 + i;
    }
    wave_sync();
    uint32_t span = 0u, topup = 0u;
    if (R > nc) {
      const int nspan = nc - 1;
      for (int m = lane; m < nspan; m += 64) {
        const int x = sh.cand[m], y = sh.cand[m + 1];
        const int g = y - x - 1;
        sh.gap[m] = g;
        sh.sigma[m] = g > 0 ? __fdiv_rn(__fadd_rn(sh.s[x], sh.s[y]), (float)(g + 2)) : 0.0f;
      }
      wave_sync();
      // rank among spans with a gap: (sigma desc, left endpoint asc)
      int nvalid_lane = 0;
      for (int m = lane; m < nspan; m += 64) {
        int r = -1;
        if (sh.gap[m] != 0) {
          const float sm = sh.sigma[m];
          r = 0;
          for (int o = 0; o < nspan; ++o) {
            if (sh.gap[o] == 0) continue;
            const float so = sh.sigma[o];
            r += (so > sm || (so == sm && o < m)) ? 1 : 0;
          }
          ++nvalid_lane;
        }
        sh.rank[m] = r;
      }
      wave_sync();
      for (int m = lane; m < nspan; m += 64)
        if (sh.rank[m] >= 0) sh.ordgap[sh.rank[m]] = sh.gap[m];
      int nvalid;
      (void)wave_excl(nvalid_lane, &nvalid);
      wave_sync();
      // inclusive prefix of the gaps in rank order
      {
        const int per = (nvalid + 63) / 64;
        const int a0 = lane * per < nvalid ? lane * per : nvalid;
        const int a1 = a0 + per < nvalid ? a0 + per : nvalid;
        int sum = 0;
        for (int r = a0; r < a1; ++r) sum += sh.ordgap[r];
        int tot;
        int run = wave_excl(sum, &tot);
        for (int r = a0; r < a1; ++r) {
          run += sh.ordgap[r];
          sh.ordgap[r] = run;
        }
      }
      wave_sync();
      const int room = R - nc;
      // accepted spans mark their interiors: span m holds the non-candidates
      // whose count of candidates so far is m + 1
      {
        int seen = cb;
#pragma unroll
        for (int i = 0; i < kP; ++i) {
          if (i >= nmine) continue;
          if ((cand >> i) & 1u) {
            ++seen;
          } else if (seen >= 1 && seen <= nspan) {
            const int r = sh.rank[seen - 1];
            if (r >= 0 && sh.ordgap[r] <= room) span |= 1u << i;
          }
        }
      }
      // tokens added by the accepted spans = the largest accepted prefix sum
      int used = 0;
      for (int m = lane; m < nspan; m += 64) {
        const int r = sh.rank[m];
        if (r >= 0 && sh.ordgap[r] <= room && sh.ordgap[r] > used) used = sh.ordgap[r];
      }
      used = wave_max(used);
      const int need = room - used;
      if (need > 0) topup = wave_select<kP>(key, valid & ~cand & ~span, need);
    }
    keep = cand | span | topup;
  }
  wave_write<kP>(keep, j0, a.retained_out + (size_t)unit * R, R);
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  if (a.n_units == 0) return hipSuccess;
  // one wave per unit, as many waves per workgroup as 64 KiB of LDS holds
  // (at most 3.5 KiB + 0.9 KiB + 20 B per candidate at C = 896, K = 64;
  // 51 KiB at C = K = 2048)
  const size_t wave_bytes = (wave_lds_bytes(a.C, a.K) + 15) / 16 * 16;
  int waves = (int)(65536 / wave_bytes);
  waves = waves < 1 ? 1 : (waves > kSelWaves ? kSelWaves : waves);
  const unsigned grid = (unsigned)((a.n_units + waves - 1) / waves);
  const size_t bytes = wave_bytes * waves;
  const int P = (a.C + 63) / 64;
  if (P <= 8)
    hipLaunchKernelGGL(select_wave_kernel<8>, dim3(grid), dim3(64 * waves), bytes, stream, a, wave_bytes);
  else if (P <= 16)
    hipLaunchKernelGGL(select_wave_kernel<16>, dim3(grid), dim3(64 * waves), bytes, stream, a, wave_bytes);
  else
    hipLaunchKernelGGL(select_wave_kernel<32>, dim3(grid), dim3(64 * waves), bytes, stream, a, wave_bytes);
  return hipGetLastError();
}

}  // namespace kara
