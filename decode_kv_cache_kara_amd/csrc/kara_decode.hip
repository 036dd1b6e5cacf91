// The decode steps on either side of the compression step.
//
// append: one decode step's K and V rows go into the paged cache at the
//   sequence's next physical position, and its query states into the
//   sequence's ring of the last W query states ("Technical Summary: Kara",
//   Methodology 1, Mechanism: all window tokens' query states score the
//   region, so they are kept until the window is scored).  Pure 16-byte
//   copies, one workgroup per (sequence, layer).
//
// decode attention: the attention of one decode step's query heads over a
//   sequence's cached tokens, read through its block table (paper, Abstract:
//   the compressed cache is served through PagedAttention).  It is bound by
//   HBM: per token and KV head it reads one K and one V row (2 * D * elt
//   bytes) and does 4 * G * D flops.  Layout of the work:
//     * a workgroup takes 512 or 1024 tokens of one (sequence, KV head)
//       ("split"; the host picks 1024 for launches with many workgroups);
//       the G query heads of the group share every K/V row it reads, and the
//       split's block ids (loaded in the same round trip as the sequence's
//       length) are staged in LDS as row indices; splits past the sequence's
//       end exit at once;
//     * bf16: QK^T of 16 tokens per wave step on the matrix cores (see
//       attention_mfma_kernel); float32: D / 4 lanes hold one token's row as
//       16-byte pieces and dot products are summed across those lanes with
//       DPP row permutations (attention_kernel);
//     * a running maximum, sum and output per query head are rescaled only
//       when a maximum moves;
//     * lane groups, waves and then splits are merged with the usual
//       (max, sum, output) rescaling; the split merge is a second kernel.
//   Logits are kept in log2 units (the dot products are scaled by
//   log2(e) / sqrt(D)) and exp2 is used throughout.

#include "kara_internal.hpp"

#include <cmath>

namespace kara {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// append
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int b = blockIdx.x / a.n_lyr_in;
  const int li = blockIdx.x - b * a.n_lyr_in;
  const int l = a.layer >= 0 ? a.layer : li;
  const int tid = threadIdx.x;

  int pos = a.positions[b];
  const int max_pos = a.MB * a.bs - 1;
  pos = pos < 0 ? 0 : (pos > max_pos ? max_pos : pos);
  int blk = a.table[(size_t)b * a.MB + pos / a.bs];
  blk = blk < 0 ? 0 : (blk >= a.NB ? a.NB - 1 : blk);
  int slot = a.slots[b];
  slot = slot < 0 ? 0 : (slot >= a.n_slots ? a.n_slots - 1 : slot);
  int n = a.counts[b];
  n = n < 0 ? 0 : n;
  const int ring_pos = n % a.W;

  const int row_pieces = a.row_bytes / 16;            // one head's row
  const int q_pieces = a.Hq * row_pieces;
  const int kv_pieces = a.Hkv * row_pieces;
  const char* qs = (const char*)a.q + ((size_t)b * a.n_lyr_in + li) * q_pieces * 16;
  char* qd = (char*)a.ring + (((size_t)slot * a.Lyr + l) * a.W + ring_pos) * q_pieces * 16;
  for (int p = tid; p < q_pieces; p += 256)
    *(u32x4*)(qd + (size_t)p * 16) = *(const u32x4*)(qs + (size_t)p * 16);

  const size_t src_off = ((size_t)b * a.n_lyr_in + li) * kv_pieces * 16;
  for (int p = tid; p < kv_pieces; p += 256) {
    const int h = p / row_pieces, pc = p - h * row_pieces;
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      const char* src = (const char*)(kv ? a.v : a.k) + src_off + (size_t)p * 16;
      char* dst = (char*)a.pool +
                  (((((size_t)l * 2 + kv) * a.NB + blk) * a.Hkv + h) * a.bs + pos % a.bs) * a.row_bytes +
                  pc * 16;
      *(u32x4*)dst = *(const u32x4*)src;
    }
  }
}

// ---------------------------------------------------------------------------
// decode attention
// ---------------------------------------------------------------------------

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / 64;
// Tokens per lane group per step.  Fetching the next step's rows ahead of the
// current step's arithmetic costs occupancy and measured slower.
constexpr int kU = 4;

template <typename T>
__device__ __forceinline__ void unpack(const u32x4& w, float* f);

template <>
__device__ __forceinline__ void unpack<__bf16>(const u32x4& w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void unpack<float>(const u32x4& w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
}

// Merges (m2, l2, o2) into (m, l, o); maxima in log2 units, -inf = empty.
template <int E>
__device__ __forceinline__ void merge(float& m, float& l, float* o, float m2, float l2, const float* o2) {
  const float mn = fmaxf(m, m2);
  const float s1 = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
  const float s2 = (m2 == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m2 - mn);
  l = l * s1 + l2 * s2;
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = o[e] * s1 + o2[e] * s2;
  m = mn;
}

template <int Ctrl>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), Ctrl, 0xF, 0xF,
                                                                   false));
}

// Sum over aligned groups of N lanes (N = 2 .. 32), every lane of a group
// receiving the group's sum: swaps within quads, then the mirrored quad of
// the half row, then the mirrored half row (DPP), then the other row.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x = dpp_add<0xB1>(x);                      // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x = dpp_add<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x = dpp_add<0x141>(x);  // row_half_mirror
  if constexpr (N >= 16) x = dpp_add<0x140>(x); // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  return x;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <typename T, int D, int G>
__global__ __launch_bounds__(kAttnThreads) void attention_kernel(AttnArgs a) {
  constexpr int E = 16 / (int)sizeof(T);        // elements per 16-byte piece
  constexpr int kLanes = D / E;                 // lanes per token row
  constexpr int kGroups = 64 / kLanes;          // tokens per wave per load
  constexpr int kRowBytes = D * (int)sizeof(T);
  constexpr bool kBf16 = sizeof(T) == 2;
  __shared__ float sh_m[kAttnWaves][G], sh_l[kAttnWaves][G];
  __shared__ float sh_o[kAttnWaves][G][D];
  __shared__ int32_t sh_blk[kAttnChunkMax + 1];

  const int split = blockIdx.x % a.n_split;
  const int h = (blockIdx.x / a.n_split) % a.Hkv;
  const int b = blockIdx.x / (a.n_split * a.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane % kLanes, grp = lane / kLanes;

  int L = a.lens[b];
  const int max_tok = a.MB * a.bs;
  L = L < 1 ? 1 : (L > max_tok ? max_tok : L);
  const int t0 = split * a.chunk;
  // splits past the sequence's end hold nothing; the combine reads only the
  // sequence's own splits (same clamped length)
  if (t0 >= L) return;
  const int t1 = min(L, t0 + a.chunk);

  // the split's block ids, clamped to the pool
  const int e0 = t0 / a.bs;
  const int n_e = t1 > t0 ? (t1 - 1) / a.bs - e0 + 1 : 0;
  for (int i = tid; i < n_e; i += kAttnThreads) {
    const int blk = a.table[(size_t)b * a.MB + e0 + i];
    sh_blk[i] = blk < 0 ? 0 : (blk >= a.NB ? a.NB - 1 : blk);
  }
  __syncthreads();

  // this lane's piece of the G query rows: packed bf16 pairs (bf16), or
  // floats (fp32); logits are scaled to log2 units after the dot product
  u32x4 qw[G];
#pragma unroll
  for (int g = 0; g < G; ++g)
    qw[g] = *(const u32x4*)((const char*)a.q + (((size_t)b * a.Hq + h * G + g) * D + sub * E) * sizeof(T));
  float m[G], l[G], o[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[g][e] = 0.0f;
  }

  const char* kbase = (const char*)a.pool + ((size_t)a.layer * 2 * a.NB * a.Hkv + h) * a.bs * kRowBytes;
  const size_t v_off = (size_t)a.NB * a.Hkv * a.bs * kRowBytes;
  const size_t blk_bytes = (size_t)a.Hkv * a.bs * kRowBytes;
  constexpr int kStep = kAttnWaves * kGroups * kU;   // tokens per workgroup step
  const int my0 = (wave * kGroups + grp) * kU;

  auto load_rows = [&](int base, u32x4* kw, u32x4* vw) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int t = base + my0 + u;
      const int tc = t < t1 ? t : t1 - 1;
      const char* p = kbase + (size_t)sh_blk[tc / a.bs - e0] * blk_bytes + (size_t)(tc % a.bs) * kRowBytes + sub * 16;
      kw[u] = __builtin_nontemporal_load((const u32x4*)p);
      vw[u] = __builtin_nontemporal_load((const u32x4*)(p + v_off));
    }
  };
  for (int base = t0; base < t1; base += kStep) {
    u32x4 kw[kU], vw[kU];
    bool ok[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) ok[u] = base + my0 + u < t1;
    load_rows(base, kw, vw);
    float x[kU][G];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d = 0.0f;
        if constexpr (kBf16) {
          // (A bit cast of an indexed vector element inside this unrolled
          // loop compiles to element 0 every time with the ROCm 7.2 clang;
          // copying the pairs out first is compiled correctly.)
          bf16x2 qp[4], kp[4];
          __builtin_memcpy(qp, &qw[g], 16);
          __builtin_memcpy(kp, &kw[u], 16);
#pragma unroll
          for (int i = 0; i < 4; ++i) d = __builtin_amdgcn_fdot2_f32_bf16(qp[i], kp[i], d, false);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) d = fmaf(__uint_as_float(qw[g][i]), __uint_as_float(kw[u][i]), d);
        }
        x[u][g] = group_sum<kLanes>(d) * a.c;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = m[g];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (!ok[u]) x[u][g] = -INFINITY;
        mx = fmaxf(mx, x[u][g]);
      }
      // rescale only when some lane's running maximum moves (rare after the
      // first tokens); lanes whose maximum did not move multiply by 1
      if (__ballot(mx > m[g])) {
        const float sc = (mx == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m[g] - mx);
        l[g] *= sc;
#pragma unroll
        for (int e = 0; e < E; ++e) o[g][e] *= sc;
        m[g] = mx;
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float vf[E];
      unpack<T>(vw[u], vf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = (x[u][g] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(x[u][g] - m[g]);
        l[g] += p;
#pragma unroll
        for (int e = 0; e < E; ++e) o[g][e] = fmaf(p, vf[e], o[g][e]);
      }
    }
  }

  // merge the lane groups of the wave (same pieces, different tokens)
#pragma unroll
  for (int off = kLanes; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float m2 = __shfl_xor(m[g], off), l2 = __shfl_xor(l[g], off);
      float o2[E];
#pragma unroll
      for (int e = 0; e < E; ++e) o2[e] = __shfl_xor(o[g][e], off);
      merge<E>(m[g], l[g], o[g], m2, l2, o2);
    }
  }
  if (grp == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (sub == 0) {
        sh_m[wave][g] = m[g];
        sh_l[wave][g] = l[g];
      }
#pragma unroll
      for (int e = 0; e < E; ++e) sh_o[wave][g][sub * E + e] = o[g][e];
    }
  }
  __syncthreads();
  // merge the waves and write this split's (max, sum, output) per query head
  const size_t part = (size_t)(b * a.Hq + h * G) * a.n_split + split;
  for (int i = tid; i < G * D; i += kAttnThreads) {
    const int g = i / D, d = i - g * D;
    float mm = sh_m[0][g], ll = sh_l[0][g], oo = sh_o[0][g][d];
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) merge<1>(mm, ll, &oo, sh_m[w][g], sh_l[w][g], &sh_o[w][g][d]);
    const size_t pg = part + (size_t)g * a.n_split;
    a.part_o[pg * D + d] = oo;
    if (d == 0) {
      a.part_ml[2 * pg] = mm;
      a.part_ml[2 * pg + 1] = ll;
    }
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int kCtrl>
__device__ __forceinline__ float dpp_max(float x) {
  return fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF,
                                                                        0xF, false)));
}

// Maximum / sum over the 16 lanes of a DPP row.
__device__ __forceinline__ float row_max16(float x) {
  x = dpp_max<0xB1>(x);     // quad_perm [1,0,3,2]
  x = dpp_max<0x4E>(x);     // quad_perm [2,3,0,1]
  x = dpp_max<0x141>(x);    // row_half_mirror
  return dpp_max<0x140>(x); // row_mirror
}

// bf16 decode attention with QK^T on the matrix cores.  Per step a wave takes
// 16 consecutive tokens of the split: v_mfma_f32_16x16x32_bf16 multiplies the
// group's query heads (A operand: head = lane & 15, zero rows past G) by the
// 16 tokens' keys (B operand, loaded straight from the cache rows: token =
// lane & 15, dims 32 ks + 8 (lane >> 4) .. + 7), giving lane l the logits of
// heads 4 (l >> 4) .. + 3 for token l & 15.  The running maximum of a head is
// then one value per 16-lane row (a DPP row maximum), so every lane of the
// wave shares it; each lane keeps the partial sum of its own token column.
// P times V stays in float32 FMAs: the probabilities go through the wave's
// LDS tile [token][head] to the V layout (D / 8 lanes per 16-byte-piece row,
// 64 / (D / 8) rows per wave-wide load), and since the maximum is common to
// the wave, the lane groups' outputs are added without rescaling at the end.
template <int D, int G>
__global__ __launch_bounds__(kAttnThreads) void attention_mfma_kernel(AttnArgs a) {
  static_assert(G >= 1 && G <= 8, "query heads per KV head");
  constexpr int kKs = D / 32;               // reduction steps of 32 dims
  constexpr int kLanes = D / 8;             // lanes per V row (16-byte pieces)
  constexpr int kGroups = 64 / kLanes;      // V rows per wave-wide load
  constexpr int kT = 16;                    // tokens per wave step
  constexpr int kV = kT / kGroups;          // V rows per lane per step
  constexpr int kRowBytes = D * 2;
  constexpr int kRG = (G + 3) / 4;          // 16-lane rows holding query heads
  __shared__ float sh_m[kAttnWaves][G], sh_l[kAttnWaves][G];
  __shared__ float sh_o[kAttnWaves][G][D];
  __shared__ int32_t sh_blk[kAttnChunkMax + 1];
  __shared__ __attribute__((aligned(16))) float sh_p[kAttnWaves][kT][8];

  const int split = blockIdx.x % a.n_split;
  const int h = (blockIdx.x / a.n_split) % a.Hkv;
  const int b = blockIdx.x / (a.n_split * a.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // The split's blocks as the index of their first K row of head h within
  // the layer (rows of kRowBytes; fits 32 bits: the layer's K rows are
  // NB Hkv bs), block ids clamped to the pool.  The table entries of the
  // whole chunk (within the table row) are loaded together with the length,
  // so that the two loads take one round trip.
  const int t0 = split * a.chunk;
  const int e0 = t0 >> a.bs_shift;
  const int n_chunk = min(((a.chunk - 1) >> a.bs_shift) + 1, a.MB - e0);
  int blk_pre[(kAttnChunkMax + kAttnThreads - 1) / kAttnThreads];
#pragma unroll
  for (int k = 0; k < (kAttnChunkMax + kAttnThreads - 1) / kAttnThreads; ++k) {
    const int i = tid + k * kAttnThreads;
    blk_pre[k] = i < n_chunk ? a.table[(size_t)b * a.MB + e0 + i] : 0;
  }
  int L = a.lens[b];
  const int max_tok = a.MB * a.bs;
  L = L < 1 ? 1 : (L > max_tok ? max_tok : L);
  // splits past the sequence's end hold nothing; the combine reads only the
  // sequence's own splits (same clamped length)
  if (t0 >= L) return;
  const int t1 = min(L, t0 + a.chunk);
  const int n_e = ((t1 - 1) >> a.bs_shift) - e0 + 1;
#pragma unroll
  for (int k = 0; k < (kAttnChunkMax + kAttnThreads - 1) / kAttnThreads; ++k) {
    const int i = tid + k * kAttnThreads;
    if (i < n_e) {
      const int blk = blk_pre[k] < 0 ? 0 : (blk_pre[k] >= a.NB ? a.NB - 1 : blk_pre[k]);
      sh_blk[i] = (int32_t)(((uint32_t)blk * (uint32_t)a.Hkv + (uint32_t)h) << a.bs_shift);
    }
  }
  // query heads as the A operand (rows past G are zero)
  const int col = lane & 15, rg = lane >> 4;
  bf16x8 qa[kKs];
#pragma unroll
  for (int ks = 0; ks < kKs; ++ks) {
    if (col < G) {
      qa[ks] = *(const bf16x8*)((const char*)a.q + (((size_t)b * a.Hq + h * G + col) * D + 32 * ks + 8 * rg) * 2);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qa[ks][e] = (__bf16)0.0f;
    }
  }
  __syncthreads();

  float mrun[4], lrun[4];                   // heads 4 rg + r: running maximum (log2), sum over this lane's tokens
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    mrun[r] = -INFINITY;
    lrun[r] = 0.0f;
  }
  const int vsub = lane % kLanes, vgrp = lane / kLanes;
  float o[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[g][e] = 0.0f;

  const char* kbase = (const char*)a.pool + (size_t)a.layer * 2 * a.NB * a.Hkv * a.bs * kRowBytes;
  const char* vbase = kbase + (size_t)a.NB * a.Hkv * a.bs * kRowBytes;
  const int bs_mask = a.bs - 1;
  // K or V row of token t (t inside the split)
  auto row_ptr = [&](const char* base, int t) -> const char* {
    const uint32_t row = (uint32_t)sh_blk[(t >> a.bs_shift) - e0] + (uint32_t)(t & bs_mask);
    return base + (size_t)row * kRowBytes;
  };
  float* pt = &sh_p[wave][0][0];

  for (int base = t0 + wave * kT; base < t1; base += kAttnWaves * kT) {
    // keys of token base + col (clamped; masked below) and this lane's V rows
    const char* kp = row_ptr(kbase, min(base + col, t1 - 1)) + 16 * rg;
    u32x4 kw[kKs];
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) kw[ks] = __builtin_nontemporal_load((const u32x4*)(kp + 64 * ks));
    u32x4 vw[kV];
#pragma unroll
    for (int j = 0; j < kV; ++j)
      vw[j] = __builtin_nontemporal_load(
          (const u32x4*)(row_ptr(vbase, min(base + vgrp + kGroups * j, t1 - 1)) + 16 * vsub));
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
      bf16x8 kf;
      __builtin_memcpy(&kf, &kw[ks], 16);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kf, acc, 0, 0, 0);
    }
    const bool tok_ok = base + col < t1;
    float x[4], mx[4];
    bool moved = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = tok_ok ? acc[r] * a.c : -INFINITY;
      mx[r] = fmaxf(mrun[r], row_max16(x[r]));
      moved |= 4 * rg + r < G && mx[r] > mrun[r];
    }
    // a head's maximum moved (rare after the first steps): rescale its sums
    // and outputs (the factor of head g is held by lane 16 (g / 4))
    if (__ballot(moved)) {
      float sc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[r] = mx[r] == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(mrun[r] - mx[r]);
        lrun[r] *= sc[r];
        mrun[r] = mx[r];
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float s = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc[g % 4]), 16 * (g / 4)));
#pragma unroll
        for (int e = 0; e < 8; ++e) o[g][e] *= s;
      }
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = x[r] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x[r] - mrun[r]);
      lrun[r] += p[r];
    }
    // probabilities to the V layout through the wave's tile [token][head]
    if (rg < kRG) *(float4*)&pt[col * 8 + 4 * rg] = make_float4(p[0], p[1], p[2], p[3]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int j = 0; j < kV; ++j) {
      const int tl = vgrp + kGroups * j;
      float pv[8];
      *(float4*)&pv[0] = *(const float4*)&pt[tl * 8];
      if (G > 4) *(float4*)&pv[4] = *(const float4*)&pt[tl * 8 + 4];
      float vf[8];
      unpack<__bf16>(vw[j], vf);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[g][e] = fmaf(pv[g], vf[e], o[g][e]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // the wave's sums over its 16 token columns, and its outputs over the lane
  // groups (same dims, different tokens, one running maximum per head)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float v = lrun[r];
    v = dpp_add<0xB1>(v);
    v = dpp_add<0x4E>(v);
    v = dpp_add<0x141>(v);
    lrun[r] = dpp_add<0x140>(v);
  }
#pragma unroll
  for (int off = kLanes; off < 64; off <<= 1)
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[g][e] += __shfl_xor(o[g][e], off);
  if (col == 0 && rg < kRG) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = 4 * rg + r;
      if (g < G) {
        sh_m[wave][g] = mrun[r];
        sh_l[wave][g] = lrun[r];
      }
    }
  }
  if (vgrp == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) sh_o[wave][g][vsub * 8 + e] = o[g][e];
  }
  __syncthreads();
  // merge the waves and write this split's (max, sum, output) per query head
  const size_t part = (size_t)(b * a.Hq + h * G) * a.n_split + split;
  for (int i = tid; i < G * D; i += kAttnThreads) {
    const int g = i / D, d = i - g * D;
    float mm = sh_m[0][g], ll = sh_l[0][g], oo = sh_o[0][g][d];
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) merge<1>(mm, ll, &oo, sh_m[w][g], sh_l[w][g], &sh_o[w][g][d]);
    const size_t pg = part + (size_t)g * a.n_split;
    a.part_o[pg * D + d] = oo;
    if (d == 0) {
      a.part_ml[2 * pg] = mm;
      a.part_ml[2 * pg + 1] = ll;
    }
  }
}

// out[b][g] = merge over splits; one workgroup per (sequence, query head).
// Splits are read eight at a time (all loads of a batch issued before any is
// used), then merged in split order.
template <int D>
__global__ __launch_bounds__(D) void combine_kernel(AttnArgs a) {
  constexpr int kB = 8;
  const int bg = blockIdx.x;
  const int d = threadIdx.x;
  // the sequence's own splits (its clamped length, as in attention_kernel)
  int L = a.lens[bg / a.Hq];
  const int max_tok = a.MB * a.bs;
  L = L < 1 ? 1 : (L > max_tok ? max_tok : L);
  const int n = min(a.n_split, (L + a.chunk - 1) / a.chunk);
  const size_t p0 = (size_t)bg * a.n_split;
  float mm = -INFINITY;
  for (int s0 = 0; s0 < n; s0 += kB) {
    float ms[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) ms[u] = s0 + u < n ? a.part_ml[2 * (p0 + s0 + u)] : -INFINITY;
#pragma unroll
    for (int u = 0; u < kB; ++u) mm = fmaxf(mm, ms[u]);
  }
  float num = 0.0f, den = 0.0f;
  for (int s0 = 0; s0 < n; s0 += kB) {
    float ms[kB], ls[kB], os[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const bool ok = s0 + u < n;
      ms[u] = ok ? a.part_ml[2 * (p0 + s0 + u)] : -INFINITY;
      ls[u] = ok ? a.part_ml[2 * (p0 + s0 + u) + 1] : 0.0f;
      os[u] = ok ? a.part_o[(p0 + s0 + u) * D + d] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      if (ms[u] == -INFINITY) continue;
      const float w = __builtin_amdgcn_exp2f(ms[u] - mm);
      den = fmaf(ls[u], w, den);
      num = fmaf(os[u], w, num);
    }
  }
  a.out[(size_t)bg * D + d] = num / den;
}

// Measurement aid, not part of the path: the bf16 attention kernel's memory
// traffic alone.  The same workgroup decomposition (one split of a.chunk
// tokens of one sequence and KV head per workgroup, empty splits exiting at
// once), the same block-id staging in LDS and the same per-wave 16-token
// steps with 16-byte nontemporal loads of the K rows (B-operand layout) and
// V rows, but no arithmetic: the loaded words are XOR-folded, and a lane
// stores its fold only if it equals a fixed value, so the loads stay live and
// nothing is written in practice (dst needs 4 bytes).
template <int D>
__global__ __launch_bounds__(kAttnThreads) void paged_read_probe_kernel(AttnArgs a, uint32_t* dst) {
  constexpr int kKs = D / 32;
  constexpr int kLanes = D / 8;
  constexpr int kGroups = 64 / kLanes;
  constexpr int kT = 16;
  constexpr int kV = kT / kGroups;
  constexpr int kRowBytes = D * 2;
  __shared__ int32_t sh_blk[kAttnChunkMax + 1];
  const int split = blockIdx.x % a.n_split;
  const int h = (blockIdx.x / a.n_split) % a.Hkv;
  const int b = blockIdx.x / (a.n_split * a.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = split * a.chunk;
  const int e0 = t0 >> a.bs_shift;
  const int n_chunk = min(((a.chunk - 1) >> a.bs_shift) + 1, a.MB - e0);
  int blk_pre[(kAttnChunkMax + kAttnThreads - 1) / kAttnThreads];
#pragma unroll
  for (int k = 0; k < (kAttnChunkMax + kAttnThreads - 1) / kAttnThreads; ++k) {
    const int i = tid + k * kAttnThreads;
    blk_pre[k] = i < n_chunk ? a.table[(size_t)b * a.MB + e0 + i] : 0;
  }
  int L = a.lens[b];
  const int max_tok = a.MB * a.bs;
  L = L < 1 ? 1 : (L > max_tok ? max_tok : L);
  if (t0 >= L) return;
  const int t1 = min(L, t0 + a.chunk);
  const int n_e = ((t1 - 1) >> a.bs_shift) - e0 + 1;
#pragma unroll
  for (int k = 0; k < (kAttnChunkMax + kAttnThreads - 1) / kAttnThreads; ++k) {
    const int i = tid + k * kAttnThreads;
    if (i < n_e) {
      const int blk = blk_pre[k] < 0 ? 0 : (blk_pre[k] >= a.NB ? a.NB - 1 : blk_pre[k]);
      sh_blk[i] = (int32_t)(((uint32_t)blk * (uint32_t)a.Hkv + (uint32_t)h) << a.bs_shift);
    }
  }
  __syncthreads();
  const int col = lane & 15, rg = lane >> 4;
  const int vsub = lane % kLanes, vgrp = lane / kLanes;
  const char* kbase = (const char*)a.pool + (size_t)a.layer * 2 * a.NB * a.Hkv * a.bs * kRowBytes;
  const char* vbase = kbase + (size_t)a.NB * a.Hkv * a.bs * kRowBytes;
  const int bs_mask = a.bs - 1;
  auto row_ptr = [&](const char* base, int t) -> const char* {
    const uint32_t row = (uint32_t)sh_blk[(t >> a.bs_shift) - e0] + (uint32_t)(t & bs_mask);
    return base + (size_t)row * kRowBytes;
  };
  u32x4 fold = {0u, 0u, 0u, 0u};
  for (int base = t0 + wave * kT; base < t1; base += kAttnWaves * kT) {
    const char* kp = row_ptr(kbase, min(base + col, t1 - 1)) + 16 * rg;
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) fold ^= __builtin_nontemporal_load((const u32x4*)(kp + 64 * ks));
#pragma unroll
    for (int j = 0; j < kV; ++j)
      fold ^= __builtin_nontemporal_load(
          (const u32x4*)(row_ptr(vbase, min(base + vgrp + kGroups * j, t1 - 1)) + 16 * vsub));
  }
  const uint32_t w = fold.x ^ fold.y ^ fold.z ^ fold.w;
  if (w == 0x9E3779B9u) dst[0] = w;
}

template <typename T, int D, int G>
hipError_t launch_attention_g(const AttnArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)a.S * a.Hkv * a.n_split;
  if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((attention_mfma_kernel<D, G>), dim3(grid), dim3(kAttnThreads), 0, s, a);
  else
    hipLaunchKernelGGL((attention_kernel<T, D, G>), dim3(grid), dim3(kAttnThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((combine_kernel<D>), dim3((unsigned)a.S * a.Hq), dim3(D), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_attention_d(const AttnArgs& a, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_attention_g<T, D, 1>(a, s);
    case 2: return launch_attention_g<T, D, 2>(a, s);
    case 3: return launch_attention_g<T, D, 3>(a, s);
    case 4: return launch_attention_g<T, D, 4>(a, s);
    case 5: return launch_attention_g<T, D, 5>(a, s);
    case 6: return launch_attention_g<T, D, 6>(a, s);
    case 7: return launch_attention_g<T, D, 7>(a, s);
    case 8: return launch_attention_g<T, D, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  if (a.S == 0) return hipSuccess;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)a.S * a.n_lyr_in), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_paged_read_probe(const AttnArgs& a, uint32_t* dst, hipStream_t stream) {
  if (a.S == 0) return hipSuccess;
  const unsigned grid = (unsigned)a.S * a.Hkv * a.n_split;
  if (a.D == 128)
    hipLaunchKernelGGL((paged_read_probe_kernel<128>), dim3(grid), dim3(kAttnThreads), 0, stream, a, dst);
  else if (a.D == 64)
    hipLaunchKernelGGL((paged_read_probe_kernel<64>), dim3(grid), dim3(kAttnThreads), 0, stream, a, dst);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, int dtype, hipStream_t stream) {
  if (a.S == 0) return hipSuccess;
  if (dtype == 1) {
    if (a.D == 128) return launch_attention_d<__bf16, 128>(a, stream);
    if (a.D == 64) return launch_attention_d<__bf16, 64>(a, stream);
  } else {
    if (a.D == 128) return launch_attention_d<float, 128>(a, stream);
    if (a.D == 64) return launch_attention_d<float, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace kara
