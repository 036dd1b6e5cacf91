// Window scoring in one pass over the logits, with the window's keys held in
// registers ("Technical Summary: Kara", Methodology 1, Mechanism and
// Rationale: every window query's softmax over all W window keys, with no
// mask, is accumulated into the scores of the keys j < C = W - B).
//
// The score of key j is  s[j] = sum_rows exp(x[row, j]) / Z[row]  with
// Z[row] = sum over all W keys of exp(x[row, k]).  A row's normaliser is known
// only after all of its keys, so a kernel that streams keys past resident
// query rows must either compute every logit twice (once for Z, once for the
// column sums) or keep every exponential until Z is known.  Here the roles are
// swapped: one workgroup holds all (up to 1024) keys of a unit's window in
// registers, 128 keys per wave of eight, and streams the unit's G*W query rows
// past them in tiles of 16 rows.  Per tile each wave computes the 16 x 128
// logits on the matrix cores (v_mfma_f32_16x16x32_bf16, the keys as the
// resident B operand, the query rows as the A operand read from LDS), turns
// them into exponentials in place, and adds its partial row sums into LDS;
// after one workgroup barrier every wave reads the tile's 16 normalisers and
// adds  exp * (1 / Z)  into per-key column accumulators.  Each logit costs one
// multiply, one exp2, one add and (for keys of the compressible region) one
// multiply-add, and its MFMA is issued once.
//
// The exponentials take no per-row reference (exp2 of the logit in log2
// units).  That is exact in the same sense as a row-maximum reference as long
// as no sum leaves float's range; a row whose normaliser lies outside
// [2^-40, 2^100] (logits beyond about +-27 / 69 nats) sends the workgroup to an
// exact rerun of the unit that first takes every row's maximum and then uses
// it as the reference (slow, never taken on ordinary data).
//
// Registers (two waves per SIMD, at most 256 each): 128 for the keys, 64 for
// two logit tiles (the next tile's MFMAs run while the VALU works on the
// current one), 16 for the query fragments, 8 column accumulators.  LDS: a
// ring of four 16-row query tiles (rows padded to 272 bytes), the per-wave row
// sums, and (exact rerun only) one reference per row.

#include "kara_internal.hpp"

#include <cmath>

namespace kara {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRWaves = 8;
constexpr int kRThreads = kRWaves * 64;
constexpr int kRRows = 16;                     // query rows per tile
constexpr int kRKs = 4;                        // 32-wide reduction steps over D = 128
constexpr int kRQStride = 272;                 // LDS bytes per staged query row (256 + pad)
constexpr int kRQSlots = 4;                    // query tiles in the LDS ring
constexpr int kRMaxRefRows = kResidentMaxRows; // rows with an LDS reference in the exact rerun

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF,
                                                               false));
}

// Sum over the 16 lanes of a DPP row (rotations by 8, 4, 2, 1 reach every lane).
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0x128>(x);   // row_ror:8
  x += dpp<0x124>(x);   // row_ror:4
  x += dpp<0x122>(x);   // row_ror:2
  x += dpp<0x121>(x);   // row_ror:1
  return x;
}

__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<0x128>(x));
  x = fmaxf(x, dpp<0x124>(x));
  x = fmaxf(x, dpp<0x122>(x));
  x = fmaxf(x, dpp<0x121>(x));
  return x;
}

// Sum over the 4 lanes of a quad.
__device__ __forceinline__ float quad_sum(float x) {
  x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]
  return x;
}

__device__ __forceinline__ float quad_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  return x;
}

// Lane 4r of the lane's DPP row (row_newbcast).
template <int kR>
__device__ __forceinline__ float row_bcast(float x) {
  return dpp<0x150 + 4 * kR>(x);
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int NT>
__global__ __launch_bounds__(kRThreads, 2) void score_resident_kernel(ScoreArgs a) {
  __shared__ __attribute__((aligned(16))) char qbuf[kRQSlots][kRRows * kRQStride];
  __shared__ __attribute__((aligned(16))) float zpart[2][kRWaves][kRRows];
  __shared__ float refs[kRMaxRefRows];
  __shared__ int s_redo;

  const int unit = blockIdx.x;
  if (unit >= a.n_units) return;
  const int h = unit % a.Hkv;
  const int bl = unit / a.Hkv;
  const int l = bl % a.Lyr;
  const int b = bl / a.Lyr;
  const int W = a.W, C = a.C, G = a.G;
  const int rows = G * W;
  const int n_tiles = (rows + kRRows - 1) / kRRows;
  const float c = a.c;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = lane >> 4;            // row group of the MFMA output: rows 4*grp .. 4*grp+3
  const int kl = lane & 15;             // key (output column) of the lane within an N-tile

  // Device lengths and tables are trusted only up to clamping.
  int L = a.lens[b];
  const int max_tok = a.MB * a.bs;
  L = L < W ? W : (L > max_tok ? max_tok : L);
  const int start = L - W;
  const int32_t* trow = a.table + (size_t)b * a.MB;
  size_t q_row0 = (size_t)bl * W;
  int ring_off = 0;
  if (a.q_slots) {
    int slot = a.q_slots[b];
    slot = slot < 0 ? 0 : (slot >= a.q_n_slots ? a.q_n_slots - 1 : slot);
    const int n = a.q_counts[b];
    q_row0 = ((size_t)slot * a.Lyr + l) * W;
    ring_off = (n < 0 ? 0 : n) % W;
  }
  const char* qbase = (const char*)a.q + (q_row0 * a.Hq + (size_t)h * G) * 256;
  const char* kbase = (const char*)a.pool + ((size_t)l * 2 * a.NB * a.Hkv * a.bs + (size_t)h * a.bs) * 256;
  const size_t blk_bytes = (size_t)a.Hkv * a.bs * 256;
  const int bs_mask = (1 << a.bs_shift) - 1;

  // ---- the wave's keys: B operand fragments, resident for the whole unit ----
  // Key of N-tile nt for this lane: k0 + 16 nt + kl; the lane holds its
  // 16-byte pieces (lane >> 4) + 4 ks, ks = 0..3, of that key's 256-byte row.
  const int k0 = wave * 16 * NT;
  bf16x8 kf[NT][kRKs];
  float n_inval = 0.0f;                 // this lane's keys past the window (their logits are 0)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int j = k0 + 16 * nt + kl;
    if (j < W) {
      const int tok = start + j;
      int bk = trow[tok >> a.bs_shift];
      bk = bk < 0 ? 0 : (bk >= a.NB ? a.NB - 1 : bk);
      const char* p = kbase + (size_t)bk * blk_bytes + (size_t)(tok & bs_mask) * 256 + grp * 16;
#pragma unroll
      for (int ks = 0; ks < kRKs; ++ks) kf[nt][ks] = *(const bf16x8*)(p + ks * 64);
    } else {
      n_inval += 1.0f;
#pragma unroll
      for (int ks = 0; ks < kRKs; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) kf[nt][ks][e] = (__bf16)0.0f;
    }
  }
  const bool col_wave = k0 < C;         // the wave holds keys of the compressible region

  // ---- query tiles: global -> registers -> LDS ring ----
  // Thread tid moves 8 bytes of a tile: row tid >> 5, bytes (tid & 31) * 8.
  const int st_row = tid >> 5;
  const int st_off = (tid & 31) * 8;
  auto q_addr = [&](int row) -> const char* {
    const int i = row / G, g = row - (row / G) * G;
    const int slot_i = i + ring_off < W ? i + ring_off : i + ring_off - W;
    return qbase + ((size_t)slot_i * a.Hq + g) * 256;
  };
  auto load_q = [&](int t) -> uint2 {
    const int row = t * kRRows + st_row;
    if (t < n_tiles && row < rows) return *(const uint2*)(q_addr(row) + st_off);
    return make_uint2(0u, 0u);
  };
  auto store_q = [&](uint2 v, int t) { *(uint2*)&qbuf[t % kRQSlots][st_row * kRQStride + st_off] = v; };
  auto qfrag = [&](int t, int ks) -> bf16x8 {
    return *(const bf16x8*)&qbuf[t % kRQSlots][kl * kRQStride + ks * 64 + grp * 16];
  };
  // 16 x (16 NT) logits of tile t: row 4 grp + r, key k0 + 16 nt + kl in acc[nt][r]
  auto tile_mfma = [&](f32x4 (&acc)[NT], int t) {
    bf16x8 qa[kRKs];
#pragma unroll
    for (int ks = 0; ks < kRKs; ++ks) qa[ks] = qfrag(t, ks);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
      acc[nt] = z;
    }
#pragma unroll
    for (int ks = 0; ks < kRKs; ++ks)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma(qa[ks], kf[nt][ks], acc[nt]);
  };

  if (tid == 0) s_redo = 0;
  float colacc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) colacc[nt] = 0.0f;

  // ======================= fast pass: references 0 =========================
  {
    store_q(load_q(0), 0);
    store_q(load_q(1), 1);
    uint2 stg0 = load_q(2), stg1 = load_q(3);
    __syncthreads();
    f32x4 acc0[NT], acc1[NT];
    tile_mfma(acc0, 0);
    bool bad = false;
    // One tile: `cur` holds its logits, the next tile's go into `nxt`; `stg`
    // carries tile t + 2 to its LDS slot and then fetches tile t + 4.
    auto step = [&](f32x4 (&cur)[NT], f32x4 (&nxt)[NT], uint2& stg, int t) {
      store_q(stg, t + 2);
      stg = load_q(t + 4);
      // The next tile's logits (past the last tile: zero rows, never used) on
      // the matrix cores while this tile's exponentials run: eight regions
      // fenced against reordering, each issuing NT / 2 independent MFMAs (the
      // same reduction step of different N-tiles) and NT / 2 of the lane's
      // 4 NT exponentials, so the wave issues VALU work while its own MFMAs
      // execute.
      bf16x8 qa[kRKs];
#pragma unroll
      for (int ks = 0; ks < kRKs; ++ks) qa[ks] = qfrag(t + 1, ks);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
        nxt[nt] = z;
      }
      float rp[4] = {-n_inval, -n_inval, -n_inval, -n_inval};
      constexpr int kPer = NT / 2;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const int mi = i * kPer + j, ks = mi / NT, nt = mi % NT;
          nxt[nt] = mfma(qa[ks], kf[nt][ks], nxt[nt]);
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const int e = i * kPer + j, nt = e / 4, r = e % 4;
          const float x = __builtin_amdgcn_exp2f(cur[nt][r] * c);
          cur[nt][r] = x;
          rp[r] += x;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) rp[r] = row_sum16(rp[r]);
      float* zp = &zpart[t & 1][0][0];
      if (kl == 0) *(float4*)&zp[wave * kRRows + 4 * grp] = make_float4(rp[0], rp[1], rp[2], rp[3]);
      __syncthreads();
      // the tile's normalisers: lane (grp, 4 m + q) adds waves 2q, 2q + 1 of row 4 grp + m
      const int m = 4 * grp + ((lane >> 2) & 3);
      const int q2 = 2 * (lane & 3);
      const float z = quad_sum(zp[q2 * kRRows + m] + zp[(q2 + 1) * kRRows + m]);
      const bool row_ok = t * kRRows + m < rows;
      bad = bad || (row_ok && !(z >= 0x1p-40f && z <= 0x1p100f));
      const float wm = row_ok ? __builtin_amdgcn_rcpf(z) : 0.0f;
      if (col_wave) {
        const float w0 = row_bcast<0>(wm), w1 = row_bcast<1>(wm), w2 = row_bcast<2>(wm),
                    w3 = row_bcast<3>(wm);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          float s = colacc[nt];
          s = fmaf(cur[nt][0], w0, s);
          s = fmaf(cur[nt][1], w1, s);
          s = fmaf(cur[nt][2], w2, s);
          s = fmaf(cur[nt][3], w3, s);
          colacc[nt] = s;
        }
      }
    };
    for (int t = 0; t < n_tiles; t += 2) {
      step(acc0, acc1, stg0, t);
      if (t + 1 < n_tiles) step(acc1, acc0, stg1, t + 1);
    }
    if (__ballot(bad) && lane == 0) s_redo = 1;
    __syncthreads();
  }

  // ============ exact rerun: every row's maximum as its reference ============
  if (s_redo) {                         // uniform over the workgroup
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) colacc[nt] = 0.0f;
    const bool keep_refs = rows <= kRMaxRefRows;
    for (int pass = 0; pass < 2; ++pass) {
      for (int t = 0; t < n_tiles; ++t) {
        __syncthreads();
        store_q(load_q(t), t);
        __syncthreads();
        f32x4 acc[NT];
        tile_mfma(acc, t);
        float rp[4];
        if (pass == 0) {
          // the row maxima over this wave's keys, then over the workgroup
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float mx = -INFINITY;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              if (k0 + 16 * nt + kl < W) mx = fmaxf(mx, acc[nt][r] * c);
            rp[r] = row_max16(mx);
          }
          if (kl == 0) *(float4*)&zpart[0][wave][4 * grp] = make_float4(rp[0], rp[1], rp[2], rp[3]);
          __syncthreads();
          if (tid < kRRows) {
            float mx = zpart[0][0][tid];
            for (int w = 1; w < kRWaves; ++w) mx = fmaxf(mx, zpart[0][w][tid]);
            if (keep_refs) refs[t * kRRows + tid] = mx;
          }
          continue;
        }
        float ref[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = t * kRRows + 4 * grp + r;
          ref[r] = (keep_refs && row < rows) ? refs[row] : 0.0f;
          rp[r] = 0.0f;
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool valid = k0 + 16 * nt + kl < W;
            const float e = valid ? __builtin_amdgcn_exp2f(acc[nt][r] * c - ref[r]) : 0.0f;
            acc[nt][r] = e;
            rp[r] += e;
          }
#pragma unroll
        for (int r = 0; r < 4; ++r) rp[r] = row_sum16(rp[r]);
        if (kl == 0) *(float4*)&zpart[0][wave][4 * grp] = make_float4(rp[0], rp[1], rp[2], rp[3]);
        __syncthreads();
        const int m = 4 * grp + ((lane >> 2) & 3);
        const int q2 = 2 * (lane & 3);
        const float z = quad_sum(zpart[0][q2][m] + zpart[0][q2 + 1][m]);
        const float wm = (t * kRRows + m < rows) ? 1.0f / z : 0.0f;
        const float w0 = row_bcast<0>(wm), w1 = row_bcast<1>(wm), w2 = row_bcast<2>(wm),
                    w3 = row_bcast<3>(wm);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          colacc[nt] += acc[nt][0] * w0 + acc[nt][1] * w1 + acc[nt][2] * w2 + acc[nt][3] * w3;
      }
    }
  }

  // ---- column sums: the four row groups of each key, written for keys < C ----
  float* out = a.out + (size_t)unit * C;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float s = colacc[nt];
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    const int j = k0 + 16 * nt + kl;
    if (lane < 16 && j < C) out[j] = s;
  }
}

template <int NT>
hipError_t launch_nt(const ScoreArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((score_resident_kernel<NT>), dim3((unsigned)a.n_units), dim3(kRThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int resident_tiles(int W) {
  const int per_wave = (W + kRWaves - 1) / kRWaves;
  const int nt = (per_wave + 15) / 16;
  return nt <= 2 ? 2 : (nt <= 4 ? 4 : (nt <= 6 ? 6 : 8));
}

hipError_t launch_score_resident(const ScoreArgs& a, hipStream_t stream) {
  if (a.n_units == 0) return hipSuccess;
  switch (resident_tiles(a.W)) {
    case 2: return launch_nt<2>(a, stream);
    case 4: return launch_nt<4>(a, stream);
    case 6: return launch_nt<6>(a, stream);
    default: return launch_nt<8>(a, stream);
  }
}

}  // namespace kara
