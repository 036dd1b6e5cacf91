// Window scoring with the window's keys resident in registers ("Technical
// Summary: Kara", Methodology 1, Mechanism and Rationale: every window query's
// softmax over all W window keys, with no mask, is accumulated into the
// scores of the keys j < C = W - B).
//
// The score of key j is  s[j] = sum_rows exp(x[row, j]) / Z[row]  with
// Z[row] = sum over all W keys of exp(x[row, k]).  A row's normaliser is known
// only after all of its keys, so a kernel that streams keys past resident
// query rows must either compute every logit twice (once for Z, once for the
// column sums) or keep every exponential until Z is known.  Here the roles are
// swapped: one workgroup holds up to 1024 keys of a unit's window in
// registers, 16 NT keys per wave of eight, and streams the unit's G*W query
// rows past them in tiles of 16 rows.  Per tile each wave computes the
// 16 x 16 NT logits on the matrix cores (v_mfma_f32_16x16x32_bf16, the keys as
// the resident B operand, the query rows as the A operand read from LDS),
// turns them into exponentials in place, and publishes its partial row sums
// in LDS; after one workgroup barrier every wave reads the tile's 16
// normalisers and adds  exp * (1 / Z)  into per-key column accumulators.
//
// Windows of up to 1024 keys take one pass (mode kWhole): every logit's MFMA
// and exp2 are issued once.  Longer windows (up to 2048 keys) take three
// launches over two key blocks, KB0 = [0, 1024) and KB1 = [1024, W):
//   kRowSums      KB1 resident: each row's partial normaliser over KB1;
//   kWithRowSums  KB0 resident: the partial normaliser over KB0 plus the one
//                 from KB1 gives Z; column sums of KB0's region keys; 1 / Z
//                 stored per row;
//   kWeighted     KB1 resident again: column sums of KB1's region keys
//                 [1024, C) with the stored 1 / Z.
// Only KB1's region keys are computed twice: 1024 + 1024 + (C - 1024) logits
// per row (2816 at W = 2048, C = 1792) instead of W + C = 3840 for a kernel
// that recomputes the whole region.
//
// The exponentials take no per-row reference (exp2 of the logit in log2
// units).  That is exact in the same sense as a row-maximum reference as long
// as no sum leaves float's range; a row whose normaliser lies outside
// [2^-40, 2^100] (logits beyond about +-27 / 69 nats) sends the unit to an
// exact route that first takes every row's maximum over all keys, then the
// normalisers with those references, then the column sums (slow, key block by
// key block; never taken on ordinary data).  For one-block windows kWhole
// marks such a unit (a negative first score) and a second, grid-stride launch
// runs the route for the marked units only, so that the route's code does not
// share the main kernel's register budget; for two-block windows the check is
// made by kWithRowSums and the route run by kWeighted.
//
// Registers (two waves per SIMD, at most 256 each): 4 NT x 4 for the keys,
// 2 x 4 NT for two logit tiles (the next tile's MFMAs run while the VALU works
// on the current one), 16 for the query fragments, NT column accumulators.
// LDS: a ring of six 16-row query tiles (4 KB each, moved from global memory
// by direct-to-LDS loads), the per-wave row sums, staged per-row normaliser
// inputs, and (exact route) one reference and one normaliser per row.

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
constexpr int kRQTile = kRRows * 256;          // LDS bytes of a staged query tile
constexpr int kRQSlots = 6;                    // query tiles in the LDS ring
constexpr int kRRowSlots = 8;                  // tiles of staged per-row inputs in LDS
constexpr int kZStride = kRWaves + 1;          // floats per row of the per-wave row sums
constexpr int kExactGrid = 512;                // workgroups of the exact launch (grid-stride)

enum Mode { kWhole = 0, kRowSums = 1, kWithRowSums = 2, kWeighted = 3, kExact = 4 };

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  const int xi = __builtin_bit_cast(int, x);
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(xi, xi, kCtrl, 0xF, 0xF, true));
}

// Sum / maximum over the 16 lanes of a DPP row (rotations by 8, 4, 2, 1).
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

// Row sums of a tile over the 16 lanes (keys) of a DPP row, transposed: the
// lane starts with its partial sums of rows 0..3 of its row group and ends with
// the full sum of row (lane & 15) >> 2.  Lanes i and 15 - i (row_mirror) and
// then i and 7 - i (row_half_mirror) swap the halves they do not keep; the
// last two steps sum within the quad.
__device__ __forceinline__ float row_sums16_transposed(const float (&rp)[4], int kl) {
  const bool hi8 = kl & 8, hi4 = kl & 4;
  const float k0 = hi8 ? rp[2] : rp[0], s0 = hi8 ? rp[0] : rp[2];
  const float k1 = hi8 ? rp[3] : rp[1], s1 = hi8 ? rp[1] : rp[3];
  const float a0 = k0 + dpp<0x140>(s0);   // row_mirror
  const float a1 = k1 + dpp<0x140>(s1);
  const float kk = hi4 ? a1 : a0, ss = hi4 ? a0 : a1;
  float v = kk + dpp<0x141>(ss);          // row_half_mirror
  v += dpp<0xB1>(v);                      // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);                      // quad_perm [2,3,0,1]
  return v;
}

// Sum over the 4 lanes of a quad.
__device__ __forceinline__ float quad_sum(float x) {
  x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]
  return x;
}

// Lane 4r of the lane's DPP row (row_newbcast).
template <int kR>
__device__ __forceinline__ float row_bcast(float x) {
  return dpp<0x150 + 4 * kR>(x);
}

// 16 bytes per lane from global memory (base + off) straight into LDS: lane i
// of the wave writes LDS bytes [lds + 16 i, lds + 16 i + 16).  The load counts
// in vmcnt like any vector load; the caller waits for it before a barrier
// that publishes the data (the compiler does not see the LDS write).
__device__ __forceinline__ void load_to_lds16(const char* base, uint32_t off, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS of one workgroup.
struct ResidentLds {
  __attribute__((aligned(16))) char qbuf[kRQSlots][kRQTile];
  __attribute__((aligned(16))) float zpart[2][kRWaves][kRRows];
  // fast pass: per-wave row sums as [row][wave] with a row stride of 9 floats,
  // so that neither the 16 writers of a wave nor the quads that read two
  // waves' sums of one row meet in an LDS bank
  float zrs[2][kRRows * kZStride];
  __attribute__((aligned(16))) float rowin[kRRowSlots][kRRows];
  float refs[kResidentMaxRows];
  float zfull[kResidentMaxRows];
  int s_redo;
};

// One unit's scores on one workgroup.  MODE kExact runs the exact route only
// (for a unit that the kWhole launch marked).
template <int NT, int MODE>
__device__ __forceinline__ void score_unit(const ScoreArgs& a, const int unit, ResidentLds& sm) {
  constexpr bool kRowSumsHere = MODE != kWeighted;     // this launch computes row normalisers
  constexpr bool kCols = MODE != kRowSums;              // this launch adds column sums
  constexpr bool kStageRow = MODE == kWithRowSums || MODE == kWeighted;   // a per-row input is staged
  constexpr int kBlockKeys = kRWaves * 16 * NT;
  auto& qbuf = sm.qbuf;
  auto& zpart = sm.zpart;
  auto& zrs = sm.zrs;
  auto& rowin = sm.rowin;
  auto& refs = sm.refs;
  auto& zfull = sm.zfull;
  auto& s_redo = sm.s_redo;

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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  float* zrow = a.zrow ? a.zrow + (size_t)unit * rows : nullptr;
  float* out = a.out + (size_t)unit * C;

  // ---- resident keys: B operand fragments ----
  // Key of N-tile nt for this lane: lo + 16 NT wave + 16 nt + kl; the lane
  // holds its 16-byte pieces (lane >> 4) + 4 ks, ks = 0..3, of that key's
  // 256-byte row.  Keys at or past `hi` are zero (logit 0).
  bf16x8 kf[NT][kRKs];
  auto load_keys = [&](int lo, int hi) -> float {
    float n_out = 0.0f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int j = lo + wave * 16 * NT + 16 * nt + kl;
      if (j < hi) {
        const int tok = start + j;
        int bk = trow[tok >> a.bs_shift];
        bk = bk < 0 ? 0 : (bk >= a.NB ? a.NB - 1 : bk);
        const char* p = kbase + (size_t)bk * blk_bytes + (size_t)(tok & bs_mask) * 256 + grp * 16;
#pragma unroll
        for (int ks = 0; ks < kRKs; ++ks) kf[nt][ks] = *(const bf16x8*)(p + ks * 64);
      } else {
        n_out += 1.0f;
#pragma unroll
        for (int ks = 0; ks < kRKs; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) kf[nt][ks][e] = (__bf16)0.0f;
      }
    }
    return n_out;
  };

  // ---- query tiles: global memory -> LDS ring ----
  // A staged tile holds rows 16 t + kr, kr = 0..15, as four 1 KB quarters:
  // quarter ks holds dims 32 ks .. 32 ks + 31 of every row, row kr at byte
  // 64 kr of the quarter, its 16-byte piece p (dims 32 ks + 8 p ..) at
  // position p ^ ((kr >> 2) & 3).  The 16 lanes that read one piece of rows
  // 0..15 then meet in no LDS bank, and the quarter is an immediate offset.
  //
  // The fast pass moves two tiles per pair of steps with one direct-to-LDS load
  // per wave: wave w moves quarter w & 3 of the pair's tile w >> 2, lane L row
  // L >> 2, position L & 3.  The lane's row advances by 32 per pair, i.e. by
  // 32 / G positions and 32 % G heads; the (position, head) pair is kept up to
  // date incrementally.  Rows past the last one read the last row again
  // (finite values; their normaliser weights are zero).  Offsets within the
  // unit's window fit 32 bits (W * Hq * 256 bytes).
  const uint32_t qlds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)&qbuf[0][0];
  const int dm_row = 16 * (wave >> 2) + (lane >> 2);
  const uint32_t dm_piece = (uint32_t)(4 * (wave & 3) + ((lane & 3) ^ ((lane >> 4) & 3))) * 16u;
  const int di = 32 / G, dg = 32 - (32 / G) * G;
  int ld_i = dm_row / G, ld_g = dm_row - (dm_row / G) * G, ld_row = dm_row;
  // Starts the wave's load of the pair of tiles tp, tp + 1 (tp even, the next
  // pair in sequence).
  auto load_pair = [&](int tp) {
    const bool ok = ld_row < rows;
    const int i = ok ? ld_i : W - 1, g = ok ? ld_g : G - 1;
    const int slot_i = i + ring_off < W ? i + ring_off : i + ring_off - W;
    const uint32_t off = (uint32_t)(slot_i * a.Hq + g) * 256u + dm_piece;
    const int slot = (tp + (wave >> 2)) % kRQSlots;
    load_to_lds16(qbase, off, qlds + (uint32_t)(slot * kRQTile + (wave & 3) * 1024));
    ld_row += 32;
    ld_i += di;
    ld_g += dg;
    if (ld_g >= G) {
      ld_g -= G;
      ld_i += 1;
    }
  };
  // Exact route: thread tid moves 8 bytes of a tile, row tid >> 5, bytes
  // (tid & 31) * 8 of the row, through registers.
  const int st_row = tid >> 5;
  const int st_off = (tid & 31) * 8;
  // the thread's piece of tile t (random access, for the exact route)
  auto load_q_at = [&](int t) -> uint2 {
    const int row = t * kRRows + st_row;
    if (row >= rows) return make_uint2(0u, 0u);
    const int i = row / G, g = row - (row / G) * G;
    const int slot_i = i + ring_off < W ? i + ring_off : i + ring_off - W;
    return *(const uint2*)(qbase + ((size_t)slot_i * a.Hq + g) * 256 + st_off);
  };
  auto store_q = [&](uint2 v, int t) {
    const int p = st_off >> 4;
    const int pos = ((p & 3) ^ ((st_row >> 2) & 3)) * 16 + (st_off & 8);
    *(uint2*)&qbuf[t % kRQSlots][(p >> 2) * 1024 + st_row * 64 + pos] = v;
  };
  const int qlane = kl * 64 + ((grp ^ ((kl >> 2) & 3)) << 4);
  auto qfrag = [&](int t, int ks) -> bf16x8 { return *(const bf16x8*)&qbuf[t % kRQSlots][ks * 1024 + qlane]; };
  // Per-row input of tile t (kWithRowSums: the partial normaliser over KB1;
  // kWeighted: 1 / Z), staged through registers into LDS and stored by threads
  // 0..15 (0 for rows past the last one).  The load is unconditional, so that
  // the compiler can wait for it by count (every wave reads row
  // t * 16 + (tid & 15), clamped to the last row).
  auto load_row = [&](int t) -> float {
    if (!kStageRow) return 0.0f;
    const int row = t * kRRows + (tid & (kRRows - 1));
    return zrow[row < rows ? row : rows - 1];
  };
  auto store_row = [&](float v, int t) {
    if (kStageRow && tid < kRRows) rowin[t % kRRowSlots][tid] = t * kRRows + tid < rows ? v : 0.0f;
  };
  // 16 x (16 NT) logits of tile t: row 4 grp + r, key (block key) 16 NT wave + 16 nt + kl
  auto tile_mfma = [&](f32x4 (&acc)[NT], int t) {
    bf16x8 qa[kRKs];
#pragma unroll
    for (int ks = 0; ks < kRKs; ++ks) qa[ks] = qfrag(t, ks);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
      acc[nt] = z;
    }
#pragma unroll
    for (int ks = 0; ks < kRKs; ++ks)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma(qa[ks], kf[nt][ks], acc[nt]);
  };
  // Column sums of the lane's keys over its row group, summed over the four
  // groups and written for keys lo + ... below min(hi, C).
  auto write_cols = [&](const float (&colacc)[NT], int lo, int hi) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float s = colacc[nt];
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      const int j = lo + wave * 16 * NT + 16 * nt + kl;
      if (lane < 16 && j < hi && j < C) out[j] = s;
    }
  };

  // ============ exact route: every row's maximum as its reference ============
  // Key blocks of kBlockKeys keys cover the window; three sweeps: row maxima,
  // normalisers, column sums of the region's keys.
  auto exact_unit = [&]() {
    for (int i = tid; i < rows; i += kRThreads) {
      refs[i] = -INFINITY;
      zfull[i] = 0.0f;
    }
    for (int sweep = 0; sweep < 3; ++sweep) {
      for (int lo = 0; lo < (sweep == 2 ? C : W); lo += kBlockKeys) {
        const int hi = min(lo + kBlockKeys, W);
        load_keys(lo, hi);
        float colacc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) colacc[nt] = 0.0f;
        for (int t = 0; t < n_tiles; ++t) {
          __syncthreads();
          store_q(load_q_at(t), t);
          __syncthreads();
          f32x4 acc[NT];
          tile_mfma(acc, t);
          float ref[4], rp[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = t * kRRows + 4 * grp + r;
            ref[r] = row < rows ? refs[row] : 0.0f;
          }
          if (sweep == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float mx = -INFINITY;
#pragma unroll
              for (int nt = 0; nt < NT; ++nt)
                if (lo + wave * 16 * NT + 16 * nt + kl < hi) mx = fmaxf(mx, acc[nt][r] * c);
              rp[r] = row_max16(mx);
            }
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) rp[r] = 0.0f;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const bool valid = lo + wave * 16 * NT + 16 * nt + kl < hi;
                const float e = valid ? __builtin_amdgcn_exp2f(acc[nt][r] * c - ref[r]) : 0.0f;
                acc[nt][r] = e;
                rp[r] += e;
              }
#pragma unroll
            for (int r = 0; r < 4; ++r) rp[r] = row_sum16(rp[r]);
          }
          if (sweep < 2) {
            if (kl == 0) *(float4*)&zpart[0][wave][4 * grp] = make_float4(rp[0], rp[1], rp[2], rp[3]);
            __syncthreads();
            if (tid < kRRows && t * kRRows + tid < rows) {
              const int row = t * kRRows + tid;
              float v = zpart[0][0][tid];
              for (int w = 1; w < kRWaves; ++w)
                v = sweep == 0 ? fmaxf(v, zpart[0][w][tid]) : v + zpart[0][w][tid];
              if (sweep == 0) refs[row] = fmaxf(refs[row], v);
              else zfull[row] += v;
            }
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = t * kRRows + 4 * grp + r;
              const float w = row < rows ? 1.0f / zfull[row] : 0.0f;
#pragma unroll
              for (int nt = 0; nt < NT; ++nt) colacc[nt] = fmaf(acc[nt][r], w, colacc[nt]);
            }
          }
        }
        if (sweep == 2) write_cols(colacc, lo, hi);
      }
    }
  };

  if (MODE == kExact) {
    exact_unit();
    return;
  }
  if (tid == 0) s_redo = 0;

  // kWeighted: a unit whose normalisers left float's comfortable range in
  // kWithRowSums is scored by the exact route instead (uniform branch).
  if (MODE == kWeighted && a.uflags[unit] != 0) {
    exact_unit();
    return;
  }

  // ======================= fast pass: references 0 =========================
  const int key_lo = a.key_lo, key_hi = a.key_hi;
  // the first two pairs of query tiles travel while the keys load
  load_pair(0);
  if (n_tiles > 2) load_pair(2);
  const float n_inval = load_keys(key_lo, key_hi);
  // keys past the block among the 16 lanes of the row group (logit 0, exp2 = 1)
  const float inval16 = row_sum16(n_inval);
  float colacc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) colacc[nt] = 0.0f;
  bool bad = false;
  {
    store_row(load_row(0), 0);
    store_row(load_row(1), 1);
    float sr0 = load_row(2), sr1 = load_row(3);
    wait_vm_all();
    __syncthreads();
    f32x4 acc0[NT], acc1[NT];
    tile_mfma(acc0, 0);
    // One tile: `cur` holds its logits, the next tile's go into `nxt`.  The
    // first step of each pair (t even) waits for this wave's loads of tiles
    // t + 2 and t + 3 (started two steps earlier; the step's barrier then
    // publishes them), stores those tiles' row inputs, and starts the loads of
    // tiles t + 4 and t + 5, so that the loads in flight when a pair starts
    // are a whole pair old.  Tiles t + 4 and t + 5 go to the slots of tiles
    // t - 2 and t - 1, whose fragments every wave read before the previous
    // step's barrier; the row inputs keep eight slots because a tile's are
    // read after its barrier.
    auto step = [&](f32x4 (&cur)[NT], f32x4 (&nxt)[NT], int t, bool stage) {
      if (stage) {
        wait_vm_all();
        store_row(sr0, t + 2);
        store_row(sr1, t + 3);
        sr0 = load_row(t + 4);
        sr1 = load_row(t + 5);
        if (t + 4 < n_tiles) load_pair(t + 4);
      }
      // The next tile's logits (past the last tile: zero rows, never used) on
      // the matrix cores while this tile's VALU work runs, in regions fenced
      // against reordering: one region per logit of the lane (its multiply,
      // exp2 and add) carries one of the first 3 NT MFMAs (reduction steps
      // 0-2; consecutive ones update different N-tiles); the last step's
      // MFMAs are issued while the normalisers' LDS reads are in flight.  A
      // wave thus issues VALU work while its own MFMAs execute.
      // query fragments of the next tile: steps 0-2 now, step 3 after the barrier
      bf16x8 qa[kRKs - 1];
#pragma unroll
      for (int ks = 0; ks < kRKs - 1; ++ks) qa[ks] = qfrag(t + 1, ks);
      float rp[4];
#pragma unroll
      for (int k = 0; k < 4 * NT; ++k) {
        if (k < 3 * NT) {
          const int ks = k / NT, nt = k % NT;
          if (ks == 0) {
            const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
            nxt[nt] = mfma(qa[0], kf[nt][0], z);
          } else {
            nxt[nt] = mfma(qa[ks], kf[nt][ks], nxt[nt]);
          }
        }
        {
          const int nt = k / 4, r = k % 4;
          const float x = __builtin_amdgcn_exp2f(cur[nt][r] * c);
          cur[nt][r] = x;
          if (kRowSumsHere) rp[r] = nt == 0 ? x : rp[r] + x;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      float* zp = &zrs[t & 1][0];
      if (kRowSumsHere) {
        // this wave's sum of row 4 grp + (kl >> 2), published by one lane of each quad
        const float zw = row_sums16_transposed(rp, kl) - inval16;
        if ((kl & 3) == 0) zp[(4 * grp + (kl >> 2)) * kZStride + wave] = zw;
      }
      __syncthreads();
      // The tile's normalisers from LDS: lane (grp, 4 m + q) adds waves 2q,
      // 2q + 1 of row 4 grp + m.  Half of the last reduction step's MFMAs are
      // issued while those reads are in flight, the other half between the
      // column sums' FMAs.
      const int m = 4 * grp + ((lane >> 2) & 3);
      const int q2 = 2 * (lane & 3);
      const bf16x8 q3 = qfrag(t + 1, kRKs - 1);
      float za = 0.0f, zb = 0.0f, zx = 0.0f;
      float4 wrow = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (kRowSumsHere) {
        za = zp[m * kZStride + q2];
        zb = zp[m * kZStride + q2 + 1];
        if (MODE == kWithRowSums) zx = rowin[t % kRRowSlots][m];
      } else {
        wrow = *(const float4*)&rowin[t % kRRowSlots][4 * grp];
      }
#pragma unroll
      for (int nt = 0; nt < NT / 2; ++nt) nxt[nt] = mfma(q3, kf[nt][3], nxt[nt]);
      __builtin_amdgcn_sched_barrier(0);
      float w0 = wrow.x, w1 = wrow.y, w2 = wrow.z, w3 = wrow.w;
      if (kRowSumsHere) {
        const float z = MODE == kWithRowSums ? quad_sum(za + zb) + zx : quad_sum(za + zb);
        const bool row_ok = t * kRRows + m < rows;
        if (MODE != kRowSums) bad |= __ballot(row_ok && !(z >= 0x1p-40f && z <= 0x1p100f)) != 0;
        if (MODE == kRowSums) {
          if (wave == 0 && (lane & 3) == 0 && row_ok) zrow[t * kRRows + m] = z;
        } else {
          const float wm = row_ok ? __builtin_amdgcn_rcpf(z) : 0.0f;
          if (MODE == kWithRowSums && wave == 0 && (lane & 3) == 0 && row_ok) zrow[t * kRRows + m] = wm;
          w0 = row_bcast<0>(wm);
          w1 = row_bcast<1>(wm);
          w2 = row_bcast<2>(wm);
          w3 = row_bcast<3>(wm);
        }
      }
      // column sums (every wave adds them, so that all waves reach the next
      // barrier together; only region keys are written)
      auto cols = [&](int nt) {
        float s = colacc[nt];
        s = fmaf(cur[nt][0], w0, s);
        s = fmaf(cur[nt][1], w1, s);
        s = fmaf(cur[nt][2], w2, s);
        s = fmaf(cur[nt][3], w3, s);
        colacc[nt] = s;
      };
#pragma unroll
      for (int nt = 0; nt < NT / 2; ++nt) {
        nxt[NT / 2 + nt] = mfma(q3, kf[NT / 2 + nt][3], nxt[NT / 2 + nt]);
        if (kCols) cols(nt);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kCols) {
#pragma unroll
        for (int nt = NT / 2; nt < NT; ++nt) cols(nt);
      }
    };
    for (int t = 0; t < n_tiles; t += 2) {
      step(acc0, acc1, t, true);
      if (t + 1 < n_tiles) step(acc1, acc0, t + 1, false);
    }
    // every tile load was waited for by a later pair; none may still be
    // writing this workgroup's LDS when it ends
    wait_vm_all();
  }

  if (MODE == kRowSums) return;
  if (bad && lane == 0) s_redo = 1;
  __syncthreads();
  if (MODE == kWithRowSums) {
    // the next launch reruns units whose normalisers left the range exactly
    if (tid == 0) a.uflags[unit] = s_redo;
    write_cols(colacc, key_lo, key_hi);
    return;
  }
  if (MODE == kWhole && s_redo) {       // uniform over the workgroup
    // marked for the exact launch: scores are never negative, and that
    // launch overwrites every score of the unit
    if (tid == 0) out[0] = -1.0f;
    return;
  }
  write_cols(colacc, key_lo, key_hi);
}

template <int NT, int MODE>
__global__ __launch_bounds__(kRThreads, 2) void score_resident_kernel(ScoreArgs a) {
  __shared__ ResidentLds sm;
  if ((int)blockIdx.x >= a.n_units) return;
  score_unit<NT, MODE>(a, blockIdx.x, sm);
}

// The exact route for the units of a one-launch window that the kWhole launch
// marked (first score negative).  A grid-stride pass: each workgroup checks
// the marks of units blockIdx.x + gridDim.x * (tid + kRThreads * r) and
// scores the marked ones one after another.  Kept apart from kWhole so that
// the route's code does not share that kernel's register budget.
template <int NT>
__global__ __launch_bounds__(kRThreads, 2) void exact_resident_kernel(ScoreArgs a) {
  __shared__ ResidentLds sm;
  __shared__ int s_list[kRThreads];
  __shared__ int s_n;
  const int stride = (int)gridDim.x * kRThreads;
  for (int u0 = blockIdx.x; u0 < a.n_units; u0 += stride) {
    const long u = (long)u0 + (long)threadIdx.x * gridDim.x;
    const bool marked = u < a.n_units && a.out[u * a.C] < 0.0f;
    if (threadIdx.x == 0) s_n = 0;
    __syncthreads();
    if (marked) s_list[atomicAdd(&s_n, 1)] = (int)u;
    __syncthreads();
    const int n = s_n;
    for (int i = 0; i < n; ++i) {
      score_unit<NT, kExact>(a, s_list[i], sm);
      __syncthreads();
    }
  }
}

template <int NT, int MODE>
hipError_t launch_one(const ScoreArgs& a, int lo, int hi, hipStream_t stream) {
  ScoreArgs b = a;
  b.key_lo = lo;
  b.key_hi = hi;
  hipLaunchKernelGGL((score_resident_kernel<NT, MODE>), dim3((unsigned)a.n_units), dim3(kRThreads), 0, stream, b);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(const ScoreArgs& a, int lo, int hi, hipStream_t stream) {
  switch (resident_tiles(hi - lo)) {
    case 2: return launch_one<2, MODE>(a, lo, hi, stream);
    case 4: return launch_one<4, MODE>(a, lo, hi, stream);
    case 6: return launch_one<6, MODE>(a, lo, hi, stream);
    default: return launch_one<8, MODE>(a, lo, hi, stream);
  }
}

}  // namespace

int resident_tiles(int n_keys) {
  const int per_wave = (n_keys + kRWaves - 1) / kRWaves;
  const int nt = (per_wave + 15) / 16;
  return nt <= 2 ? 2 : (nt <= 4 ? 4 : (nt <= 6 ? 6 : 8));
}

hipError_t launch_score_resident(const ScoreArgs& a, hipStream_t stream) {
  if (a.n_units == 0) return hipSuccess;
  if (a.W <= kResidentBlock) {
    hipError_t e = launch_mode<kWhole>(a, 0, a.W, stream);
    if (e != hipSuccess) return e;
    ScoreArgs b = a;
    b.key_lo = 0;
    b.key_hi = a.W;
    const unsigned grid = (unsigned)(a.n_units < kExactGrid ? a.n_units : kExactGrid);
    hipLaunchKernelGGL((exact_resident_kernel<8>), dim3(grid), dim3(kRThreads), 0, stream, b);
    return hipGetLastError();
  }
  if (!a.zrow || !a.uflags) return hipErrorInvalidValue;
  hipError_t e;
  if ((e = launch_mode<kRowSums>(a, kResidentBlock, a.W, stream)) != hipSuccess) return e;
  if ((e = launch_mode<kWithRowSums>(a, 0, kResidentBlock, stream)) != hipSuccess) return e;
  // KB1's region keys (none if C <= 1024: the launch then only runs the exact route where flagged)
  const int hi = a.C > kResidentBlock ? a.C : kResidentBlock + 1;
  return launch_mode<kWeighted>(a, kResidentBlock, hi, stream);
}

}  // namespace kara
