// Tile machinery shared by every contraction of the streaming LM-head loss.
//
// One shape of contraction serves the whole path: C[m][n] = sum_k A[m][k] B[n][k]
// with both operands K-contiguous ("NT").  The forward and the recompute take
// A = W (vocabulary rows) and B = hidden rows; the backward contractions take
// the staged logit gradient and transposed copies of W and of the hidden chunk,
// so they are NT as well.
//
// gfx950 mapping:
//  * 256 threads = 4 wave64s in a 2 x 2 grid; a wave owns a (BM/2) x (BN/2)
//    sub-tile made of 16 x 16 MFMA fragments (v_mfma_f32_16x16x32_bf16 for
//    bf16, v_mfma_f32_16x16x4_f32 for fp32), fp32 accumulators.  The 16x16
//    shape moves half the accumulator traffic per flop of the 32x32 one,
//    which measures faster on this power-limited part.
//  * K advances in slabs of 128 bytes per row (64 bf16 / 32 fp32).  A slab of
//    A and B sits in LDS as rows of eight 16-byte chunks, chunk c of row r
//    stored at position c ^ (r & 7): eight consecutive rows read at the same
//    logical chunk hit eight different bank groups (conflict-free ds_read_b128).
//  * Two LDS stages filled by direct-to-LDS loads: the next slab streams in
//    while the MFMAs consume the current stage (one barrier per slab).
//  * Workgroups are dealt round-robin to the 8 XCDs; `tile_of` renumbers them
//    so each XCD walks a compact block of tiles and its private L2 sees the
//    same A and B slabs from several tiles at once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specloss {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

typedef uint16_t bf16_bits;  // storage type of bf16 tensors

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T>
struct ElemTraits;
template <>
struct ElemTraits<bf16_bits> {
  static constexpr int kPerChunk = 8;
};
template <>
struct ElemTraits<float> {
  static constexpr int kPerChunk = 4;
};

constexpr int kFrag = 16;   // MFMA output fragment: 16 x 16
constexpr int kSteps = 2;   // k-steps per slab (4 chunks of 16 bytes per step)

template <typename T, int BM_, int BN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int KC = ElemTraits<T>::kPerChunk;  // elements per 16-byte chunk
  static constexpr int BK = 8 * KC;                    // elements per slab row (128 bytes)
  static constexpr int WM = BM / 2, WN = BN / 2;       // wave sub-tile
  static constexpr int FM = WM / kFrag, FN = WN / kFrag;  // 16x16 fragments per wave
  static constexpr int STAGE = (BM + BN) * kRowBytes;  // bytes of one LDS stage
  static constexpr int LDS_BYTES = 2 * STAGE;
};

// Rows of a K-contiguous operand.  Tile row r reads source row
// map ? map[r] : r (relative to `base`), clamped into [0, n_rows): rows past
// the end or unmapped rows still load valid memory and their results are
// discarded by the epilogues.
template <typename T>
struct Operand {
  const T* base;
  int64_t ld;            // elements between rows
  int32_t n_rows;        // valid source rows
  const int32_t* map;    // optional gather map indexed by tile row (already offset)
  int32_t map_len;       // entries readable in map
};

__device__ __forceinline__ int32_t clamp_row(int32_t r, int32_t n) {
  return r < 0 ? 0 : (r >= n ? n - 1 : r);
}

template <typename T>
__device__ __forceinline__ const T* row_ptr(const Operand<T>& op, int32_t r) {
  int32_t src = r;
  if (op.map != nullptr) src = op.map[r < op.map_len ? r : op.map_len - 1];
  src = clamp_row(src, op.n_rows);
  return op.base + (int64_t)src * op.ld;
}

// Accumulator fragment element -> tile coordinates (16x16 MFMA output layout):
// register r of lane l holds row 4*(l/16) + r and column l%16, so the four
// lanes l%16 == c share column c and each holds four consecutive rows.
__device__ __forceinline__ int frag_row(int r, int lane) { return ((lane >> 4) << 2) + r; }
__device__ __forceinline__ int frag_col(int lane) { return lane & 15; }

template <typename T>
__device__ __forceinline__ void mfma_slab_step(f32x4_t& acc, const i32x4_t& a, const i32x4_t& b);

// bf16: lane l holds 8 consecutive k of row l%16 (k group l/16)
template <>
__device__ __forceinline__ void mfma_slab_step<bf16_bits>(f32x4_t& acc, const i32x4_t& a,
                                                          const i32x4_t& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

// fp32: each lane holds four consecutive k of its row; instruction e pairs
// element e of the four lane groups.  A and B use the same k assignment, so
// the four instructions together sum over all sixteen k of the step.
template <>
__device__ __forceinline__ void mfma_slab_step<float>(f32x4_t& acc, const i32x4_t& a,
                                                      const i32x4_t& b) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a[e]), __int_as_float(b[e]), acc,
                                               0, 0, 0);
}

// MFMA instructions per (A fragment, B fragment) pair and k-step
template <typename T>
constexpr int kMfmaPerPair = sizeof(T) == 2 ? 1 : 4;

// Wait until this wave's outstanding vector-memory operations (including
// direct-to-LDS loads) have completed: s_waitcnt vmcnt(0), other counters
// left alone (gfx9 encoding: expcnt 7, lgkmcnt 15).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ lds_void_t* to_lds(char* p) {
  return (lds_void_t*)((__attribute__((address_space(3))) char*)(p));
}

// A wave's share of one slab: PER_WAVE groups of 8 rows, each group one
// direct-to-LDS load of 1 KB.  Every group reads from a wave-uniform base
// pointer (kept in SGPRs) plus a per-lane 32-bit byte offset, so a load costs
// one scalar M0 write and the load itself, with no per-load vector address
// arithmetic.
template <int PER_WAVE>
struct SlabLoads {
  const char* base[PER_WAVE];  // uniform per group
  uint32_t off[PER_WAVE];      // per lane: row offset + swizzled chunk
  char* dst;                   // uniform: LDS address of group 0 in stage 0
};

// Issue groups [U0, U1) of a slab at byte offset kbytes along K into `stage`.
// The builtin exists only for the device pass of the single-source compile.
template <int PER_WAVE, int U0, int U1, typename Cfg>
__device__ __forceinline__ void issue_groups(const SlabLoads<PER_WAVE>& L, int stage,
                                             int64_t kbytes) {
#if defined(__HIP_DEVICE_COMPILE__)
  char* dst = L.dst + stage * Cfg::STAGE;
#pragma unroll
  for (int u = U0; u < U1; ++u)
    __builtin_amdgcn_global_load_lds(L.base[u] + kbytes + L.off[u], to_lds(dst + u * 1024), 16,
                                     0, 0);
#endif
}

template <typename T>
__device__ __forceinline__ void group_source(const Operand<T>& op, int32_t row0, int r,
                                             int lchunk, const char*& base, uint32_t& off) {
  if (op.map != nullptr) {
    // gathered rows: offsets from the operand base (host checks they fit 32 bits)
    const int32_t idx = row0 + r;
    const int32_t src = clamp_row(op.map[idx < op.map_len ? idx : op.map_len - 1], op.n_rows);
    base = reinterpret_cast<const char*>(op.base);
    off = (uint32_t)((int64_t)src * op.ld * (int64_t)sizeof(T)) + lchunk * 16;
  } else {
    // contiguous rows: offsets from the tile's first row
    const int32_t src = clamp_row(row0 + r, op.n_rows);
    base = reinterpret_cast<const char*>(op.base + (int64_t)row0 * op.ld);
    off = (uint32_t)((int64_t)(src - row0) * op.ld * (int64_t)sizeof(T)) + lchunk * 16;
  }
}

template <typename Cfg>
__device__ __forceinline__ void read_frags(const char* sa, const char* sb, int s, int lane,
                                           int wm, int wn, i32x4_t (&af)[Cfg::FM],
                                           i32x4_t (&bf)[Cfg::FN]) {
  const int frow = lane & 15;
  const int chunk = 4 * s + (lane >> 4);
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i) {
    const int r = wm * Cfg::WM + i * kFrag + frow;
    af[i] = *reinterpret_cast<const i32x4_t*>(sa + r * kRowBytes + ((chunk ^ (r & 7)) << 4));
  }
#pragma unroll
  for (int j = 0; j < Cfg::FN; ++j) {
    const int r = wn * Cfg::WN + j * kFrag + frow;
    bf[j] = *reinterpret_cast<const i32x4_t*>(sb + r * kRowBytes + ((chunk ^ (r & 7)) << 4));
  }
}

// One slab = two k-steps of MFMAs.  Step 0 issues the second half of slab
// k+1's loads (unless FIRST: the prologue loaded all of it) and reads step
// 1's fragments; step 1 (unless LAST) waits for slab k+1, meets the other
// waves at the barrier (all of them now hold step 1's fragments, so this
// stage is free), issues the first half of slab k+2 into it and reads slab
// k+1's step-0 fragments.  Inside a step, fragment reads and
// loads are interleaved with the MFMAs so they land while the rest run.
template <typename T, typename Cfg, int PER_WAVE, bool FIRST, bool LAST>
__device__ __forceinline__ void slab_steps(f32x4_t (&acc)[Cfg::FM][Cfg::FN],
                                           i32x4_t (&fa)[2][Cfg::FM], i32x4_t (&fb)[2][Cfg::FN],
                                           char* smem, int stage, int lane, int wm, int wn,
                                           const SlabLoads<PER_WAVE>& L, int64_t next_kbytes,
                                           int64_t pend_kbytes) {
  constexpr int kR = Cfg::FM + Cfg::FN;
  constexpr int kH = PER_WAVE / 2;
  constexpr int kSlots = Cfg::FM * Cfg::FN - kR;  // MFMA slots left after the reads
  constexpr int kPerSlot = (PER_WAVE + kSlots - 1) / kSlots;
  const char* sa = smem + stage * Cfg::STAGE;
  const char* sb = sa + Cfg::BM * kRowBytes;
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const bool loads = (s == 0 && !FIRST) || (s == kSteps - 1 && !LAST);
    if (s == 0 && !FIRST) issue_groups<PER_WAVE, kH, PER_WAVE, Cfg>(L, stage ^ 1, pend_kbytes);
    if (s < kSteps - 1) {
      read_frags<Cfg>(sa, sb, s + 1, lane, wm, wn, fa[(s + 1) & 1], fb[(s + 1) & 1]);
    } else if (!LAST) {
      wait_vmem();
      __syncthreads();
      issue_groups<PER_WAVE, 0, kH, Cfg>(L, stage, next_kbytes);
      const char* na = smem + (stage ^ 1) * Cfg::STAGE;
      read_frags<Cfg>(na, na + Cfg::BM * kRowBytes, 0, lane, wm, wn, fa[0], fb[0]);
    }
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j) mfma_slab_step<T>(acc[i][j], fa[s & 1][i], fb[s & 1][j]);
    if (s < kSteps - 1 || !LAST) {
#pragma unroll
      for (int q = 0; q < kR; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPerPair<T>, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                 // LDS read
      }
      if (loads) {
#pragma unroll
        for (int q = 0; q < kSlots; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPerPair<T>, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x020, kPerSlot, 0);          // slab loads
        }
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, kSlots * kMfmaPerPair<T>, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// C_tile = A[a_row0 : a_row0+BM, 0:k_len] * B[b_row0 : b_row0+BN, 0:k_len]^T,
// accumulated into `acc` (which the caller zeroes).  k_len is a multiple of
// Cfg::BK.  Ends with a barrier, so LDS is free for the epilogue.
//
// Slab rows (A rows, then B rows) reach LDS by direct-to-LDS loads
// (global_load_lds_dwordx4): one wave instruction fills 1 KB = 8 slab rows,
// lane i landing at byte 16 i; lane i therefore fetches logical chunk
// (i % 8) ^ (row % 8) of row i / 8, which realises the XOR swizzle.
template <typename T, typename Cfg>
__device__ __forceinline__ void tile_mainloop(f32x4_t (&acc)[Cfg::FM][Cfg::FN],
                                              const Operand<T>& A, int32_t a_row0,
                                              const Operand<T>& B, int32_t b_row0, int32_t k_len,
                                              char* smem) {
  constexpr int ROWS = Cfg::BM + Cfg::BN;
  constexpr int GROUPS = ROWS / 8;      // 1 KB load instructions per slab
  constexpr int PER_WAVE = GROUPS / 4;  // per wave
  static_assert(GROUPS % 4 == 0 && PER_WAVE % 2 == 0 && Cfg::BM % 8 == 0,
                "slab must split into 8-row groups");
  static_assert(Cfg::FM * Cfg::FN > Cfg::FM + Cfg::FN, "too few MFMAs per step");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int prow = lane >> 3;
  const int lchunk = (lane & 7) ^ prow;

  SlabLoads<PER_WAVE> L;
#pragma unroll
  for (int u = 0; u < PER_WAVE; ++u) {
    const int g = wave * PER_WAVE + u;  // uniform: which 8-row group
    if (g * 8 < Cfg::BM) group_source(A, a_row0, g * 8 + prow, lchunk, L.base[u], L.off[u]);
    else group_source(B, b_row0, g * 8 - Cfg::BM + prow, lchunk, L.base[u], L.off[u]);
  }
  L.dst = smem + wave * PER_WAVE * 1024;

  const int nslab = k_len / Cfg::BK;
  const int64_t last_kbytes = (int64_t)(nslab - 1) * kRowBytes;
  // slab 0 into stage 0; slab 1 (with a single slab, a harmless reload of
  // slab 0) into stage 1
  issue_groups<PER_WAVE, 0, PER_WAVE, Cfg>(L, 0, 0);
  wait_vmem();
  __syncthreads();
  issue_groups<PER_WAVE, 0, PER_WAVE, Cfg>(L, 1, nslab > 1 ? kRowBytes : 0);
  i32x4_t fa[2][Cfg::FM], fb[2][Cfg::FN];
  read_frags<Cfg>(smem, smem + Cfg::BM * kRowBytes, 0, lane, wm, wn, fa[0], fb[0]);
  __builtin_amdgcn_sched_barrier(0);

  // slab k+2's loads (clamped to the last slab: a reload into a stage that is
  // never read again) start at slab k's step 3 and finish at slab k+1's step 0
  auto clampk = [&](int k) { return k < nslab ? (int64_t)k * kRowBytes : last_kbytes; };
  if (nslab > 1) {
    slab_steps<T, Cfg, PER_WAVE, true, false>(acc, fa, fb, smem, 0, lane, wm, wn, L, clampk(2), 0);
    for (int ks = 1; ks + 1 < nslab; ++ks)
      slab_steps<T, Cfg, PER_WAVE, false, false>(acc, fa, fb, smem, ks & 1, lane, wm, wn, L,
                                                 clampk(ks + 2), clampk(ks + 1));
    slab_steps<T, Cfg, PER_WAVE, false, true>(acc, fa, fb, smem, (nslab - 1) & 1, lane, wm, wn, L,
                                              0, clampk(nslab));
  } else {
    slab_steps<T, Cfg, PER_WAVE, true, true>(acc, fa, fb, smem, 0, lane, wm, wn, L, 0, 0);
  }
  wait_vmem();      // reloads must land before LDS is reused
  __syncthreads();  // LDS is handed to the epilogue
}

template <typename Cfg>
__device__ __forceinline__ void zero_acc(f32x4_t (&acc)[Cfg::FM][Cfg::FN]) {
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;
}

// Workgroup -> tile.  Workgroups are dealt to the 8 XCDs round-robin
// (workgroup b runs on XCD b % 8); renumber so XCD x owns the contiguous range
// [x * per_xcd, (x+1) * per_xcd) of a grouped raster order in which
// `group_m` consecutive tile-rows are walked column by column.  The grid must
// have 8 * ceil(tiles / 8) workgroups; returns false for the padding ones.
__device__ __forceinline__ bool tile_of(int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int per_xcd = (total + 7) >> 3;
  const int b = blockIdx.x;
  const int logical = (b & 7) * per_xcd + (b >> 3);
  if (logical >= total) return false;
  const int group_size = group_m * tiles_n;
  const int g = logical / group_size;
  const int first_m = g * group_m;
  const int gm = min(group_m, tiles_m - first_m);
  const int idx = logical - g * group_size;
  tm = first_m + idx % gm;
  tn = idx / gm;
  return true;
}

__host__ __device__ inline int grid_for_tiles(int tiles) { return ((tiles + 7) / 8) * 8; }

}  // namespace specloss
