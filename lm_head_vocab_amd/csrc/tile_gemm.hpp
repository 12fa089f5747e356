// Tile machinery shared by every contraction of the streaming LM-head loss.
//
// Every contraction is C[m][n] = sum_k A[m][k] B[n][k].  An operand is either
// K-major (row m holds its k values contiguously: W and the hidden rows in the
// forward, the staged logit gradient dz in the dh contraction) or MN-major
// (k-row k holds the m values contiguously: W as the right operand of dh, and
// dz and the hidden chunk as the operands of dW), so no transposed copy is
// ever made of a bf16 operand.
//
// gfx950 mapping:
//  * 256 threads = 4 wave64s in a 2 x 2 grid (or 512 = 8 in 2 x 4, two per
//    SIMD); a wave owns a (BM/2) x (BN/WNW) sub-tile made of 16 x 16 MFMA fragments (v_mfma_f32_16x16x32_bf16 for
//    bf16, v_mfma_f32_16x16x4_f32 for fp32), fp32 accumulators.  The 16x16
//    shape moves half the accumulator traffic per flop of the 32x32 one,
//    which measures faster on this power-limited part.
//  * K advances in slabs of 128 bytes per row (64 bf16 / 32 fp32).  A slab of
//    A and B sits in LDS as rows of eight 16-byte chunks, chunk c of row r
//    stored at position c ^ (r & 7): eight consecutive rows read at the same
//    logical chunk hit eight different bank groups (conflict-free ds_read_b128).
//  * An MN-major slab is 64 k-rows of BM (or BN) values; the 16-byte chunk c
//    of k-row k is stored at position c ^ f(k), f(k) = 2 ((k & 3) | (k & 8) >> 1),
//    and fragments are read with the transposing LDS load ds_read_b64_tr_b16:
//    in each 16-lane group, lane L receives element L % 4 of the 8-byte loads
//    of lanes 4 j + L / 4 (j = 0..3), so lanes that load four consecutive m
//    of k-rows kb + j hand every lane four consecutive k of one m.  The
//    swizzle puts the four k-rows of a 16-lane group, and the two groups of
//    a 32-lane half, in different bank groups.
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
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_tr_t;
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

// LGAP: MFMAs between consecutive slab loads of a step.  WNW: waves along N
// (2: 4 waves, one per SIMD; 4: 8 waves, two per SIMD).
template <typename T, int BM_, int BN_, int LGAP_ = 1, int WNW_ = 2>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, LGAP = LGAP_, WNW = WNW_;
  static constexpr int WAVES = 2 * WNW, THREADS = 64 * WAVES;
  static constexpr int KC = ElemTraits<T>::kPerChunk;  // elements per 16-byte chunk
  static constexpr int BK = 8 * KC;                    // elements per slab row (128 bytes)
  static constexpr int WM = BM / 2, WN = BN / WNW;     // wave sub-tile
  static constexpr int FM = WM / kFrag, FN = WN / kFrag;  // 16x16 fragments per wave
  static constexpr int STAGE = (BM + BN) * kRowBytes;  // bytes of one LDS stage
  static constexpr int LDS_BYTES = 2 * STAGE;
};

// A K-major operand: tile row r reads source row map ? map[r] : r (relative
// to `base`), clamped into [0, n_rows): rows past the end or unmapped rows
// still load valid memory and their results are discarded by the epilogues.
// An MN-major operand (bf16 only): element (m, k) at base[k * ld + m]; m is
// clamped below n_rows (a multiple of 8) and k below k_valid the same way,
// so every load stays inside the tensor.
template <typename T>
struct Operand {
  const T* base;
  int64_t ld;            // elements between rows (K-major) or k-rows (MN-major)
  int32_t n_rows;        // valid source rows (K-major) or m values (MN-major)
  const int32_t* map;    // optional gather map indexed by tile row (K-major only)
  int32_t map_len;       // entries readable in map
  int32_t k_valid;       // MN-major: k-rows readable from the start of the contraction
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
//
// A wave's groups all belong to one operand when an operand is MN-major (the
// 256 x 256 tiles); `kstride` is the bytes one slab advances in that operand
// (128 for K-major, 64 k-rows for MN-major).  For an MN-major operand a group
// is two k-rows; in a slab that runs past k_valid the k-rows are clamped to
// the last valid one (only such slabs pay for the clamp).
template <int PER_WAVE>
struct SlabLoads {
  const char* base[PER_WAVE];  // uniform per group
  uint32_t off[PER_WAVE];      // per lane: row offset + swizzled chunk
  char* dst;                   // uniform: LDS address of group 0 in stage 0
  int64_t kstride;             // uniform: bytes per slab along K
  uint32_t ldb;                // uniform (MN-major): bytes between k-rows
  int32_t kvalid;              // uniform (MN-major): readable k-rows, else INT32_MAX
  int32_t krow0;               // uniform (MN-major): k-row of group 0's first half
};

// Issue groups [U0, U1) of slab `slab` into `stage`.  The builtin exists only
// for the device pass of the single-source compile.
template <int PER_WAVE, int U0, int U1, typename Cfg>
__device__ __forceinline__ void issue_groups(const SlabLoads<PER_WAVE>& L, int stage, int slab) {
#if defined(__HIP_DEVICE_COMPILE__)
  char* dst = L.dst + stage * Cfg::STAGE;
  const int64_t kb = (int64_t)slab * L.kstride;
  if ((slab + 1) * 64 > L.kvalid) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int u = U0; u < U1; ++u) {
      // k-rows past the last valid one read that row (signed: the slab may
      // start past it)
      const int over = slab * 64 + L.krow0 + 2 * u + (lane >> 5) - (L.kvalid - 1);
      const int64_t back = over > 0 ? (int64_t)over * L.ldb : 0;
      __builtin_amdgcn_global_load_lds(L.base[u] + kb + (int64_t)L.off[u] - back,
                                       to_lds(dst + u * 1024), 16, 0, 0);
    }
  } else {
#pragma unroll
    for (int u = U0; u < U1; ++u)
      __builtin_amdgcn_global_load_lds(L.base[u] + kb + L.off[u], to_lds(dst + u * 1024), 16,
                                       0, 0);
  }
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
    // contiguous rows: offsets from the tile's first row, itself clamped into
    // the tensor (a tile may start past the last row; the offsets stay >= 0)
    const int32_t first = clamp_row(row0, op.n_rows);
    const int32_t src = clamp_row(row0 + r, op.n_rows);
    base = reinterpret_cast<const char*>(op.base + (int64_t)first * op.ld);
    off = (uint32_t)((int64_t)(src - first) * op.ld * (int64_t)sizeof(T)) + lchunk * 16;
  }
}

// MN-major slab of one operand: group source of the two k-rows 2 ga, 2 ga + 1.
// Lane p loads k-row 2 ga + p / 32, logical chunk (p % 32) ^ f(k) of the
// tile's m range [m0, m0 + 256), the chunk clamped into the valid m.
template <typename T>
__device__ __forceinline__ void group_source_mn(const Operand<T>& op, int32_t m0, int ga,
                                                int lane, const char*& base, uint32_t& off) {
  const int k = 2 * ga + (lane >> 5);
  int chunk = (lane & 31) ^ (2 * ((k & 3) | ((k & 8) >> 1)));
  const int last = (op.n_rows - m0) / 8 - 1;  // last chunk holding valid m
  if (chunk > last) chunk = last < 0 ? 0 : last;
  base = reinterpret_cast<const char*>(op.base + m0);
  off = (uint32_t)((int64_t)k * op.ld * (int64_t)sizeof(T)) + chunk * 16;
}

// Fragments of one K-major operand for k-step s (rows of kRowBytes).
template <int F>
__device__ __forceinline__ void read_frags_k(const char* so, int s, int lane, int m_wave,
                                             i32x4_t (&f)[F]) {
  const int frow = lane & 15;
  const int chunk = 4 * s + (lane >> 4);
#pragma unroll
  for (int i = 0; i < F; ++i) {
    const int r = m_wave + i * kFrag + frow;
    f[i] = *reinterpret_cast<const i32x4_t*>(so + r * kRowBytes + ((chunk ^ (r & 7)) << 4));
  }
}

// Fragments of one MN-major operand (k-rows of `pitch` bytes) for k-step s:
// two transposing loads per fragment, k-rows 32 s + 8 g + j and + 4, where
// lane l = 16 g + 4 j + q loads m values 4 q .. 4 q + 3 of the fragment.
template <int F, int PITCH>
__device__ __forceinline__ void read_frags_mn(const char* so, int s, int lane, int m_wave,
                                              i32x4_t (&f)[F]) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int g = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
  const int x = (2 * (j | ((g & 1) << 2))) | (q >> 1);
  const char* row = so + (32 * s + 8 * g + j) * PITCH + (q & 1) * 8;
#pragma unroll
  for (int i = 0; i < F; ++i) {
    const char* p = row + ((((m_wave + i * kFrag) >> 3) ^ x) << 4);
    typedef __attribute__((address_space(3))) bf16x4_tr_t lds_bf16x4;
    const bf16x4_tr_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4*)((__attribute__((address_space(3))) char*)(p)));
    const bf16x4_tr_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4*)((__attribute__((address_space(3))) char*)(p + 4 * PITCH)));
    const i32x2_t l2 = __builtin_bit_cast(i32x2_t, lo), h2 = __builtin_bit_cast(i32x2_t, hi);
    f[i] = i32x4_t{l2[0], l2[1], h2[0], h2[1]};
  }
#else
  (void)so, (void)s, (void)lane, (void)m_wave;
#pragma unroll
  for (int i = 0; i < F; ++i) f[i] = i32x4_t{0, 0, 0, 0};
#endif
}

template <typename Cfg, bool A_MN, bool B_MN>
__device__ __forceinline__ void read_frags(const char* sa, const char* sb, int s, int lane,
                                           int wm, int wn, i32x4_t (&af)[Cfg::FM],
                                           i32x4_t (&bf)[Cfg::FN]) {
  if constexpr (A_MN) read_frags_mn<Cfg::FM, Cfg::BM * 2>(sa, s, lane, wm * Cfg::WM, af);
  else read_frags_k<Cfg::FM>(sa, s, lane, wm * Cfg::WM, af);
  if constexpr (B_MN) read_frags_mn<Cfg::FN, Cfg::BN * 2>(sb, s, lane, wn * Cfg::WN, bf);
  else read_frags_k<Cfg::FN>(sb, s, lane, wn * Cfg::WN, bf);
}

// Transposed copy of the A operand, taken from its LDS slabs (the dh
// contraction: A = dz [rows][V], K-major).  Each (slab, tile row) pair is
// written by exactly one workgroup, the one whose tile column equals the
// slab's global index modulo `every`, so across a launch every 64-column slab
// of every 256-row tile goes out once as 64 rows of `out` (row = k, 256
// values = the tile's A rows), with values of rows at or past n_valid as 0.
struct SlabDump {
  bf16_bits* out;  // out[k * ld + col0 + n]
  int64_t ld;
  int32_t col0;     // first A row of the tile
  int32_t n_valid;  // A rows of the tile that hold data (may exceed 256)
  int32_t every;    // tile columns of the launch
  int32_t phase;    // this workgroup's tile column
  int32_t slab0;    // global index of the workgroup's first slab (split K)
};

// Eight waves: wave w writes k-rows 16 (w % 4) .. + 15 of the slab for tile
// rows 128 (w / 4) .. + 127.  A transposing LDS read in a 16-lane group gives
// lane L four consecutive tile rows of k-row kb + L (source lane 4 j + q reads
// tile row n0 + j at k kb + 4 q .. + 3, and lane L receives element L % 4 of
// lanes 4 j + L / 4); two such reads make 8 rows, stored as one 16-byte piece.
template <typename Cfg>
__device__ __forceinline__ void dump_slab_t(const char* sa, const SlabDump& D, int slab, int lane,
                                            int wave) {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(Cfg::WAVES == 8 && Cfg::BM == 256 && sizeof(bf16_bits) == 2, "8 waves, 256 rows");
  const int g = lane >> 4, L = lane & 15, j = L >> 2, q = L & 3;
  const int kb = 16 * (wave & 3), nh = 128 * (wave >> 2);
  const int kbyte = (kb + 4 * q) * 2;
  const int kch = kbyte >> 4, koff = kbyte & 15;
  bf16_bits* orow = D.out + (int64_t)(slab * 64 + kb + L) * D.ld + D.col0;
  typedef __attribute__((address_space(3))) bf16x4_tr_t lds_bf16x4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n0 = nh + 32 * i + 8 * g;
    const int ra = n0 + j, rb = ra + 4;
    const char* pa = sa + ra * kRowBytes + ((kch ^ (ra & 7)) << 4) + koff;
    const char* pb = sa + rb * kRowBytes + ((kch ^ (rb & 7)) << 4) + koff;
    const bf16x4_tr_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4*)((__attribute__((address_space(3))) char*)(pa)));
    const bf16x4_tr_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4*)((__attribute__((address_space(3))) char*)(pb)));
    const i32x2_t l2 = __builtin_bit_cast(i32x2_t, lo), h2 = __builtin_bit_cast(i32x2_t, hi);
    i32x4_t w = i32x4_t{l2[0], l2[1], h2[0], h2[1]};
    if (n0 + 8 > D.n_valid) {
      // keep only the bf16 halves of rows below n_valid (element e: word e / 2,
      // low half when e is even)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (n0 + e >= D.n_valid) w[e >> 1] &= (e & 1) ? 0x0000ffff : (int)0xffff0000;
    }
    *reinterpret_cast<i32x4_t*>(orow + n0) = w;
  }
#else
  (void)sa, (void)D, (void)slab, (void)lane, (void)wave;
#endif
}

// One slab = two k-steps of MFMAs.  Step 0 issues the second half of slab
// k+1's loads (unless FIRST: the prologue loaded all of it) and reads step
// 1's fragments; step 1 (unless LAST) waits for slab k+1, meets the other
// waves at the barrier (all of them now hold step 1's fragments, so this
// stage is free), issues the first half of slab k+2 into it and reads slab
// k+1's step-0 fragments.  Inside a step, loads and fragment reads are
// interleaved with the MFMAs so they land while the rest run.  With DUMP and
// dump_slab >= 0 the wave also writes its share of slab k+1's transposed A
// right after that barrier (slab k+1 stays in its stage for a whole slab, so
// the stores have a slab's time before the next barrier waits for them;
// measured 0.1 ms per step better than writing a slab during its own step 0).
template <typename T, typename Cfg, int PER_WAVE, bool FIRST, bool LAST, bool A_MN, bool B_MN,
          bool DUMP = false>
__device__ __forceinline__ void slab_steps(f32x4_t (&acc)[Cfg::FM][Cfg::FN],
                                           i32x4_t (&fa)[2][Cfg::FM], i32x4_t (&fb)[2][Cfg::FN],
                                           char* smem, int stage, int lane, int wm, int wn,
                                           const SlabLoads<PER_WAVE>& L, int next_slab,
                                           int pend_slab, const SlabDump* D = nullptr,
                                           int dump_slab = -1) {
  // LDS read instructions per step: one per K-major fragment, two per MN-major one
  constexpr int kR = Cfg::FM * (A_MN ? 2 : 1) + Cfg::FN * (B_MN ? 2 : 1);
  constexpr int kH = PER_WAVE / 2;
  constexpr int kRest = Cfg::FM * Cfg::FN - kH * Cfg::LGAP - kR;  // MFMAs after loads and reads
  static_assert(kRest >= 0, "too few MFMAs per step for the interleave");
  const char* sa = smem + stage * Cfg::STAGE;
  const char* sb = sa + Cfg::BM * kRowBytes;
  // MFMAs of step 1 issued before the slab barrier: they need only fragments
  // already in registers and keep the MFMA pipe busy while the wave waits
  // (16 measured best of 0, 8, 16 and 32)
  constexpr int kEarly = 16 < kRest ? 16 : kRest;
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const bool loads = (s == 0 && !FIRST) || (s == kSteps - 1 && !LAST);
    const int early = (s == kSteps - 1 && !LAST) ? kEarly : 0;
    if (s == 0 && !FIRST) issue_groups<PER_WAVE, kH, PER_WAVE, Cfg>(L, stage ^ 1, pend_slab);
    if (s < kSteps - 1) {
      read_frags<Cfg, A_MN, B_MN>(sa, sb, s + 1, lane, wm, wn, fa[(s + 1) & 1], fb[(s + 1) & 1]);
    } else if (!LAST) {
#pragma unroll
      for (int q = 0; q < kEarly; ++q)
        mfma_slab_step<T>(acc[q / Cfg::FN][q % Cfg::FN], fa[s & 1][q / Cfg::FN],
                          fb[s & 1][q % Cfg::FN]);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmem();
      __syncthreads();
      issue_groups<PER_WAVE, 0, kH, Cfg>(L, stage, next_slab);
      const char* na = smem + (stage ^ 1) * Cfg::STAGE;
      if constexpr (DUMP) {
        // the next slab, complete in the other stage since this barrier and
        // kept there until the next one: a slab's time for the stores
        if (dump_slab >= 0) dump_slab_t<Cfg>(na, *D, dump_slab, lane, wm * Cfg::WNW + wn);
      }
      read_frags<Cfg, A_MN, B_MN>(na, na + Cfg::BM * kRowBytes, 0, lane, wm, wn, fa[0], fb[0]);
    }
#pragma unroll
    for (int q = early; q < Cfg::FM * Cfg::FN; ++q)
      mfma_slab_step<T>(acc[q / Cfg::FN][q % Cfg::FN], fa[s & 1][q / Cfg::FN],
                        fb[s & 1][q % Cfg::FN]);
    if (s < kSteps - 1 || !LAST) {
      // the step's slab loads go first, one per LGAP MFMAs, then the fragment
      // reads for the next step, one per MFMA, then the remaining MFMAs
      // (measured about 2% faster than reads first)
      if (loads) {
#pragma unroll
        for (int q = 0; q < kH; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, Cfg::LGAP * kMfmaPerPair<T>, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // slab load
        }
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, kH * Cfg::LGAP * kMfmaPerPair<T>, 0);
      }
#pragma unroll
      for (int q = 0; q < kR; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPerPair<T>, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                 // LDS read
      }
      if (early) __builtin_amdgcn_sched_group_barrier(0x008, (kRest - kEarly) * kMfmaPerPair<T>, 0);
      else __builtin_amdgcn_sched_group_barrier(0x008, kRest * kMfmaPerPair<T>, 0);
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
template <typename T, typename Cfg, bool A_MN = false, bool B_MN = false, bool DUMP = false>
__device__ __forceinline__ void tile_mainloop(f32x4_t (&acc)[Cfg::FM][Cfg::FN],
                                              const Operand<T>& A, int32_t a_row0,
                                              const Operand<T>& B, int32_t b_row0, int32_t k_len,
                                              char* smem, const SlabDump* D = nullptr) {
  constexpr int ROWS = Cfg::BM + Cfg::BN;
  constexpr int GROUPS = ROWS / 8;               // 1 KB load instructions per slab
  constexpr int PER_WAVE = GROUPS / Cfg::WAVES;  // per wave
  static_assert(GROUPS % Cfg::WAVES == 0 && PER_WAVE % 2 == 0 && Cfg::BM % 8 == 0,
                "slab must split into 8-row groups");
  static_assert(Cfg::FM * Cfg::FN > Cfg::FM * (A_MN ? 2 : 1) + Cfg::FN * (B_MN ? 2 : 1),
                "too few MFMAs per step");
  static_assert(!(A_MN || B_MN) || (sizeof(T) == 2 && Cfg::BM == 256 && Cfg::BN == 256),
                "MN-major operands: bf16, 256 x 256 tiles (a wave's groups in one operand)");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / Cfg::WNW, wn = wave % Cfg::WNW;
  const int prow = lane >> 3;
  const int lchunk = (lane & 7) ^ prow;

  SlabLoads<PER_WAVE> L;
  const bool wave_b = wave * PER_WAVE * 8 >= Cfg::BM;  // uniform: this wave loads B
  const bool wave_mn = wave_b ? B_MN : A_MN;
  const Operand<T>& O = wave_b ? B : A;
  L.kstride = wave_mn ? (int64_t)64 * O.ld * (int64_t)sizeof(T) : kRowBytes;
  L.ldb = (uint32_t)(O.ld * (int64_t)sizeof(T));
  L.kvalid = wave_mn ? O.k_valid : 0x7fffffff;
  L.krow0 = 2 * (wave * PER_WAVE - (wave_b ? Cfg::BM / 8 : 0));
#pragma unroll
  for (int u = 0; u < PER_WAVE; ++u) {
    const int g = wave * PER_WAVE + u;  // uniform: which 1 KB group
    if (g * 8 < Cfg::BM) {
      if (A_MN) group_source_mn(A, a_row0, g, lane, L.base[u], L.off[u]);
      else group_source(A, a_row0, g * 8 + prow, lchunk, L.base[u], L.off[u]);
    } else {
      if (B_MN) group_source_mn(B, b_row0, g - Cfg::BM / 8, lane, L.base[u], L.off[u]);
      else group_source(B, b_row0, g * 8 - Cfg::BM + prow, lchunk, L.base[u], L.off[u]);
    }
  }
  L.dst = smem + wave * PER_WAVE * 1024;

  const int nslab = k_len / Cfg::BK;
  // slab 0 into stage 0; slab 1 (with a single slab, a harmless reload of
  // slab 0) into stage 1
  issue_groups<PER_WAVE, 0, PER_WAVE, Cfg>(L, 0, 0);
  wait_vmem();
  __syncthreads();
  issue_groups<PER_WAVE, 0, PER_WAVE, Cfg>(L, 1, nslab > 1 ? 1 : 0);
  i32x4_t fa[2][Cfg::FM], fb[2][Cfg::FN];
  read_frags<Cfg, A_MN, B_MN>(smem, smem + Cfg::BM * kRowBytes, 0, lane, wm, wn, fa[0], fb[0]);
  __builtin_amdgcn_sched_barrier(0);

  // slab k+2's loads (clamped to the last slab: a reload into a stage that is
  // never read again) start at slab k's last step and finish at slab k+1's step 0
  auto clampk = [&](int k) { return k < nslab ? k : nslab - 1; };
  // DUMP: slabs whose global index is phase modulo every go out transposed;
  // `until` counts the slabs left before the next one (uniform)
  int until = 0;
  if constexpr (DUMP) {
    until = (D->phase - D->slab0) % D->every;
    if (until < 0) until += D->every;
  }
  auto dump_at = [&](int ks) {
    if constexpr (!DUMP) return -1;
    if (until != 0) {
      --until;
      return -1;
    }
    until = D->every - 1;
    return D->slab0 + ks;
  };
  if constexpr (DUMP) {
    // slab 0 from stage 0 (visible since the prologue barrier, kept until
    // the barrier of its step 1); slab k + 1 after slab k's barrier
    const int d0 = dump_at(0);
    if (d0 >= 0) dump_slab_t<Cfg>(smem, *D, d0, lane, wave);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (nslab > 1) {
    slab_steps<T, Cfg, PER_WAVE, true, false, A_MN, B_MN, DUMP>(acc, fa, fb, smem, 0, lane, wm, wn,
                                                                L, clampk(2), 0, D, dump_at(1));
    for (int ks = 1; ks + 1 < nslab; ++ks)
      slab_steps<T, Cfg, PER_WAVE, false, false, A_MN, B_MN, DUMP>(
          acc, fa, fb, smem, ks & 1, lane, wm, wn, L, clampk(ks + 2), clampk(ks + 1), D,
          dump_at(ks + 1));
    slab_steps<T, Cfg, PER_WAVE, false, true, A_MN, B_MN, DUMP>(acc, fa, fb, smem, (nslab - 1) & 1,
                                                                lane, wm, wn, L, 0, clampk(nslab));
  } else {
    slab_steps<T, Cfg, PER_WAVE, true, true, A_MN, B_MN, DUMP>(acc, fa, fb, smem, 0, lane, wm, wn,
                                                               L, 0, 0);
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
