// HIP kernels of the streaming LM-head loss for gfx950.
//
// Vocab-tiled passes (one workgroup per 256-row vocabulary tile x token tile;
// the logits tile lives only in accumulator registers):
//   k_stats  pass 1: per (vocab tile, token) running max and sum of exp of the
//            logits (and the argmax for the target side): blog "Streaming Cross
//            Entropy", the logsumexp of every token without its logits row.
//   k_div    pass 2: recomputes draft and target tiles and sums, per token,
//            min(p,q), q*1[q<p], p log(p/q), q log(q/p) and the JSD terms with
//            the final logsumexps (speculators "Available Losses" table).
//   k_dz     backward recompute: forms the logit gradient of the weighted loss
//            in registers and stages it (bf16 for bf16 inputs) for the two
//            contractions (blog "Backward pass").
//   k_stats_stage  pass 1 of the single forward+backward call: as k_stats,
//            and stores e = exp(z - m_tile) of every (token, vocab) for the
//            backward, so no logits tile is computed twice.
// Memory-bound passes of the single call: k_dz_stage forms the logit
// gradient of the cross-entropies from the staged values, in place, plus its
// transpose for the dW contraction; for the divergences pass 1 keeps both
// raw logit rows, and k_div_raw (the second sweep's sums) and k_dz_raw (the
// logit gradient and its transpose) read them.
// Plain contraction k_gemm: dh = dz W and dW (+)= dz^T h.
// Row kernels: validity/counts, label-logit gather, partial merges, means,
// gradient seeds, transposes and head alignment.
//
// Every reduction runs in a fixed order (no floating-point atomics), so
// results are bitwise repeatable.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "launch.hpp"
#include "tile_gemm.hpp"

namespace specloss {

// Height (in tiles) of the tile blocks each XCD walks, see tile_of: blocks of
// 4 x 8 tiles measured best for every contraction of the path (1, 2 and 8
// were slower at the 8B shape).
constexpr int kGroupM = 4;
// MFMAs between consecutive slab loads in pass 1 (3) and in the plain
// contractions (1): measured best of 1 to 4 on each at the 8B shape.
constexpr int kStatsLoadGap = 3;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

template <typename T>
__device__ __forceinline__ Operand<T> as_op(const GemmOperand& g) {
  return Operand<T>{static_cast<const T*>(g.base), g.ld, g.n_rows, g.map, g.map_len, g.k_valid};
}

// The four lanes l, l^16, l^32, l^48 hold the same output column.  These
// butterflies combine their values in a fixed order (lower lane first at each
// level), so every lane ends with the same, repeatable result.
__device__ __forceinline__ float col_sum(float x, int lane) {
  float o = __shfl_xor(x, 16);
  x = (lane & 16) ? o + x : x + o;
  o = __shfl_xor(x, 32);
  return (lane & 32) ? o + x : x + o;
}
__device__ __forceinline__ float col_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

// Tile entries past the vocabulary's end (the last vocabulary tile) become
// -inf, so that the max and exp loops need no per-entry test: exp2(-inf) = 0
// adds nothing to a sum.  The loops then take the maximum with the IEEE
// maximum (v_maximum3_f32 on gfx950, NaN-propagating), which needs no
// canonicalising of the accumulators that fmaxf would add.
template <typename Cfg>
__device__ __forceinline__ void mask_vocab_tail(f32x4_t (&acc)[Cfg::FM][Cfg::FN], int v_base,
                                                int lane, int vocab) {
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (v_base + i * kFrag + frag_row(r, lane) >= vocab) acc[i][j][r] = -INFINITY;
}

// Merge two (max, sum of exp(x - max)) pairs; `a` is the lower-index side.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * fast_exp2((m - mn) * kLog2e) + s2 * fast_exp2((m2 - mn) * kLog2e);
  m = mn;
}

// as lse_merge, also carrying q = sum exp(2 (x - m)) (the squared norm of the
// unnormalised distribution) relative to the same running maximum
__device__ __forceinline__ void lse_merge_sq(float& m, float& s, float& q, float m2, float s2,
                                             float q2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  const float a = fast_exp2((m - mn) * kLog2e), b = fast_exp2((m2 - mn) * kLog2e);
  s = s * a + s2 * b;
  q = q * a * a + q2 * b * b;
  m = mn;
}

// log of the mixture m = (p + q) / 2 for the Jensen-Shannon terms.  Where
// both probabilities are below the smallest normal float (exp underflow) the
// terms p (log p - log m) and q (log q - log m) are below 1e-36 (x log x ->
// 0), and any finite value serves; the hardware logarithm takes a denormal
// input as 0, which would give 0 * inf.
__device__ __forceinline__ float log_mixture(float p, float q) {
  const float m = 0.5f * (p + q);
  return m >= 1.17549435e-38f ? fast_log2(m) * kLn2 : 0.0f;
}

template <typename T>
__device__ __forceinline__ void store4(T* dst, float a0, float a1, float a2, float a3);
template <>
__device__ __forceinline__ void store4<bf16_bits>(bf16_bits* dst, float a0, float a1, float a2,
                                                  float a3) {
  bf16x4_t v = {(__bf16)a0, (__bf16)a1, (__bf16)a2, (__bf16)a3};
  *reinterpret_cast<bf16x4_t*>(dst) = v;
}
template <>
__device__ __forceinline__ void store4<float>(float* dst, float a0, float a1, float a2, float a3) {
  f32x4_t v = {a0, a1, a2, a3};
  *reinterpret_cast<f32x4_t*>(dst) = v;
}
// Two accumulator fragments that share their 16 rows and sit in adjacent
// 16-column blocks, stored through a layout whose rows are contiguous and
// whose columns are `ld` apart; p0 addresses (row 0, column 0) of the first.
// Each lane holds rows 4 g .. 4 g + 3 (g = lane / 16) of column lane % 16 of
// both (`a`, `b`).  For bf16, v_permlane16_swap exchanges the odd 16-lane rows
// of the first with the even rows of the second, after which lanes of row g
// hold the eight rows 8 (g / 2) .. + 7 of column block g % 2: one 16-byte
// store per lane instead of two 8-byte ones.
template <typename T>
__device__ __forceinline__ void store_frag_pair(T* p0, int64_t ld, const float (&a)[4],
                                                const float (&b)[4], int lane) {
  if constexpr (sizeof(T) == 2) {
    const bf16x4_t va = {(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3]};
    const bf16x4_t vb = {(__bf16)b[0], (__bf16)b[1], (__bf16)b[2], (__bf16)b[3]};
    const i32x2_t ia = __builtin_bit_cast(i32x2_t, va), ib = __builtin_bit_cast(i32x2_t, vb);
    const auto s0 = __builtin_amdgcn_permlane16_swap(ia[0], ib[0], false, false);
    const auto s1 = __builtin_amdgcn_permlane16_swap(ia[1], ib[1], false, false);
    const int g = lane >> 4;
    const i32x4_t out = {(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
    *reinterpret_cast<i32x4_t*>(p0 + (int64_t)(16 * (g & 1) + (lane & 15)) * ld + 8 * (g >> 1)) =
        out;
  } else {
    const int r0 = 4 * (lane >> 4), c = lane & 15;
    store4<T>(p0 + (int64_t)c * ld + r0, a[0], a[1], a[2], a[3]);
    store4<T>(p0 + (int64_t)(16 + c) * ld + r0, b[0], b[1], b[2], b[3]);
  }
}

template <typename T>
__device__ __forceinline__ float load1(const T* src) {
  if constexpr (sizeof(T) == 2) return (float)*reinterpret_cast<const __bf16*>(src);
  else return *src;
}

template <typename T>
__device__ __forceinline__ void store1(T* dst, float x);
template <>
__device__ __forceinline__ void store1<bf16_bits>(bf16_bits* dst, float x) {
  *reinterpret_cast<__bf16*>(dst) = (__bf16)x;
}
template <>
__device__ __forceinline__ void store1<float>(float* dst, float x) {
  *dst = x;
}

// 16 bytes of T (8 bf16 or 4 fp32) widened to fp32
template <typename T, int KC>
__device__ __forceinline__ void load_chunk(const T* src, float (&out)[KC]) {
  const i32x4_t raw = *reinterpret_cast<const i32x4_t*>(src);
  if constexpr (sizeof(T) == 2) {
    const bf16x8_t b = __builtin_bit_cast(bf16x8_t, raw);
#pragma unroll
    for (int q = 0; q < KC; ++q) out[q] = (float)b[q];
  } else {
#pragma unroll
    for (int q = 0; q < KC; ++q) out[q] = __int_as_float(raw[q]);
  }
}

// A tile's values (in the accumulator layout) stored to a row-major output
// whose rows are the tile's M index, as 16-byte pieces: the tile goes out in
// two halves of 128 rows, each staged through LDS as fp32 (rows padded to
// BN * 4 + 16 bytes so the row groups of a fragment store land in different
// banks), then streamed row by row.  Rounding to T happens at the store.
template <typename T, typename Cfg>
__device__ __forceinline__ void store_tile_rows(const f32x4_t (&acc)[Cfg::FM][Cfg::FN], T* out,
                                                int64_t ld, int64_t row0, int64_t col0,
                                                char* smem) {
  constexpr int kHalf = Cfg::BM / 2;
  constexpr int kStride = Cfg::BN * 4 + 16;
  constexpr int kPieces = Cfg::BN / 8;  // 8-value pieces per row
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / Cfg::WNW, wn = wave % Cfg::WNW;
#pragma unroll 1
  for (int h = 0; h < 2; ++h) {
    if (wm == h) {
#pragma unroll
      for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = i * kFrag + frag_row(r, lane);
            const int col = wn * Cfg::WN + j * kFrag + frag_col(lane);
            *reinterpret_cast<float*>(smem + row * kStride + col * 4) = acc[i][j][r];
          }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < kHalf * kPieces; idx += Cfg::THREADS) {
      const int row = idx / kPieces, pc = idx % kPieces;
      const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(smem + row * kStride + pc * 32);
      const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(smem + row * kStride + pc * 32 + 16);
      T* p = out + (row0 + h * kHalf + row) * ld + col0 + pc * 8;
      if constexpr (sizeof(T) == 2) {
        const bf16x8_t b = {(__bf16)x0[0], (__bf16)x0[1], (__bf16)x0[2], (__bf16)x0[3],
                            (__bf16)x1[0], (__bf16)x1[1], (__bf16)x1[2], (__bf16)x1[3]};
        *reinterpret_cast<bf16x8_t*>(p) = b;
      } else {
        *reinterpret_cast<f32x4_t*>(p) = x0;
        *reinterpret_cast<f32x4_t*>(p + 4) = x1;
      }
    }
    __syncthreads();
  }
}

// ============================================================================
// pass 1: per-tile softmax statistics
// ============================================================================
// TARGET (the target distribution p): also the lowest-index argmax and the sum
// of e^2, e = exp(u - m_tile), from which the flatness score is formed.
// RAW: the tile's logits also go out as fp32 (a.raw), each lane storing its
// four consecutive vocabulary entries of a row as one 16-byte nontemporal
// store before the statistics are formed, so the stores drain under that
// arithmetic.
template <typename T, bool TARGET, int WNW = 2, bool RAW = false>
__global__ __launch_bounds__(128 * WNW, 1) void k_stats(StatsLaunch a) {
  constexpr bool ARGMAX = TARGET;
  using Cfg = TileCfg<T, 256, 256, (WNW == 2 ? kStatsLoadGap : 1), WNW>;
  __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS_BYTES];
  int tm, tn;
  if (!tile_of(a.tiles_m, a.tiles_n, kGroupM, tm, tn)) return;

  f32x4_t acc[Cfg::FM][Cfg::FN];
  zero_acc<Cfg>(acc);
  tile_mainloop<T, Cfg>(acc, as_op<T>(a.A), tm * Cfg::BM, as_op<T>(a.B), tn * Cfg::BN, a.k_len,
                        smem);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WNW, wn = wave % WNW;
  const int v_base = tm * Cfg::BM + wm * Cfg::WM;
  const bool tail = tm * Cfg::BM + Cfg::BM > a.vocab;

  if constexpr (RAW) {
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
      const int c = tn * Cfg::BN + wn * Cfg::WN + j * kFrag + frag_col(lane);
      if (c < a.ncols) {
        float* row = a.raw + (int64_t)c * a.ld_raw + v_base + frag_row(0, lane);
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
          __builtin_nontemporal_store(acc[i][j], reinterpret_cast<f32x4_t*>(row + i * kFrag));
      }
    }
  }

  if (tail) mask_vocab_tail<Cfg>(acc, v_base, lane, a.vocab);
  float mj[Cfg::FN], sj[Cfg::FN], qj[Cfg::FN];
  int ij[Cfg::FN];
#pragma unroll
  for (int j = 0; j < Cfg::FN; ++j) {
    float mx = -INFINITY;
    int idx = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = acc[i][j][r];
        if (ARGMAX) {
          // strict: keeps the lowest index
          if (x > mx) { mx = x; idx = v_base + i * kFrag + frag_row(r, lane); }
        } else {
          mx = __builtin_elementwise_maximum(mx, x);
        }
      }
    const float m = col_max(mx);
    float s = 0.0f, q = 0.0f;
    if (m != -INFINITY) {
      const float mb = m * kLog2e;
#pragma unroll
      for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = fast_exp2(fmaf(acc[i][j][r], kLog2e, -mb));
          s += e;
          if (TARGET) q = fmaf(e, e, q);
        }
    }
    mj[j] = m;
    sj[j] = col_sum(s, lane);
    qj[j] = TARGET ? col_sum(q, lane) : 0.0f;
    if (ARGMAX) {
      // lowest index among the lanes that reach the column maximum
      int cand = (mx == m) ? idx : 0x7fffffff;
      cand = min(cand, __shfl_xor(cand, 16));
      ij[j] = min(cand, __shfl_xor(cand, 32));
    } else {
      ij[j] = 0;
    }
  }

  // the two wave rows (wm) share token columns: wm = 1 hands its values over
  float* red = reinterpret_cast<float*>(smem);
  if (wm == 1 && lane < kFrag) {
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
      const int c = wn * Cfg::WN + j * kFrag + lane;
      red[c * 4 + 0] = mj[j];
      red[c * 4 + 1] = sj[j];
      red[c * 4 + 2] = __int_as_float(ij[j]);
      red[c * 4 + 3] = qj[j];
    }
  }
  __syncthreads();
  if (wm == 0 && lane < kFrag) {
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
      const int c = wn * Cfg::WN + j * kFrag + lane;
      float m = mj[j], s = sj[j], q = qj[j];
      int id = ij[j];
      const float m2 = red[c * 4 + 0], s2 = red[c * 4 + 1];
      const int i2 = __float_as_int(red[c * 4 + 2]);
      if (ARGMAX) id = (m2 > m) ? i2 : ((m2 == m) ? min(id, i2) : id);
      if (TARGET)
        lse_merge_sq(m, s, q, m2, s2, red[c * 4 + 3]);
      else
        lse_merge(m, s, m2, s2);
      const int col = tn * Cfg::BN + c;
      if (col < a.ncols) {
        const int64_t o = (int64_t)tm * a.ldp + col;
        a.pm[o] = m;
        a.ps[o] = s;
        if (ARGMAX) a.pi[o] = id;
        if (TARGET) a.pq[o] = q;
      }
    }
  }
}

// (max, sum exp(x - max), sum exp(x - max) y) triples: y-sums merge as the sums do
__device__ __forceinline__ void lse_merge_x(float& m, float& s, float& x, float m2, float s2,
                                            float x2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  const float a = fast_exp2((m - mn) * kLog2e), b = fast_exp2((m2 - mn) * kLog2e);
  s = s * a + s2 * b;
  x = x * a + x2 * b;
  m = mn;
}

// Pass 1 of both sides of a row at once: the draft tile z and the target tile
// u are both kept in registers (256 x 128 tiles, as in pass 2), so besides
// the statistics of k_stats for each side the tile also yields the log-ratio
// sums of the two Kullback-Leibler divergences relative to the tile maxima:
// pa = sum exp(u - m_u) (u - z) and pr = sum exp(z - m_z) (z - u).
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void k_stats_dual(DualStatsLaunch a) {
  using Cfg = TileCfg<T, 256, 128>;
  __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS_BYTES];
  int tm, tn;
  if (!tile_of(a.tiles_m, a.tiles_n, kGroupM, tm, tn)) return;

  f32x4_t az[Cfg::FM][Cfg::FN], au[Cfg::FM][Cfg::FN];
  zero_acc<Cfg>(az);
  zero_acc<Cfg>(au);
  tile_mainloop<T, Cfg>(az, as_op<T>(a.Az), tm * Cfg::BM, as_op<T>(a.Bz), tn * Cfg::BN, a.k_len,
                        smem);
  tile_mainloop<T, Cfg>(au, as_op<T>(a.Au), tm * Cfg::BM, as_op<T>(a.Bu), tn * Cfg::BN, a.k_len,
                        smem);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int v_base = tm * Cfg::BM + wm * Cfg::WM;
  const bool tail = tm * Cfg::BM + Cfg::BM > a.vocab;

  // per column: m_z, s_z, pr, m_u, s_u, argmax, q_u, pa
  constexpr int NV = 8;
  float val[Cfg::FN][NV];
#pragma unroll
  for (int j = 0; j < Cfg::FN; ++j) {
    float mz = -INFINITY, mu = -INFINITY;
    int iu = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = v_base + i * kFrag + frag_row(r, lane);
        if (tail && v >= a.vocab) continue;
        mz = fmaxf(mz, az[i][j][r]);
        if (au[i][j][r] > mu) { mu = au[i][j][r]; iu = v; }  // strict: lowest index
      }
    const float Mz = col_max(mz), Mu = col_max(mu);
    float sz = 0.0f, pr = 0.0f, su = 0.0f, qu = 0.0f, pa = 0.0f;
    if (Mz != -INFINITY) {  // then Mu is finite too: the same entries are valid
      const float mzb = Mz * kLog2e, mub = Mu * kLog2e;
#pragma unroll
      for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int v = v_base + i * kFrag + frag_row(r, lane);
          if (tail && v >= a.vocab) continue;
          const float z = az[i][j][r], u = au[i][j][r], d = u - z;
          const float ez = fast_exp2(fmaf(z, kLog2e, -mzb));
          const float eu = fast_exp2(fmaf(u, kLog2e, -mub));
          sz += ez;
          pr = fmaf(ez, -d, pr);
          su += eu;
          qu = fmaf(eu, eu, qu);
          pa = fmaf(eu, d, pa);
        }
    }
    int cand = (mu == Mu) ? iu : 0x7fffffff;
    cand = min(cand, __shfl_xor(cand, 16));
    cand = min(cand, __shfl_xor(cand, 32));
    val[j][0] = Mz;
    val[j][1] = col_sum(sz, lane);
    val[j][2] = col_sum(pr, lane);
    val[j][3] = Mu;
    val[j][4] = col_sum(su, lane);
    val[j][5] = __int_as_float(cand);
    val[j][6] = col_sum(qu, lane);
    val[j][7] = col_sum(pa, lane);
  }

  // the two wave rows (wm) share token columns: wm = 1 hands its values over
  float* red = reinterpret_cast<float*>(smem);  // [BN][NV]
  if (wm == 1 && lane < kFrag) {
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
      const int c = wn * Cfg::WN + j * kFrag + lane;
#pragma unroll
      for (int f = 0; f < NV; ++f) red[c * NV + f] = val[j][f];
    }
  }
  __syncthreads();
  if (wm == 0 && lane < kFrag) {
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
      const int c = wn * Cfg::WN + j * kFrag + lane;
      const int col = tn * Cfg::BN + c;
      if (col >= a.ncols) continue;
      const float* o2 = red + c * NV;
      float mz = val[j][0], sz = val[j][1], pr = val[j][2];
      lse_merge_x(mz, sz, pr, o2[0], o2[1], o2[2]);
      float mu = val[j][3], su = val[j][4], qu = val[j][6], pa = val[j][7];
      int id = __float_as_int(val[j][5]);
      const int i2 = __float_as_int(o2[5]);
      id = (o2[3] > mu) ? i2 : ((o2[3] == mu) ? min(id, i2) : id);
      {
        // the pair (s, q) and the pair (s, pa) share the rescaling of s
        float s1 = su, q1 = qu, m1 = mu;
        lse_merge_sq(m1, s1, q1, o2[3], o2[4], o2[6]);
        lse_merge_x(mu, su, pa, o2[3], o2[4], o2[7]);
        qu = q1;
      }
      const int64_t o = (int64_t)tm * a.ldp + col;
      a.pm_z[o] = mz;
      a.ps_z[o] = sz;
      a.pr_z[o] = pr;
      a.pm_u[o] = mu;
      a.ps_u[o] = su;
      a.pi_u[o] = id;
      a.pq_u[o] = qu;
      a.pa_u[o] = pa;
    }
  }
}

// ============================================================================
// pass 1 with staging: the tile's column maxima are merged across the two
// half-waves and the two wave rows first, then e = exp(z - m_tile) is summed
// for the partials and stored for the backward (rounded to the storage type),
// scaled to the row's reference when one is given: e' = e exp(m_tile - ref) =
// exp(z - ref), unless the tile's max exceeds ref + kStageRange (then e
// itself, so nothing overflows; such rows are rescaled by k_stage_fix), and 0
// on rows whose seed is 0.  With stage_t the values also go out transposed,
// as 16-byte pieces of rows through the LDS-staged row epilogue.
template <typename T, int WNW>
__global__ __launch_bounds__(128 * WNW, 1) void k_stats_stage(StatsStageLaunch a) {
  // four waves: a load every three MFMAs; eight: every MFMA (as the contractions)
  using Cfg = TileCfg<T, 256, 256, (WNW == 2 ? kStatsLoadGap : 1), WNW>;
  constexpr int kRowsSmem = (Cfg::BM / 2) * (Cfg::BN * 4 + 16);  // store_tile_rows staging
  constexpr int kSmem = Cfg::LDS_BYTES > kRowsSmem ? Cfg::LDS_BYTES : kRowsSmem;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  const StatsLaunch& st = a.st;
  int tm, tn;
  if (!tile_of(st.tiles_m, st.tiles_n, kGroupM, tm, tn)) return;

  f32x4_t acc[Cfg::FM][Cfg::FN];
  zero_acc<Cfg>(acc);
  tile_mainloop<T, Cfg>(acc, as_op<T>(st.A), tm * Cfg::BM, as_op<T>(st.B), tn * Cfg::BN,
                        st.k_len, smem);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / Cfg::WNW, wn = wave % Cfg::WNW;
  const int v_base = tm * Cfg::BM + wm * Cfg::WM;
  const bool tail = tm * Cfg::BM + Cfg::BM > st.vocab;
  float* red = reinterpret_cast<float*>(smem);  // [2 wave rows][BN]

  if (tail) mask_vocab_tail<Cfg>(acc, v_base, lane, st.vocab);
  float mj[Cfg::FN];
#pragma unroll
  for (int j = 0; j < Cfg::FN; ++j) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = __builtin_elementwise_maximum(mx, acc[i][j][r]);
    mj[j] = col_max(mx);
    if (lane < kFrag) red[wm * Cfg::BN + wn * Cfg::WN + j * kFrag + lane] = mj[j];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < Cfg::FN; ++j) {
    const int c = wn * Cfg::WN + j * kFrag + frag_col(lane);
    mj[j] = fmaxf(red[c], red[Cfg::BN + c]);
  }

  // the fp32 logit at each row's labels, from the one tile that holds it (the
  // staged bf16 value near 1 would lose the difference q_y - 1)
  if (a.ref) {
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
      const int c = tn * Cfg::BN + wn * Cfg::WN + j * kFrag + frag_col(lane);
      if (c >= st.ncols) continue;
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int32_t* yv = w ? a.y2 : a.y1;
        if (!yv) continue;
        const int y = yv[c];
        if (y < 0 || (y >> 8) != tm) continue;
        const int local = (y & 255) - wm * Cfg::WM;  // row within this wave's rows
        if (local < 0 || local >= Cfg::WM || ((local & 15) >> 2) != (lane >> 4)) continue;
        float z = 0.0f;
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (i == (local >> 4) && r == (local & 3)) z = acc[i][j][r];
        (w ? a.zt2 : a.zt1)[c] = z;
      }
    }
  }

  T* E = static_cast<T*>(a.stage);
  float sj[Cfg::FN];
  static_assert(Cfg::FN % 2 == 0, "column blocks are stored in pairs");
#pragma unroll
  for (int j = 0; j < Cfg::FN; j += 2) {
    // E row = chunk row (this tile's column), contiguous along the vocabulary
    T* e0 = E + (int64_t)(tn * Cfg::BN + wn * Cfg::WN + j * kFrag) * a.ld_stage + v_base;
    const float mb0 = mj[j] * kLog2e, mb1 = mj[j + 1] * kLog2e;
    // staging factors of the two columns: exp(m_tile - ref), 1 or 0
    float f0 = 1.0f, f1 = 1.0f;
    if (a.ref) {
      float fh[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = tn * Cfg::BN + wn * Cfg::WN + (j + h) * kFrag + frag_col(lane);
        const float m = mj[j + h];
        float f = 0.0f;
        if (c < st.ncols && a.seed[c] != 0.0f) {
          const float d = m - a.ref[c];
          f = d > kStageRange ? 1.0f : fast_exp2(d * kLog2e);
        }
        fh[h] = f;
      }
      f0 = fh[0];
      f1 = fh[1];
    }
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
      float e[4], f[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        e[r] = fast_exp2(fmaf(acc[i][j][r], kLog2e, -mb0));
        f[r] = fast_exp2(fmaf(acc[i][j + 1][r], kLog2e, -mb1));
        s0 += e[r];
        s1 += f[r];
        e[r] *= f0;
        f[r] *= f1;
        acc[i][j][r] = e[r];
        acc[i][j + 1][r] = f[r];
      }
      store_frag_pair<T>(e0 + i * kFrag, a.ld_stage, e, f, lane);
    }
    sj[j] = col_sum(s0, lane);
    sj[j + 1] = col_sum(s1, lane);
  }
  __syncthreads();
  if (lane < kFrag) {
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j)
      red[wm * Cfg::BN + wn * Cfg::WN + j * kFrag + lane] = sj[j];
  }
  __syncthreads();
  if (wm == 0 && lane < kFrag) {
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
      const int c = wn * Cfg::WN + j * kFrag + lane;
      const int col = tn * Cfg::BN + c;
      if (col < st.ncols) {
        const int64_t o = (int64_t)tm * st.ldp + col;
        st.pm[o] = mj[j];
        st.ps[o] = red[c] + red[Cfg::BN + c];
      }
    }
  }
  if (a.stage_t) {
    __syncthreads();  // the row epilogue reuses the reduction space
    store_tile_rows<T, Cfg>(acc, static_cast<T*>(a.stage_t), a.ld_stage_t, (int64_t)tm * Cfg::BM,
                            (int64_t)tn * Cfg::BN, smem);
  }
}

// dz^T rows of one (256-entry vocabulary tile, 64 chunk rows) block from
// its LDS copy: row rr of the block holds its 16-byte chunk ch at position
// ch ^ (rr / KC), so the KC-row column reads hit distinct banks.
template <typename T>
__device__ __forceinline__ void store_dzt_block(const char* tile, T* dzt, int64_t ld_dzt, int vt,
                                                int rb) {
  constexpr int VT = kVocabTile, RB = 64;
  constexpr int KC = ElemTraits<T>::kPerChunk;
  constexpr int STRIDE = VT * (int)sizeof(T);
  constexpr int PER_ROW = RB / KC;  // 16-byte pieces per dz^T row segment
  for (int idx = threadIdx.x; idx < VT * PER_ROW; idx += 256) {
    const int v = idx / PER_ROW, q = idx % PER_ROW;
    i32x4_t out;
    const char* col = tile + (((v / KC) ^ q) << 4) + (v % KC) * (int)sizeof(T);
    if constexpr (sizeof(T) == 2) {
      bf16x8_t b;
#pragma unroll
      for (int e = 0; e < KC; ++e)
        b[e] = *reinterpret_cast<const __bf16*>(col + (q * KC + e) * STRIDE);
      out = __builtin_bit_cast(i32x4_t, b);
    } else {
#pragma unroll
      for (int e = 0; e < KC; ++e)
        out[e] = *reinterpret_cast<const int*>(col + (q * KC + e) * STRIDE);
    }
    *reinterpret_cast<i32x4_t*>(dzt + (int64_t)(vt * VT + v) * ld_dzt + rb * RB + q * KC) = out;
  }
}

// dz of the label / argmax cross-entropies from the staged e = exp(z - m_tile),
// one workgroup per (256-wide vocabulary tile, 64 rows): rows are read and
// written back coalesced (16 bytes per lane), and the block is transposed
// through LDS into dz^T.
//   dz = seed ((w_lab + w_arg) e exp(m_tile - lse) - w_lab [v = y_lab] - w_arg [v = y_arg])
template <typename T>
__global__ __launch_bounds__(256) void k_dz_stage(DzStageLaunch a) {
  constexpr int VT = kVocabTile, RB = 64;
  constexpr int KC = ElemTraits<T>::kPerChunk;       // elements per 16 bytes
  constexpr int CPR = VT / KC;                        // 16-byte chunks per row
  // LDS: row rr holds its 16-byte chunk ch at position ch ^ (rr / KC), so the
  // KC-row column reads of the transpose hit distinct banks
  constexpr int STRIDE = VT * (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) char tile[RB * STRIDE];
  const int vt = blockIdx.x % a.tiles_m;
  const int rb = blockIdx.x / a.tiles_m;
  T* dz = static_cast<T*>(a.dz);
  T* dzt = static_cast<T*>(a.dzt);

  constexpr int IT = RB * CPR / 256;  // 16-byte chunks per thread
  static_assert(RB * CPR % 256 == 0, "chunks must split evenly over the block");
  i32x4_t raw[IT];
  // all of this thread's loads first, so they are in flight together
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * 256 + threadIdx.x;
    const int rr = idx / CPR, ch = idx % CPR;
    const int64_t o = (int64_t)(rb * RB + rr) * a.ld_dz + vt * VT + ch * KC;
    raw[it] = *reinterpret_cast<const i32x4_t*>(dz + o);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * 256 + threadIdx.x;
    const int rr = idx / CPR, ch = idx % CPR;
    const int c = rb * RB + rr;                    // chunk row
    const int v0 = vt * VT + ch * KC;
    T* p = dz + (int64_t)c * a.ld_dz + v0;
    float e[KC];
    if constexpr (sizeof(T) == 2) {
      const bf16x8_t b = __builtin_bit_cast(bf16x8_t, raw[it]);
#pragma unroll
      for (int q = 0; q < KC; ++q) e[q] = (float)b[q];
    } else {
#pragma unroll
      for (int q = 0; q < KC; ++q) e[q] = __int_as_float(raw[it][q]);
    }
    float sd = 0.0f, scale = 0.0f;
    int yl = -1, ya = -1;
    if (c < a.ncols) {
      const int64_t gr = a.r0 + c;
      sd = a.seed[gr];
      if (sd != 0.0f) {
        scale = sd * (a.w_lab + a.w_arg) *
                fast_exp2((a.pm[(int64_t)vt * a.ldp + c] - a.sv.lse_q[gr]) * kLog2e);
        yl = a.sv.y_label[gr];
        ya = a.sv.y_arg[gr];
      }
    }
    float d[KC];
#pragma unroll
    for (int q = 0; q < KC; ++q) {
      const int v = v0 + q;
      float x = e[q] * scale;
      if (v == yl) x -= sd * a.w_lab;
      if (v == ya) x -= sd * a.w_arg;
      d[q] = (sd != 0.0f && v < a.vocab) ? x : 0.0f;
    }
    i32x4_t out;
    if constexpr (sizeof(T) == 2) {
      bf16x8_t b;
#pragma unroll
      for (int q = 0; q < KC; ++q) b[q] = (__bf16)d[q];
      out = __builtin_bit_cast(i32x4_t, b);
    } else {
#pragma unroll
      for (int q = 0; q < KC; ++q) out[q] = __float_as_int(d[q]);
    }
    *reinterpret_cast<i32x4_t*>(p) = out;
    if (dzt) *reinterpret_cast<i32x4_t*>(tile + rr * STRIDE + ((ch ^ (rr / KC)) << 4)) = out;
  }
  if (!dzt) return;  // bf16: the dW contraction reads dz itself
  __syncthreads();
  store_dzt_block<T>(tile, dzt, a.ld_dzt, vt, rb);
}

// ============================================================================
// pass 2: divergence sums with the final logsumexps
// ============================================================================
// NEED != 0: the set of sums as a compile-time constant (the common sets),
// so the per-element tests of `need` disappear; NEED == 0 reads a.need.
template <typename T, int WNW, uint32_t NEED = 0>
__global__ __launch_bounds__(128 * WNW, 1) void k_div(DivLaunch a) {
  using Cfg = TileCfg<T, 256, 128, 1, WNW>;
  __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS_BYTES];
  int tm, tn;
  if (!tile_of(a.tiles_m, a.tiles_n, kGroupM, tm, tn)) return;

  f32x4_t az[Cfg::FM][Cfg::FN], au[Cfg::FM][Cfg::FN];
  zero_acc<Cfg>(az);
  zero_acc<Cfg>(au);
  tile_mainloop<T, Cfg>(az, as_op<T>(a.Az), tm * Cfg::BM, as_op<T>(a.Bz), tn * Cfg::BN, a.k_len,
                        smem);
  tile_mainloop<T, Cfg>(au, as_op<T>(a.Au), tm * Cfg::BM, as_op<T>(a.Bu), tn * Cfg::BN, a.k_len,
                        smem);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WNW, wn = wave % WNW;
  const int v_base = tm * Cfg::BM + wm * Cfg::WM;
  const bool tail = tm * Cfg::BM + Cfg::BM > a.vocab;
  const uint32_t need = NEED ? NEED : a.need;

  float sums[Cfg::FN][kNumSums];
#pragma unroll
  for (int j = 0; j < Cfg::FN; ++j) {
    const int c_tile = tn * Cfg::BN + wn * Cfg::WN + j * kFrag + frag_col(lane);  // chunk row
    const int col = min(c_tile, a.ncols - 1);
    const float lq0 = a.lse_q[col], lp0 = a.lse_p[col];
    float s_alpha = 0.f, s_s = 0.f, s_kl = 0.f, s_rkl = 0.f, s_jsd = 0.f, s_eqg = 0.f;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = v_base + i * kFrag + frag_row(r, lane);
        if (tail && v >= a.vocab) continue;
        const float lq = az[i][j][r] - lq0;
        const float lp = au[i][j][r] - lp0;
        const float q = fast_exp2(lq * kLog2e);
        const float p = fast_exp2(lp * kLog2e);
        if (need & SUM_ALPHA) s_alpha += fminf(p, q);
        if (need & SUM_S) s_s += (q < p) ? q : ((q == p) ? 0.5f * q : 0.0f);
        if (need & SUM_KL) s_kl += p * (lp - lq);
        if (need & SUM_RKL) s_rkl += q * (lq - lp);
        if (need & (SUM_JSD | SUM_EQG)) {
          const float lm = log_mixture(p, q);
          if (need & SUM_JSD) s_jsd += 0.5f * (p * (lp - lm) + q * (lq - lm));
          if (need & SUM_EQG) s_eqg += 0.5f * q * (lq - lm);
        }
      }
    }
    const float v6[kNumSums] = {s_alpha, s_s, s_kl, s_rkl, s_jsd, s_eqg};
#pragma unroll
    for (int f = 0; f < kNumSums; ++f) sums[j][f] = col_sum(v6[f], lane);
  }

  float* red = reinterpret_cast<float*>(smem);  // [BN][kNumSums]
  if (wm == 1 && lane < kFrag) {
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
      const int c = wn * Cfg::WN + j * kFrag + lane;
#pragma unroll
      for (int f = 0; f < kNumSums; ++f) red[c * kNumSums + f] = sums[j][f];
    }
  }
  __syncthreads();
  if (wm == 0 && lane < kFrag) {
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
      const int c = wn * Cfg::WN + j * kFrag + lane;
      const int col = tn * Cfg::BN + c;
      if (col >= a.ncols) continue;
#pragma unroll
      for (int f = 0; f < kNumSums; ++f)
        if (need & (1u << f))
          a.part[f * a.part_stride + (int64_t)tm * a.ldp + col] = sums[j][f] + red[c * kNumSums + f];
    }
  }
}

// Pass 2 for aligned heads: a tile covers 256 vocabulary rows and 64 target
// rows, and the target tile u is computed once for the K draft rows each
// target row serves.  The draft tile has 64 K columns ordered so that wave
// column wn holds, for each head k, the same 32 target rows as its u
// columns: z column wn * 32 K + k * 32 + jj pairs with u column wn * 32 + jj
// (the map puts the matching draft row there).  Per (vocabulary row, draft
// row) the arithmetic is that of k_div, in the same order, so the sums are
// the same bits.
template <typename T, int K, uint32_t NEED = 0>
__global__ __launch_bounds__(kThreads, 1) void k_div_heads(DivHeadsLaunch h) {
  using CfgZ = TileCfg<T, 256, 64 * K>;
  using CfgU = TileCfg<T, 256, 64>;
  constexpr int kSmem = CfgZ::LDS_BYTES > CfgU::LDS_BYTES ? CfgZ::LDS_BYTES : CfgU::LDS_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  const DivLaunch& a = h.d;
  int tm, tn;
  if (!tile_of(a.tiles_m, a.tiles_n, kGroupM, tm, tn)) return;

  f32x4_t az[CfgZ::FM][CfgZ::FN], au[CfgU::FM][CfgU::FN];
  zero_acc<CfgZ>(az);
  zero_acc<CfgU>(au);
  tile_mainloop<T, CfgZ>(az, as_op<T>(a.Az), tm * CfgZ::BM, as_op<T>(a.Bz), tn * CfgZ::BN,
                         a.k_len, smem);
  tile_mainloop<T, CfgU>(au, as_op<T>(a.Au), tm * CfgU::BM, as_op<T>(a.Bu), tn * CfgU::BN,
                         a.k_len, smem);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int v_base = tm * CfgU::BM + wm * CfgU::WM;
  const bool tail = tm * CfgU::BM + CfgU::BM > a.vocab;
  const uint32_t need = NEED ? NEED : a.need;  // as in k_div
  static_assert(CfgU::FN == 2 && CfgZ::FN == 2 * K && CfgU::WN == 32, "heads tile layout");

  // per (head, u fragment column): chunk row or -1, and the six sums
  float sums[K][CfgU::FN][kNumSums];
  int crow[K][CfgU::FN];
#pragma unroll
  for (int j = 0; j < CfgU::FN; ++j) {
    const int64_t tj = h.jlo + tn * 64 + wn * CfgU::WN + j * kFrag + frag_col(lane);  // target row
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int64_t lr = (tj - h.shifts[k]) * K + k - h.r0;  // chunk row of head k
      const bool ok = tj - h.shifts[k] >= 0 && lr >= 0 && lr < h.rows;
      crow[k][j] = ok ? (int)lr : -1;
      const int col = ok ? (int)lr : 0;
      const float lq0 = a.lse_q[col], lp0 = a.lse_p[col];
      float s_alpha = 0.f, s_s = 0.f, s_kl = 0.f, s_rkl = 0.f, s_jsd = 0.f, s_eqg = 0.f;
#pragma unroll
      for (int i = 0; i < CfgU::FM; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int v = v_base + i * kFrag + frag_row(r, lane);
          if (tail && v >= a.vocab) continue;
          const float lq = az[i][k * CfgU::FN + j][r] - lq0;
          const float lp = au[i][j][r] - lp0;
          const float q = fast_exp2(lq * kLog2e);
          const float p = fast_exp2(lp * kLog2e);
          if (need & SUM_ALPHA) s_alpha += fminf(p, q);
          if (need & SUM_S) s_s += (q < p) ? q : ((q == p) ? 0.5f * q : 0.0f);
          if (need & SUM_KL) s_kl += p * (lp - lq);
          if (need & SUM_RKL) s_rkl += q * (lq - lp);
          if (need & (SUM_JSD | SUM_EQG)) {
            const float lm = log_mixture(p, q);
            if (need & SUM_JSD) s_jsd += 0.5f * (p * (lp - lm) + q * (lq - lm));
            if (need & SUM_EQG) s_eqg += 0.5f * q * (lq - lm);
          }
        }
      }
      const float v6[kNumSums] = {s_alpha, s_s, s_kl, s_rkl, s_jsd, s_eqg};
#pragma unroll
      for (int f = 0; f < kNumSums; ++f) sums[k][j][f] = col_sum(v6[f], lane);
    }
  }

  // the two wave rows (wm) share target columns: wm = 1 hands its sums over
  float* red = reinterpret_cast<float*>(smem);  // [K][64][kNumSums]
  if (wm == 1 && lane < kFrag) {
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
      for (int j = 0; j < CfgU::FN; ++j) {
        const int c = wn * CfgU::WN + j * kFrag + lane;
#pragma unroll
        for (int f = 0; f < kNumSums; ++f) red[(k * 64 + c) * kNumSums + f] = sums[k][j][f];
      }
  }
  __syncthreads();
  if (wm == 0 && lane < kFrag) {
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
      for (int j = 0; j < CfgU::FN; ++j) {
        const int c = wn * CfgU::WN + j * kFrag + lane;
        const int col = crow[k][j];
        if (col < 0) continue;
#pragma unroll
        for (int f = 0; f < kNumSums; ++f)
          if (need & (1u << f))
            a.part[f * a.part_stride + (int64_t)tm * a.ldp + col] =
                sums[k][j][f] + red[(k * 64 + c) * kNumSums + f];
      }
  }
}

// Draft rows of the heads tiles: entry tn * 64 K + r is the chunk row of z
// tile row r of tile column tn (clamped into the chunk; rows outside it are
// discarded by the kernel).
__global__ __launch_bounds__(256) void k_heads_map(int32_t* map, int32_t tiles_n, int32_t K,
                                                   ShiftArg sh, int64_t jlo, int64_t r0,
                                                   int32_t rows) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n = (int64_t)tiles_n * 64 * K;
  if (idx >= n) return;
  const int tn = (int)(idx / (64 * K)), r = (int)(idx % (64 * K));
  const int wn = r / (32 * K), k = (r % (32 * K)) / 32, jj = r % 32;
  const int64_t tj = jlo + (int64_t)tn * 64 + wn * 32 + jj;
  int64_t lr = (tj - sh.v[k]) * K + k - r0;
  if (tj - sh.v[k] < 0 || lr < 0) lr = 0;
  if (lr >= rows) lr = rows - 1;
  map[idx] = (int32_t)lr;
}

// ============================================================================
// pass 2 and the logit gradient from raw logits (single call, divergences)
// ============================================================================
// Pass 1 of the single call keeps both raw fp32 logit rows of the chunk
// (z: draft, u: target), so the second sweep and the logit gradient are
// memory passes over them instead of two recomputed contractions.

__device__ __forceinline__ int raw_urow(const RawRows& r, int c) {
  if (!r.urow) return c;
  const int64_t x = (int64_t)r.urow[c] - r.ushift;
  return (int)(x < 0 ? 0 : (x >= r.n_u ? r.n_u - 1 : x));
}

// Sum of the eight lanes of a row (lanes 8 k .. 8 k + 7, lane 8 k + 4 h + g):
// (g0 + g1) + (g2 + g3) within each h, then h0 + h1, the lower lane first at
// each level, so every lane ends with the same value.
__device__ __forceinline__ float row8_sum(float x, int lane) {
#pragma unroll
  for (int m = 1; m < 8; m <<= 1) {
    const float o = __shfl_xor(x, m);
    x = (lane & m) ? o + x : x + o;
  }
  return x;
}

// One workgroup per (256-entry vocabulary tile, 64 chunk rows), eight lanes
// per row.  Lane (h, g) of a row sums the 32 entries h 128 + i 16 + 4 g + r
// (i < 8, r < 4) in that order (eight 16-byte loads per side), and the eight
// partials meet in row8_sum: the order in which k_div forms the same sums
// from its accumulators (a wave row h, lane group g, fragments i, registers
// r, then col_sum and the two wave rows), so both second sweeps give the same
// bits.  The element terms are those of k_div (speculators "Available
// Losses" rows).
template <uint32_t NEED = 0>
__global__ __launch_bounds__(256) void k_div_raw(DivRawLaunch a) {
  const int vt = blockIdx.x % a.tiles_m;
  const int rb = blockIdx.x / a.tiles_m;
  const int lane = threadIdx.x & 63;
  const int sub = lane & 7, g = sub & 3, hh = sub >> 2;
  const uint32_t need = NEED ? NEED : a.need;
  const int vb = vt * kVocabTile + hh * 128 + 4 * g;  // entry (i, r): vb + 16 i + r
  const bool tail = (vt + 1) * kVocabTile > a.vocab;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int c = rb * 64 + it * 32 + (threadIdx.x >> 3);  // chunk row of this lane's group
    const int cc = c < a.ncols ? c : a.ncols - 1;
    const float* zr = a.r.z + (int64_t)cc * a.r.ld_z + vb;
    const float* ur = a.r.u + (int64_t)raw_urow(a.r, cc) * a.r.ld_u + vb;
    f32x4_t zz[8], uu[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      zz[i] = *reinterpret_cast<const f32x4_t*>(zr + 16 * i);
      uu[i] = *reinterpret_cast<const f32x4_t*>(ur + 16 * i);
    }
    const float lq0 = a.lse_q[cc], lp0 = a.lse_p[cc];
    float s_alpha = 0.f, s_s = 0.f, s_kl = 0.f, s_rkl = 0.f, s_jsd = 0.f, s_eqg = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (tail && vb + 16 * i + r >= a.vocab) continue;
        const float lq = zz[i][r] - lq0;
        const float lp = uu[i][r] - lp0;
        const float q = fast_exp2(lq * kLog2e);
        const float p = fast_exp2(lp * kLog2e);
        if (need & SUM_ALPHA) s_alpha += fminf(p, q);
        if (need & SUM_S) s_s += (q < p) ? q : ((q == p) ? 0.5f * q : 0.0f);
        if (need & SUM_KL) s_kl += p * (lp - lq);
        if (need & SUM_RKL) s_rkl += q * (lq - lp);
        if (need & (SUM_JSD | SUM_EQG)) {
          const float lm = log_mixture(p, q);
          if (need & SUM_JSD) s_jsd += 0.5f * (p * (lp - lm) + q * (lq - lm));
          if (need & SUM_EQG) s_eqg += 0.5f * q * (lq - lm);
        }
      }
    const float v6[kNumSums] = {s_alpha, s_s, s_kl, s_rkl, s_jsd, s_eqg};
#pragma unroll
    for (int f = 0; f < kNumSums; ++f) {
      if (!(need & (1u << f))) continue;
      const float x = row8_sum(v6[f], lane);
      if (sub == 0 && c < a.ncols) a.part[f * a.part_stride + (int64_t)vt * a.ldp + c] = x;
    }
  }
}

// dz from raw logits (the formula at DzRawLaunch), one workgroup per
// (256-entry vocabulary tile, 64 chunk rows): q, d = q - p and l = log q -
// log p formed in fp32 (and c = [q < p] from the sign of that d, as the S
// sums of k_div_raw decide it).  The block is written row-major and,
// transposed through LDS, into dz^T.
template <typename T, bool LOG>
__global__ __launch_bounds__(256) void k_dz_raw(DzRawLaunch a) {
  constexpr int VT = kVocabTile, RB = 64;
  constexpr int KC = ElemTraits<T>::kPerChunk;  // output values per 16 bytes
  constexpr int CPR = VT / KC;
  constexpr int NL = KC / 4;                    // 16-byte fp32 loads per chunk and side
  constexpr int STRIDE = VT * (int)sizeof(T);
  constexpr int IT = RB * CPR / 256;
  static_assert(RB * CPR % 256 == 0, "chunks must split evenly over the block");
  __shared__ __attribute__((aligned(16))) char tile[RB * STRIDE];
  const int vt = blockIdx.x % a.tiles_m;
  const int rb = blockIdx.x / a.tiles_m;
  T* dz = static_cast<T*>(a.dz);
  T* dzt = static_cast<T*>(a.dzt);

  f32x4_t zz[IT][NL], uu[IT][NL];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * 256 + threadIdx.x;
    const int rr = idx / CPR, ch = idx % CPR;
    const int c = rb * RB + rr;
    const int cc = c < a.ncols ? c : a.ncols - 1;
    const float* zr = a.r.z + (int64_t)cc * a.r.ld_z + vt * VT + ch * KC;
    const float* ur = a.r.u + (int64_t)raw_urow(a.r, cc) * a.r.ld_u + vt * VT + ch * KC;
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      zz[it][l] = *reinterpret_cast<const f32x4_t*>(zr + 4 * l);
      uu[it][l] = *reinterpret_cast<const f32x4_t*>(ur + 4 * l);
    }
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * 256 + threadIdx.x;
    const int rr = idx / CPR, ch = idx % CPR;
    const int c = rb * RB + rr;
    const int v0 = vt * VT + ch * KC;
    float sd = 0.0f, scale = 0.0f, cb = 0.0f, cc = 0.0f, S = 0.0f;
    float cr = 0.0f, cj = 0.0f, rkl = 0.0f, eqg = 0.0f, lq0 = 0.0f, lp0 = 0.0f;
    int yl = -1, ya = -1;
    if (c < a.ncols) {
      const int64_t gr = a.r0 + c;
      sd = a.seed[gr];
      if (sd != 0.0f) {
        const float alpha = a.sv.alpha[gr];
        const float lam = __expf(-3.0f * alpha);
        scale = sd * (a.w_lab + a.w_arg);
        cb = sd * (a.w_kl + a.w_lk * lam);
        cc = sd * (a.w_tv + (a.w_nla != 0.0f ? a.w_nla / alpha : 0.0f) + a.w_lk * (1.0f - lam));
        S = a.sv.S[gr];
        if (LOG) {
          cr = sd * a.w_rkl;
          cj = sd * a.w_jsd;
          rkl = a.sv.rkl[gr];
          eqg = a.sv.eqg[gr];
        }
        yl = a.sv.y_label[gr];
        ya = a.sv.y_arg[gr];
        lq0 = a.sv.lse_q[gr];
        lp0 = a.sv.lse_p[gr];
      }
    }
    float d[KC];
#pragma unroll
    for (int q = 0; q < KC; ++q) {
      const int v = v0 + q;
      const float lq = zz[it][q / 4][q % 4] - lq0;
      const float lp = uu[it][q / 4][q % 4] - lp0;
      const float qq = fast_exp2(lq * kLog2e);
      const float pp = fast_exp2(lp * kLog2e);
      const float dd = qq - pp;
      const float ci = dd < 0.0f ? 1.0f : (dd == 0.0f ? 0.5f : 0.0f);
      float x = fmaf(cb, dd, qq * scale) - cc * qq * (ci - S);
      if (LOG) {
        // softplus(-l) = max(-l, 0) + log(1 + exp(-|l|))
        const float l = lq - lp;
        const float sp = fmaxf(-l, 0.0f) + fast_log2(1.0f + fast_exp2(-fabsf(l) * kLog2e)) * kLn2;
        const float g = 0.5f * (kLn2 - sp);
        x += qq * (cr * (l - rkl) + cj * (g - eqg));
      }
      if (v == yl) x -= sd * a.w_lab;
      if (v == ya) x -= sd * a.w_arg;
      d[q] = (sd != 0.0f && v < a.vocab) ? x : 0.0f;
    }
    i32x4_t out;
    if constexpr (sizeof(T) == 2) {
      bf16x8_t b;
#pragma unroll
      for (int q = 0; q < KC; ++q) b[q] = (__bf16)d[q];
      out = __builtin_bit_cast(i32x4_t, b);
    } else {
#pragma unroll
      for (int q = 0; q < KC; ++q) out[q] = __float_as_int(d[q]);
    }
    *reinterpret_cast<i32x4_t*>(dz + (int64_t)c * a.ld_dz + v0) = out;
    if (dzt) *reinterpret_cast<i32x4_t*>(tile + rr * STRIDE + ((ch ^ (rr / KC)) << 4)) = out;
  }
  if (!dzt) return;
  __syncthreads();
  store_dzt_block<T>(tile, dzt, a.ld_dzt, vt, rb);
}

// ============================================================================
// backward recompute: logit gradient tile -> staged chunk (two layouts)
// ============================================================================
struct RowCoef {
  float seed, lse_q, lse_p, alpha, S, rkl, eqg, lam;
  int y_lab, y_arg;
};

template <bool DUAL>
__device__ __forceinline__ float dz_elem(const RowCoef& c, const float* w, float z, float u,
                                         int v) {
  const float lq = z - c.lse_q;
  const float q = fast_exp2(lq * kLog2e);
  float g = 0.0f;
  if (w[0] != 0.0f) g += w[0] * (q - (v == c.y_lab ? 1.0f : 0.0f));
  if (w[1] != 0.0f) g += w[1] * (q - (v == c.y_arg ? 1.0f : 0.0f));
  if (DUAL) {
    const float lp = u - c.lse_p;
    const float p = fast_exp2(lp * kLog2e);
    if (w[2] != 0.0f) g += w[2] * (q - p);
    if (w[3] != 0.0f) g += w[3] * q * (lq - lp - c.rkl);
    if (w[4] != 0.0f) {
      const float lm = log_mixture(p, q);
      g += w[4] * q * (0.5f * (lq - lm) - c.eqg);
    }
    if (w[5] != 0.0f || w[6] != 0.0f || w[7] != 0.0f) {
      const float cc = (q < p) ? 1.0f : ((q == p) ? 0.5f : 0.0f);
      const float tv = -q * (cc - c.S);
      if (w[5] != 0.0f) g += w[5] * tv;
      if (w[6] != 0.0f) g += w[6] * tv / c.alpha;
      if (w[7] != 0.0f) g += w[7] * (c.lam * (q - p) + (1.0f - c.lam) * tv);
    }
  }
  return g;
}

template <typename T, bool DUAL, int WNW = 2>
__global__ __launch_bounds__(128 * WNW, 1) void k_dz(DzLaunch a) {
  using Cfg = TileCfg<T, 256, (DUAL ? 128 : 256), 1, WNW>;
  constexpr int kRowsSmem = (Cfg::BM / 2) * (Cfg::BN * 4 + 16);  // store_tile_rows staging
  constexpr int kSmem = Cfg::LDS_BYTES > kRowsSmem ? Cfg::LDS_BYTES : kRowsSmem;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  int tm, tn;
  if (!tile_of(a.tiles_m, a.tiles_n, kGroupM, tm, tn)) return;

  f32x4_t az[Cfg::FM][Cfg::FN];
  f32x4_t au[DUAL ? Cfg::FM : 1][DUAL ? Cfg::FN : 1];
  zero_acc<Cfg>(az);
  tile_mainloop<T, Cfg>(az, as_op<T>(a.Az), tm * Cfg::BM, as_op<T>(a.Bz), tn * Cfg::BN, a.k_len,
                        smem);
  if constexpr (DUAL) {
    zero_acc<Cfg>(au);
    tile_mainloop<T, Cfg>(au, as_op<T>(a.Au), tm * Cfg::BM, as_op<T>(a.Bu), tn * Cfg::BN,
                          a.k_len, smem);
  }

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WNW, wn = wave % WNW;
  const int v_base = tm * Cfg::BM + wm * Cfg::WM;
  T* dz = static_cast<T*>(a.dz);
  T* dzt = static_cast<T*>(a.dzt);

  // dz rows (chunk row, contiguous along the vocabulary): column blocks j,
  // j + 1 go out together as 16-byte pieces; the values replace the
  // accumulators for the dz^T epilogue
  static_assert(Cfg::FN % 2 == 0, "column blocks are stored in pairs");
#pragma unroll
  for (int j = 0; j < Cfg::FN; j += 2) {
    RowCoef rc[2];
    bool live[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = tn * Cfg::BN + wn * Cfg::WN + (j + h) * kFrag + frag_col(lane);  // chunk row
      const int64_t gr = a.r0 + min(c, a.ncols - 1);
      rc[h].seed = (c < a.ncols) ? a.seed[gr] : 0.0f;
      rc[h].lse_q = a.sv.lse_q[gr];
      rc[h].y_lab = a.sv.y_label[gr] >= 0 ? a.sv.y_label[gr] - a.vocab_offset : -1;
      rc[h].y_arg = a.sv.y_arg[gr] >= 0 ? a.sv.y_arg[gr] - a.vocab_offset : -1;
      if (DUAL) {
        rc[h].lse_p = a.sv.lse_p[gr];
        rc[h].alpha = a.sv.alpha[gr];
        rc[h].S = a.sv.S[gr];
        rc[h].rkl = a.sv.rkl[gr];
        rc[h].eqg = a.sv.eqg[gr];
        rc[h].lam = __expf(-3.0f * rc[h].alpha);
      }
      live[h] = rc[h].seed != 0.0f;
    }
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
      float o[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int v = v_base + i * kFrag + frag_row(r, lane);
          float d = 0.0f;
          if (live[h] && v < a.vocab) {
            const float u = DUAL ? au[DUAL ? i : 0][DUAL ? j + h : 0][r] : 0.0f;
            d = rc[h].seed * dz_elem<DUAL>(rc[h], a.w, az[i][j + h][r], u, v);
          }
          o[h][r] = d;
          az[i][j + h][r] = d;
        }
      store_frag_pair<T>(dz + (int64_t)(tn * Cfg::BN + wn * Cfg::WN + j * kFrag) * a.ld_dz + v_base +
                             i * kFrag,
                         a.ld_dz, o[0], o[1], lane);
    }
  }
  // dz^T rows (vocabulary entry, contiguous along the chunk rows)
  if (dzt)
    store_tile_rows<T, Cfg>(az, dzt, a.ld_dzt, (int64_t)tm * Cfg::BM, (int64_t)tn * Cfg::BN, smem);
}

// ============================================================================
// plain contraction with store / accumulate epilogue
// ============================================================================
// ROLE 0: dh = dz W, A = dz, B = W^T; ROLE 1: dW = dz^T h, A = dz^T, B = h^T,
// all K-major (transposed copies).  LEAN (bf16 only): no copies; dh reads W
// as an MN-major B (its rows are k), dW reads dz and the hidden chunk as
// MN-major A and B.
//
// DUMP (dh, bf16): the contraction also writes A's transpose (dz^T, from dz)
// as it streams A's slabs through LDS; each workgroup writes the slabs whose
// index equals its tile column modulo the tile columns, so every slab of
// every row tile goes out once (tile_gemm.hpp, SlabDump).
//
// Epilogue: the tile goes out in two halves of 128 rows.  The two waves that
// own a half write their accumulators into LDS (rows padded to 1040 bytes so
// the four row groups of a store land in different banks); then all threads
// stream the half's rows: 16-byte loads of the old values (accumulate), add,
// 16-byte stores, eight pieces in flight per thread.  fp32 outputs are read
// and written nontemporally: the next touch of a dW row is a whole chunk
// later, and cached dW lines would only displace the operand slabs that the
// other tiles of a round re-read (measured: gemm_dW 2.6 % faster).
constexpr int kHalfRows = 128;
constexpr int kEpiStride = 256 * 4 + 16;  // bytes per staged row

template <typename T, typename OutT, int ROLE, bool LEAN, int WNW, bool DUMP = false>
__global__ __launch_bounds__(128 * WNW, 1) void k_gemm(GemmLaunch a) {
  using Cfg = TileCfg<T, 256, 256, 1, WNW>;
  constexpr bool kA_MN = LEAN && ROLE == 1;
  constexpr bool kB_MN = LEAN;
  constexpr int kSmem = Cfg::LDS_BYTES > kHalfRows * kEpiStride ? Cfg::LDS_BYTES
                                                               : kHalfRows * kEpiStride;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  int tm, tn;
  if (!tile_of(a.tiles_m * a.splits, a.tiles_n, kGroupM, tm, tn)) return;
  // split-K slice of this tile row: its K range and its partial output
  const int split = tm / a.tiles_m;
  tm -= split * a.tiles_m;
  Operand<T> opA = as_op<T>(a.A), opB = as_op<T>(a.B);
  int32_t k_len = a.k_len;
  OutT* C = static_cast<OutT*>(a.C);
  if (split > 0) {
    const int64_t k0 = (int64_t)split * a.k_split;
    if (kA_MN) {
      opA.base += k0 * opA.ld;
      opA.k_valid -= (int32_t)k0;
    } else {
      opA.base += k0;
    }
    if (kB_MN) {
      opB.base += k0 * opB.ld;
      opB.k_valid -= (int32_t)k0;
    } else {
      opB.base += k0;
    }
    k_len -= (int32_t)k0;
    C += split * a.part_stride;
  }
  if (a.splits > 1 && k_len > a.k_split) k_len = a.k_split;
  f32x4_t acc[Cfg::FM][Cfg::FN];
  zero_acc<Cfg>(acc);
  if constexpr (DUMP) {
    static_assert(ROLE == 0 && !kA_MN && sizeof(T) == 2, "A's transpose: dh, bf16, K-major A");
    SlabDump D;
    D.out = static_cast<bf16_bits*>(a.at_out);
    D.ld = a.ld_at;
    D.col0 = tm * Cfg::BM;
    D.n_valid = a.m_valid - tm * Cfg::BM;
    D.every = a.tiles_n;
    D.phase = tn;
    D.slab0 = split * (a.k_split / Cfg::BK);
    tile_mainloop<T, Cfg, kA_MN, kB_MN, true>(acc, opA, tm * Cfg::BM, opB, tn * Cfg::BN, k_len,
                                              smem, &D);
  } else {
    tile_mainloop<T, Cfg, kA_MN, kB_MN>(acc, opA, tm * Cfg::BM, opB, tn * Cfg::BN, k_len, smem);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / Cfg::WNW, wn = wave % Cfg::WNW;
  constexpr int kPieces = kHalfRows * 64;              // 16-byte pieces (4 values) per half
  constexpr int kPerThread = kPieces / Cfg::THREADS;
  constexpr int kBatch = 8;
#pragma unroll 1
  for (int h = 0; h < 2; ++h) {
    if (wm == h) {
#pragma unroll
      for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = i * kFrag + frag_row(r, lane);
            const int col = wn * Cfg::WN + j * kFrag + frag_col(lane);
            *reinterpret_cast<float*>(smem + row * kEpiStride + col * 4) = acc[i][j][r];
          }
    }
    __syncthreads();
#pragma unroll 1
    for (int b0 = 0; b0 < kPerThread; b0 += kBatch) {
      f32x4_t old[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int piece = (b0 + q) * Cfg::THREADS + threadIdx.x;
        const int row = piece >> 6, c4 = (piece & 63) * 4;
        const int grow = tm * Cfg::BM + h * kHalfRows + row, gcol = tn * Cfg::BN + c4;
        old[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (a.accumulate && grow < a.m_valid && gcol < a.n_valid) {
          const OutT* p = C + (int64_t)grow * a.ldc + gcol;
          if constexpr (sizeof(OutT) == 4) {
            old[q] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
          } else {
            const bf16x4_t v = *reinterpret_cast<const bf16x4_t*>(p);
            old[q] = f32x4_t{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
          }
        }
      }
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int piece = (b0 + q) * Cfg::THREADS + threadIdx.x;
        const int row = piece >> 6, c4 = (piece & 63) * 4;
        const int grow = tm * Cfg::BM + h * kHalfRows + row, gcol = tn * Cfg::BN + c4;
        if (grow >= a.m_valid || gcol >= a.n_valid) continue;
        f32x4_t x = *reinterpret_cast<const f32x4_t*>(smem + row * kEpiStride + c4 * 4);
        if (a.rscale) x *= a.rscale[grow];
        x += old[q];
        OutT* p = C + (int64_t)grow * a.ldc + gcol;
        if constexpr (sizeof(OutT) == 4) __builtin_nontemporal_store(x, reinterpret_cast<f32x4_t*>(p));
        else store4<bf16_bits>(reinterpret_cast<bf16_bits*>(p), x[0], x[1], x[2], x[3]);
      }
    }
    __syncthreads();
  }
}

// ============================================================================
// row kernels
// ============================================================================
__global__ __launch_bounds__(1024) void k_validity(ValidityLaunch a) {
  __shared__ int64_t red[2][1024];
  int64_t nv = 0, nb = 0;
  for (int64_t r = threadIdx.x; r < a.n; r += 1024) {
    int valid = a.mask ? (a.mask[r] != 0) : 1;
    int bad = 0;
    int lab = -1;
    if (a.use_labels) {
      lab = a.labels[r];
      if (lab == -100) {
        valid = 0;
      } else if (lab < 0 || lab >= a.vocab) {
        bad = valid;
        valid = 0;
      }
    }
    if (a.use_target && a.target_row) {
      const int tr = a.target_row[r];
      const bool off_layout =
          a.n_heads > 0 && (int64_t)tr != r / a.n_heads + a.shifts[r % a.n_heads];
      if (tr < 0 || tr >= a.n_target || off_layout) {
        bad |= valid;
        valid = 0;
      }
    }
    a.flags[r] = valid;
    a.y_label[r] = (a.use_labels && valid) ? lab : -1;
    nv += valid;
    nb += bad;
  }
  red[0][threadIdx.x] = nv;
  red[1][threadIdx.x] = nb;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      red[0][threadIdx.x] += red[0][threadIdx.x + o];
      red[1][threadIdx.x] += red[1][threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    a.counts[0] = red[0][0];
    a.counts[1] = red[1][0];
  }
}

// one wave per row: z_y = W[y] . h[row] in fp32, fixed lane/tree order
template <typename T>
__global__ __launch_bounds__(256) void k_rowdot(RowdotLaunch a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.ncols) return;
  const T* h = static_cast<const T*>(a.h) + (int64_t)row * a.H;
  const T* W = static_cast<const T*>(a.W);
  constexpr int KC = ElemTraits<T>::kPerChunk;
  for (int which = 0; which < 2; ++which) {
    const int32_t* y = which ? a.y2 : a.y1;
    float* out = which ? a.out2 : a.out1;
    if (!y) continue;
    const int lab = y[row] >= 0 ? y[row] - a.vocab_offset : -1;
    const bool ok = lab >= 0 && lab < a.vocab;
    float acc = 0.0f;
    if (ok) {
      const T* wr = W + (int64_t)lab * a.H;
      for (int64_t k = (int64_t)lane * KC; k < a.H; k += 64 * KC) {
        const i32x4_t hv = *reinterpret_cast<const i32x4_t*>(h + k);
        const i32x4_t wv = *reinterpret_cast<const i32x4_t*>(wr + k);
        if constexpr (sizeof(T) == 2) {
          const bf16x8_t hb = __builtin_bit_cast(bf16x8_t, hv);
          const bf16x8_t wb = __builtin_bit_cast(bf16x8_t, wv);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc = fmaf((float)hb[e], (float)wb[e], acc);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = fmaf(__int_as_float(hv[e]), __int_as_float(wv[e]), acc);
        }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) out[row] = ok ? acc : a.outside;
  }
}

// One workgroup per 32 rows; the 8 threads of a row each merge a contiguous
// segment of vocabulary tiles (max pass, then sum pass), then the segments
// are merged in order.  The argmax keeps the first tile holding the maximum,
// i.e. the lowest vocabulary index.
// pq (may be null): per-tile sums of e^2, merged into q the same way
// k_combine1: 32 rows per block, each row's vocabulary tiles split over
// kCombine1Threads / 32 segments (merged in segment order)
constexpr int kCombine1Threads = 1024;

// px (may be null): per-tile sums relative to the tile maximum, merged into x
// as s is
__device__ __forceinline__ void seg_lse(const float* pm, const float* ps, const float* pq,
                                        const float* px, int64_t ldp, int c, int t0, int t1,
                                        float& m, float& s, float& q, float& x, int& best) {
  m = -INFINITY;
  best = -1;
  for (int t = t0; t < t1; ++t) {
    const float v = pm[(int64_t)t * ldp + c];
    if (v > m) { m = v; best = t; }
  }
  s = 0.0f;
  q = 0.0f;
  x = 0.0f;
  if (m != -INFINITY)
    for (int t = t0; t < t1; ++t) {
      const int64_t o = (int64_t)t * ldp + c;
      const float f = fast_exp2((pm[o] - m) * kLog2e);
      s += ps[o] * f;
      if (pq) q += pq[o] * f * f;
      if (px) x += px[o] * f;
    }
}

__global__ __launch_bounds__(kCombine1Threads) void k_combine1(Combine1Launch a) {
  constexpr int SEG = kCombine1Threads / 32, RPB = 32;
  __shared__ float sm[2][SEG][RPB], ss[2][SEG][RPB], sx[2][SEG][RPB], sq[SEG][RPB];
  __shared__ int sb[SEG][RPB];
  const int rr = threadIdx.x % RPB, seg = threadIdx.x / RPB;
  const int c = blockIdx.x * RPB + rr;
  const int per = (a.tiles_m + SEG - 1) / SEG;
  const int t0 = min(a.tiles_m, seg * per), t1 = min(a.tiles_m, t0 + per);
  const bool ratio = a.pa_u != nullptr;  // log-ratio partials of the dual pass 1
  if (c < a.ncols) {
    float m, s, q, x;
    int best;
    if (a.pm_z) {
      seg_lse(a.pm_z, a.ps_z, nullptr, a.pr_z, a.ldp, c, t0, t1, m, s, q, x, best);
      sm[0][seg][rr] = m;
      ss[0][seg][rr] = s;
      sx[0][seg][rr] = x;
    }
    if (a.pm_u) {
      seg_lse(a.pm_u, a.ps_u, a.pq_u, a.pa_u, a.ldp, c, t0, t1, m, s, q, x, best);
      sm[1][seg][rr] = m;
      ss[1][seg][rr] = s;
      sx[1][seg][rr] = x;
      sq[seg][rr] = q;
      sb[seg][rr] = best;
    }
  }
  __syncthreads();
  if (seg != 0 || c >= a.ncols) return;
  float lse_side[2] = {0.0f, 0.0f}, ex_side[2] = {0.0f, 0.0f};
  for (int side = a.pm_z ? 0 : 1; side < (a.pm_u ? 2 : 1); ++side) {
    float m = -INFINITY;
    int bseg = 0;
    for (int g = 0; g < SEG; ++g)
      if (sm[side][g][rr] > m) { m = sm[side][g][rr]; bseg = g; }
    float s = 0.0f, q = 0.0f, x = 0.0f;
    for (int g = 0; g < SEG; ++g)
      if (sm[side][g][rr] != -INFINITY) {
        const float f = fast_exp2((sm[side][g][rr] - m) * kLog2e);
        s += ss[side][g][rr] * f;
        if (ratio) x += sx[side][g][rr] * f;
        if (side == 1) q += sq[g][rr] * f * f;
      }
    // expectation of the side's log-ratio under its own distribution:
    // E_q[z - u] (side 0), E_p[u - z] (side 1)
    if (ratio) ex_side[side] = x / s;
    const int bt_best = side == 1 ? sb[bseg][rr] : -1;
    if (a.raw_m[0]) {
      // a vocabulary shard's record: the merged partials themselves
      a.raw_m[side][c] = m;
      a.raw_s[side][c] = s;
      if (side == 1) {
        a.raw_q2[c] = q;
        a.raw_idx[c] = bt_best >= 0 ? a.pi_u[(int64_t)bt_best * a.ldp + c] + a.idx_offset : -1;
      }
      continue;
    }
    const float lse = m + logf(s);
    lse_side[side] = lse;
    if (side == 0) {
      a.lse_q[c] = lse;
      if (a.row_max) a.row_max[c] = m;
    } else {
      a.lse_p[c] = lse;
      const int bt = sb[bseg][rr];  // -1 only when no tile has a finite maximum
      a.y_arg[c] = bt >= 0 ? a.pi_u[(int64_t)bt * a.ldp + c] : -1;
      // cos(p, uniform) = sum p / (sqrt(V) |p|) = s / (sqrt(V q)), with p = e / s
      a.flat[c] = (bt >= 0 && (!a.flags || a.flags[c])) ? s / sqrtf((float)a.vocab * q) : 0.0f;
    }
  }
  if (a.target_absent && !a.raw_m[0]) {
    a.lse_p[c] = 0.0f;
    a.y_arg[c] = -1;
    a.flat[c] = 0.0f;
  }
  if (ratio) {
    // KL(p||q) = E_p[u - z] - lse_p + lse_q, KL(q||p) = E_q[z - u] - lse_q + lse_p
    const float dl = lse_side[1] - lse_side[0];
    if (a.kl_out) a.kl_out[c] = ex_side[1] - dl;
    if (a.rkl_out) a.rkl_out[c] = ex_side[0] + dl;
  }
}

// Target statistics of rows that share target rows: row gr takes those of
// its target row (valid rows), or the no-target values.
__global__ __launch_bounds__(256) void k_target_gather(TargetGatherLaunch a) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= a.ncols) return;
  const int64_t gr = a.r0 + c;
  const bool valid = a.flags[gr] != 0;
  const int32_t t = valid ? a.target_row[gr] : 0;  // in range on valid rows
  a.lse_p[gr] = valid ? a.t_lse_p[t] : 0.0f;
  a.y_arg[gr] = valid ? a.t_y_arg[t] : -1;
  a.flat[gr] = valid ? a.t_flat[t] : 0.0f;
}

// Sums over the vocabulary tiles of the pass-2 partials of kSegRows rows:
// the tiles of a row are split into kSegs contiguous segments, one thread
// each, and the segment sums are added in segment order (a fixed order, so
// results are bitwise repeatable).  Threads (rr, seg) = (tid % kSegRows,
// tid / kSegRows); on return, threads of segment 0 hold the row's sums.
constexpr int kSegRows = 32, kSegs = 32;
__device__ __forceinline__ void tile_sums(const float* part, int64_t part_stride, int64_t ldp,
                                          int tiles_m, uint32_t need, int c, bool row_ok,
                                          float (&sum)[kNumSums]) {
  __shared__ float sp[kNumSums][kSegs][kSegRows];
  const int rr = threadIdx.x % kSegRows, seg = threadIdx.x / kSegRows;
  const int per = (tiles_m + kSegs - 1) / kSegs;
  const int t0 = min(tiles_m, seg * per), t1 = min(tiles_m, t0 + per);
#pragma unroll
  for (int f = 0; f < kNumSums; ++f) {
    float acc = 0.0f;
    if (row_ok && (need & (1u << f))) {
      const float* p = part + f * part_stride + c;
      int t = t0;
      for (; t + 4 <= t1; t += 4) {
        const float x0 = p[(int64_t)t * ldp], x1 = p[(int64_t)(t + 1) * ldp];
        const float x2 = p[(int64_t)(t + 2) * ldp], x3 = p[(int64_t)(t + 3) * ldp];
        acc += x0;
        acc += x1;
        acc += x2;
        acc += x3;
      }
      for (; t < t1; ++t) acc += p[(int64_t)t * ldp];
    }
    sp[f][seg][rr] = acc;
  }
  __syncthreads();
#pragma unroll
  for (int f = 0; f < kNumSums; ++f) {
    float acc = 0.0f;
    if (seg == 0)
      for (int g = 0; g < kSegs; ++g) acc += sp[f][g][rr];
    sum[f] = acc;
  }
}

// sums over the vocabulary tiles of one shard: out[f][c] = sum_t part[f][t][c]
// (fixed order) for every requested sum f
__global__ __launch_bounds__(kSegRows * kSegs) void k_tile_sum(TileSumLaunch a) {
  const int c = blockIdx.x * kSegRows + (int)(threadIdx.x % kSegRows);
  float sum[kNumSums];
  tile_sums(a.part, a.part_stride, a.ldp, a.tiles_m, a.need, c, c < a.ncols, sum);
  if (threadIdx.x >= kSegRows || c >= a.ncols) return;
  for (int f = 0; f < kNumSums; ++f)
    if (a.need & (1u << f)) a.out[f * a.out_stride + c] = sum[f];
}

// out[i] = sum_g parts[g][i] in shard order (fp32 partials; fp32 or bf16 out)
template <typename OutT>
__global__ __launch_bounds__(256) void k_sum_parts(const float* parts, int64_t n, int32_t n_parts,
                                                   OutT* out) {
  const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i4 >= n) return;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const int lim = (int)(n - i4 < 4 ? n - i4 : 4);
  for (int g = 0; g < n_parts; ++g) {
    const float* src = parts + (int64_t)g * n + i4;
    if (lim == 4) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(src);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += v[e];
    } else {
      for (int e = 0; e < lim; ++e) acc[e] += src[e];
    }
  }
  for (int e = 0; e < lim; ++e) store1<OutT>(out + i4 + e, acc[e]);
}

__global__ __launch_bounds__(kSegRows * kSegs) void k_combine2(Combine2Launch a) {
  const int c = blockIdx.x * kSegRows + (int)(threadIdx.x % kSegRows);
  float sum[kNumSums];
  tile_sums(a.part, a.part_stride, a.ldp, a.tiles_m, a.need, c, c < a.ncols, sum);
  if (threadIdx.x >= kSegRows || c >= a.ncols) return;
  const float alpha = sum[0], S = sum[1], kl = sum[2], rkl = sum[3], jsd = sum[4], eqg = sum[5];
  const bool valid = a.flags[c] != 0;
  float L[kNumKinds];
  float zl = -INFINITY, za = -INFINITY;
  for (int g = 0; g < a.zy_count; ++g) {  // one entry, or one per vocabulary shard
    if (a.zy_lab) zl = fmaxf(zl, a.zy_lab[g * a.zy_stride + c]);
    if (a.zy_arg) za = fmaxf(za, a.zy_arg[g * a.zy_stride + c]);
  }
  L[0] = a.zy_lab ? a.lse_q[c] - zl : 0.0f;
  L[1] = a.zy_arg ? a.lse_q[c] - za : 0.0f;
  L[2] = kl;
  L[3] = rkl;
  L[4] = jsd;
  L[5] = 1.0f - alpha;
  L[6] = -logf(alpha);
  const float lam = expf(-3.0f * alpha);
  L[7] = lam * kl + (1.0f - lam) * (1.0f - alpha);
  float total = 0.0f;
#pragma unroll
  for (int k = 0; k < kNumKinds; ++k) {
    if (a.w[k] == 0.0f) continue;
    const float lk = valid ? L[k] : 0.0f;
    total += a.w[k] * lk;
    if (a.term) a.term[k * a.term_stride + c] = lk;
  }
  a.loss[c] = valid ? total : 0.0f;
  a.alpha[c] = (a.need & SUM_ALPHA) ? alpha : 1.0f;
  a.S[c] = S;
  a.rkl[c] = rkl;
  a.eqg[c] = eqg;
}

__global__ __launch_bounds__(1024) void k_reduce(ReduceLaunch a) {
  __shared__ double red[1024];
  const int64_t nv = a.counts[0];
  for (int q = 0; q <= kNumKinds; ++q) {
    const float* src;
    if (q == 0) {
      src = a.loss;
    } else {
      if (!(a.active & (1u << (q - 1)))) {
        if (threadIdx.x == 0) a.reduced[q] = 0.0f;
        continue;
      }
      src = a.term + (int64_t)(q - 1) * a.term_stride;
    }
    double s = 0.0;
    for (int64_t r = threadIdx.x; r < a.n; r += 1024) s += (double)src[r];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int o = 512; o > 0; o >>= 1) {
      if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
      __syncthreads();
    }
    if (threadIdx.x == 0) a.reduced[q] = nv > 0 ? (float)(red[0] / (double)nv) : 0.0f;
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void k_seed(SeedLaunch a) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= a.n) return;
  const int64_t nv = a.counts[0];
  float s = 0.0f;
  if (a.flags[r]) {
    if (a.grad_loss) s += a.grad_loss[r];
    if (a.grad_mean && nv > 0) s += a.grad_mean[0] / (float)nv;
  }
  a.seed[r] = s;
}

// 64 x 64 tile transpose through LDS with 16-byte global loads and stores.
// Source rows past `rows` read as zeros, which pads output columns
// [rows, ld_out) with zeros.  cols and ld_out are multiples of 64 (the host
// requires a hidden size that is a multiple of 64; ld_out is the padded
// vocabulary or chunk size).  In LDS, source row y keeps its 16-byte chunk
// ch at position ch ^ (y / KC): the column gathers of the second half read
// KC rows y = KC q + e at one chunk, and the XOR with q spreads them over
// distinct banks.
template <typename T>
__global__ __launch_bounds__(256) void k_transpose(const T* in, int64_t rows, int64_t cols, T* out,
                                                   int64_t ld_out, const float* rscale) {
  constexpr int KC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = 64 / KC;             // chunks per 64-element row
  constexpr int IT = 64 * CPR / 256;       // chunks per thread
  constexpr int ROWB = 64 * (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) char tile[64 * ROWB];
  const int64_t c0 = (int64_t)blockIdx.x * 64;  // source row block (becomes out columns)
  const int64_t j0 = (int64_t)blockIdx.y * 64;  // source column block (becomes out rows)
  i32x4_t v[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * 256 + threadIdx.x;
    const int y = idx / CPR, ch = idx % CPR;
    const int64_t r = c0 + y;
    v[it] = r < rows ? *reinterpret_cast<const i32x4_t*>(in + r * cols + j0 + ch * KC)
                     : i32x4_t{0, 0, 0, 0};
    if (rscale && r < rows) {
      const float f = rscale[r];
      if constexpr (sizeof(T) == 2) {
        bf16x8_t b = __builtin_bit_cast(bf16x8_t, v[it]);
#pragma unroll
        for (int e = 0; e < KC; ++e) b[e] = (__bf16)((float)b[e] * f);
        v[it] = __builtin_bit_cast(i32x4_t, b);
      } else {
#pragma unroll
        for (int e = 0; e < KC; ++e) v[it][e] = __float_as_int(__int_as_float(v[it][e]) * f);
      }
    }
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * 256 + threadIdx.x;
    const int y = idx / CPR, ch = idx % CPR;
    *reinterpret_cast<i32x4_t*>(tile + y * ROWB + ((ch ^ (y / KC)) << 4)) = v[it];
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = it * 256 + threadIdx.x;
    const int x = idx / CPR, q = idx % CPR;  // out row j0 + x, chunk q = source rows KC q ..
    const char* col = tile + (((x / KC) ^ q) << 4) + (x % KC) * (int)sizeof(T);
    i32x4_t o;
    if constexpr (sizeof(T) == 2) {
      bf16x8_t b;
#pragma unroll
      for (int e = 0; e < KC; ++e) b[e] = *reinterpret_cast<const __bf16*>(col + (q * KC + e) * ROWB);
      o = __builtin_bit_cast(i32x4_t, b);
    } else {
#pragma unroll
      for (int e = 0; e < KC; ++e) o[e] = *reinterpret_cast<const int*>(col + (q * KC + e) * ROWB);
    }
    *reinterpret_cast<i32x4_t*>(out + (j0 + x) * ld_out + c0 + q * KC) = o;
  }
}

__global__ __launch_bounds__(256) void k_align(AlignLaunch a) {
  const int64_t n = (int64_t)a.n_heads * a.batch * a.seq_len;
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= n) return;
  // token-major: row r = (b * seq_len + t) * n_heads + k
  const int k = (int)(r % a.n_heads);
  const int64_t bt = r / a.n_heads;
  const int64_t t = bt % a.seq_len;
  const int64_t b = bt / a.seq_len;
  const int64_t tt = t + a.shifts[k];
  int32_t tr = -1;
  uint8_t m = 0;
  if (tt < a.seq_len) {
    const int64_t src = b * a.seq_len + tt;
    if (!a.loss_mask || a.loss_mask[src]) {
      tr = (int32_t)src;
      m = 1;
    }
  }
  a.target_row[r] = tr;
  a.mask[r] = m;
}

// ============================================================================
// staged cross-entropy values: row factor, rescue of far rows, one-hot terms
// ============================================================================
// One workgroup per chunk row.  The row's staged values are exp(z - ref) (and
// exp(z - m_tile) in tiles whose max exceeds ref + kStageRange).  Normal rows
// keep them, with factor seed (w_lab + w_arg) exp(ref - lse): dz = factor *
// staged.  A row with such a tile is rescaled in place to exp(z - lse) (each
// tile by exp(t_ref - lse) <= 1, t_ref the reference it was staged with), with
// factor seed (w_lab + w_arg).  The entries of the row's labels, where dz =
// seed ((w_lab + w_arg) q - w_lab [v = y_lab] - w_arg [v = y_arg]) carries the
// one-hot terms, are rewritten from the tile's fp32 logit there (see
// label_entry), by the thread that owns entry y (entry i of every tile
// belongs to thread i).
template <typename T>
__global__ __launch_bounds__(256) void k_stage_fix(StageFixLaunch a) {
  const int c = blockIdx.x;
  const int64_t gr = a.r0 + c;
  const float sd = a.seed[gr];
  if (sd == 0.0f) {  // staged as zeros
    if (threadIdx.x == 0) a.rscale[c] = 0.0f;
    return;
  }
  const float lse = a.sv.lse_q[gr], ref = a.ref[c];
  const bool far = a.row_max[c] - ref > kStageRange;
  const float eref = far ? lse : ref;
  const float factor = sd * (a.w_lab + a.w_arg) * fast_exp2((eref - lse) * kLog2e);
  const int yl = a.w_lab != 0.0f ? a.sv.y_label[gr] : -1;
  const int ya = a.w_arg != 0.0f ? a.sv.y_arg[gr] : -1;
  // entry y of dz / factor = exp(lse - eref) (q_y - w_y / W), W = w_lab + w_arg,
  // w_y the weights whose label is y; formed as expm1(z_y - lse) + (W - w_y) / W
  // from the tile's fp32 logit so that q_y near 1 keeps its difference from 1
  const float wsum = a.w_lab + a.w_arg;
  auto label_entry = [&](int y, float zt) {
    const float wy = (y == yl ? a.w_lab : 0.0f) + (y == ya ? a.w_arg : 0.0f);
    return fast_exp2((lse - eref) * kLog2e) * (expm1f(zt - lse) + (wsum - wy) / wsum);
  };
  T* E = static_cast<T*>(a.stage) + (int64_t)c * a.ld_stage;
  T* Et = static_cast<T*>(a.stage_t);
  auto put = [&](int64_t v, float x) {
    store1<T>(E + v, x);
    if (Et) store1<T>(Et + v * a.ld_stage_t + c, x);
  };
  if (threadIdx.x == 0) a.rscale[c] = factor;
  if (far) {
    // thread i owns entry i of every tile
    for (int t = 0; t < a.tiles_m; ++t) {
      const float m = a.pm[(int64_t)t * a.ldp + c];
      const float tref = m - ref > kStageRange ? m : ref;
      const float f = fast_exp2((tref - lse) * kLog2e);
      const int64_t v = (int64_t)t * kVocabTile + threadIdx.x;
      if (v != yl && v != ya) put(v, load1<T>(E + v) * f);
    }
  }
  // the label entries, by the thread that owns them
  if (yl >= 0 && (yl & 255) == (int)threadIdx.x) put(yl, label_entry(yl, a.zt_lab[c]));
  if (ya >= 0 && ya != yl && (ya & 255) == (int)threadIdx.x)
    put(ya, label_entry(ya, a.zt_arg[c]));
}

// ============================================================================
// scratch of the allocation-free forward
// ============================================================================
// One array per device (each device holds its own copy), kept until the
// process ends.  Host code never uses the array's name as an address: the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  static std::mutex mu;
  static void* per_device[kMaxScratchDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

// ============================================================================
// launchers
// ============================================================================
// bf16 pass 1 without staging: eight waves too (lk_hybrid stats_p and stats_q
// 1.6 % faster than with four)
constexpr int kStatsWNW = 4;
hipError_t launch_stats(bool bf16, bool target, const StatsLaunch& a, hipStream_t s) {
  const dim3 grid(grid_for_tiles(a.tiles_m * a.tiles_n)), block(kThreads);
  constexpr int W = kStatsWNW;
  const bool raw = a.raw != nullptr;
  if (bf16) {
    const dim3 b8(128 * W);
    if (raw && target) hipLaunchKernelGGL((k_stats<bf16_bits, true, W, true>), grid, b8, 0, s, a);
    else if (raw) hipLaunchKernelGGL((k_stats<bf16_bits, false, W, true>), grid, b8, 0, s, a);
    else if (target) hipLaunchKernelGGL((k_stats<bf16_bits, true, W>), grid, b8, 0, s, a);
    else hipLaunchKernelGGL((k_stats<bf16_bits, false, W>), grid, b8, 0, s, a);
  } else {
    if (raw && target) hipLaunchKernelGGL((k_stats<float, true, 2, true>), grid, block, 0, s, a);
    else if (raw) hipLaunchKernelGGL((k_stats<float, false, 2, true>), grid, block, 0, s, a);
    else if (target) hipLaunchKernelGGL((k_stats<float, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_stats<float, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

// bf16 pass 1 with staging runs eight waves (two per SIMD): 3 % faster than
// four at the 8B shape despite a few spills outside its inner loop
constexpr int kStageWNW = 4;
hipError_t launch_stats_stage(bool bf16, const StatsStageLaunch& a, hipStream_t s) {
  const dim3 grid(grid_for_tiles(a.st.tiles_m * a.st.tiles_n)), block(kThreads);
  if (bf16) hipLaunchKernelGGL((k_stats_stage<bf16_bits, kStageWNW>), grid,
                               dim3(128 * kStageWNW), 0, s, a);
  else hipLaunchKernelGGL((k_stats_stage<float, 2>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dz_stage(bool bf16, const DzStageLaunch& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.tiles_m * a.row_blocks)), block(256);
  if (bf16) hipLaunchKernelGGL(k_dz_stage<bf16_bits>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(k_dz_stage<float>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_stats_dual(bool bf16, const DualStatsLaunch& a, hipStream_t s) {
  const dim3 grid(grid_for_tiles(a.tiles_m * a.tiles_n)), block(kThreads);
  if (bf16)
    hipLaunchKernelGGL(k_stats_dual<bf16_bits>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(k_stats_dual<float>, grid, block, 0, s, a);
  return hipGetLastError();
}

// four waves (2 x 2); eight (2 x 4, two per SIMD) measured the same
constexpr int kDivWNW = 2;

hipError_t launch_heads_map(int32_t* map, int32_t tiles_n, int32_t n_heads, const int32_t* shifts,
                            int64_t jlo, int64_t r0, int32_t rows, hipStream_t s) {
  ShiftArg sh{};
  for (int k = 0; k < n_heads && k < kMaxHeads; ++k) sh.v[k] = shifts[k];
  const int64_t n = (int64_t)tiles_n * 64 * n_heads;
  hipLaunchKernelGGL(k_heads_map, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, map,
                     tiles_n, n_heads, sh, jlo, r0, rows);
  return hipGetLastError();
}

hipError_t launch_div_heads(bool bf16, const DivHeadsLaunch& a, hipStream_t s) {
  if (!bf16 || a.n_heads < 2 || a.n_heads > 3) return hipErrorInvalidValue;
  const dim3 grid(grid_for_tiles(a.d.tiles_m * a.d.tiles_n)), block(kThreads);
  if (a.n_heads == 2) hipLaunchKernelGGL((k_div_heads<bf16_bits, 2>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((k_div_heads<bf16_bits, 3>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_div_raw(const DivRawLaunch& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.tiles_m * ((a.ncols + 63) / 64))), block(256);
  constexpr uint32_t kLk = SUM_ALPHA | SUM_S | SUM_KL, kTv = SUM_ALPHA | SUM_S;
  if (a.need == kLk) hipLaunchKernelGGL((k_div_raw<kLk>), grid, block, 0, s, a);
  else if (a.need == kTv) hipLaunchKernelGGL((k_div_raw<kTv>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((k_div_raw<0>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dz_raw(bool bf16, const DzRawLaunch& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.tiles_m * a.row_blocks)), block(256);
  const bool log = a.w_rkl != 0.0f || a.w_jsd != 0.0f;
  if (bf16) {
    if (log) hipLaunchKernelGGL((k_dz_raw<bf16_bits, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_dz_raw<bf16_bits, false>), grid, block, 0, s, a);
  } else {
    if (log) hipLaunchKernelGGL((k_dz_raw<float, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_dz_raw<float, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_div(bool bf16, const DivLaunch& a, hipStream_t s) {
  constexpr int W = kDivWNW;
  const dim3 grid(grid_for_tiles(a.tiles_m * a.tiles_n)), block(128 * W);
  // the common sum sets (lk_hybrid; tv / nla) as constants: measured 2%
  // faster than reading them per element
  constexpr uint32_t kLk = SUM_ALPHA | SUM_S | SUM_KL, kTv = SUM_ALPHA | SUM_S;
  if (bf16) {
    if (a.need == kLk) hipLaunchKernelGGL((k_div<bf16_bits, W, kLk>), grid, block, 0, s, a);
    else if (a.need == kTv) hipLaunchKernelGGL((k_div<bf16_bits, W, kTv>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_div<bf16_bits, W>), grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL((k_div<float, 2>), dim3(grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_dz(bool bf16, bool dual, const DzLaunch& a, hipStream_t s) {
  const dim3 grid(grid_for_tiles(a.tiles_m * a.tiles_n)), block(kThreads);
  if (bf16) {
    // the single-contraction recompute runs eight waves like pass 1 (two-call
    // CE step 0.3 % faster); the dual one keeps four
    if (dual) hipLaunchKernelGGL((k_dz<bf16_bits, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_dz<bf16_bits, false, 4>), grid, dim3(512), 0, s, a);
  } else {
    if (dual) hipLaunchKernelGGL((k_dz<float, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_dz<float, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

// Waves along N of the plain bf16 contractions with K-major operands: 4 (eight
// waves, 128 x 64 each, two per SIMD).  Measured against four waves at the 8B
// shape: gemm_dW 26.3 vs 27.5 ms per step (its fp32 read-modify-write
// epilogue runs on twice the threads), gemm_dh about 1% faster.  The
// contractions with MN-major operands (W or the hidden rows read in place)
// run eight waves too despite a few spills outside the inner loop: the dh
// contraction of the 405B shape (W in place) 56.1 -> 46.7 ms per step.  bf16
// pass 1 runs eight as well, with a load every MFMA (kStageWNW, kStatsWNW).
constexpr int kGemmWNW = 4;
constexpr int kLeanWNW = 4;

template <int ROLE>
static void launch_gemm_role(bool bf16, const GemmLaunch& a, hipStream_t s) {
  constexpr int W = kGemmWNW;
  const dim3 grid(grid_for_tiles(a.tiles_m * a.splits * a.tiles_n)), block(128 * W);
  if constexpr (ROLE == 0) {
    if (bf16 && a.at_out) {
      static_assert(kGemmWNW == 4 && kLeanWNW == 4, "A's transpose needs eight waves");
      if (a.lean) {
        if (a.out_bf16) hipLaunchKernelGGL((k_gemm<bf16_bits, bf16_bits, 0, true, 4, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((k_gemm<bf16_bits, float, 0, true, 4, true>), grid, block, 0, s, a);
      } else {
        if (a.out_bf16) hipLaunchKernelGGL((k_gemm<bf16_bits, bf16_bits, 0, false, 4, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((k_gemm<bf16_bits, float, 0, false, 4, true>), grid, block, 0, s, a);
      }
      return;
    }
  }
  if (bf16 && a.lean) {
    constexpr int LW = kLeanWNW;
    if (a.out_bf16) hipLaunchKernelGGL((k_gemm<bf16_bits, bf16_bits, ROLE, true, LW>), grid, dim3(128 * LW), 0, s, a);
    else hipLaunchKernelGGL((k_gemm<bf16_bits, float, ROLE, true, LW>), grid, dim3(128 * LW), 0, s, a);
  } else if (bf16) {
    if (a.out_bf16) hipLaunchKernelGGL((k_gemm<bf16_bits, bf16_bits, ROLE, false, W>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_gemm<bf16_bits, float, ROLE, false, W>), grid, block, 0, s, a);
  } else {
    if (a.out_bf16) hipLaunchKernelGGL((k_gemm<float, bf16_bits, ROLE, false, 2>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_gemm<float, float, ROLE, false, 2>), grid, dim3(256), 0, s, a);
  }
}

hipError_t launch_gemm(bool bf16, const GemmLaunch& a, hipStream_t s) {
  if (a.splits < 1 || (a.splits > 1 && (a.k_split <= 0 || a.k_split % 64 != 0 ||
                                        (int64_t)(a.splits - 1) * a.k_split >= a.k_len)))
    return hipErrorInvalidValue;
  if (a.at_out && (a.role != 0 || !bf16 || a.ld_at % 8 != 0 ||
                   reinterpret_cast<uintptr_t>(a.at_out) % 16 != 0 ||
                   (int64_t)a.tiles_m * 256 > a.ld_at || a.k_len % 64 != 0))
    return hipErrorInvalidValue;
  if (a.role == 0) launch_gemm_role<0>(bf16, a, s);
  else launch_gemm_role<1>(bf16, a, s);
  return hipGetLastError();
}

hipError_t launch_validity(const ValidityLaunch& a, hipStream_t s) {
  hipLaunchKernelGGL(k_validity, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rowdot(bool bf16, const RowdotLaunch& a, hipStream_t s) {
  const dim3 grid((a.ncols + 3) / 4), block(256);
  if (bf16) hipLaunchKernelGGL(k_rowdot<bf16_bits>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(k_rowdot<float>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine1(const Combine1Launch& a, hipStream_t s) {
  hipLaunchKernelGGL(k_combine1, dim3((a.ncols + 31) / 32), dim3(kCombine1Threads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine2(const Combine2Launch& a, hipStream_t s) {
  hipLaunchKernelGGL(k_combine2, dim3((a.ncols + kSegRows - 1) / kSegRows), dim3(kSegRows * kSegs),
                     0, s, a);
  return hipGetLastError();
}

hipError_t launch_target_gather(const TargetGatherLaunch& a, hipStream_t s) {
  hipLaunchKernelGGL(k_target_gather, dim3((a.ncols + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_tile_sum(const TileSumLaunch& a, hipStream_t s) {
  hipLaunchKernelGGL(k_tile_sum, dim3((a.ncols + kSegRows - 1) / kSegRows), dim3(kSegRows * kSegs),
                     0, s, a);
  return hipGetLastError();
}

hipError_t launch_sum_parts(const float* parts, int64_t n, int32_t n_parts, void* out,
                            bool out_bf16, hipStream_t s) {
  const dim3 grid((unsigned)((n + 1023) / 1024)), block(256);
  if (out_bf16)
    hipLaunchKernelGGL(k_sum_parts<bf16_bits>, grid, block, 0, s, parts, n, n_parts,
                       static_cast<bf16_bits*>(out));
  else
    hipLaunchKernelGGL(k_sum_parts<float>, grid, block, 0, s, parts, n, n_parts,
                       static_cast<float*>(out));
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceLaunch& a, hipStream_t s) {
  hipLaunchKernelGGL(k_reduce, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_seed(const SeedLaunch& a, hipStream_t s) {
  hipLaunchKernelGGL(k_seed, dim3((unsigned)((a.n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_transpose(bool bf16, const void* in, int64_t rows, int64_t cols, void* out,
                            int64_t width, int64_t ld_out, hipStream_t s, const float* rscale) {
  // whole 64 x 64 tiles on both sides and 16-byte aligned rows
  if (cols % 64 != 0 || width % 64 != 0 || ld_out % 64 != 0 || rows > width || width > ld_out)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)(width / 64), (unsigned)(cols / 64)), block(256);
  if (bf16)
    hipLaunchKernelGGL(k_transpose<bf16_bits>, grid, block, 0, s,
                       static_cast<const bf16_bits*>(in), rows, cols, static_cast<bf16_bits*>(out),
                       ld_out, rscale);
  else
    hipLaunchKernelGGL(k_transpose<float>, grid, block, 0, s, static_cast<const float*>(in), rows,
                       cols, static_cast<float*>(out), ld_out, rscale);
  return hipGetLastError();
}

hipError_t launch_stage_fix(bool bf16, const StageFixLaunch& a, hipStream_t s) {
  if (a.ncols <= 0) return hipSuccess;
  if (bf16) hipLaunchKernelGGL(k_stage_fix<bf16_bits>, dim3(a.ncols), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_stage_fix<float>, dim3(a.ncols), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_align(const AlignLaunch& a, hipStream_t s) {
  const int64_t n = (int64_t)a.n_heads * a.batch * a.seq_len;
  hipLaunchKernelGGL(k_align, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace specloss
