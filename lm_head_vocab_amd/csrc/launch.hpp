// Internal launch interface between the C-ABI host code (api.cpp) and the
// HIP kernels (kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace specloss {

// Sums produced by the second (divergence) pass, one partial array each.
enum : uint32_t {
  SUM_ALPHA = 1u << 0,  // sum_v min(p, q)
  SUM_S = 1u << 1,      // sum_v q * c, c = 1[q < p] (1/2 on ties)
  SUM_KL = 1u << 2,     // sum_v p (log p - log q)
  SUM_RKL = 1u << 3,    // sum_v q (log q - log p)
  SUM_JSD = 1u << 4,    // sum_v (p (log p - log m) + q (log q - log m)) / 2
  SUM_EQG = 1u << 5,    // sum_v q (log q - log m) / 2
};
constexpr int kNumSums = 6;
constexpr int kNumKinds = 8;
constexpr int kVocabTile = 256;  // vocabulary rows per tile in every vocab-tiled pass

// Per-row saved state (struct of arrays, global row index).
struct SavedView {
  float* lse_q;
  float* lse_p;
  int32_t* y_label;  // label of ce_label, -1 when none/invalid
  int32_t* y_arg;    // argmax p (lowest index), -1 when none
  float* alpha;
  float* S;
  float* rkl;
  float* eqg;
  int32_t* flags;    // 1 = valid row
  float* flat;       // flatness of p: cos(p, uniform), 0 when no target or invalid
};

// K-major: row r at base + r * ld (n_rows valid, optional gather map).
// MN-major (bf16 contractions of the backward): element (m, k) at
// base + k * ld + m, n_rows valid m, k_valid readable k-rows.
struct GemmOperand {
  const void* base;
  int64_t ld;
  int32_t n_rows;
  const int32_t* map;
  int32_t map_len;
  int32_t k_valid;
};

// ---- vocab-tiled passes (A = a vocabulary-row weight, B = hidden rows) ----
struct StatsLaunch {
  GemmOperand A, B;
  int32_t k_len, vocab, tiles_m, tiles_n, ncols, ldp;
  float* pm;
  float* ps;
  int32_t* pi;  // target variant only: lowest-index argmax per tile
  float* pq;    // target variant only: sum exp(2 (u - m_tile)) per tile
};
// target: the variant for the target logits u (argmax and e^2 sums as well)
hipError_t launch_stats(bool bf16, bool target, const StatsLaunch& a, hipStream_t s);

// pass 1 for the single-call forward+backward: also stores
// e = exp(z - m_tile) of every (row, vocab) into `stage` ([cap][Vp], row-major)
struct StatsStageLaunch {
  StatsLaunch st;
  void* stage;
  int64_t ld_stage;
};
hipError_t launch_stats_stage(bool bf16, const StatsStageLaunch& a, hipStream_t s);

// logit gradient from staged values, written over them and, transposed, into
// dzt ([Vp][cap]).  Without dd (label / argmax cross-entropies) the buffer
// holds e = exp(z - m_tile):
//   dz = seed * ((w_lab + w_arg) e exp(m_tile - lse) - w_lab [v == y_lab] - w_arg [v == y_arg]);
// with dd it holds q and dd holds q - p, and the divergence terms
// (kl_div, tv, nla, lk_hybrid) are added from the saved alpha and S.
struct DzStageLaunch {
  int32_t tiles_m, ncols, vocab, ldp;
  int64_t r0;
  const float* pm;     // chunk partial maxima [tiles_m][ldp] (e mode only)
  const float* seed;   // [N], global rows
  SavedView sv;        // global rows
  float w_lab, w_arg;
  float w_kl, w_tv, w_nla, w_lk;  // divergence weights (dd mode only)
  const void* dd;      // [cap][Vp] q - p, or null
  void* dz;            // in: e or q, out: dz; [cap][Vp]
  int64_t ld_dz;
  void* dzt;           // [Vp][cap], or null (not needed by bf16 contractions)
  int64_t ld_dzt;
  int32_t row_blocks;  // 64-row blocks covered (multiple of the 256-row tiles)
};
hipError_t launch_dz_stage(bool bf16, const DzStageLaunch& a, hipStream_t s);

struct DivLaunch {
  GemmOperand Az, Bz, Au, Bu;
  int32_t k_len, vocab, tiles_m, tiles_n, ncols, ldp;
  const float* lse_q;  // chunk-local (already offset by the chunk start)
  const float* lse_p;
  uint32_t need;
  float* part;          // [kNumSums][tiles_m][ldp]
  int64_t part_stride;  // tiles_m * ldp
  void* stage_q;        // null, or [cap][ld_stage]: q of every (chunk row, vocab)
  void* stage_d;        // [cap][ld_stage]: q - p (with stage_q)
  int64_t ld_stage;
};
hipError_t launch_div(bool bf16, const DivLaunch& a, hipStream_t s);

struct DzLaunch {
  GemmOperand Az, Bz, Au, Bu;
  int32_t k_len, vocab, tiles_m, tiles_n, ncols;
  int64_t r0;
  const float* seed;  // [N], global rows
  SavedView sv;       // global rows
  float w[kNumKinds];
  void* dz;           // [cap][Vp], row = chunk row
  int64_t ld_dz;
  void* dzt;          // [Vp][cap], or null (not needed by bf16 contractions)
  int64_t ld_dzt;
  int32_t vocab_offset;  // first vocabulary row of A (saved labels are global indices)
};
// dual: also recompute the target logits (kinds that need p)
hipError_t launch_dz(bool bf16, bool dual, const DzLaunch& a, hipStream_t s);

// ---- plain contraction C[m][n] (+)= sum_k A[m][k] B[n][k] ----
struct GemmLaunch {
  GemmOperand A, B;
  int32_t k_len, tiles_m, tiles_n, m_valid, n_valid;
  void* C;
  int64_t ldc;
  int accumulate;
  int out_bf16;
  int role;  // 0: dh, 1: dW (separate kernel names in profiles)
  int lean;  // bf16 only: B (and for dW also A) are MN-major, read without copies
};
hipError_t launch_gemm(bool bf16, const GemmLaunch& a, hipStream_t s);

// ---- row kernels ----
struct ValidityLaunch {
  int64_t n;
  const uint8_t* mask;
  const int32_t* labels;
  int use_labels;
  const int32_t* target_row;
  int64_t n_target;
  int use_target;
  int32_t vocab;
  int32_t* flags;
  int32_t* y_label;
  int64_t* counts;
};
hipError_t launch_validity(const ValidityLaunch& a, hipStream_t s);

struct RowdotLaunch {
  const void* W;
  const void* h;        // chunk base
  int64_t H;
  int32_t ncols;
  int32_t vocab;        // rows of W
  int32_t vocab_offset; // global index of W's first row; labels outside
                        // [offset, offset + vocab) give `outside` and are never dereferenced
  float outside;
  const int32_t* y1;    // chunk-local label arrays (global indices), or null
  const int32_t* y2;
  float* out1;
  float* out2;
};
hipError_t launch_rowdot(bool bf16, const RowdotLaunch& a, hipStream_t s);

// pm_z null: target side only; flags null: every column counts as valid
struct Combine1Launch {
  int32_t tiles_m, ncols, ldp;
  const float* pm_z;
  const float* ps_z;
  const float* pm_u;  // null when no target
  const float* ps_u;
  const int32_t* pi_u;
  const float* pq_u;
  int32_t vocab;
  const int32_t* flags;  // chunk-local
  float* lse_q;  // chunk-local
  float* lse_p;
  int32_t* y_arg;
  float* flat;
  // record mode (raw_m[0] != null): write the merged partials of this call's
  // tiles instead of the final values: m and sum-exp per side, e^2 sum and
  // argmax (plus idx_offset) of the target side
  float* raw_m[2];
  float* raw_s[2];
  float* raw_q2;
  int32_t* raw_idx;
  int32_t idx_offset;
};
hipError_t launch_combine1(const Combine1Launch& a, hipStream_t s);

// per-row target statistics from per-target-row ones (rows sharing target rows)
struct TargetGatherLaunch {
  int32_t ncols;
  int64_t r0;                 // global row of chunk column 0
  const int32_t* flags;       // [N] global
  const int32_t* target_row;  // [N] global
  const float* t_lse_p;       // [n_target_rows]
  const int32_t* t_y_arg;
  const float* t_flat;
  float* lse_p;               // [N] global
  int32_t* y_arg;
  float* flat;
};
hipError_t launch_target_gather(const TargetGatherLaunch& a, hipStream_t s);

struct TileSumLaunch {
  int32_t tiles_m, ncols, ldp;
  uint32_t need;
  const float* part;    // [kNumSums][tiles_m][ldp]
  int64_t part_stride;
  float* out;           // [kNumSums][out_stride]
  int64_t out_stride;
};
hipError_t launch_tile_sum(const TileSumLaunch& a, hipStream_t s);

// out[i] = sum over g < n_parts of parts[g * n + i] (fixed order)
hipError_t launch_sum_parts(const float* parts, int64_t n, int32_t n_parts, void* out,
                            bool out_bf16, hipStream_t s);

struct Combine2Launch {
  int32_t tiles_m, ncols, ldp;
  const float* part;
  int64_t part_stride;
  uint32_t need;
  float w[kNumKinds];
  const int32_t* flags;   // chunk-local
  const float* lse_q;
  const float* zy_lab;    // chunk-local label logits (null if unused)
  const float* zy_arg;
  int32_t zy_count;       // entries per row (max taken): 1, or one per vocabulary shard
  int64_t zy_stride;
  float* loss;            // chunk-local
  float* term;            // chunk-local, stride term_stride between kinds
  int64_t term_stride;
  float* alpha;           // chunk-local saved fields
  float* S;
  float* rkl;
  float* eqg;
};
hipError_t launch_combine2(const Combine2Launch& a, hipStream_t s);

struct ReduceLaunch {
  int64_t n;
  const float* loss;
  const float* term;
  int64_t term_stride;
  uint32_t active;  // bit k = kind k on
  const int64_t* counts;
  float* reduced;   // [1 + kNumKinds]
};
hipError_t launch_reduce(const ReduceLaunch& a, hipStream_t s);

struct SeedLaunch {
  int64_t n;
  const int32_t* flags;
  const float* grad_loss;
  const float* grad_mean;
  const int64_t* counts;
  float* seed;
};
hipError_t launch_seed(const SeedLaunch& a, hipStream_t s);

// out[j][c] = c < rows ? in[c][j] : 0 for j < cols, c < ld_out
hipError_t launch_transpose(bool bf16, const void* in, int64_t rows, int64_t cols, void* out,
                            int64_t ld_out, hipStream_t s);

struct AlignLaunch {
  int64_t seq_len, batch;
  int32_t n_heads;
  int32_t shifts[64];
  const uint8_t* loss_mask;
  int32_t* target_row;
  uint8_t* mask;
};
hipError_t launch_align(const AlignLaunch& a, hipStream_t s);

}  // namespace specloss
