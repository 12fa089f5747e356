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
constexpr int kMaxHeads = 4;  // aligned heads a problem may declare
struct ShiftArg {
  int32_t v[kMaxHeads];
};
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
  // optional: the tile's raw fp32 logits, row c (< ncols) of B at
  // raw[c * ld_raw + v] for every v of the padded vocabulary (v >= vocab
  // holds values of clamped weight rows, never read as logits)
  float* raw;
  int64_t ld_raw;
};
// target: the variant for the target logits u (argmax and e^2 sums as well)
hipError_t launch_stats(bool bf16, bool target, const StatsLaunch& a, hipStream_t s);

// pass 1 of both sides at once (draft z = W h and target u = W_t g of the
// same rows, 256 x 128 tiles): the per-tile statistics of launch_stats for
// each side, plus, relative to the same tile maxima, the unnormalised
// expectations of the log-ratio pa_u = sum_v exp(u_v - m_u) (u_v - z_v) and
// pr_z = sum_v exp(z_v - m_z) (z_v - u_v), from which the combine forms
// KL(p||q) = pa_u / s_u - lse_p + lse_q and KL(q||p) = pr_z / s_z - lse_q +
// lse_p without a second sweep.
struct DualStatsLaunch {
  GemmOperand Az, Bz, Au, Bu;
  int32_t k_len, vocab, tiles_m, tiles_n, ncols, ldp;
  float* pm_z;
  float* ps_z;
  float* pr_z;
  float* pm_u;
  float* ps_u;
  int32_t* pi_u;
  float* pq_u;
  float* pa_u;
};
hipError_t launch_stats_dual(bool bf16, const DualStatsLaunch& a, hipStream_t s);

// pass 1 for the single-call forward+backward: also stores staged values of
// every (row, vocab) into `stage` ([cap][Vp], row-major) and, when stage_t is
// set, transposed into stage_t ([Vp][cap]).  Without `ref` a row's values are
// e = exp(z - m_tile).  With `ref` (per chunk row) they are e' = exp(z - ref)
// in the tiles whose max is at most ref + kStageRange, e = exp(z - m_tile) in
// the others (a row with such a tile is rescaled after the forward), and 0 on
// rows whose seed is 0.
constexpr float kStageRange = 64.0f;
struct StatsStageLaunch {
  StatsLaunch st;
  void* stage;
  int64_t ld_stage;
  void* stage_t;
  int64_t ld_stage_t;
  const float* ref;   // chunk-local, or null
  const float* seed;  // chunk-local (with ref)
  // with ref: the tile holding a row's label y1 (y2) writes the row's fp32
  // logit there into zt1 (zt2); chunk-local, null when unused
  const int32_t* y1;
  const int32_t* y2;
  float* zt1;
  float* zt2;
};
hipError_t launch_stats_stage(bool bf16, const StatsStageLaunch& a, hipStream_t s);

// logit gradient of the label / argmax cross-entropies from the staged
// e = exp(z - m_tile), written over it and, transposed, into dzt ([Vp][cap]):
//   dz = seed * ((w_lab + w_arg) e exp(m_tile - lse) - w_lab [v == y_lab] - w_arg [v == y_arg])
struct DzStageLaunch {
  int32_t tiles_m, ncols, vocab, ldp;
  int64_t r0;
  const float* pm;     // chunk partial maxima [tiles_m][ldp]
  const float* seed;   // [N], global rows
  SavedView sv;        // global rows
  float w_lab, w_arg;
  void* dz;            // in: e, out: dz; [cap][Vp]
  int64_t ld_dz;
  void* dzt;           // [Vp][cap], or null (not needed by bf16 contractions)
  int64_t ld_dzt;
  int32_t row_blocks;  // 64-row blocks covered (multiple of the 256-row tiles)
};
hipError_t launch_dz_stage(bool bf16, const DzStageLaunch& a, hipStream_t s);

// Second sweep over raw logits kept from pass 1 (single call, divergences):
// the draft row c of the chunk is z[c * ld_z + v], its target row is
// u[r * ld_u + v] with r = c, or with urow set r = urow[c] - ushift clamped
// into [0, n_u) (rows that share target rows keep one copy).  q and p are
// formed with the final logsumexps exactly as in launch_div.
struct RawRows {
  const float* z;
  int64_t ld_z;
  const float* u;
  int64_t ld_u;
  const int32_t* urow;  // chunk-local, or null
  int64_t ushift;
  int32_t n_u;
};

// The pass-2 sums from raw logits, memory-bound: per (256-entry vocabulary
// tile, chunk row) partials in the layout of launch_div.
struct DivRawLaunch {
  RawRows r;
  int32_t tiles_m, ncols, vocab, ldp;
  const float* lse_q;  // chunk-local
  const float* lse_p;
  uint32_t need;
  float* part;          // [kNumSums][tiles_m][ldp]
  int64_t part_stride;
};
hipError_t launch_div_raw(const DivRawLaunch& a, hipStream_t s);

// The logit gradient of the divergences (and of label / argmax
// cross-entropies mixed with them) from raw logits, with q = exp(z - lse_q),
// p = exp(u - lse_p), d = q - p, c = [q < p] (1/2 on ties) and
// l = log q - log p formed in fp32:
//   dz = seed (A q + B d - C q (c - S) + q (w_rkl (l - rKL) + w_jsd (g - E_q[g])))
//        - seed (w_lab [v = y_lab] + w_arg [v = y_arg])
// where A = w_lab + w_arg, B = w_kl + w_lk lam, C = w_tv + w_nla / alpha +
// w_lk (1 - lam), lam = exp(-3 alpha), g = (ln 2 - softplus(-l)) / 2 =
// (log q - log m) / 2, m = (p + q) / 2, and alpha, S, rKL, E_q[g] the row's
// saved sums.  dz ([cap][ld_dz], input dtype) and, transposed, dzt
// ([Vp][ld_dzt], or null).
struct DzRawLaunch {
  RawRows r;
  int32_t tiles_m, ncols, vocab;
  int64_t r0;
  const float* seed;  // [N], global rows
  SavedView sv;       // global rows
  float w_lab, w_arg, w_kl, w_tv, w_nla, w_lk, w_rkl, w_jsd;
  void* dz;
  int64_t ld_dz;
  void* dzt;
  int64_t ld_dzt;
  int32_t row_blocks;  // 64-row blocks covered
};
hipError_t launch_dz_raw(bool bf16, const DzRawLaunch& a, hipStream_t s);

struct DivLaunch {
  GemmOperand Az, Bz, Au, Bu;
  int32_t k_len, vocab, tiles_m, tiles_n, ncols, ldp;
  const float* lse_q;  // chunk-local (already offset by the chunk start)
  const float* lse_p;
  uint32_t need;
  float* part;          // [kNumSums][tiles_m][ldp]
  int64_t part_stride;  // tiles_m * ldp
};
hipError_t launch_div(bool bf16, const DivLaunch& a, hipStream_t s);

// pass 2 for aligned heads (rows token-major: chunk row r - r0 of global row
// r = T * K + k is head k at token T, whose target row is T + shifts[k]):
// tiles of 256 vocabulary rows x 64 target rows j = jlo + tn * 64 + c, each
// target tile computed once for the K <= 3 draft rows (j - shifts[k]) * K + k
// it serves that lie in the chunk.  Bz rows come through `map` (filled by
// launch_heads_map: [tiles_n][64 K] chunk-local rows, clamped into the
// chunk); Bu starts at target row jlo.  Sums and partials as for launch_div,
// indexed by chunk row.
struct DivHeadsLaunch {
  DivLaunch d;     // Bz: the chunk's rows with `map`; Bu: target rows from jlo
  int32_t n_heads;
  int32_t shifts[kMaxHeads];
  int64_t jlo;     // first target row of the tiles
  int64_t r0;      // global row of chunk row 0
  int32_t rows;    // chunk rows
};
hipError_t launch_div_heads(bool bf16, const DivHeadsLaunch& a, hipStream_t s);
hipError_t launch_heads_map(int32_t* map, int32_t tiles_n, int32_t n_heads, const int32_t* shifts,
                            int64_t jlo, int64_t r0, int32_t rows, hipStream_t s);

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
  const float* rscale;  // per output row m, or null: C = rscale[m] * (A B^T) (no accumulate)
  // split K: `splits` (>= 1) slices of k_split along K (the last one shorter);
  // slice s writes its partial product to C + s * part_stride elements.
  // The grid covers tiles_m * splits tile rows.
  int32_t splits, k_split;
  int64_t part_stride;
  // dh only (bf16), or null: A's transpose, at_out[k * ld_at + m] for every
  // k < k_len and m of the row tiles (0 at m >= m_valid), written from A's
  // LDS slabs as the contraction streams them
  void* at_out;
  int64_t ld_at;
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
  // aligned heads (n_heads > 0): a valid row r must have target row
  // r / n_heads + shifts[r % n_heads]; a row that does not is bad
  int32_t n_heads;
  int32_t shifts[kMaxHeads];
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
  float* row_max;        // chunk-local max of z per row, or null
  int32_t target_absent; // no target in the problem: write its no-target values
  // log-ratio partials of launch_stats_dual (or null): the merged KL(p||q)
  // and KL(q||p) go to kl_out and rkl_out (chunk-local)
  const float* pa_u;
  const float* pr_z;
  float* kl_out;
  float* rkl_out;
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

// Finish the staged values of the label / argmax cross-entropies (single
// call, pass 1 with `ref`), one workgroup per chunk row: the row factor
// rscale = seed (w_lab + w_arg) exp(eref - lse_q) with eref = ref, or lse_q
// for a row whose max exceeds ref + kStageRange (its tiles are first rescaled
// to exp(z - lse_q)); then the one-hot terms go into the staged entries of
// the row's labels, so that dz = rscale * staged in both layouts.
struct StageFixLaunch {
  int32_t ncols, tiles_m, ldp;
  int64_t r0;            // global row of chunk column 0
  const float* pm;       // [tiles_m][ldp] per-tile max of z
  const float* ref;      // chunk-local
  const float* row_max;  // chunk-local
  const float* seed;     // global
  SavedView sv;          // global
  const float* zt_lab;   // chunk-local: the tile's logit at y_label (see StatsStageLaunch)
  const float* zt_arg;   // chunk-local: the tile's logit at y_arg
  float w_lab, w_arg;
  void* stage;           // [cap][ld_stage]
  int64_t ld_stage;
  void* stage_t;         // [Vp][ld_stage_t]
  int64_t ld_stage_t;
  float* rscale;         // chunk-local output
};
hipError_t launch_stage_fix(bool bf16, const StageFixLaunch& a, hipStream_t s);

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

// out[j][c] = c < rows ? in[c][j] : 0 for j < cols, c < width (row stride ld_out)
// rscale (optional, per source row): out = rscale[row] * in, rounded to the type
hipError_t launch_transpose(bool bf16, const void* in, int64_t rows, int64_t cols, void* out,
                            int64_t width, int64_t ld_out, hipStream_t s,
                            const float* rscale = nullptr);

struct AlignLaunch {
  int64_t seq_len, batch;
  int32_t n_heads;
  int32_t shifts[64];
  const uint8_t* loss_mask;
  int32_t* target_row;
  uint8_t* mask;
};
hipError_t launch_align(const AlignLaunch& a, hipStream_t s);

// ---- the allocation-free forward ----
// Bytes of the file-scope device scratch array behind lmhead_loss_fwd_noalloc
// (SPECLOSS_NOALLOC_SCRATCH_BYTES in the public header).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
// Device address of the current device's scratch array: looked up with
// hipGetSymbolAddress on the first call on each device (that device current)
// and kept per device.
hipError_t noalloc_scratch(void** ptr);

}  // namespace specloss
