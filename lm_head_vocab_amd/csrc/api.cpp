// C-ABI of libspecloss: argument checks, workspace plan and launch sequence.
//
// Forward, per chunk of rows (blog "Streaming Cross Entropy": tokens are
// independent, so rows are processed in chunks and only per-row statistics
// survive a chunk):
//   pass 1   k_stats on (W, hidden)        -> per (vocab tile, row) max / sum-exp
//            k_stats on (W_t, target rows) -> same plus argmax (target kinds)
//   merge    k_combine1 -> logsumexp of q and p, argmax p
//   gather   k_rowdot   -> label logit z_y (ce_label) and z at argmax p (ce)
//   pass 2   k_div      -> alpha, S, KL, rKL, JSD, E_q[g] partials (divergences)
//   losses   k_combine2 -> per-row weighted loss, unweighted terms, saved stats
// then k_reduce -> sum / n_valid (blog "Backward pass": one denominator).
// Backward, per chunk (blog "Backward pass": per-chunk logits, gradients for
// the chunk's hidden states, LM-head gradient accumulated over chunks):
//   k_dz (recompute + logit gradient) -> staged dz chunk, both layouts
//   k_gemm dh = dz W^T^T  and  k_gemm dW (+)= dz^T h, chunks in order.
#include <math.h>
#include <string.h>

#include <new>

#include "launch.hpp"
#include "specloss.h"

using namespace specloss;

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kDefaultChunk = 8192;
constexpr int64_t kChunkQuantum = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
int64_t cdiv(int64_t x, int64_t m) { return (x + m - 1) / m; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct KindSet {
  uint32_t active = 0;  // bit k = weight k nonzero
  bool label = false;   // ce_label on
  bool target = false;  // any kind needing the target side
  bool pass2 = false;   // any divergence needing a second sweep
  bool dual_bwd = false;
  bool stage_div = false;  // single call: pass 2 stages q and q - p (no rkl / jsd)
  uint32_t need = 0;    // SUM_* bits
};

KindSet kinds_of(const float* w) {
  KindSet k;
  for (int i = 0; i < kNumKinds; ++i)
    if (w[i] != 0.0f) k.active |= 1u << i;
  auto on = [&](int i) { return (k.active >> i) & 1u; };
  k.label = on(SPECLOSS_CE_LABEL);
  k.target = (k.active & ~(1u << SPECLOSS_CE_LABEL)) != 0;
  if (on(SPECLOSS_KL)) k.need |= SUM_KL;
  if (on(SPECLOSS_RKL)) k.need |= SUM_RKL;
  if (on(SPECLOSS_JSD)) k.need |= SUM_JSD | SUM_EQG;
  if (on(SPECLOSS_TV) || on(SPECLOSS_NLA)) k.need |= SUM_ALPHA | SUM_S;
  if (on(SPECLOSS_LK_HYBRID)) k.need |= SUM_ALPHA | SUM_S | SUM_KL;
  if (k.need) k.need |= SUM_ALPHA;  // alpha is reported whenever a second sweep runs
  k.pass2 = k.need != 0;
  k.dual_bwd = (k.active & ~((1u << SPECLOSS_CE_LABEL) | (1u << SPECLOSS_CE_ARGMAX_P))) != 0;
  k.stage_div = k.dual_bwd && !on(SPECLOSS_RKL) && !on(SPECLOSS_JSD);
  return k;
}

size_t elem_size(const specloss_problem* p) { return p->in_dtype == SPECLOSS_BF16 ? 2 : 4; }

int check_problem(const specloss_problem* p, KindSet* ks) {
  if (!p) return SPECLOSS_E_INVAL;
  if (p->n_rows <= 0 || p->hidden <= 0 || p->vocab <= 0) return SPECLOSS_E_INVAL;
  if (p->n_rows > INT32_MAX / 2 || p->vocab > INT32_MAX / 2 || p->hidden > INT32_MAX / 2)
    return SPECLOSS_E_UNSUPPORTED;
  if (p->flags != 0 && p->flags != SPECLOSS_FLAG_COPIES && p->flags != SPECLOSS_FLAG_NO_COPIES)
    return SPECLOSS_E_INVAL;
  if (p->in_dtype != SPECLOSS_F32 && p->in_dtype != SPECLOSS_BF16) return SPECLOSS_E_UNSUPPORTED;
  if (p->hidden % 64 != 0) return SPECLOSS_E_UNSUPPORTED;
  if (p->flags == SPECLOSS_FLAG_NO_COPIES && p->in_dtype != SPECLOSS_BF16)
    return SPECLOSS_E_UNSUPPORTED;
  if (!p->hidden_states || !p->W) return SPECLOSS_E_INVAL;
  if (!aligned(p->hidden_states, 16) || !aligned(p->W, 16)) return SPECLOSS_E_UNSUPPORTED;
  for (int i = 0; i < kNumKinds; ++i)
    if (!isfinite(p->weights[i])) return SPECLOSS_E_INVAL;
  KindSet k = kinds_of(p->weights);
  if (!k.active) return SPECLOSS_E_INVAL;
  if (k.label) {
    if (!p->labels) return SPECLOSS_E_INVAL;
    if (!aligned(p->labels, 4)) return SPECLOSS_E_UNSUPPORTED;
  }
  if (k.target) {
    if (!p->target_hidden || !p->W_t || p->n_target_rows <= 0) return SPECLOSS_E_INVAL;
    if (p->n_target_rows > INT32_MAX / 2) return SPECLOSS_E_UNSUPPORTED;
    if (!aligned(p->target_hidden, 16) || !aligned(p->W_t, 16)) return SPECLOSS_E_UNSUPPORTED;
    if (p->target_row) {
      if (!aligned(p->target_row, 4)) return SPECLOSS_E_UNSUPPORTED;
      // gathered rows are addressed by 32-bit byte offsets from the tensor base
      if ((uint64_t)p->n_target_rows * (uint64_t)p->hidden * elem_size(p) > 0xFFFFFFFFull)
        return SPECLOSS_E_UNSUPPORTED;
    } else if (p->n_target_rows < p->n_rows) {
      return SPECLOSS_E_INVAL;  // identity map needs a target row per row
    }
  }
  *ks = k;
  return SPECLOSS_OK;
}

// Workspace: a head used by both directions, then the forward and backward
// regions, which overlap (the two directions never run at the same time on
// one workspace).
struct Layout {
  int64_t N, H, V, Vp, Tv, Nc;
  size_t es;
  bool copies;  // the backward contractions read transposed copies (W^T, h^T, dz^T)
  // head
  size_t terms, saved, seed, tstat, head_end;
  // rows share target rows (a row map onto fewer target rows than rows): the
  // target statistics are computed once per target row, then gathered
  bool shared_target;
  int64_t Nt;
  // forward
  size_t pz, pu, p2, zy, fwd_end;
  // backward
  size_t wt, ht, dz, dzt, bwd_end;
  // single-call forward+backward: forward partials and backward buffers at once
  size_t f_pz, f_pu, f_p2, f_zy, f_wt, f_ht, f_dz, f_dd, f_dzt, fused_end;
};

// copies: make transposed copies for the backward contractions (always for
// fp32).  Without them (bf16 only) the contractions read W, h and dz as
// MN-major operands through the transposing LDS load, which needs about half
// the workspace but runs the contractions about 1.5x slower.
Layout plan(const specloss_problem* p, const KindSet& k, int64_t Nc, bool copies = true) {
  Layout L;
  L.N = p->n_rows;
  L.H = p->hidden;
  L.V = p->vocab;
  L.Vp = round_up(L.V, kVocabTile);
  L.Tv = L.Vp / kVocabTile;
  L.Nc = Nc;
  L.es = elem_size(p);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, kAlign);
    return at;
  };
  L.shared_target = k.target && p->target_row && p->n_target_rows < p->n_rows;
  L.Nt = p->n_target_rows;
  L.terms = take((size_t)kNumKinds * L.N * 4);
  L.saved = take(specloss_saved_bytes(L.N));
  L.seed = take((size_t)L.N * 4);
  L.tstat = take(L.shared_target ? 3 * align_up((size_t)L.Nt * 4, kAlign) : 0);
  L.head_end = o;
  const size_t tile_cols = (size_t)L.Tv * Nc * 4;
  L.pz = take(2 * tile_cols);
  L.pu = take(k.target ? 4 * tile_cols : 0);
  L.p2 = take(k.pass2 ? (size_t)kNumSums * tile_cols : 0);
  L.zy = take(2 * (size_t)Nc * 4);
  L.fwd_end = o;
  L.copies = copies || L.es == 4;
  o = L.head_end;
  L.wt = take(L.copies ? (size_t)L.H * L.Vp * L.es : 0);
  L.ht = take(L.copies ? (size_t)L.H * Nc * L.es : 0);
  L.dz = take((size_t)Nc * L.Vp * L.es);
  L.dzt = take(L.copies ? (size_t)L.Vp * Nc * L.es : 0);
  L.bwd_end = o;
  o = L.head_end;
  L.f_pz = take(2 * tile_cols);
  L.f_pu = take(k.target ? 4 * tile_cols : 0);
  L.f_p2 = take(k.stage_div ? (size_t)kNumSums * tile_cols : 0);
  L.f_zy = take(2 * (size_t)Nc * 4);
  L.f_wt = take(L.copies ? (size_t)L.H * L.Vp * L.es : 0);
  L.f_ht = take(L.copies ? (size_t)L.H * Nc * L.es : 0);
  L.f_dz = take((size_t)Nc * L.Vp * L.es);
  L.f_dd = take(k.stage_div ? (size_t)Nc * L.Vp * L.es : 0);
  L.f_dzt = take(L.copies ? (size_t)L.Vp * Nc * L.es : 0);
  L.fused_end = o;
  return L;
}

// largest chunk (multiple of 256, at most the padded row count) whose region fits
enum Region { REGION_FWD, REGION_BWD, REGION_FUSED };

size_t region_end(const Layout& L, Region r) {
  return r == REGION_FWD ? L.fwd_end : (r == REGION_BWD ? L.bwd_end : L.fused_end);
}

// Largest chunk (multiple of 256) whose region fits.
int64_t largest_chunk(const specloss_problem* p, const KindSet& k, size_t ws_bytes,
                      Region region, bool copies) {
  const int64_t top = round_up(p->n_rows, kChunkQuantum);
  int64_t lo = 1, hi = top / kChunkQuantum, best = 0;
  while (lo <= hi) {  // the requirement grows with the chunk
    const int64_t mid = (lo + hi) / 2;
    const Layout L = plan(p, k, mid * kChunkQuantum, copies);
    if (region_end(L, region) <= ws_bytes) {
      best = mid;
      lo = mid + 1;
    } else {
      hi = mid - 1;
    }
  }
  return best * kChunkQuantum;
}

// Chunk for a region, and (backward regions) whether to make transposed
// copies: with copies when the workspace holds them at a chunk of at least
// min(N, 1024) rows; otherwise (bf16) without, if that allows a larger chunk.
// (The copy-free contractions run about 1.5x slower; below about 1000 rows
// per chunk the fp32 read-modify-write of dW per chunk costs more than that
// at the large shapes.)
// flags force the choice (SPECLOSS_FLAG_COPIES / _NO_COPIES).
int64_t pick_chunk(const specloss_problem* p, const KindSet& k, size_t ws_bytes, Region region,
                   bool* copies = nullptr) {
  if (copies && p->flags == SPECLOSS_FLAG_NO_COPIES) {
    *copies = false;
    return largest_chunk(p, k, ws_bytes, region, false);
  }
  int64_t nc = largest_chunk(p, k, ws_bytes, region, true);
  if (copies) *copies = true;
  if (!copies) return nc;
  const int64_t top = round_up(p->n_rows, kChunkQuantum);
  if (p->flags == 0 && p->in_dtype == SPECLOSS_BF16 && nc < (top < 1024 ? top : 1024)) {
    const int64_t without = largest_chunk(p, k, ws_bytes, region, false);
    if (without > nc) {
      *copies = false;
      return without;
    }
  }
  return nc;
}

SavedView saved_view(void* base, int64_t n) {
  const size_t stride = align_up((size_t)n * 4, kAlign);
  char* b = static_cast<char*>(base);
  SavedView v;
  v.lse_q = reinterpret_cast<float*>(b + 0 * stride);
  v.lse_p = reinterpret_cast<float*>(b + 1 * stride);
  v.y_label = reinterpret_cast<int32_t*>(b + 2 * stride);
  v.y_arg = reinterpret_cast<int32_t*>(b + 3 * stride);
  v.alpha = reinterpret_cast<float*>(b + 4 * stride);
  v.S = reinterpret_cast<float*>(b + 5 * stride);
  v.rkl = reinterpret_cast<float*>(b + 6 * stride);
  v.eqg = reinterpret_cast<float*>(b + 7 * stride);
  v.flags = reinterpret_cast<int32_t*>(b + 8 * stride);
  v.flat = reinterpret_cast<float*>(b + 9 * stride);
  return v;
}

GemmOperand op(const void* base, int64_t ld, int64_t n_rows, const int32_t* map = nullptr,
               int64_t map_len = 0) {
  GemmOperand g{};
  g.base = base;
  g.ld = ld;
  g.n_rows = (int32_t)n_rows;
  g.map = map;
  g.map_len = (int32_t)map_len;
  return g;
}

const void* offset_rows(const void* base, int64_t rows, int64_t H, size_t es) {
  return static_cast<const char*>(base) + (size_t)rows * H * es;
}

// target-side B operand for chunk rows [r0, r0 + rows)
GemmOperand target_operand(const specloss_problem* p, int64_t r0, int64_t rows, size_t es) {
  if (p->target_row) return op(p->target_hidden, p->hidden, p->n_target_rows, p->target_row + r0, rows);
  return op(offset_rows(p->target_hidden, r0, p->hidden, es), p->hidden, rows);
}

#define HIP_TRY(expr)                                   \
  do {                                                  \
    if ((expr) != hipSuccess) return SPECLOSS_E_HIP;    \
  } while (0)

enum KernelId : int32_t {
  K_VALIDITY, K_STATS_Q, K_STATS_P, K_COMBINE1, K_ROWDOT, K_DIV, K_COMBINE2, K_REDUCE, K_COPY,
  K_SEED, K_TRANSPOSE_W, K_TRANSPOSE_H, K_DZ, K_GEMM_DH, K_GEMM_DW, K_STATS_STAGE, K_DZ_STAGE,
  K_DIV_STAGE, K_DZ_DIV, K_TILE_SUM, K_SUM_PARTS, K_TARGET_GATHER, K_NUM_IDS
};
const char* const kKernelNames[K_NUM_IDS] = {
    "validity", "stats_q", "stats_p", "combine1", "rowdot", "div", "combine2", "reduce",
    "copy_lse", "seed", "transpose_W", "transpose_h", "dz", "gemm_dh", "gemm_dW",
    "stats_stage", "dz_stage", "div_stage", "dz_div", "tile_sum", "sum_partials",
    "target_gather"};

// Brackets launches with the trace's events when the problem carries one.
struct Tracer {
  specloss_trace* t;
  hipStream_t s;
  int begin(int32_t id, double work);
  void end(int i);
};

#define TRACED(tr, id, work, expr)                       \
  do {                                                   \
    const int ti_ = (tr).begin((id), (work));            \
    const hipError_t e_ = (expr);                        \
    (tr).end(ti_);                                       \
    if (e_ != hipSuccess) return SPECLOSS_E_HIP;         \
  } while (0)

}  // namespace

struct specloss_trace {
  int32_t capacity;
  int32_t count;
  hipEvent_t* ev;  // 2 * capacity: begin, end
  int32_t* ids;
  double* work;
};

namespace {
int Tracer::begin(int32_t id, double w) {
  if (!t) return -1;
  const int i = t->count++;
  if (i >= t->capacity) return -1;
  t->ids[i] = id;
  t->work[i] = w;
  (void)hipEventRecord(t->ev[2 * i], s);
  return i;
}
void Tracer::end(int i) {
  if (t && i >= 0) (void)hipEventRecord(t->ev[2 * i + 1], s);
}
}  // namespace

namespace {

struct FwdBufs {
  float* pz;   // q-side partials [2][Tv][Nc]
  float* pu;   // p-side partials [4][Tv][Nc]
  float* p2;   // pass-2 partials [kNumSums][Tv][Nc]
  float* zy;   // gathered logits [2][Nc]
  int64_t Nc;
  void* tstat = nullptr;  // per-target-row lse_p, argmax, flatness (shared targets)
};

// Target statistics once per target row (rows that share target rows):
// pass 1 of W_t over target_hidden in chunks of Nc rows, merged per target row
// into b.tstat.
int target_prepass(const specloss_problem* p, const Layout& L, const FwdBufs& b, Tracer& tr,
                   hipStream_t stream) {
  const bool bf16 = p->in_dtype == SPECLOSS_BF16;
  const int64_t H = L.H, Nc = b.Nc, tile_cols = L.Tv * Nc;
  char* tb = static_cast<char*>(b.tstat);
  const size_t fs = align_up((size_t)L.Nt * 4, kAlign);
  for (int64_t t0 = 0; t0 < L.Nt; t0 += Nc) {
    const int64_t rows = (L.Nt - t0) < Nc ? (L.Nt - t0) : Nc;
    StatsLaunch su{};
    su.A = op(p->W_t, H, p->vocab);
    su.B = op(offset_rows(p->target_hidden, t0, H, L.es), H, rows);
    su.k_len = (int32_t)H;
    su.vocab = (int32_t)p->vocab;
    su.tiles_m = (int32_t)L.Tv;
    su.tiles_n = (int32_t)cdiv(rows, 256);
    su.ncols = (int32_t)rows;
    su.ldp = (int32_t)Nc;
    su.pm = b.pu;
    su.ps = b.pu + tile_cols;
    su.pi = reinterpret_cast<int32_t*>(b.pu + 2 * tile_cols);
    su.pq = b.pu + 3 * tile_cols;
    TRACED(tr, K_STATS_P, 2.0 * rows * H * p->vocab, launch_stats(bf16, true, su, stream));
    Combine1Launch c1{};
    c1.tiles_m = (int32_t)L.Tv;
    c1.ncols = (int32_t)rows;
    c1.ldp = (int32_t)Nc;
    c1.pm_u = b.pu;
    c1.ps_u = b.pu + tile_cols;
    c1.pi_u = reinterpret_cast<const int32_t*>(b.pu + 2 * tile_cols);
    c1.pq_u = b.pu + 3 * tile_cols;
    c1.vocab = (int32_t)p->vocab;
    c1.lse_p = reinterpret_cast<float*>(tb) + t0;
    c1.y_arg = reinterpret_cast<int32_t*>(tb + fs) + t0;
    c1.flat = reinterpret_cast<float*>(tb + 2 * fs) + t0;
    TRACED(tr, K_COMBINE1, 4.0 * L.Tv * rows * 4, launch_combine1(c1, stream));
  }
  return SPECLOSS_OK;
}

int launch_validity_for(const specloss_problem* p, const KindSet& k, const SavedView& sv,
                        int64_t* counts, Tracer& tr, hipStream_t stream, int64_t vocab = 0) {
  ValidityLaunch va{};
  va.n = p->n_rows;
  va.mask = p->mask;
  va.labels = p->labels;
  va.use_labels = k.label;
  va.target_row = p->target_row;
  va.n_target = p->n_target_rows;
  va.use_target = k.target;
  va.vocab = (int32_t)(vocab > 0 ? vocab : p->vocab);
  va.flags = sv.flags;
  va.y_label = sv.y_label;
  va.counts = counts;
  TRACED(tr, K_VALIDITY, (double)p->n_rows * 10, launch_validity(va, stream));
  return SPECLOSS_OK;
}

// Forward of chunk rows [r0, r0 + rows): pass 1 (q side; p side with argmax
// and flatness), merge, label-logit gather, pass 2 and the per-row losses.
// Staging for the logit gradient ([Nc][Vp] buffers): with `stage` alone,
// pass 1 stores e = exp(z - m_tile) there; with `stage` and `stage_d`,
// pass 2 stores q there and q - p in stage_d.
// Pass-1 contractions of chunk rows [r0, r0 + rows) into the per-(tile, row)
// partials b.pz (and b.pu for the target side); `stage` as for fwd_chunk.
int launch_pass1(const specloss_problem* p, const KindSet& k, const Layout& L, const FwdBufs& b,
                 int64_t r0, int64_t rows, void* stage, Tracer& tr, hipStream_t stream,
                 bool skip_target = false) {
  const bool bf16 = p->in_dtype == SPECLOSS_BF16;
  const int64_t H = L.H, Nc = b.Nc;
  const int64_t tile_cols = L.Tv * Nc;
  const GemmOperand Bh = op(offset_rows(p->hidden_states, r0, H, L.es), H, rows);

  StatsLaunch sz{};
  sz.A = op(p->W, H, p->vocab);
  sz.B = Bh;
  sz.k_len = (int32_t)H;
  sz.vocab = (int32_t)p->vocab;
  sz.tiles_m = (int32_t)L.Tv;
  sz.tiles_n = (int32_t)cdiv(rows, 256);
  sz.ncols = (int32_t)rows;
  sz.ldp = (int32_t)Nc;
  sz.pm = b.pz;
  sz.ps = b.pz + tile_cols;
  sz.pi = nullptr;
  sz.pq = nullptr;
  if (stage) {
    StatsStageLaunch ss{};
    ss.st = sz;
    ss.stage = stage;
    ss.ld_stage = L.Vp;
    TRACED(tr, K_STATS_STAGE, 2.0 * rows * H * p->vocab, launch_stats_stage(bf16, ss, stream));
  } else {
    TRACED(tr, K_STATS_Q, 2.0 * rows * H * p->vocab, launch_stats(bf16, false, sz, stream));
  }

  if (k.target && !skip_target) {
    StatsLaunch su = sz;
    su.A = op(p->W_t, H, p->vocab);
    su.B = target_operand(p, r0, rows, L.es);
    su.pm = b.pu;
    su.ps = b.pu + tile_cols;
    su.pi = reinterpret_cast<int32_t*>(b.pu + 2 * tile_cols);
    su.pq = b.pu + 3 * tile_cols;
    TRACED(tr, K_STATS_P, 2.0 * rows * H * p->vocab, launch_stats(bf16, true, su, stream));
  }
  return SPECLOSS_OK;
}

// Pass-2 divergence sums of chunk rows [r0, r0 + rows) into b.p2, with the
// final logsumexps in `sv`; stage_q / stage_d as for fwd_chunk (or null).
int launch_pass2(const specloss_problem* p, const KindSet& k, const Layout& L, const FwdBufs& b,
                 const SavedView& sv, int64_t r0, int64_t rows, void* stage_q, void* stage_d,
                 Tracer& tr, hipStream_t stream) {
  const bool bf16 = p->in_dtype == SPECLOSS_BF16;
  const int64_t H = L.H, Nc = b.Nc;
  DivLaunch dv{};
  dv.Az = op(p->W, H, p->vocab);
  dv.Bz = op(offset_rows(p->hidden_states, r0, H, L.es), H, rows);
  dv.Au = op(p->W_t, H, p->vocab);
  dv.Bu = target_operand(p, r0, rows, L.es);
  dv.k_len = (int32_t)H;
  dv.vocab = (int32_t)p->vocab;
  dv.tiles_m = (int32_t)L.Tv;
  dv.tiles_n = (int32_t)cdiv(rows, 128);
  dv.ncols = (int32_t)rows;
  dv.ldp = (int32_t)Nc;
  dv.lse_q = sv.lse_q + r0;
  dv.lse_p = sv.lse_p + r0;
  dv.need = k.need;
  dv.part = b.p2;
  dv.part_stride = L.Tv * Nc;
  dv.stage_q = stage_d ? stage_q : nullptr;
  dv.stage_d = stage_d;
  dv.ld_stage = L.Vp;
  TRACED(tr, stage_d ? K_DIV_STAGE : K_DIV, 4.0 * rows * H * p->vocab,
         launch_div(bf16, dv, stream));
  return SPECLOSS_OK;
}

int fwd_chunk(const specloss_problem* p, const KindSet& k, const Layout& L, const FwdBufs& b,
              const SavedView& sv, float* loss, float* terms, int64_t r0, int64_t rows,
              void* stage, void* stage_d, Tracer& tr, hipStream_t stream) {
  const bool bf16 = p->in_dtype == SPECLOSS_BF16;
  const int64_t H = L.H, Nc = b.Nc;
  const int64_t tile_cols = L.Tv * Nc;
  const bool own_target = k.target && !L.shared_target;
  {
    const int rc = launch_pass1(p, k, L, b, r0, rows, stage_d ? nullptr : stage, tr, stream,
                                !own_target);
    if (rc) return rc;
  }

  Combine1Launch c1{};
  c1.tiles_m = (int32_t)L.Tv;
  c1.ncols = (int32_t)rows;
  c1.ldp = (int32_t)Nc;
  c1.pm_z = b.pz;
  c1.ps_z = b.pz + tile_cols;
  c1.pm_u = own_target ? b.pu : nullptr;
  c1.ps_u = own_target ? b.pu + tile_cols : nullptr;
  c1.pi_u = own_target ? reinterpret_cast<const int32_t*>(b.pu + 2 * tile_cols) : nullptr;
  c1.pq_u = own_target ? b.pu + 3 * tile_cols : nullptr;
  c1.vocab = (int32_t)p->vocab;
  c1.flags = sv.flags + r0;
  c1.lse_q = sv.lse_q + r0;
  c1.lse_p = sv.lse_p + r0;
  c1.y_arg = sv.y_arg + r0;
  c1.flat = sv.flat + r0;
  TRACED(tr, K_COMBINE1, (own_target ? 6.0 : 2.0) * L.Tv * rows * 4, launch_combine1(c1, stream));
  if (L.shared_target) {
    const char* tb = reinterpret_cast<const char*>(b.tstat);
    const size_t fs = align_up((size_t)L.Nt * 4, kAlign);
    TargetGatherLaunch tg{};
    tg.ncols = (int32_t)rows;
    tg.r0 = r0;
    tg.flags = sv.flags;
    tg.target_row = p->target_row;
    tg.t_lse_p = reinterpret_cast<const float*>(tb);
    tg.t_y_arg = reinterpret_cast<const int32_t*>(tb + fs);
    tg.t_flat = reinterpret_cast<const float*>(tb + 2 * fs);
    tg.lse_p = sv.lse_p;
    tg.y_arg = sv.y_arg;
    tg.flat = sv.flat;
    TRACED(tr, K_TARGET_GATHER, (double)rows * 24, launch_target_gather(tg, stream));
  }

  const bool ce_lab = (k.active >> SPECLOSS_CE_LABEL) & 1u;
  const bool ce_arg = (k.active >> SPECLOSS_CE_ARGMAX_P) & 1u;
  if (ce_lab || ce_arg) {
    RowdotLaunch rd{};
    rd.W = p->W;
    rd.h = offset_rows(p->hidden_states, r0, H, L.es);
    rd.H = H;
    rd.ncols = (int32_t)rows;
    rd.vocab = (int32_t)p->vocab;
    rd.y1 = ce_lab ? sv.y_label + r0 : nullptr;
    rd.y2 = ce_arg ? sv.y_arg + r0 : nullptr;
    rd.out1 = b.zy;
    rd.out2 = b.zy + Nc;
    TRACED(tr, K_ROWDOT, 2.0 * rows * H * L.es * ((ce_lab ? 1 : 0) + (ce_arg ? 1 : 0)),
           launch_rowdot(bf16, rd, stream));
  }

  if (k.pass2) {
    const int rc = launch_pass2(p, k, L, b, sv, r0, rows, stage, stage_d, tr, stream);
    if (rc) return rc;
  }

  Combine2Launch c2{};
  c2.tiles_m = (int32_t)L.Tv;
  c2.ncols = (int32_t)rows;
  c2.ldp = (int32_t)Nc;
  c2.part = b.p2;
  c2.part_stride = tile_cols;
  c2.need = k.need;
  memcpy(c2.w, p->weights, sizeof(c2.w));
  c2.flags = sv.flags + r0;
  c2.lse_q = sv.lse_q + r0;
  c2.zy_lab = ce_lab ? b.zy : nullptr;
  c2.zy_arg = ce_arg ? b.zy + Nc : nullptr;
  c2.zy_count = 1;
  c2.loss = loss + r0;
  c2.term = terms + r0;
  c2.term_stride = p->n_rows;
  c2.alpha = sv.alpha + r0;
  c2.S = sv.S + r0;
  c2.rkl = sv.rkl + r0;
  c2.eqg = sv.eqg + r0;
  TRACED(tr, K_COMBINE2, (double)rows * 4 * (2 + __builtin_popcount(k.need) * L.Tv),
         launch_combine2(c2, stream));
  return SPECLOSS_OK;
}

int launch_reduce_for(const specloss_problem* p, const KindSet& k, const float* loss,
                      const float* terms, const int64_t* counts, float* reduced, Tracer& tr,
                      hipStream_t stream) {
  ReduceLaunch rl{};
  rl.n = p->n_rows;
  rl.loss = loss;
  rl.term = terms;
  rl.term_stride = p->n_rows;
  rl.active = k.active;
  rl.counts = counts;
  rl.reduced = reduced;
  TRACED(tr, K_REDUCE, (double)p->n_rows * 4 * (1 + __builtin_popcount(k.active)),
         launch_reduce(rl, stream));
  return SPECLOSS_OK;
}

int launch_seed_for(const specloss_problem* p, const SavedView& sv, const float* grad_loss,
                    const float* grad_mean, const int64_t* counts, float* seed, Tracer& tr,
                    hipStream_t stream) {
  SeedLaunch sd{};
  sd.n = p->n_rows;
  sd.flags = sv.flags;
  sd.grad_loss = grad_loss;
  sd.grad_mean = grad_mean;
  sd.counts = counts;
  sd.seed = seed;
  TRACED(tr, K_SEED, (double)p->n_rows * 12, launch_seed(sd, stream));
  return SPECLOSS_OK;
}

// dh rows [r0, r0 + rows) = dz W for one chunk from the staged dz [Nc][Vp]
// and the copy W^T [H][Vp]; without copies (bf16), W is read as it is (an
// MN-major operand).
int contract_dh(const specloss_problem* p, const Layout& L, int64_t Nc, const void* dz,
                const void* wt, int64_t r0, int64_t rows, void* dhidden, int32_t dh_dtype,
                Tracer& tr, hipStream_t stream) {
  const bool bf16 = p->in_dtype == SPECLOSS_BF16;
  const int64_t H = L.H, V = L.V, Vp = L.Vp;
  const size_t dh_es = dh_dtype == SPECLOSS_BF16 ? 2 : 4;
  GemmLaunch g{};
  g.A = op(dz, Vp, Nc);
  g.lean = !L.copies;
  if (g.lean) {
    g.B = op(p->W, H, H);  // element (h, v) at W[v * H + h]
    g.B.k_valid = (int32_t)V;
    g.k_len = (int32_t)round_up(V, 64);
  } else {
    g.B = op(wt, Vp, H);
    g.k_len = (int32_t)Vp;
  }
  g.tiles_m = (int32_t)cdiv(rows, 256);
  g.tiles_n = (int32_t)cdiv(H, 256);
  g.m_valid = (int32_t)rows;
  g.n_valid = (int32_t)H;
  g.C = static_cast<char*>(dhidden) + (size_t)r0 * H * dh_es;
  g.ldc = H;
  g.accumulate = 0;
  g.out_bf16 = dh_dtype == SPECLOSS_BF16;
  g.role = 0;
  TRACED(tr, K_GEMM_DH, 2.0 * rows * H * V, launch_gemm(bf16, g, stream));
  return SPECLOSS_OK;
}

// dW (+)= dz^T h over `rows` consecutive rows starting at global row r0:
// with copies from dz^T [Vp][ld] and h^T [H][ld] (their first `rows` columns;
// columns up to the next multiple of 64 hold zeros); without copies (bf16)
// from dz [Nc][Vp] and the hidden rows themselves (MN-major operands).
int contract_dW(const specloss_problem* p, const Layout& L, int64_t Nc, const void* dz,
                const void* dzt, const void* ht, int64_t ld, int64_t r0, int64_t rows,
                bool accumulate, float* dW, Tracer& tr, hipStream_t stream) {
  const bool bf16 = p->in_dtype == SPECLOSS_BF16;
  const int64_t H = L.H, V = L.V, Vp = L.Vp;
  GemmLaunch g{};
  g.k_len = (int32_t)round_up(rows, 64);
  g.lean = !L.copies;
  if (g.lean) {
    g.A = op(dz, Vp, Vp);  // element (v, c) at dz[c * Vp + v]; rows >= `rows` hold 0
    g.A.k_valid = (int32_t)Nc;
    g.B = op(offset_rows(p->hidden_states, r0, H, L.es), H, H);  // (h, c) at h[c * H + h]
    g.B.k_valid = (int32_t)(L.N - r0);
  } else {
    g.A = op(dzt, ld, Vp);
    g.B = op(ht, ld, H);
  }
  g.tiles_m = (int32_t)L.Tv;
  g.tiles_n = (int32_t)cdiv(H, 256);
  g.m_valid = (int32_t)V;
  g.n_valid = (int32_t)H;
  g.C = dW;
  g.ldc = H;
  g.accumulate = accumulate ? 1 : 0;
  g.out_bf16 = 0;
  g.role = 1;
  TRACED(tr, K_GEMM_DW, 2.0 * rows * H * V, launch_gemm(bf16, g, stream));
  return SPECLOSS_OK;
}

#define TRY(expr)                   \
  do {                              \
    const int rc_ = (expr);         \
    if (rc_) return rc_;            \
  } while (0)

int check_fwd_outputs(const float* loss, const float* term_loss, const float* lse_q,
                      const void* saved, const int64_t* counts, const float* reduced) {
  if (!loss || !counts) return SPECLOSS_E_INVAL;
  if (!aligned(loss, 4) || !aligned(term_loss, 4) || !aligned(lse_q, 4) || !aligned(saved, 4) ||
      !aligned(counts, 8) || !aligned(reduced, 4))
    return SPECLOSS_E_UNSUPPORTED;
  return SPECLOSS_OK;
}

int check_bwd_args(const float* grad_loss, const float* grad_mean, void* dhidden,
                   int32_t dh_dtype, float* dW) {
  if (!grad_loss && !grad_mean) return SPECLOSS_E_INVAL;
  if (!dhidden && !dW) return SPECLOSS_E_INVAL;
  if (dh_dtype != SPECLOSS_F32 && dh_dtype != SPECLOSS_BF16) return SPECLOSS_E_UNSUPPORTED;
  if (!aligned(grad_loss, 4) || !aligned(grad_mean, 4) || !aligned(dW, 16) ||
      !aligned(dhidden, 16))
    return SPECLOSS_E_UNSUPPORTED;
  return SPECLOSS_OK;
}

int check_bwd_inputs(const float* grad_loss, const float* grad_mean, const int64_t* counts,
                     const void* saved, void* dhidden, int32_t dh_dtype, float* dW,
                     void* workspace) {
  if (!saved || !counts) return SPECLOSS_E_INVAL;
  TRY(check_bwd_args(grad_loss, grad_mean, dhidden, dh_dtype, dW));
  if (!aligned(counts, 8) || !aligned(saved, 4)) return SPECLOSS_E_UNSUPPORTED;
  if (!workspace || !aligned(workspace, kAlign)) return SPECLOSS_E_WORKSPACE;
  return SPECLOSS_OK;
}

// Backward by recompute: per chunk, the logit gradient tile is recomputed from
// the saved per-row state, staged in two layouts and contracted into dh, dW.
// vocab_offset: global index of W's first row (saved labels are global).
int bwd_recompute(const specloss_problem* p, const KindSet& k, const float* grad_loss,
                  const float* grad_mean, const int64_t* counts, const void* saved,
                  void* workspace, size_t ws_bytes, void* dhidden, int32_t dh_dtype, float* dW,
                  int accumulate_dW, int64_t vocab_offset, hipStream_t stream) {
  bool with_copies = true;
  const int64_t Nc = pick_chunk(p, k, ws_bytes, REGION_BWD, &with_copies);
  if (Nc <= 0) return SPECLOSS_E_WORKSPACE;
  const Layout L = plan(p, k, Nc, with_copies);
  char* ws = static_cast<char*>(workspace);
  const bool bf16 = p->in_dtype == SPECLOSS_BF16;
  const int64_t N = L.N, H = L.H, V = L.V, Vp = L.Vp;
  const SavedView sv = saved_view(const_cast<void*>(saved), N);
  float* seed = reinterpret_cast<float*>(ws + L.seed);
  const bool copies = L.copies;
  void* wt = copies ? ws + L.wt : nullptr;
  void* ht = copies ? ws + L.ht : nullptr;
  void* dz = ws + L.dz;
  void* dzt = copies ? ws + L.dzt : nullptr;
  Tracer tr{p->trace, stream};

  TRY(launch_seed_for(p, sv, grad_loss, grad_mean, counts, seed, tr, stream));
  if (dhidden && copies)
    TRACED(tr, K_TRANSPOSE_W, 2.0 * Vp * H * L.es, launch_transpose(bf16, p->W, V, H, wt, Vp, stream));

  int chunk = 0;
  for (int64_t r0 = 0; r0 < N; r0 += Nc, ++chunk) {
    const int64_t rows = (N - r0) < Nc ? (N - r0) : Nc;
    const void* hc = offset_rows(p->hidden_states, r0, H, L.es);
    if (dW && copies)
      TRACED(tr, K_TRANSPOSE_H, 2.0 * Nc * H * L.es, launch_transpose(bf16, hc, rows, H, ht, Nc, stream));

    DzLaunch dl{};
    dl.Az = op(p->W, H, V);
    dl.Bz = op(hc, H, rows);
    if (k.dual_bwd) {
      dl.Au = op(p->W_t, H, V);
      dl.Bu = target_operand(p, r0, rows, L.es);
    } else {
      dl.Au = dl.Az;
      dl.Bu = dl.Bz;
    }
    dl.k_len = (int32_t)H;
    dl.vocab = (int32_t)V;
    dl.tiles_m = (int32_t)L.Tv;
    dl.tiles_n = (int32_t)cdiv(rows, k.dual_bwd ? 128 : 256);
    dl.ncols = (int32_t)rows;
    dl.r0 = r0;
    dl.seed = seed;
    dl.sv = sv;
    memcpy(dl.w, p->weights, sizeof(dl.w));
    dl.dz = dz;
    dl.ld_dz = Vp;
    dl.dzt = dzt;
    dl.ld_dzt = Nc;
    dl.vocab_offset = (int32_t)vocab_offset;
    TRACED(tr, K_DZ, (k.dual_bwd ? 4.0 : 2.0) * rows * H * V, launch_dz(bf16, k.dual_bwd, dl, stream));
    if (dhidden) TRY(contract_dh(p, L, Nc, dz, wt, r0, rows, dhidden, dh_dtype, tr, stream));
    if (dW)
      TRY(contract_dW(p, L, Nc, dz, dzt, ht, Nc, r0, rows, chunk > 0 || accumulate_dW, dW, tr,
                      stream));
  }
  return SPECLOSS_OK;
}

// ---- vocabulary-parallel variant ----
// Exchange buffer: part 1 = m_q, s_q, m_p, s_p, q2_p, argmax (global index);
// part 2 = the kNumSums divergence sums, label logit, argmax-p logit.  Each
// field is [G][Ns] 4-byte entries, Ns = N rounded up to 64.
constexpr int kExch1 = 6, kExch2 = kNumSums + 2;

struct Exchange {
  char* base;
  int64_t Ns;
  int32_t G;
  float* f(int field) const { return reinterpret_cast<float*>(base) + (int64_t)field * G * Ns; }
  float* at(int field, int g, int64_t r0 = 0) const { return f(field) + (int64_t)g * Ns + r0; }
};

Exchange exchange_of(const specloss_shard* sh, int64_t n) {
  return Exchange{static_cast<char*>(sh->exchange), round_up(n, 64), sh->n_shards};
}

int check_shard(const specloss_problem* p, const specloss_shard* sh) {
  if (!sh || !sh->exchange) return SPECLOSS_E_INVAL;
  if (!aligned(sh->exchange, kAlign)) return SPECLOSS_E_UNSUPPORTED;
  if (sh->n_shards < 1 || sh->shard < 0 || sh->shard >= sh->n_shards) return SPECLOSS_E_INVAL;
  if (sh->vocab_total <= 0 || sh->vocab_total > INT32_MAX / 2) return SPECLOSS_E_INVAL;
  if (sh->vocab_offset < 0 || sh->vocab_offset + p->vocab > sh->vocab_total)
    return SPECLOSS_E_INVAL;
  return SPECLOSS_OK;
}

}  // namespace

extern "C" {

size_t specloss_saved_bytes(int64_t n_rows) {
  if (n_rows <= 0) return 0;
  return (size_t)SPECLOSS_SAVED_FIELDS * align_up((size_t)n_rows * 4, kAlign);
}

int specloss_saved_offset(int64_t n_rows, int32_t field, size_t* offset) {
  if (n_rows <= 0 || field < 0 || field >= SPECLOSS_SAVED_FIELDS || !offset)
    return SPECLOSS_E_INVAL;
  *offset = (size_t)field * align_up((size_t)n_rows * 4, kAlign);
  return SPECLOSS_OK;
}

int lmhead_loss_workspace_size(const specloss_problem* p, int64_t max_chunk_rows, size_t* bytes) {
  KindSet k;
  const int rc = check_problem(p, &k);
  if (rc) return rc;
  if (!bytes) return SPECLOSS_E_INVAL;
  int64_t nc = max_chunk_rows <= 0 ? kDefaultChunk : max_chunk_rows;
  nc = round_up(nc, kChunkQuantum);
  nc = nc < round_up(p->n_rows, kChunkQuantum) ? nc : round_up(p->n_rows, kChunkQuantum);
  const Layout L = plan(p, k, nc);
  size_t b = L.fwd_end > L.bwd_end ? L.fwd_end : L.bwd_end;
  if (L.fused_end > b) b = L.fused_end;
  *bytes = b;
  return SPECLOSS_OK;
}

int lmhead_loss_fwd(const specloss_problem* p, void* workspace, size_t ws_bytes, float* loss,
                    float* term_loss, float* lse_q, void* saved, int64_t* counts, float* reduced,
                    hipStream_t stream) {
  KindSet k;
  TRY(check_problem(p, &k));
  TRY(check_fwd_outputs(loss, term_loss, lse_q, saved, counts, reduced));
  if (!workspace || !aligned(workspace, kAlign)) return SPECLOSS_E_WORKSPACE;
  const int64_t Nc = pick_chunk(p, k, ws_bytes, REGION_FWD);
  if (Nc <= 0) return SPECLOSS_E_WORKSPACE;
  const Layout L = plan(p, k, Nc);
  char* ws = static_cast<char*>(workspace);
  const int64_t N = L.N;
  const SavedView sv = saved_view(saved ? saved : ws + L.saved, N);
  float* terms = term_loss ? term_loss : reinterpret_cast<float*>(ws + L.terms);
  const FwdBufs b{reinterpret_cast<float*>(ws + L.pz), reinterpret_cast<float*>(ws + L.pu),
                  reinterpret_cast<float*>(ws + L.p2), reinterpret_cast<float*>(ws + L.zy), Nc,
                  ws + L.tstat};
  Tracer tr{p->trace, stream};

  TRY(launch_validity_for(p, k, sv, counts, tr, stream));
  if (L.shared_target) TRY(target_prepass(p, L, b, tr, stream));
  for (int64_t r0 = 0; r0 < N; r0 += Nc) {
    const int64_t rows = (N - r0) < Nc ? (N - r0) : Nc;
    TRY(fwd_chunk(p, k, L, b, sv, loss, terms, r0, rows, nullptr, nullptr, tr, stream));
  }
  if (reduced) TRY(launch_reduce_for(p, k, loss, terms, counts, reduced, tr, stream));
  if (lse_q)
    TRACED(tr, K_COPY, (double)N * 8,
           hipMemcpyAsync(lse_q, sv.lse_q, (size_t)N * 4, hipMemcpyDeviceToDevice, stream));
  return SPECLOSS_OK;
}

int lmhead_loss_bwd(const specloss_problem* p, const float* grad_loss, const float* grad_mean,
                    const int64_t* counts, const void* saved, void* workspace, size_t ws_bytes,
                    void* dhidden, int32_t dh_dtype, float* dW, int accumulate_dW,
                    hipStream_t stream) {
  KindSet k;
  TRY(check_problem(p, &k));
  TRY(check_bwd_inputs(grad_loss, grad_mean, counts, saved, dhidden, dh_dtype, dW, workspace));
  return bwd_recompute(p, k, grad_loss, grad_mean, counts, saved, workspace, ws_bytes, dhidden,
                       dh_dtype, dW, accumulate_dW, 0, stream);
}

int lmhead_loss_fwd_bwd(const specloss_problem* p, void* workspace, size_t ws_bytes, float* loss,
                        float* term_loss, float* lse_q, void* saved, int64_t* counts,
                        float* reduced, const float* grad_loss, const float* grad_mean,
                        void* dhidden, int32_t dh_dtype, float* dW, int accumulate_dW,
                        hipStream_t stream) {
  KindSet k;
  TRY(check_problem(p, &k));
  TRY(check_fwd_outputs(loss, term_loss, lse_q, saved, counts, reduced));
  TRY(check_bwd_args(grad_loss, grad_mean, dhidden, dh_dtype, dW));
  if (!workspace || !aligned(workspace, kAlign)) return SPECLOSS_E_WORKSPACE;
  if (k.dual_bwd && !k.stage_div) {
    // rkl / jsd gradients need log p and log m per element: the forward and
    // backward sequences run back to back on the same workspace
    char* ws = static_cast<char*>(workspace);
    const Layout L0 = plan(p, k, kChunkQuantum);
    void* sv_base = saved ? saved : ws + L0.saved;
    TRY(lmhead_loss_fwd(p, workspace, ws_bytes, loss, term_loss, lse_q, sv_base, counts, reduced,
                        stream));
    return lmhead_loss_bwd(p, grad_loss, grad_mean, counts, sv_base, workspace, ws_bytes, dhidden,
                           dh_dtype, dW, accumulate_dW, stream);
  }
  // label / argmax cross-entropies: pass 1 stages e = exp(z - m_tile) per
  // chunk; with kl_div / tv / nla / lk_hybrid, pass 2 stages q and q - p.  The
  // logit gradient is formed from the staged values without recomputing logits.
  bool with_copies = true;
  const int64_t Nc = pick_chunk(p, k, ws_bytes, REGION_FUSED, &with_copies);
  if (Nc <= 0) return SPECLOSS_E_WORKSPACE;
  const Layout L = plan(p, k, Nc, with_copies);
  char* ws = static_cast<char*>(workspace);
  const bool bf16 = p->in_dtype == SPECLOSS_BF16;
  const int64_t N = L.N, H = L.H, V = L.V, Vp = L.Vp;
  const SavedView sv = saved_view(saved ? saved : ws + L.saved, N);
  float* terms = term_loss ? term_loss : reinterpret_cast<float*>(ws + L.terms);
  float* seed = reinterpret_cast<float*>(ws + L.seed);
  const FwdBufs b{reinterpret_cast<float*>(ws + L.f_pz), reinterpret_cast<float*>(ws + L.f_pu),
                  k.stage_div ? reinterpret_cast<float*>(ws + L.f_p2) : nullptr,
                  reinterpret_cast<float*>(ws + L.f_zy), Nc, ws + L.tstat};
  const bool copies = L.copies;
  void* wt = copies ? ws + L.f_wt : nullptr;
  void* ht = copies ? ws + L.f_ht : nullptr;
  void* dz = ws + L.f_dz;
  void* dd = k.stage_div ? ws + L.f_dd : nullptr;
  void* dzt = copies ? ws + L.f_dzt : nullptr;
  Tracer tr{p->trace, stream};

  TRY(launch_validity_for(p, k, sv, counts, tr, stream));
  TRY(launch_seed_for(p, sv, grad_loss, grad_mean, counts, seed, tr, stream));
  if (L.shared_target) TRY(target_prepass(p, L, b, tr, stream));
  if (dhidden && copies)
    TRACED(tr, K_TRANSPOSE_W, 2.0 * Vp * H * L.es, launch_transpose(bf16, p->W, V, H, wt, Vp, stream));
  int chunk = 0;
  for (int64_t r0 = 0; r0 < N; r0 += Nc, ++chunk) {
    const int64_t rows = (N - r0) < Nc ? (N - r0) : Nc;
    TRY(fwd_chunk(p, k, L, b, sv, loss, terms, r0, rows, dz, dd, tr, stream));
    DzStageLaunch ds{};
    ds.tiles_m = (int32_t)L.Tv;
    ds.ncols = (int32_t)rows;
    ds.vocab = (int32_t)V;
    ds.ldp = (int32_t)Nc;
    ds.r0 = r0;
    ds.pm = b.pz;
    ds.seed = seed;
    ds.sv = sv;
    ds.w_lab = p->weights[SPECLOSS_CE_LABEL];
    ds.w_arg = p->weights[SPECLOSS_CE_ARGMAX_P];
    ds.w_kl = p->weights[SPECLOSS_KL];
    ds.w_tv = p->weights[SPECLOSS_TV];
    ds.w_nla = p->weights[SPECLOSS_NLA];
    ds.w_lk = p->weights[SPECLOSS_LK_HYBRID];
    ds.dd = dd;
    ds.dz = dz;
    ds.ld_dz = Vp;
    ds.dzt = dzt;
    ds.ld_dzt = Nc;
    ds.row_blocks = (int32_t)(cdiv(rows, 256) * 4);
    TRACED(tr, dd ? K_DZ_DIV : K_DZ_STAGE,
           (double)ds.row_blocks * 64 * Vp * L.es * ((dd ? 3 : 2) + (dzt ? 1 : 0)),
           launch_dz_stage(bf16, ds, stream));
    const void* hc = offset_rows(p->hidden_states, r0, H, L.es);
    if (dW && copies)
      TRACED(tr, K_TRANSPOSE_H, 2.0 * Nc * H * L.es, launch_transpose(bf16, hc, rows, H, ht, Nc, stream));
    if (dhidden) TRY(contract_dh(p, L, Nc, dz, wt, r0, rows, dhidden, dh_dtype, tr, stream));
    if (dW)
      TRY(contract_dW(p, L, Nc, dz, dzt, ht, Nc, r0, rows, chunk > 0 || accumulate_dW, dW, tr,
                      stream));
  }
  if (reduced) TRY(launch_reduce_for(p, k, loss, terms, counts, reduced, tr, stream));
  if (lse_q)
    TRACED(tr, K_COPY, (double)N * 8,
           hipMemcpyAsync(lse_q, sv.lse_q, (size_t)N * 4, hipMemcpyDeviceToDevice, stream));
  return SPECLOSS_OK;
}

int specloss_align_heads(int64_t seq_len, int64_t batch, int32_t n_heads, const int32_t* shifts,
                         const uint8_t* loss_mask, int32_t* target_row_out, uint8_t* mask_out,
                         hipStream_t stream) {
  if (seq_len <= 0 || batch <= 0 || n_heads <= 0 || !shifts || !target_row_out || !mask_out)
    return SPECLOSS_E_INVAL;
  if (n_heads > 64 || seq_len * batch > INT32_MAX / 2 ||
      (int64_t)n_heads * batch * seq_len > INT32_MAX / 2)
    return SPECLOSS_E_UNSUPPORTED;
  if (!aligned(target_row_out, 4)) return SPECLOSS_E_UNSUPPORTED;
  AlignLaunch a{};
  a.seq_len = seq_len;
  a.batch = batch;
  a.n_heads = n_heads;
  for (int i = 0; i < 64; ++i) a.shifts[i] = 0;
  for (int i = 0; i < n_heads; ++i) {
    if (shifts[i] < 0) return SPECLOSS_E_INVAL;
    a.shifts[i] = shifts[i];
  }
  a.loss_mask = loss_mask;
  a.target_row = target_row_out;
  a.mask = mask_out;
  HIP_TRY(launch_align(a, stream));
  return SPECLOSS_OK;
}

specloss_trace* specloss_trace_create(int32_t capacity) {
  if (capacity <= 0 || capacity > (1 << 20)) return nullptr;
  specloss_trace* t = new (std::nothrow) specloss_trace;
  if (!t) return nullptr;
  t->capacity = capacity;
  t->count = 0;
  t->ev = new (std::nothrow) hipEvent_t[2 * (size_t)capacity];
  t->ids = new (std::nothrow) int32_t[capacity];
  t->work = new (std::nothrow) double[capacity];
  int made = 0;
  bool ok = t->ev && t->ids && t->work;
  for (; ok && made < 2 * capacity; ++made)
    if (hipEventCreate(&t->ev[made]) != hipSuccess) ok = false;
  if (!ok) {
    for (int i = 0; i + 1 < made; ++i) (void)hipEventDestroy(t->ev[i]);
    t->capacity = 0;
    specloss_trace_destroy(t);
    return nullptr;
  }
  return t;
}

void specloss_trace_destroy(specloss_trace* t) {
  if (!t) return;
  if (t->ev)
    for (int i = 0; i < 2 * t->capacity; ++i) (void)hipEventDestroy(t->ev[i]);
  delete[] t->ev;
  delete[] t->ids;
  delete[] t->work;
  delete t;
}

void specloss_trace_reset(specloss_trace* t) {
  if (t) t->count = 0;
}

int specloss_trace_read(specloss_trace* t, int32_t max, int32_t* kernel_id, float* ms,
                        double* work, int32_t* count) {
  if (!t || !count || max < 0) return SPECLOSS_E_INVAL;
  *count = t->count;
  const int n = t->count < t->capacity ? t->count : t->capacity;
  for (int i = 0; i < n && i < max; ++i) {
    if (hipEventSynchronize(t->ev[2 * i + 1]) != hipSuccess) return SPECLOSS_E_HIP;
    float e = 0.0f;
    if (hipEventElapsedTime(&e, t->ev[2 * i], t->ev[2 * i + 1]) != hipSuccess) return SPECLOSS_E_HIP;
    if (kernel_id) kernel_id[i] = t->ids[i];
    if (ms) ms[i] = e;
    if (work) work[i] = t->work[i];
  }
  return SPECLOSS_OK;
}

const char* specloss_kernel_name(int32_t id) {
  if (id < 0 || id >= K_NUM_IDS) return nullptr;
  return kKernelNames[id];
}

const char* specloss_strerror(int code) {
  switch (code) {
    case SPECLOSS_OK: return "success";
    case SPECLOSS_E_INVAL: return "invalid argument";
    case SPECLOSS_E_UNSUPPORTED: return "unsupported shape, dtype or alignment";
    case SPECLOSS_E_WORKSPACE: return "workspace missing or too small";
    case SPECLOSS_E_HIP: return "HIP launch failed";
    default: return "unknown error";
  }
}

const char* specloss_kind_name(int kind) {
  static const char* names[kNumKinds] = {"ce_label", "ce", "kl_div", "rkl",
                                         "jsd",      "tv", "nla",    "lk_hybrid"};
  if (kind < 0 || kind >= kNumKinds) return nullptr;
  return names[kind];
}

}  // extern "C"

extern "C" {

size_t specloss_exchange_bytes(int64_t n_rows, int32_t n_shards) {
  if (n_rows <= 0 || n_shards <= 0) return 0;
  return (size_t)(kExch1 + kExch2) * n_shards * round_up(n_rows, 64) * 4;
}

int lmhead_shard_pass1(const specloss_problem* p, const specloss_shard* sh, void* workspace,
                       size_t ws_bytes, hipStream_t stream) {
  KindSet k;
  TRY(check_problem(p, &k));
  TRY(check_shard(p, sh));
  if (!workspace || !aligned(workspace, kAlign)) return SPECLOSS_E_WORKSPACE;
  const int64_t Nc = pick_chunk(p, k, ws_bytes, REGION_FWD);
  if (Nc <= 0) return SPECLOSS_E_WORKSPACE;
  const Layout L = plan(p, k, Nc);
  char* ws = static_cast<char*>(workspace);
  const FwdBufs b{reinterpret_cast<float*>(ws + L.pz), reinterpret_cast<float*>(ws + L.pu),
                  reinterpret_cast<float*>(ws + L.p2), reinterpret_cast<float*>(ws + L.zy), Nc};
  const Exchange X = exchange_of(sh, L.N);
  const int g = sh->shard;
  const int64_t tile_cols = L.Tv * Nc;
  Tracer tr{p->trace, stream};
  for (int64_t r0 = 0; r0 < L.N; r0 += Nc) {
    const int64_t rows = (L.N - r0) < Nc ? (L.N - r0) : Nc;
    TRY(launch_pass1(p, k, L, b, r0, rows, nullptr, tr, stream));
    Combine1Launch c1{};
    c1.tiles_m = (int32_t)L.Tv;
    c1.ncols = (int32_t)rows;
    c1.ldp = (int32_t)Nc;
    c1.pm_z = b.pz;
    c1.ps_z = b.pz + tile_cols;
    c1.pm_u = k.target ? b.pu : nullptr;
    c1.ps_u = k.target ? b.pu + tile_cols : nullptr;
    c1.pi_u = k.target ? reinterpret_cast<const int32_t*>(b.pu + 2 * tile_cols) : nullptr;
    c1.pq_u = k.target ? b.pu + 3 * tile_cols : nullptr;
    c1.vocab = (int32_t)p->vocab;
    c1.raw_m[0] = X.at(0, g, r0);
    c1.raw_s[0] = X.at(1, g, r0);
    c1.raw_m[1] = X.at(2, g, r0);
    c1.raw_s[1] = X.at(3, g, r0);
    c1.raw_q2 = X.at(4, g, r0);
    c1.raw_idx = reinterpret_cast<int32_t*>(X.at(5, g, r0));
    c1.idx_offset = (int32_t)sh->vocab_offset;
    TRACED(tr, K_COMBINE1, (k.target ? 6.0 : 2.0) * L.Tv * rows * 4, launch_combine1(c1, stream));
  }
  return SPECLOSS_OK;
}

int lmhead_shard_merge1(const specloss_problem* p, const specloss_shard* sh, void* saved,
                        int64_t* counts, hipStream_t stream) {
  KindSet k;
  TRY(check_problem(p, &k));
  TRY(check_shard(p, sh));
  if (!saved || !counts) return SPECLOSS_E_INVAL;
  if (!aligned(saved, 4) || !aligned(counts, 8)) return SPECLOSS_E_UNSUPPORTED;
  const int64_t N = p->n_rows;
  const SavedView sv = saved_view(saved, N);
  const Exchange X = exchange_of(sh, N);
  Tracer tr{p->trace, stream};
  TRY(launch_validity_for(p, k, sv, counts, tr, stream, sh->vocab_total));
  Combine1Launch c1{};
  c1.tiles_m = X.G;  // the G shard records merge like G vocabulary tiles
  c1.ncols = (int32_t)N;
  c1.ldp = (int32_t)X.Ns;
  c1.pm_z = X.f(0);
  c1.ps_z = X.f(1);
  c1.pm_u = k.target ? X.f(2) : nullptr;
  c1.ps_u = k.target ? X.f(3) : nullptr;
  c1.pq_u = k.target ? X.f(4) : nullptr;
  c1.pi_u = k.target ? reinterpret_cast<const int32_t*>(X.f(5)) : nullptr;
  c1.vocab = (int32_t)sh->vocab_total;
  c1.flags = sv.flags;
  c1.lse_q = sv.lse_q;
  c1.lse_p = sv.lse_p;
  c1.y_arg = sv.y_arg;
  c1.flat = sv.flat;
  TRACED(tr, K_COMBINE1, (k.target ? 6.0 : 2.0) * X.G * N * 4, launch_combine1(c1, stream));
  return SPECLOSS_OK;
}

int lmhead_shard_pass2(const specloss_problem* p, const specloss_shard* sh, const void* saved,
                       void* workspace, size_t ws_bytes, hipStream_t stream) {
  KindSet k;
  TRY(check_problem(p, &k));
  TRY(check_shard(p, sh));
  if (!saved) return SPECLOSS_E_INVAL;
  if (!aligned(saved, 4)) return SPECLOSS_E_UNSUPPORTED;
  if (!workspace || !aligned(workspace, kAlign)) return SPECLOSS_E_WORKSPACE;
  const int64_t Nc = pick_chunk(p, k, ws_bytes, REGION_FWD);
  if (Nc <= 0) return SPECLOSS_E_WORKSPACE;
  const Layout L = plan(p, k, Nc);
  char* ws = static_cast<char*>(workspace);
  const FwdBufs b{reinterpret_cast<float*>(ws + L.pz), reinterpret_cast<float*>(ws + L.pu),
                  reinterpret_cast<float*>(ws + L.p2), reinterpret_cast<float*>(ws + L.zy), Nc};
  const bool bf16 = p->in_dtype == SPECLOSS_BF16;
  const SavedView sv = saved_view(const_cast<void*>(saved), L.N);
  const Exchange X = exchange_of(sh, L.N);
  const int g = sh->shard;
  const bool ce_lab = (k.active >> SPECLOSS_CE_LABEL) & 1u;
  const bool ce_arg = (k.active >> SPECLOSS_CE_ARGMAX_P) & 1u;
  Tracer tr{p->trace, stream};
  for (int64_t r0 = 0; r0 < L.N; r0 += Nc) {
    const int64_t rows = (L.N - r0) < Nc ? (L.N - r0) : Nc;
    if (ce_lab || ce_arg) {
      RowdotLaunch rd{};
      rd.W = p->W;
      rd.h = offset_rows(p->hidden_states, r0, L.H, L.es);
      rd.H = L.H;
      rd.ncols = (int32_t)rows;
      rd.vocab = (int32_t)p->vocab;
      rd.vocab_offset = (int32_t)sh->vocab_offset;
      rd.outside = -INFINITY;  // the shard holding the row's label supplies the logit
      rd.y1 = ce_lab ? sv.y_label + r0 : nullptr;
      rd.y2 = ce_arg ? sv.y_arg + r0 : nullptr;
      rd.out1 = X.at(kExch1 + kNumSums, g, r0);
      rd.out2 = X.at(kExch1 + kNumSums + 1, g, r0);
      TRACED(tr, K_ROWDOT, 2.0 * rows * L.H * L.es * ((ce_lab ? 1 : 0) + (ce_arg ? 1 : 0)),
             launch_rowdot(bf16, rd, stream));
    }
    if (k.pass2) {
      TRY(launch_pass2(p, k, L, b, sv, r0, rows, nullptr, nullptr, tr, stream));
      TileSumLaunch ts{};
      ts.tiles_m = (int32_t)L.Tv;
      ts.ncols = (int32_t)rows;
      ts.ldp = (int32_t)Nc;
      ts.need = k.need;
      ts.part = b.p2;
      ts.part_stride = L.Tv * Nc;
      ts.out = X.at(kExch1, g, r0);
      ts.out_stride = (int64_t)X.G * X.Ns;
      TRACED(tr, K_TILE_SUM, (double)__builtin_popcount(k.need) * (L.Tv + 1) * rows * 4,
             launch_tile_sum(ts, stream));
    }
  }
  return SPECLOSS_OK;
}

int lmhead_shard_merge2(const specloss_problem* p, const specloss_shard* sh, void* saved,
                        const int64_t* counts, float* loss, float* term_loss, float* lse_q,
                        float* reduced, hipStream_t stream) {
  KindSet k;
  TRY(check_problem(p, &k));
  TRY(check_shard(p, sh));
  if (!saved) return SPECLOSS_E_INVAL;
  TRY(check_fwd_outputs(loss, term_loss, lse_q, saved, counts, reduced));
  if (reduced && !term_loss) return SPECLOSS_E_INVAL;  // the per-kind means read the terms
  const int64_t N = p->n_rows;
  const SavedView sv = saved_view(saved, N);
  const Exchange X = exchange_of(sh, N);
  const bool ce_lab = (k.active >> SPECLOSS_CE_LABEL) & 1u;
  const bool ce_arg = (k.active >> SPECLOSS_CE_ARGMAX_P) & 1u;
  Tracer tr{p->trace, stream};
  Combine2Launch c2{};
  c2.tiles_m = X.G;  // the G shard sums add like G vocabulary tiles
  c2.ncols = (int32_t)N;
  c2.ldp = (int32_t)X.Ns;
  c2.part = X.f(kExch1);
  c2.part_stride = (int64_t)X.G * X.Ns;
  c2.need = k.need;
  memcpy(c2.w, p->weights, sizeof(c2.w));
  c2.flags = sv.flags;
  c2.lse_q = sv.lse_q;
  c2.zy_lab = ce_lab ? X.f(kExch1 + kNumSums) : nullptr;
  c2.zy_arg = ce_arg ? X.f(kExch1 + kNumSums + 1) : nullptr;
  c2.zy_count = X.G;
  c2.zy_stride = X.Ns;
  c2.loss = loss;
  c2.term = term_loss;
  c2.term_stride = N;
  c2.alpha = sv.alpha;
  c2.S = sv.S;
  c2.rkl = sv.rkl;
  c2.eqg = sv.eqg;
  TRACED(tr, K_COMBINE2, (double)N * 4 * (2 + __builtin_popcount(k.need) * X.G),
         launch_combine2(c2, stream));
  if (reduced) TRY(launch_reduce_for(p, k, loss, term_loss, counts, reduced, tr, stream));
  if (lse_q)
    TRACED(tr, K_COPY, (double)N * 8,
           hipMemcpyAsync(lse_q, sv.lse_q, (size_t)N * 4, hipMemcpyDeviceToDevice, stream));
  return SPECLOSS_OK;
}

int lmhead_shard_bwd(const specloss_problem* p, const specloss_shard* sh, const float* grad_loss,
                     const float* grad_mean, const int64_t* counts, const void* saved,
                     void* workspace, size_t ws_bytes, float* dh_partial, float* dW,
                     int accumulate_dW, hipStream_t stream) {
  KindSet k;
  TRY(check_problem(p, &k));
  TRY(check_shard(p, sh));
  TRY(check_bwd_inputs(grad_loss, grad_mean, counts, saved, dh_partial, SPECLOSS_F32, dW,
                       workspace));
  return bwd_recompute(p, k, grad_loss, grad_mean, counts, saved, workspace, ws_bytes, dh_partial,
                       SPECLOSS_F32, dW, accumulate_dW, sh->vocab_offset, stream);
}

int specloss_sum_partials(const float* parts, int64_t n, int32_t n_parts, void* out,
                          int32_t out_dtype, hipStream_t stream) {
  if (!parts || !out || n <= 0 || n_parts < 1) return SPECLOSS_E_INVAL;
  if (out_dtype != SPECLOSS_F32 && out_dtype != SPECLOSS_BF16) return SPECLOSS_E_UNSUPPORTED;
  if (!aligned(parts, 16) || n % 4 != 0 || !aligned(out, out_dtype == SPECLOSS_F32 ? 4 : 2))
    return SPECLOSS_E_UNSUPPORTED;
  HIP_TRY(launch_sum_parts(parts, n, n_parts, out, out_dtype == SPECLOSS_BF16, stream));
  return SPECLOSS_OK;
}

}  // extern "C"
