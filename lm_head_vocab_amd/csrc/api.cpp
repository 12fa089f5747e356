// C-ABI of libspecloss: argument checks, workspace plan and launch sequence.
//
// Forward, per chunk of rows (blog "Streaming Cross Entropy": tokens are
// independent, so rows are processed in chunks and only per-row statistics
// survive a chunk):
//   pass 1   k_stats on (W, hidden)        -> per (vocab tile, row) max / sum-exp
//            k_stats on (W_t, target rows) -> same plus argmax (target kinds)
//   merge    k_combine1 -> logsumexp of q and p, argmax p
//   gather   k_rowdot   -> label logit z_y (ce_label) and z at argmax p (ce)
//   pass 2   k_div      -> alpha, S, KL, rKL, JSD, E_q[g] partials (divergences),
//            or k_div_raw over the raw logit rows pass 1 kept (k_stats RAW)
//   losses   k_combine2 -> per-row weighted loss, unweighted terms, saved stats
// then k_reduce -> sum / n_valid (blog "Backward pass": one denominator).
// Backward, per chunk (blog "Backward pass": per-chunk logits, gradients for
// the chunk's hidden states, LM-head gradient accumulated over chunks):
//   k_dz (recompute + logit gradient), or for the divergences raw logit rows
//   recomputed by pass 1's contraction and k_dz_raw -> dz chunk, both layouts
//   k_gemm dh = dz W^T^T  and  k_gemm dW (+)= dz^T h, chunks in order.
// The single call (lmhead_loss_fwd_bwd) forms dz from what its forward kept:
// the staged exp(z - label logit) of the cross-entropies, or the raw rows.
// With both gradients the cross-entropies' pass 1 stages dz only, and the dh
// contraction writes dz^T from the dz slabs it streams through LDS.
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
  bool stage_div = false;  // single call: pass 1 keeps both raw logit rows (every divergence)
  // the only sums needed are the Kullback-Leibler ones: the two-call forward
  // takes them from a dual pass 1 (no second sweep) when each row has its
  // own target row
  bool ratio_only = false;
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
  // alpha is reported whenever a kind other than the Kullback-Leibler ones needs a
  // second sweep
  if (k.need & ~(SUM_KL | SUM_RKL)) k.need |= SUM_ALPHA;
  k.pass2 = k.need != 0;
  k.ratio_only = k.pass2 && (k.need & ~(SUM_KL | SUM_RKL)) == 0;
  k.dual_bwd = (k.active & ~((1u << SPECLOSS_CE_LABEL) | (1u << SPECLOSS_CE_ARGMAX_P))) != 0;
  k.stage_div = k.dual_bwd;
  return k;
}

size_t elem_size(const specloss_problem* p) { return p->in_dtype == SPECLOSS_BF16 ? 2 : 4; }

int check_problem(const specloss_problem* p, KindSet* ks) {
  if (!p) return SPECLOSS_E_INVAL;
  if (p->n_rows <= 0 || p->hidden <= 0 || p->vocab <= 0) return SPECLOSS_E_INVAL;
  if (p->n_rows > INT32_MAX / 2 || p->vocab > INT32_MAX / 2 || p->hidden > INT32_MAX / 2)
    return SPECLOSS_E_UNSUPPORTED;
  if (p->flags != 0 && p->flags != SPECLOSS_FLAG_COPIES && p->flags != SPECLOSS_FLAG_NO_COPIES &&
      p->flags != SPECLOSS_FLAG_NO_WEIGHT_COPY)
    return SPECLOSS_E_INVAL;
  if (p->in_dtype != SPECLOSS_F32 && p->in_dtype != SPECLOSS_BF16) return SPECLOSS_E_UNSUPPORTED;
  if (p->hidden % 64 != 0) return SPECLOSS_E_UNSUPPORTED;
  if ((p->flags == SPECLOSS_FLAG_NO_COPIES || p->flags == SPECLOSS_FLAG_NO_WEIGHT_COPY) &&
      p->in_dtype != SPECLOSS_BF16)
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
  if (p->n_heads != 0) {
    if (p->n_heads < 1 || p->n_heads > SPECLOSS_MAX_HEADS || p->n_rows % p->n_heads != 0)
      return SPECLOSS_E_INVAL;
    for (int i = 0; i < p->n_heads; ++i)
      if (p->head_shift[i] < 0 || p->head_shift[i] > 65536) return SPECLOSS_E_INVAL;
    if (k.target && !p->target_row) return SPECLOSS_E_INVAL;
  }
  *ks = k;
  return SPECLOSS_OK;
}

// Which transposed copies the backward contractions read.  A K-major copy
// lets a contraction read 16-byte fragments; without it the operand is read
// in place (MN-major) through the transposing LDS load (bf16 only).
enum BwdLayout : int32_t {
  LAYOUT_COPIES = 0,     // W^T for dh; h^T and dz^T for dW
  LAYOUT_DW_COPIES = 1,  // dh reads W in place; h^T and dz^T for dW
  LAYOUT_NONE = 2        // dh reads W, dW reads dz and the hidden rows in place
};

// Workspace: a head used by both directions, then the forward and backward
// regions, which overlap (the two directions never run at the same time on
// one workspace).
struct Layout {
  int64_t N, H, V, Vp, Tv, Nc;
  size_t es;
  int32_t layout;   // BwdLayout
  int32_t dh_splits;  // split-K slices of the dh contraction (1: none)
  bool wt_copy;     // dh reads the copy W^T [H][Vp]
  bool dw_copies;   // dW reads the copies h^T [H][ld_t] and dz^T [Vp][ld_t]
  // chunks one dW contraction takes (copies only): chunk c writes its copies'
  // columns [(c mod dw_group) Nc, + Nc); ld_t = dw_group Nc
  int32_t dw_group;
  int64_t ld_t;
  // head
  size_t terms, saved, seed, tstat, head_end;
  // rows share target rows (a row map onto fewer target rows than rows): the
  // target statistics are computed once per target row, then gathered
  bool shared_target;
  int64_t Nt;
  // forward (fwd_raw: the two-call forward keeps both raw logit rows, zr and
  // ur, as the single call does)
  bool fwd_raw;
  size_t pz, pu, p2, zy, hmap, zr, ur, fwd_end;
  // backward (bwd_raw: the divergences' logit rows are recomputed into raw
  // buffers, b_zr and b_ur, with partial scratch b_pz / b_pu, as in pass 1)
  bool bwd_raw;
  size_t wt, ht, dz, dzt, dhp, b_pz, b_pu, b_zr, b_ur, bwd_end;
  // single-call forward+backward: forward partials and backward buffers at once;
  // the divergences keep the chunk's raw fp32 logits (f_zr: Nc draft rows,
  // f_ur: Nu target rows; the same in the forward region with fwd_raw) and
  // the target partials have pu_cols columns
  int64_t Nu, pu_cols;
  size_t f_pz, f_pu, f_p2, f_zy, f_wt, f_ht, f_dz, f_zr, f_ur, f_dzt, f_rs, f_dhp, fused_end;
};

// The second sweep of a problem with aligned heads shares target tiles
// between the heads (k_div_heads): K = 2 or 3, bf16, a target side with a
// row map.  The tiles of a chunk of Nc rows span at most Nc / K + 2 tokens
// plus the spread of the shifts.
bool heads_pass2(const specloss_problem* p, const KindSet& k) {
  return k.pass2 && k.target && p->target_row && p->in_dtype == SPECLOSS_BF16 &&
         (p->n_heads == 2 || p->n_heads == 3);
}

// The kinds whose second sweep can read raw logits kept by pass 1 (all that
// need one, except kl_div / rkl alone, which the dual pass 1 yields).
bool raw_second_sweep(const KindSet& k) { return k.target && k.pass2 && !k.ratio_only; }

void shift_range(const specloss_problem* p, int32_t& lo, int32_t& hi) {
  lo = p->head_shift[0];
  hi = p->head_shift[0];
  for (int i = 1; i < p->n_heads; ++i) {
    lo = p->head_shift[i] < lo ? p->head_shift[i] : lo;
    hi = p->head_shift[i] > hi ? p->head_shift[i] : hi;
  }
}

// Target rows [jlo, jhi) that chunk rows [r0, r0 + rows) of a problem with
// aligned heads use (token-major rows: row T K + k has target T + shift_k).
void heads_span(const specloss_problem* p, int64_t r0, int64_t rows, int64_t& jlo, int64_t& jhi) {
  const int32_t K = p->n_heads;
  int32_t s_lo, s_hi;
  shift_range(p, s_lo, s_hi);
  jlo = r0 / K + s_lo;
  jhi = (r0 + rows - 1) / K + 1 + s_hi;
}

// at most Nc / K + 2 tokens plus the spread of the shifts
int64_t heads_span_cap(const specloss_problem* p, int64_t Nc) {
  int32_t lo, hi;
  shift_range(p, lo, hi);
  return Nc / p->n_heads + 2 + (hi - lo);
}

int64_t heads_map_entries(const specloss_problem* p, int64_t Nc) {
  return cdiv(heads_span_cap(p, Nc), 64) * 64 * p->n_heads;
}

// Split-K slices of the dh contraction of a chunk of Nc rows: its grid has
// ceil(Nc / 256) x ceil(H / 256) tiles, and with few of them (small chunks)
// most of the 256 CUs would idle.  S slices of the vocabulary run as
// S times the tiles, each 1/S as long; S in [1, 8] minimises
// ceil(tiles S / 256) / S (the launch's rounds of one slice's length), the
// smallest S on ties.  The partials are added in slice order afterwards.
int32_t dh_splits(int64_t Nc, int64_t H) {
  const int64_t tiles = cdiv(Nc, 256) * cdiv(H, 256);
  int32_t best = 1;
  double best_t = (double)cdiv(tiles, 256);
  for (int32_t s = 2; s <= 8; ++s) {
    const double t = (double)cdiv(tiles * s, 256) / s;
    if (t < best_t - 1e-9) {
      best_t = t;
      best = s;
    }
  }
  return best;
}

// fp32 inputs always take LAYOUT_COPIES (the transposing LDS load is bf16).
Layout plan(const specloss_problem* p, const KindSet& k, int64_t Nc,
            int32_t layout = LAYOUT_COPIES, bool fwd_raw = false, bool bwd_raw = false,
            int32_t dw_group = 1) {
  Layout L;
  L.N = p->n_rows;
  L.H = p->hidden;
  L.V = p->vocab;
  L.Vp = round_up(L.V, kVocabTile);
  L.Tv = L.Vp / kVocabTile;
  L.Nc = Nc;
  L.es = elem_size(p);
  L.layout = L.es == 4 ? LAYOUT_COPIES : layout;
  L.wt_copy = L.layout == LAYOUT_COPIES;
  L.dw_copies = L.layout != LAYOUT_NONE;
  L.dw_group = L.dw_copies ? dw_group : 1;
  L.ld_t = L.dw_group * Nc;
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
  L.fwd_raw = fwd_raw && raw_second_sweep(k);
  L.Nu = (k.stage_div || L.fwd_raw) ? (heads_pass2(p, k) ? heads_span_cap(p, Nc) : Nc) : 0;
  L.pu_cols = L.Nu > Nc ? L.Nu : Nc;
  const size_t pu_bytes = k.target ? 4 * (size_t)L.Tv * L.pu_cols * 4 : 0;
  L.pz = take(2 * tile_cols);
  L.pu = take(pu_bytes);
  L.p2 = take(k.pass2 ? (size_t)kNumSums * tile_cols : 0);
  L.zy = take(2 * (size_t)Nc * 4);
  const size_t hmap_bytes =
      heads_pass2(p, k) && !L.fwd_raw ? (size_t)heads_map_entries(p, Nc) * 4 : 0;
  L.hmap = take(hmap_bytes);
  L.zr = take(L.fwd_raw ? (size_t)Nc * L.Vp * 4 : 0);
  L.ur = take(L.fwd_raw ? (size_t)L.Nu * L.Vp * 4 : 0);
  L.fwd_end = o;
  o = L.head_end;
  L.wt = take(L.wt_copy ? (size_t)L.H * L.Vp * L.es : 0);
  L.ht = take(L.dw_copies ? (size_t)L.H * L.ld_t * L.es : 0);
  L.dz = take((size_t)Nc * L.Vp * L.es);
  L.dzt = take(L.dw_copies ? (size_t)L.Vp * L.ld_t * L.es : 0);
  L.dh_splits = dh_splits(Nc, L.H);
  const size_t dhp_bytes = L.dh_splits > 1 ? (size_t)L.dh_splits * Nc * L.H * 4 : 0;
  L.dhp = take(dhp_bytes);
  L.bwd_raw = bwd_raw && k.stage_div;
  L.b_pz = take(L.bwd_raw ? 2 * tile_cols : 0);
  L.b_pu = take(L.bwd_raw ? pu_bytes : 0);
  L.b_zr = take(L.bwd_raw ? (size_t)Nc * L.Vp * 4 : 0);
  L.b_ur = take(L.bwd_raw ? (size_t)L.Nu * L.Vp * 4 : 0);
  L.bwd_end = o;
  o = L.head_end;
  L.f_pz = take(2 * tile_cols);
  L.f_pu = take(pu_bytes);
  L.f_p2 = take(k.stage_div ? (size_t)kNumSums * tile_cols : 0);
  L.f_zy = take(2 * (size_t)Nc * 4);
  L.f_wt = take(L.wt_copy ? (size_t)L.H * L.Vp * L.es : 0);
  L.f_ht = take(L.dw_copies ? (size_t)L.H * L.ld_t * L.es : 0);
  L.f_dz = take((size_t)Nc * L.Vp * L.es);
  L.f_zr = take(k.stage_div ? (size_t)Nc * L.Vp * 4 : 0);
  L.f_ur = take(k.stage_div ? (size_t)L.Nu * L.Vp * 4 : 0);
  L.f_dzt = take(L.dw_copies ? (size_t)L.Vp * L.ld_t * L.es : 0);
  L.f_rs = take(4 * (size_t)Nc * 4);
  L.f_dhp = take(dhp_bytes);
  L.fused_end = o;
  return L;
}

enum Region { REGION_FWD, REGION_BWD, REGION_FUSED };

size_t region_end(const Layout& L, Region r) {
  return r == REGION_FWD ? L.fwd_end : (r == REGION_BWD ? L.bwd_end : L.fused_end);
}

size_t workspace_end(const Layout& L) {
  size_t b = L.fwd_end > L.bwd_end ? L.fwd_end : L.bwd_end;
  return L.fused_end > b ? L.fused_end : b;
}

// Largest chunk (multiple of 256, at most `top` rows) whose region fits
// `ws_bytes` (strictly below it when `strict`).  The requirement is not
// monotonic in the chunk (a chunk with few row tiles adds split-K partials of
// dh, e.g. 1792 rows at H = 16384 take more than 2048), so every candidate is
// tried from the top; a plan costs a few arithmetic operations.
int64_t largest_chunk(const specloss_problem* p, const KindSet& k, size_t ws_bytes,
                      Region region, int32_t layout, int64_t top, bool strict = false,
                      bool raw = false, int32_t dw_group = 1) {
  for (int64_t m = top / kChunkQuantum; m >= 1; --m) {
    const Layout L = plan(p, k, m * kChunkQuantum, layout, raw && region == REGION_FWD,
                          raw && region == REGION_BWD, dw_group);
    const size_t need = region_end(L, region);
    if (strict ? need < ws_bytes : need <= ws_bytes) return m * kChunkQuantum;
  }
  return 0;
}

int32_t forced_layout(const specloss_problem* p) {
  switch (p->flags) {
    case SPECLOSS_FLAG_COPIES: return LAYOUT_COPIES;
    case SPECLOSS_FLAG_NO_WEIGHT_COPY: return LAYOUT_DW_COPIES;
    case SPECLOSS_FLAG_NO_COPIES: return LAYOUT_NONE;
    default: return -1;
  }
}

// Smallest chunk a layout is taken with (pick_chunk) and smallest chunk of a
// dW group: min(N, 1024) rows.
int64_t wanted_chunk(const specloss_problem* p) {
  const int64_t top = round_up(p->n_rows, kChunkQuantum);
  return top < 1024 ? top : 1024;
}

// Largest chunk of one layout and its dW group.  Each dW contraction reads and
// writes the whole fp32 dW (2 V H 4 bytes) beside its 2 rows H V flops, so at
// small chunks it is bound by that traffic.  With the copies, G consecutive
// chunks can share one contraction (dw_group G: their dz^T and h^T columns
// side by side, K = G Nc).  The copies of G chunks take a smaller chunk, which
// costs the other kernels some efficiency, so a group is taken when
//   - its chunk still has min(N, 1024) rows,
//   - it is at most kDwGroupDepth rows deep (on MI355X the contraction ran
//     at 1.32 PFLOP/s with K = 8192 and 1.26 with K = 16384 at H = 4096,
//     V = 128256), and
//   - it saves at least two of dW's read-modify-writes per call over single
//     chunks (measured whole-call changes: one saved at N = 8192, H = 2048
//     lost 2.6 %; two at the three-head H = 16384 shape gained 3.4 %, four at
//     N = 16384, H = 4096 with a target gained 4.6 %);
// among those, the group with the fewest read-modify-writes (the smaller
// group on a tie).
constexpr int64_t kDwGroupDepth = 8192;
constexpr int32_t kMaxDwGroup = 4;

// Read-modify-writes of dW per call with chunks of n rows in groups of g.
int64_t dw_passes(const specloss_problem* p, int64_t n, int32_t g) {
  return cdiv(cdiv(p->n_rows, n), g);
}

// The dW group (1 if none) for single chunks of n1 rows, given the largest
// chunk ng[g] that fits with groups of g (g = 2 .. kMaxDwGroup; <= 0: none).
int32_t choose_dw_group(const specloss_problem* p, int64_t n1, const int64_t* ng) {
  const int64_t N = p->n_rows;
  if (n1 <= 0 || n1 >= N) return 1;
  int32_t best = 1;
  int64_t best_passes = dw_passes(p, n1, 1) - 1;  // a group must save at least two
  for (int32_t g = 2; g <= kMaxDwGroup; ++g) {
    const int64_t n = ng[g];
    if (n < wanted_chunk(p) || g * n > kDwGroupDepth) continue;
    const int64_t passes = dw_passes(p, n, g);
    if (passes < best_passes) {
      best = g;
      best_passes = passes;
    }
  }
  return best;
}

int64_t fit_chunk(const specloss_problem* p, const KindSet& k, size_t ws_bytes, Region region,
                  int32_t layout, int64_t top, bool strict, bool raw, int32_t* dw_group) {
  *dw_group = 1;
  const int64_t n1 = largest_chunk(p, k, ws_bytes, region, layout, top, strict, raw, 1);
  if (region == REGION_FWD || n1 <= 0 || n1 >= p->n_rows || !plan(p, k, n1, layout).dw_copies)
    return n1;
  int64_t ng[kMaxDwGroup + 1] = {};
  for (int32_t g = 2; g <= kMaxDwGroup; ++g)
    ng[g] = largest_chunk(p, k, ws_bytes, region, layout, top, strict, raw, g);
  *dw_group = choose_dw_group(p, n1, ng);
  return *dw_group > 1 ? ng[*dw_group] : n1;
}

// Chunk for a region and the backward layout.  With every copy when the
// workspace holds them at a chunk of at least min(N, 1024) rows; otherwise
// (bf16) without the W^T copy, then without any copy, whichever allows a
// larger chunk.  (The in-place operands run the contractions slower; below
// about 1000 rows per chunk the fp32 read-modify-write of dW per chunk costs
// more than that at the large shapes.)  flags force the layout.  Each layout's chunk comes with
// its dW group (fit_chunk).
int64_t pick_chunk(const specloss_problem* p, const KindSet& k, size_t ws_bytes, Region region,
                   int32_t* layout = nullptr, int32_t* dw_group = nullptr) {
  const int64_t top = round_up(p->n_rows, kChunkQuantum);
  const int32_t forced = forced_layout(p);
  int32_t g = 1;
  int64_t best;
  if (forced >= 0) {
    if (layout) *layout = forced;
    best = fit_chunk(p, k, ws_bytes, region, forced, top, false, false, &g);
  } else {
    best = fit_chunk(p, k, ws_bytes, region, LAYOUT_COPIES, top, false, false, &g);
    if (layout) *layout = LAYOUT_COPIES;
    if (layout && p->in_dtype == SPECLOSS_BF16) {
      for (int32_t lay : {LAYOUT_DW_COPIES, LAYOUT_NONE}) {
        if (best >= wanted_chunk(p)) break;
        int32_t gl = 1;
        const int64_t nc = fit_chunk(p, k, ws_bytes, region, lay, top, false, false, &gl);
        if (nc > best) {
          best = nc;
          *layout = lay;
          g = gl;
        }
      }
    }
  }
  if (dw_group) *dw_group = g;
  return best;
}

// Chunk of the two-call forward.  The kinds of raw_second_sweep keep both raw
// logit rows (the second sweep is then a memory pass) when the workspace
// holds them for a chunk of at least min(N, 1024) rows; otherwise their
// second sweep recomputes both tiles, with the largest chunk that fits.
int64_t pick_fwd_chunk(const specloss_problem* p, const KindSet& k, size_t ws_bytes, bool* raw) {
  *raw = false;
  if (raw_second_sweep(k)) {
    const int64_t top = round_up(p->n_rows, kChunkQuantum);
    const int64_t want = top < 1024 ? top : 1024;
    const int64_t nc = largest_chunk(p, k, ws_bytes, REGION_FWD, LAYOUT_COPIES, top, false, true);
    if (nc >= want) {
      *raw = true;
      return nc;
    }
  }
  return pick_chunk(p, k, ws_bytes, REGION_FWD);
}

// Chunk and layout of the two-call backward.  The divergences recompute both
// raw logit rows with the pass-1 contraction and form dz from them
// (k_dz_raw) when the workspace holds them for a chunk of at least min(N,
// 1024) rows in some layout (tried in pick_chunk's order); otherwise, and for
// vocabulary shards, one dual recompute kernel forms dz from the tiles.
int64_t pick_bwd_chunk(const specloss_problem* p, const KindSet& k, size_t ws_bytes,
                       int32_t* layout, bool* raw, bool shard, int32_t* dw_group) {
  *raw = false;
  if (k.stage_div && !shard) {
    const int64_t top = round_up(p->n_rows, kChunkQuantum);
    const int64_t want = wanted_chunk(p);
    const int32_t forced = forced_layout(p);
    int32_t lays[3] = {LAYOUT_COPIES, LAYOUT_DW_COPIES, LAYOUT_NONE};
    int n_lays = p->in_dtype == SPECLOSS_BF16 ? 3 : 1;
    if (forced >= 0) {
      lays[0] = forced;
      n_lays = 1;
    }
    for (int i = 0; i < n_lays; ++i) {
      const int64_t nc = fit_chunk(p, k, ws_bytes, REGION_BWD, lays[i], top, false, true, dw_group);
      if (nc >= want) {
        *layout = lays[i];
        *raw = true;
        return nc;
      }
    }
  }
  return pick_chunk(p, k, ws_bytes, REGION_BWD, layout, dw_group);
}

// The default chunk (workspace size for max_chunk_rows <= 0).  Blog, "Backward
// pass" and "Choosing the chunk size": the loss path holds about
// chunk x vocab x dtype x 2 bytes of logits-sized data and never the whole
// [tokens, vocab] logits.  So the default streams the token set in at least
// four balanced chunks of at most kDefaultChunk rows, with the whole workspace
// (staged chunk buffers, transposed copies, partials) strictly below
// N x V x (input dtype size) bytes, the size of the full logits; layouts are
// tried in the order of pick_chunk.  Problems too small for any chunk to fit
// below that size (the W^T copy alone exceeds it) take 256-row chunks.
int64_t default_chunk(const specloss_problem* p, const KindSet& k, int32_t* layout,
                      int32_t* dw_group) {
  const int64_t N = p->n_rows;
  const int64_t top = round_up(N, kChunkQuantum);
  int64_t cap = round_up(cdiv(N, 4), kChunkQuantum);
  if (cap > kDefaultChunk) cap = kDefaultChunk;
  const size_t limit = (size_t)N * (size_t)p->vocab * elem_size(p);
  const int64_t want = top < 1024 ? top : 1024;
  const int32_t forced = forced_layout(p);
  int32_t lays[3] = {LAYOUT_COPIES, LAYOUT_DW_COPIES, LAYOUT_NONE};
  int n_lays = p->in_dtype == SPECLOSS_BF16 ? 3 : 1;
  if (forced >= 0) {
    lays[0] = forced;
    n_lays = 1;
  }
  // the chunk every region fits with the copies of dw_group chunks
  auto fits = [&](int32_t lay, int32_t g) {
    int64_t nc = largest_chunk(p, k, limit, REGION_FWD, lay, cap, true);
    const int64_t nb = largest_chunk(p, k, limit, REGION_BWD, lay, cap, true, false, g);
    const int64_t nf = largest_chunk(p, k, limit, REGION_FUSED, lay, cap, true, false, g);
    nc = nb < nc ? nb : nc;
    return nf < nc ? nf : nc;
  };
  *dw_group = 1;
  for (int i = 0; i < n_lays; ++i) {
    int64_t nc = fits(lays[i], 1);
    if (nc <= 0 || (nc < want && i + 1 < n_lays)) continue;
    // a dW group as in fit_chunk
    if (nc < N && plan(p, k, nc, lays[i]).dw_copies) {
      int64_t ng[kMaxDwGroup + 1] = {};
      for (int32_t g = 2; g <= kMaxDwGroup; ++g) ng[g] = fits(lays[i], g);
      *dw_group = choose_dw_group(p, nc, ng);
      if (*dw_group > 1) nc = ng[*dw_group];
    }
    // balance: the fewest chunks of that size, then equal chunks
    const int64_t nch = cdiv(N, nc);
    *layout = lays[i];
    return round_up(cdiv(N, nch), kChunkQuantum);
  }
  *layout = n_lays == 1 ? lays[0] : LAYOUT_COPIES;
  return kChunkQuantum;
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

#define TRY(expr)                   \
  do {                              \
    const int rc_ = (expr);         \
    if (rc_) return rc_;            \
  } while (0)

#define HIP_TRY(expr)                                   \
  do {                                                  \
    if ((expr) != hipSuccess) return SPECLOSS_E_HIP;    \
  } while (0)

enum KernelId : int32_t {
  K_VALIDITY, K_STATS_Q, K_STATS_P, K_COMBINE1, K_ROWDOT, K_DIV, K_COMBINE2, K_REDUCE, K_COPY,
  K_SEED, K_TRANSPOSE_W, K_TRANSPOSE_H, K_DZ, K_GEMM_DH, K_GEMM_DW, K_STATS_STAGE, K_DZ_STAGE,
  K_TILE_SUM, K_SUM_PARTS, K_TARGET_GATHER, K_STAGE_FIX, K_STATS_DUAL, K_DIV_HEADS, K_HEADS_MAP,
  K_DIV_RAW, K_DZ_RAW, K_SPAN_CARRY, K_GEMM_DH_DZT, K_NUM_IDS
};
const char* const kKernelNames[K_NUM_IDS] = {
    "validity", "stats_q", "stats_p", "combine1", "rowdot", "div", "combine2", "reduce",
    "copy_lse", "seed", "transpose_W", "transpose_h", "dz", "gemm_dh", "gemm_dW",
    "stats_stage", "dz_stage", "tile_sum", "sum_partials", "target_gather", "stage_fix",
    "stats_dual", "div_heads", "heads_map", "div_raw", "dz_raw", "span_carry",
    "gemm_dh_dzt"};

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
  int32_t* hmap = nullptr;  // row map of the aligned-heads second sweep
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
  if (k.target && p->target_row && p->n_heads > 0) {
    va.n_heads = p->n_heads;
    for (int i = 0; i < p->n_heads; ++i) va.shifts[i] = p->head_shift[i];
  }
  TRACED(tr, K_VALIDITY, (double)p->n_rows * 10, launch_validity(va, stream));
  return SPECLOSS_OK;
}

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

// Pass 1 of both sides with the log-ratio sums (k_stats_dual), for problems
// whose only divergences are kl_div and rkl: the per-tile log-ratio partials
// go to the rows of b.p2 that hold the sums they replace (SUM_KL: pa, SUM_RKL:
// pr), and the combine writes the merged divergences into tile row 0 there.
int launch_pass1_dual(const specloss_problem* p, const Layout& L, const FwdBufs& b, int64_t r0,
                      int64_t rows, Tracer& tr, hipStream_t stream) {
  const bool bf16 = p->in_dtype == SPECLOSS_BF16;
  const int64_t H = L.H, Nc = b.Nc;
  const int64_t tile_cols = L.Tv * Nc;
  DualStatsLaunch d{};
  d.Az = op(p->W, H, p->vocab);
  d.Bz = op(offset_rows(p->hidden_states, r0, H, L.es), H, rows);
  d.Au = op(p->W_t, H, p->vocab);
  d.Bu = target_operand(p, r0, rows, L.es);
  d.k_len = (int32_t)H;
  d.vocab = (int32_t)p->vocab;
  d.tiles_m = (int32_t)L.Tv;
  d.tiles_n = (int32_t)cdiv(rows, 128);
  d.ncols = (int32_t)rows;
  d.ldp = (int32_t)Nc;
  d.pm_z = b.pz;
  d.ps_z = b.pz + tile_cols;
  d.pr_z = b.p2 + 3 * tile_cols;
  d.pm_u = b.pu;
  d.ps_u = b.pu + tile_cols;
  d.pi_u = reinterpret_cast<int32_t*>(b.pu + 2 * tile_cols);
  d.pq_u = b.pu + 3 * tile_cols;
  d.pa_u = b.p2 + 2 * tile_cols;
  TRACED(tr, K_STATS_DUAL, 4.0 * rows * H * p->vocab, launch_stats_dual(bf16, d, stream));
  return SPECLOSS_OK;
}

// Pass-2 divergence sums of chunk rows [r0, r0 + rows) into b.p2, with the
// final logsumexps in `sv` (the second sweep recomputes both tiles).
int launch_pass2(const specloss_problem* p, const KindSet& k, const Layout& L, const FwdBufs& b,
                 const SavedView& sv, int64_t r0, int64_t rows, Tracer& tr, hipStream_t stream) {
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
  if (heads_pass2(p, k) && b.hmap) {
    // aligned heads: target rows [jlo, jhi) serve the chunk's rows, each
    // target tile computed once
    const int32_t K = p->n_heads;
    int32_t s_lo, s_hi;
    shift_range(p, s_lo, s_hi);
    const int64_t t_lo = r0 / K, t_hi = (r0 + rows - 1) / K + 1;
    const int64_t jlo = t_lo + s_lo, jhi = t_hi + s_hi;
    const int32_t tiles_n = (int32_t)cdiv(jhi - jlo, 64);
    if ((int64_t)tiles_n * 64 * K > heads_map_entries(p, Nc)) return SPECLOSS_E_INVAL;
    TRACED(tr, K_HEADS_MAP, (double)tiles_n * 64 * K * 4,
           launch_heads_map(b.hmap, tiles_n, K, p->head_shift, jlo, r0, (int32_t)rows, stream));
    DivHeadsLaunch hv{};
    hv.d = dv;
    hv.d.Bz = op(offset_rows(p->hidden_states, r0, H, L.es), H, rows, b.hmap,
                 (int64_t)tiles_n * 64 * K);
    const int64_t jb = jlo < p->n_target_rows ? jlo : p->n_target_rows - 1;
    hv.d.Bu = op(offset_rows(p->target_hidden, jb, H, L.es), H, p->n_target_rows - jb);
    hv.d.tiles_n = tiles_n;
    hv.n_heads = K;
    for (int i = 0; i < K; ++i) hv.shifts[i] = p->head_shift[i];
    hv.jlo = jlo;
    hv.r0 = r0;
    hv.rows = (int32_t)rows;
    TRACED(tr, K_DIV_HEADS, 2.0 * (double)(rows + (jhi - jlo)) * H * p->vocab,
           launch_div_heads(bf16, hv, stream));
    return SPECLOSS_OK;
  }
  TRACED(tr, K_DIV, 4.0 * rows * H * p->vocab, launch_div(bf16, dv, stream));
  return SPECLOSS_OK;
}

// Merge of a chunk's pass-1 partials: both sides when each row has its own
// target row (with the log-ratio sums of the dual pass 1 when `dual`), the
// draft side plus the gathered per-target-row statistics otherwise.
int merge_pass1(const specloss_problem* p, const KindSet& k, const Layout& L, const FwdBufs& b,
                const SavedView& sv, int64_t r0, int64_t rows, bool dual, Tracer& tr,
                hipStream_t stream) {
  const int64_t Nc = b.Nc, tile_cols = L.Tv * Nc;
  const bool own_target = k.target && !L.shared_target;
  Combine1Launch c1{};
  c1.tiles_m = (int32_t)L.Tv;
  c1.ncols = (int32_t)rows;
  c1.ldp = (int32_t)Nc;
  c1.pm_z = b.pz;
  c1.ps_z = b.pz + tile_cols;
  c1.pm_u = own_target ? b.pu : nullptr;
  c1.target_absent = k.target ? 0 : 1;
  c1.ps_u = own_target ? b.pu + tile_cols : nullptr;
  c1.pi_u = own_target ? reinterpret_cast<const int32_t*>(b.pu + 2 * tile_cols) : nullptr;
  c1.pq_u = own_target ? b.pu + 3 * tile_cols : nullptr;
  c1.vocab = (int32_t)p->vocab;
  c1.flags = sv.flags + r0;
  c1.lse_q = sv.lse_q + r0;
  c1.lse_p = sv.lse_p + r0;
  c1.y_arg = sv.y_arg + r0;
  c1.flat = sv.flat + r0;
  if (dual) {
    c1.pa_u = b.p2 + 2 * tile_cols;
    c1.pr_z = b.p2 + 3 * tile_cols;
    c1.kl_out = (k.need & SUM_KL) ? b.p2 + 2 * tile_cols : nullptr;
    c1.rkl_out = (k.need & SUM_RKL) ? b.p2 + 3 * tile_cols : nullptr;
  }
  TRACED(tr, K_COMBINE1, (own_target ? (dual ? 8.0 : 6.0) : 2.0) * L.Tv * rows * 4,
         launch_combine1(c1, stream));
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
  return SPECLOSS_OK;
}

// The label logit z_y (ce_label) and z at argmax p (ce) of each chunk row.
int gather_label_logits(const specloss_problem* p, const KindSet& k, const Layout& L,
                        const FwdBufs& b, const SavedView& sv, int64_t r0, int64_t rows,
                        Tracer& tr, hipStream_t stream) {
  const bool ce_lab = (k.active >> SPECLOSS_CE_LABEL) & 1u;
  const bool ce_arg = (k.active >> SPECLOSS_CE_ARGMAX_P) & 1u;
  if (!ce_lab && !ce_arg) return SPECLOSS_OK;
  RowdotLaunch rd{};
  rd.W = p->W;
  rd.h = offset_rows(p->hidden_states, r0, L.H, L.es);
  rd.H = L.H;
  rd.ncols = (int32_t)rows;
  rd.vocab = (int32_t)p->vocab;
  rd.y1 = ce_lab ? sv.y_label + r0 : nullptr;
  rd.y2 = ce_arg ? sv.y_arg + r0 : nullptr;
  rd.out1 = b.zy;
  rd.out2 = b.zy + b.Nc;
  TRACED(tr, K_ROWDOT, 2.0 * rows * L.H * L.es * ((ce_lab ? 1 : 0) + (ce_arg ? 1 : 0)),
         launch_rowdot(p->in_dtype == SPECLOSS_BF16, rd, stream));
  return SPECLOSS_OK;
}

// Per-row weighted losses, unweighted terms and saved sums of a chunk from
// the pass-2 partials (tiles_m tile rows of them).
int combine_losses(const specloss_problem* p, const KindSet& k, const Layout& L, const FwdBufs& b,
                   const SavedView& sv, float* loss, float* terms, int64_t r0, int64_t rows,
                   int32_t tiles_m, Tracer& tr, hipStream_t stream) {
  const int64_t Nc = b.Nc;
  const bool ce_lab = (k.active >> SPECLOSS_CE_LABEL) & 1u;
  const bool ce_arg = (k.active >> SPECLOSS_CE_ARGMAX_P) & 1u;
  Combine2Launch c2{};
  c2.tiles_m = tiles_m;
  c2.ncols = (int32_t)rows;
  c2.ldp = (int32_t)Nc;
  c2.part = b.p2;
  c2.part_stride = L.Tv * Nc;
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
  TRACED(tr, K_COMBINE2, (double)rows * 4 * (2 + __builtin_popcount(k.need) * c2.tiles_m),
         launch_combine2(c2, stream));
  return SPECLOSS_OK;
}

// Forward of chunk rows [r0, r0 + rows): pass 1 (q side; p side with argmax
// and flatness), merge, label-logit gather, pass 2 and the per-row losses.
// With `stage` ([Nc][Vp], label / argmax cross-entropies of the single call)
// pass 1 also stores e = exp(z - m_tile) there for the logit gradient.
int fwd_chunk(const specloss_problem* p, const KindSet& k, const Layout& L, const FwdBufs& b,
              const SavedView& sv, float* loss, float* terms, int64_t r0, int64_t rows,
              void* stage, Tracer& tr, hipStream_t stream) {
  const bool own_target = k.target && !L.shared_target;
  // kl_div / rkl as the only divergences of a forward without staging: both
  // sides in one pass that also yields the divergences
  const bool dual = k.ratio_only && own_target && !stage;
  if (dual) TRY(launch_pass1_dual(p, L, b, r0, rows, tr, stream));
  else TRY(launch_pass1(p, k, L, b, r0, rows, stage, tr, stream, !own_target));
  TRY(merge_pass1(p, k, L, b, sv, r0, rows, dual, tr, stream));
  TRY(gather_label_logits(p, k, L, b, sv, r0, rows, tr, stream));
  if (k.pass2 && !dual) TRY(launch_pass2(p, k, L, b, sv, r0, rows, tr, stream));
  // dual: the divergences themselves, in tile row 0
  return combine_losses(p, k, L, b, sv, loss, terms, r0, rows, dual ? 1 : (int32_t)L.Tv, tr,
                        stream);
}

// The previous chunk's span of target rows (aligned heads).  Consecutive
// chunks' spans overlap by a few rows (the spread of the shifts plus one or
// two): those rows move to the front of ur instead of being computed again,
// so every chunk after the first contracts only its Nc / K new target rows
// (whole 256-row tiles when Nc / K is a multiple of 256).
struct SpanCarry {
  int64_t jlo = 0, jhi = 0;
  bool valid = false;
};

// The raw fp32 logit rows of chunk rows [r0, r0 + rows) with pass 1's
// contractions: z into zr [Nc][Vp], u into ur [Nu][Vp]; `rr` describes them.
// With aligned heads the target side runs once over the chunk's span of
// target rows [jlo, jhi) (ur holds one row per token of the span, read
// through target_row - jlo); otherwise u is kept per chunk row.  `stats`:
// also the pass-1 statistics (partials in b.pz / b.pu and, for aligned
// heads, merged per target row into b.tstat; other shared target rows take
// theirs from the prepass), else the partials are scratch.
int raw_pass1(const specloss_problem* p, const KindSet& k, const Layout& L, const FwdBufs& b,
              int64_t r0, int64_t rows, float* zr, float* ur, RawRows& rr, SpanCarry& carry,
              bool stats, Tracer& tr, hipStream_t stream) {
  const bool bf16 = p->in_dtype == SPECLOSS_BF16;
  const int64_t H = L.H, Nc = b.Nc, tile_cols = L.Tv * Nc;
  rr = RawRows{zr, L.Vp, ur, L.Vp, nullptr, 0, (int32_t)Nc};

  StatsLaunch sz{};
  sz.A = op(p->W, H, p->vocab);
  sz.B = op(offset_rows(p->hidden_states, r0, H, L.es), H, rows);
  sz.k_len = (int32_t)H;
  sz.vocab = (int32_t)p->vocab;
  sz.tiles_m = (int32_t)L.Tv;
  sz.tiles_n = (int32_t)cdiv(rows, 256);
  sz.ncols = (int32_t)rows;
  sz.ldp = (int32_t)Nc;
  sz.pm = b.pz;
  sz.ps = b.pz + tile_cols;
  sz.raw = zr;
  sz.ld_raw = L.Vp;
  TRACED(tr, K_STATS_Q, 2.0 * rows * H * p->vocab, launch_stats(bf16, false, sz, stream));

  StatsLaunch su = sz;
  su.A = op(p->W_t, H, p->vocab);
  su.raw = ur;
  if (L.shared_target && heads_pass2(p, k)) {
    int64_t jlo, jhi;
    heads_span(p, r0, rows, jlo, jhi);
    const int64_t nu = jhi - jlo, Nt = p->n_target_rows;
    if (nu > L.Nu) return SPECLOSS_E_INVAL;
    int64_t keep = 0;  // leading rows of the span already computed
    if (carry.valid && jlo >= carry.jlo && jlo < carry.jhi) {
      keep = (carry.jhi < jhi ? carry.jhi : jhi) - jlo;
      const int64_t from = jlo - carry.jlo;  // their rows in ur
      if (from < keep) {
        keep = 0;  // source and destination would overlap: compute them again
      } else {
        const size_t bytes = (size_t)keep * L.Vp * 4;
        TRACED(tr, K_SPAN_CARRY, 2.0 * bytes,
               hipMemcpyAsync(ur, ur + from * L.Vp, bytes, hipMemcpyDeviceToDevice, stream));
      }
    }
    carry = SpanCarry{jlo, jhi, true};
    const int64_t j0 = jlo + keep, nn = jhi - j0;  // new rows [j0, jhi)
    if (nn > 0) {
      // rows past the last target row serve masked rows only: the operand
      // clamps them into the tensor
      const int64_t jb = j0 < Nt ? j0 : Nt - 1;
      const int64_t ucols = L.pu_cols, ufield = L.Tv * ucols;
      su.B = op(offset_rows(p->target_hidden, jb, H, L.es), H, Nt - jb);
      su.tiles_n = (int32_t)cdiv(nn, 256);
      su.ncols = (int32_t)nn;
      su.ldp = (int32_t)ucols;
      su.pm = b.pu;
      su.ps = b.pu + ufield;
      su.pi = reinterpret_cast<int32_t*>(b.pu + 2 * ufield);
      su.pq = b.pu + 3 * ufield;
      su.raw = ur + keep * L.Vp;
      TRACED(tr, K_STATS_P, 2.0 * nn * H * p->vocab, launch_stats(bf16, stats, su, stream));
      if (stats && j0 < Nt) {
        // statistics per target row
        char* tb = static_cast<char*>(b.tstat);
        const size_t fs = align_up((size_t)Nt * 4, kAlign);
        const int64_t nt = nn < Nt - j0 ? nn : Nt - j0;
        Combine1Launch c1{};
        c1.tiles_m = (int32_t)L.Tv;
        c1.ncols = (int32_t)nt;
        c1.ldp = (int32_t)ucols;
        c1.pm_u = su.pm;
        c1.ps_u = su.ps;
        c1.pi_u = su.pi;
        c1.pq_u = su.pq;
        c1.vocab = (int32_t)p->vocab;
        c1.lse_p = reinterpret_cast<float*>(tb) + j0;
        c1.y_arg = reinterpret_cast<int32_t*>(tb + fs) + j0;
        c1.flat = reinterpret_cast<float*>(tb + 2 * fs) + j0;
        TRACED(tr, K_COMBINE1, 4.0 * L.Tv * nt * 4, launch_combine1(c1, stream));
      }
    }
    rr.urow = p->target_row + r0;
    rr.ushift = jlo;
    rr.n_u = (int32_t)nu;
  } else {
    su.B = target_operand(p, r0, rows, L.es);
    su.pm = b.pu;
    su.ps = b.pu + tile_cols;
    su.pi = reinterpret_cast<int32_t*>(b.pu + 2 * tile_cols);
    su.pq = b.pu + 3 * tile_cols;
    // shared target rows: the statistics come from the prepass, only u is kept
    TRACED(tr, K_STATS_P, 2.0 * rows * H * p->vocab,
           launch_stats(bf16, stats && !L.shared_target, su, stream));
  }
  return SPECLOSS_OK;
}

// Forward of chunk rows [r0, r0 + rows) for the divergences that keep raw
// logits (the single call, and the two-call forward when its workspace holds
// them): raw_pass1 with statistics, the merge, the label logits, the second
// sweep's sums from the raw rows (k_div_raw) and the per-row losses (blog
// "Backward pass": at most chunk x vocab x 2 logits-sized values are held,
// here in fp32).  Fills `rr` for the logit gradient.
int div_chunk_raw(const specloss_problem* p, const KindSet& k, const Layout& L, const FwdBufs& b,
                  const SavedView& sv, float* loss, float* terms, int64_t r0, int64_t rows,
                  float* zr, float* ur, RawRows& rr, SpanCarry& carry, Tracer& tr,
                  hipStream_t stream) {
  const int64_t Nc = b.Nc, tile_cols = L.Tv * Nc;
  TRY(raw_pass1(p, k, L, b, r0, rows, zr, ur, rr, carry, true, tr, stream));
  TRY(merge_pass1(p, k, L, b, sv, r0, rows, false, tr, stream));
  TRY(gather_label_logits(p, k, L, b, sv, r0, rows, tr, stream));

  DivRawLaunch dv{};
  dv.r = rr;
  dv.tiles_m = (int32_t)L.Tv;
  dv.ncols = (int32_t)rows;
  dv.vocab = (int32_t)p->vocab;
  dv.ldp = (int32_t)Nc;
  dv.lse_q = sv.lse_q + r0;
  dv.lse_p = sv.lse_p + r0;
  dv.need = k.need;
  dv.part = b.p2;
  dv.part_stride = tile_cols;
  TRACED(tr, K_DIV_RAW, (double)rows * L.Vp * 8, launch_div_raw(dv, stream));
  return combine_losses(p, k, L, b, sv, loss, terms, r0, rows, (int32_t)L.Tv, tr, stream);
}

// Forward of chunk rows [r0, r0 + rows) for the label / argmax
// cross-entropies in the single call, staging the logit gradient for both
// contractions without a pass of its own: the target side first (argmax p),
// then the label logits, which are each row's staging reference, then pass 1
// of the draft side, staging exp(z - reference) in both layouts, the merges,
// the per-row losses and k_stage_fix (row factors, far rows, one-hot terms).
// Afterwards dz = rscale[row] * e in e ([Nc][Vp]) and et ([Vp][Nc], or null).
int ce_chunk_staged(const specloss_problem* p, const KindSet& k, const Layout& L,
                    const FwdBufs& b, const SavedView& sv, float* loss, float* terms,
                    const float* seed, int64_t r0, int64_t rows, void* e, void* et,
                    float* rscale, Tracer& tr, hipStream_t stream) {
  // rscale [Nc], then row maxima and the tiles' label logits ([Nc] each)
  float* row_max = rscale + b.Nc;
  float* zt_lab = rscale + 2 * b.Nc;
  float* zt_arg = rscale + 3 * b.Nc;
  const bool bf16 = p->in_dtype == SPECLOSS_BF16;
  const int64_t H = L.H, Nc = b.Nc, tile_cols = L.Tv * Nc;
  const bool ce_lab = (k.active >> SPECLOSS_CE_LABEL) & 1u;
  const bool ce_arg = (k.active >> SPECLOSS_CE_ARGMAX_P) & 1u;

  StatsLaunch sz{};
  sz.A = op(p->W, H, p->vocab);
  sz.B = op(offset_rows(p->hidden_states, r0, H, L.es), H, rows);
  sz.k_len = (int32_t)H;
  sz.vocab = (int32_t)p->vocab;
  sz.tiles_m = (int32_t)L.Tv;
  sz.tiles_n = (int32_t)cdiv(rows, 256);
  sz.ncols = (int32_t)rows;
  sz.ldp = (int32_t)Nc;
  sz.pm = b.pz;
  sz.ps = b.pz + tile_cols;

  // target side: lse_p, argmax p, flatness
  if (k.target && !L.shared_target) {
    StatsLaunch su = sz;
    su.A = op(p->W_t, H, p->vocab);
    su.B = target_operand(p, r0, rows, L.es);
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
    c1.flags = sv.flags + r0;
    c1.lse_p = sv.lse_p + r0;
    c1.y_arg = sv.y_arg + r0;
    c1.flat = sv.flat + r0;
    TRACED(tr, K_COMBINE1, 4.0 * L.Tv * rows * 4, launch_combine1(c1, stream));
  } else if (L.shared_target) {
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

  // label logits (each row's staging reference; also the losses' z_y)
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

  // draft side: pass 1 with staging relative to the reference
  StatsStageLaunch ss{};
  ss.st = sz;
  ss.stage = e;
  ss.ld_stage = L.Vp;
  ss.stage_t = et;
  ss.ld_stage_t = L.ld_t;
  ss.ref = ce_lab ? b.zy : b.zy + Nc;
  ss.seed = seed + r0;
  ss.y1 = ce_lab ? sv.y_label + r0 : nullptr;
  ss.y2 = ce_arg ? sv.y_arg + r0 : nullptr;
  ss.zt1 = zt_lab;
  ss.zt2 = zt_arg;
  TRACED(tr, K_STATS_STAGE, 2.0 * rows * H * p->vocab, launch_stats_stage(bf16, ss, stream));
  Combine1Launch c1{};
  c1.tiles_m = (int32_t)L.Tv;
  c1.ncols = (int32_t)rows;
  c1.ldp = (int32_t)Nc;
  c1.pm_z = b.pz;
  c1.ps_z = b.pz + tile_cols;
  c1.vocab = (int32_t)p->vocab;
  c1.flags = sv.flags + r0;
  c1.lse_q = sv.lse_q + r0;
  c1.lse_p = sv.lse_p + r0;
  c1.y_arg = sv.y_arg + r0;
  c1.flat = sv.flat + r0;
  c1.row_max = row_max;
  c1.target_absent = k.target ? 0 : 1;
  TRACED(tr, K_COMBINE1, 2.0 * L.Tv * rows * 4, launch_combine1(c1, stream));

  Combine2Launch c2{};
  c2.tiles_m = (int32_t)L.Tv;
  c2.ncols = (int32_t)rows;
  c2.ldp = (int32_t)Nc;
  c2.part = b.p2;
  c2.part_stride = tile_cols;
  c2.need = 0;
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
  TRACED(tr, K_COMBINE2, (double)rows * 4 * 2, launch_combine2(c2, stream));

  StageFixLaunch sf{};
  sf.ncols = (int32_t)rows;
  sf.tiles_m = (int32_t)L.Tv;
  sf.ldp = (int32_t)Nc;
  sf.r0 = r0;
  sf.pm = b.pz;
  sf.ref = ss.ref;
  sf.row_max = row_max;
  sf.seed = seed;
  sf.sv = sv;
  sf.zt_lab = zt_lab;
  sf.zt_arg = zt_arg;
  sf.w_lab = p->weights[SPECLOSS_CE_LABEL];
  sf.w_arg = p->weights[SPECLOSS_CE_ARGMAX_P];
  sf.stage = e;
  sf.ld_stage = L.Vp;
  sf.stage_t = et;
  sf.ld_stage_t = L.ld_t;
  sf.rscale = rscale;
  TRACED(tr, K_STAGE_FIX, (double)rows * 32, launch_stage_fix(bf16, sf, stream));
  return SPECLOSS_OK;
}

// dz (and dz^T when dzt is set) of chunk rows [r0, r0 + rows) from the raw
// logit rows `rr`, the seeds and the saved per-row sums.
int dz_from_raw(const specloss_problem* p, const Layout& L, const RawRows& rr, int64_t r0,
                int64_t rows, const float* seed, const SavedView& sv, void* dz, void* dzt,
                Tracer& tr, hipStream_t stream) {
  DzRawLaunch dr{};
  dr.r = rr;
  dr.tiles_m = (int32_t)L.Tv;
  dr.ncols = (int32_t)rows;
  dr.vocab = (int32_t)L.V;
  dr.r0 = r0;
  dr.seed = seed;
  dr.sv = sv;
  dr.w_lab = p->weights[SPECLOSS_CE_LABEL];
  dr.w_arg = p->weights[SPECLOSS_CE_ARGMAX_P];
  dr.w_kl = p->weights[SPECLOSS_KL];
  dr.w_tv = p->weights[SPECLOSS_TV];
  dr.w_nla = p->weights[SPECLOSS_NLA];
  dr.w_lk = p->weights[SPECLOSS_LK_HYBRID];
  dr.w_rkl = p->weights[SPECLOSS_RKL];
  dr.w_jsd = p->weights[SPECLOSS_JSD];
  dr.dz = dz;
  dr.ld_dz = L.Vp;
  dr.dzt = dzt;
  dr.ld_dzt = L.ld_t;
  dr.row_blocks = (int32_t)(cdiv(rows, 256) * 4);
  TRACED(tr, K_DZ_RAW, (double)dr.row_blocks * 64 * L.Vp * (8.0 + L.es * (dzt ? 2 : 1)),
         launch_dz_raw(p->in_dtype == SPECLOSS_BF16, dr, stream));
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
// and the copy W^T [H][Vp]; without that copy (bf16), W is read as it is (an
// MN-major operand).
int contract_dh(const specloss_problem* p, const Layout& L, int64_t Nc, const void* dz,
                const void* wt, int64_t r0, int64_t rows, void* dhidden, int32_t dh_dtype,
                Tracer& tr, hipStream_t stream, const float* rscale = nullptr,
                float* dhp = nullptr, void* dzt = nullptr, int64_t ld_dzt = 0) {
  const bool bf16 = p->in_dtype == SPECLOSS_BF16;
  const int64_t H = L.H, V = L.V, Vp = L.Vp;
  const size_t dh_es = dh_dtype == SPECLOSS_BF16 ? 2 : 4;
  GemmLaunch g{};
  g.A = op(dz, Vp, Nc);
  g.lean = !L.wt_copy;
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
  char* out = static_cast<char*>(dhidden) + (size_t)r0 * H * dh_es;
  g.C = out;
  g.ldc = H;
  g.accumulate = 0;
  g.out_bf16 = dh_dtype == SPECLOSS_BF16;
  g.role = 0;
  g.rscale = rscale;
  g.at_out = dzt;
  g.ld_at = ld_dzt;
  g.splits = 1;
  if (L.dh_splits > 1 && dhp) {
    // slices of K, fp32 partials in the workspace, added in slice order
    g.splits = L.dh_splits;
    g.k_split = (int32_t)round_up(cdiv(g.k_len, g.splits), 64);
    while (g.splits > 1 && (int64_t)(g.splits - 1) * g.k_split >= g.k_len) --g.splits;
    g.C = dhp;
    g.out_bf16 = 0;
    g.part_stride = (int64_t)rows * H;
  }
  // the dh contraction that also writes dz^T has a trace name of its own
  TRACED(tr, g.at_out ? K_GEMM_DH_DZT : K_GEMM_DH, 2.0 * rows * H * V,
         launch_gemm(bf16, g, stream));
  if (g.splits > 1)
    TRACED(tr, K_SUM_PARTS, 4.0 * rows * H * (g.splits + 1),
           launch_sum_parts(dhp, rows * H, g.splits, out, dh_dtype == SPECLOSS_BF16, stream));
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
  g.lean = !L.dw_copies;
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
  g.splits = 1;
  TRACED(tr, K_GEMM_DW, 2.0 * rows * H * V, launch_gemm(bf16, g, stream));
  return SPECLOSS_OK;
}

// The dW contraction after chunk `chunk` (rows [r0, r0 + rows)): once the
// last chunk of its dW group, or of the problem, has written its copies'
// columns; K spans the group's rows.  Groups accumulate in order, the first
// overwrites dW unless accumulate_dW.
int dw_after_chunk(const specloss_problem* p, const Layout& L, int chunk, int64_t r0,
                   int64_t rows, const void* dz, const void* dzt, const void* ht,
                   int accumulate_dW, float* dW, Tracer& tr, hipStream_t stream) {
  const int32_t G = L.dw_group;
  const int64_t slot = chunk % G;
  if (slot != G - 1 && r0 + rows < L.N) return SPECLOSS_OK;
  const int64_t g0 = r0 - slot * L.Nc;
  return contract_dW(p, L, L.Nc, dz, dzt, ht, L.ld_t, g0, r0 + rows - g0,
                     chunk >= G || accumulate_dW, dW, tr, stream);
}

// The copies' columns of chunk `chunk` (dw_group slots of Nc columns).
void* slot_cols(void* base, const Layout& L, int chunk) {
  return base ? static_cast<char*>(base) + (size_t)(chunk % L.dw_group) * L.Nc * L.es : nullptr;
}

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
                  int accumulate_dW, int64_t vocab_offset, bool shard, hipStream_t stream) {
  int32_t layout = LAYOUT_COPIES, group = 1;
  bool raw = false;
  const int64_t Nc = pick_bwd_chunk(p, k, ws_bytes, &layout, &raw, shard, &group);
  if (Nc <= 0) return SPECLOSS_E_WORKSPACE;
  const Layout L = plan(p, k, Nc, layout, false, raw, group);
  char* ws = static_cast<char*>(workspace);
  const bool bf16 = p->in_dtype == SPECLOSS_BF16;
  const int64_t N = L.N, H = L.H, V = L.V, Vp = L.Vp;
  const SavedView sv = saved_view(const_cast<void*>(saved), N);
  float* seed = reinterpret_cast<float*>(ws + L.seed);
  void* wt = L.wt_copy ? ws + L.wt : nullptr;
  void* ht = L.dw_copies ? ws + L.ht : nullptr;
  void* dz = ws + L.dz;
  void* dzt = L.dw_copies ? ws + L.dzt : nullptr;
  Tracer tr{p->trace, stream};
  // raw logit rows: partials are scratch, the span carry as in the forward
  const FwdBufs rb{reinterpret_cast<float*>(ws + L.b_pz), reinterpret_cast<float*>(ws + L.b_pu),
                   nullptr, nullptr, Nc, nullptr, nullptr};
  SpanCarry carry;

  TRY(launch_seed_for(p, sv, grad_loss, grad_mean, counts, seed, tr, stream));
  if (dhidden && L.wt_copy)
    TRACED(tr, K_TRANSPOSE_W, 2.0 * Vp * H * L.es, launch_transpose(bf16, p->W, V, H, wt, Vp, Vp, stream));

  int chunk = 0;
  for (int64_t r0 = 0; r0 < N; r0 += Nc, ++chunk) {
    const int64_t rows = (N - r0) < Nc ? (N - r0) : Nc;
    const void* hc = offset_rows(p->hidden_states, r0, H, L.es);
    void* htc = slot_cols(ht, L, chunk);
    void* dztc = slot_cols(dzt, L, chunk);
    if (dW && L.dw_copies)
      TRACED(tr, K_TRANSPOSE_H, 2.0 * Nc * H * L.es,
             launch_transpose(bf16, hc, rows, H, htc, Nc, L.ld_t, stream));

    if (raw) {
      RawRows rr{};
      TRY(raw_pass1(p, k, L, rb, r0, rows, reinterpret_cast<float*>(ws + L.b_zr),
                    reinterpret_cast<float*>(ws + L.b_ur), rr, carry, false, tr, stream));
      TRY(dz_from_raw(p, L, rr, r0, rows, seed, sv, dz, dztc, tr, stream));
      if (dhidden)
        TRY(contract_dh(p, L, Nc, dz, wt, r0, rows, dhidden, dh_dtype, tr, stream, nullptr,
                        reinterpret_cast<float*>(ws + L.dhp)));
      if (dW)
        TRY(dw_after_chunk(p, L, chunk, r0, rows, dz, dzt, ht, accumulate_dW, dW, tr, stream));
      continue;
    }
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
    dl.dzt = dztc;
    dl.ld_dzt = L.ld_t;
    dl.vocab_offset = (int32_t)vocab_offset;
    TRACED(tr, K_DZ, (k.dual_bwd ? 4.0 : 2.0) * rows * H * V, launch_dz(bf16, k.dual_bwd, dl, stream));
    if (dhidden)
      TRY(contract_dh(p, L, Nc, dz, wt, r0, rows, dhidden, dh_dtype, tr, stream, nullptr,
                      reinterpret_cast<float*>(ws + L.dhp)));
    if (dW)
      TRY(dw_after_chunk(p, L, chunk, r0, rows, dz, dzt, ht, accumulate_dW, dW, tr, stream));
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
  int32_t layout = LAYOUT_COPIES, group = 1;
  int64_t nc;
  if (max_chunk_rows <= 0) {
    nc = default_chunk(p, k, &layout, &group);
  } else {
    const int32_t forced = forced_layout(p);
    layout = forced >= 0 ? forced : LAYOUT_COPIES;
    nc = round_up(max_chunk_rows, kChunkQuantum);
    nc = nc < round_up(p->n_rows, kChunkQuantum) ? nc : round_up(p->n_rows, kChunkQuantum);
  }
  *bytes = workspace_end(plan(p, k, nc, layout, false, false, group));
  return SPECLOSS_OK;
}

int lmhead_loss_chunk(const specloss_problem* p, size_t ws_bytes, int32_t call,
                      int64_t* chunk_rows, int32_t* layout, int32_t* dw_group) {
  KindSet k;
  TRY(check_problem(p, &k));
  if (!chunk_rows || !layout || call < 0 || call > 2) return SPECLOSS_E_INVAL;
  int32_t lay = LAYOUT_COPIES, group = 1;
  int64_t nc;
  if (call == 0) {
    bool raw;
    nc = pick_fwd_chunk(p, k, ws_bytes, &raw);
  } else if (call == 1) {
    bool raw;
    nc = pick_bwd_chunk(p, k, ws_bytes, &lay, &raw, false, &group);
  } else {
    nc = pick_chunk(p, k, ws_bytes, REGION_FUSED, &lay, &group);
  }
  if (nc <= 0) return SPECLOSS_E_WORKSPACE;
  const Layout L = plan(p, k, nc, lay, false, false, group);
  *chunk_rows = nc;
  *layout = L.layout;
  if (dw_group) *dw_group = L.dw_group;
  return SPECLOSS_OK;
}

int lmhead_loss_fwd(const specloss_problem* p, void* workspace, size_t ws_bytes, float* loss,
                    float* term_loss, float* lse_q, void* saved, int64_t* counts, float* reduced,
                    hipStream_t stream) {
  KindSet k;
  TRY(check_problem(p, &k));
  TRY(check_fwd_outputs(loss, term_loss, lse_q, saved, counts, reduced));
  if (!workspace || !aligned(workspace, kAlign)) return SPECLOSS_E_WORKSPACE;
  bool raw = false;
  const int64_t Nc = pick_fwd_chunk(p, k, ws_bytes, &raw);
  if (Nc <= 0) return SPECLOSS_E_WORKSPACE;
  const Layout L = plan(p, k, Nc, LAYOUT_COPIES, raw);
  char* ws = static_cast<char*>(workspace);
  const int64_t N = L.N;
  const SavedView sv = saved_view(saved ? saved : ws + L.saved, N);
  float* terms = term_loss ? term_loss : reinterpret_cast<float*>(ws + L.terms);
  const FwdBufs b{reinterpret_cast<float*>(ws + L.pz), reinterpret_cast<float*>(ws + L.pu),
                  reinterpret_cast<float*>(ws + L.p2), reinterpret_cast<float*>(ws + L.zy), Nc,
                  ws + L.tstat, raw ? nullptr : reinterpret_cast<int32_t*>(ws + L.hmap)};
  Tracer tr{p->trace, stream};

  TRY(launch_validity_for(p, k, sv, counts, tr, stream));
  // aligned heads with raw logits: the target statistics come per chunk
  if (L.shared_target && !(raw && heads_pass2(p, k))) TRY(target_prepass(p, L, b, tr, stream));
  SpanCarry carry;
  for (int64_t r0 = 0; r0 < N; r0 += Nc) {
    const int64_t rows = (N - r0) < Nc ? (N - r0) : Nc;
    if (raw) {
      RawRows rr{};
      TRY(div_chunk_raw(p, k, L, b, sv, loss, terms, r0, rows, reinterpret_cast<float*>(ws + L.zr),
                        reinterpret_cast<float*>(ws + L.ur), rr, carry, tr, stream));
    } else {
      TRY(fwd_chunk(p, k, L, b, sv, loss, terms, r0, rows, nullptr, tr, stream));
    }
  }
  if (reduced) TRY(launch_reduce_for(p, k, loss, terms, counts, reduced, tr, stream));
  if (lse_q)
    TRACED(tr, K_COPY, (double)N * 8,
           hipMemcpyAsync(lse_q, sv.lse_q, (size_t)N * 4, hipMemcpyDeviceToDevice, stream));
  return SPECLOSS_OK;
}

int lmhead_loss_fwd_noalloc(const specloss_problem* p, float* loss, float* term_loss,
                            float* lse_q, void* saved, int64_t* counts, float* reduced,
                            hipStream_t stream) {
  KindSet k;
  TRY(check_problem(p, &k));
  TRY(check_fwd_outputs(loss, term_loss, lse_q, saved, counts, reduced));
  // the forward region at its smallest chunk must fit the fixed scratch
  if (pick_chunk(p, k, kNoAllocScratchBytes, REGION_FWD) <= 0) return SPECLOSS_E_WORKSPACE;
  void* ws = nullptr;
  HIP_TRY(noalloc_scratch(&ws));
  return lmhead_loss_fwd(p, ws, kNoAllocScratchBytes, loss, term_loss, lse_q, saved, counts,
                         reduced, stream);
}

int lmhead_loss_bwd(const specloss_problem* p, const float* grad_loss, const float* grad_mean,
                    const int64_t* counts, const void* saved, void* workspace, size_t ws_bytes,
                    void* dhidden, int32_t dh_dtype, float* dW, int accumulate_dW,
                    hipStream_t stream) {
  KindSet k;
  TRY(check_problem(p, &k));
  TRY(check_bwd_inputs(grad_loss, grad_mean, counts, saved, dhidden, dh_dtype, dW, workspace));
  return bwd_recompute(p, k, grad_loss, grad_mean, counts, saved, workspace, ws_bytes, dhidden,
                       dh_dtype, dW, accumulate_dW, 0, false, stream);
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
  // label / argmax cross-entropies: pass 1 stages exp(z - ref) per chunk
  // (ce_chunk_staged); with divergences, pass 1 keeps both raw logit rows
  // (div_chunk_raw), from which the sums and then the logit gradient are
  // formed.  No logits tile is computed twice.
  int32_t layout = LAYOUT_COPIES, group = 1;
  const int64_t Nc = pick_chunk(p, k, ws_bytes, REGION_FUSED, &layout, &group);
  if (Nc <= 0) return SPECLOSS_E_WORKSPACE;
  const Layout L = plan(p, k, Nc, layout, false, false, group);
  char* ws = static_cast<char*>(workspace);
  const bool bf16 = p->in_dtype == SPECLOSS_BF16;
  const int64_t N = L.N, H = L.H, V = L.V, Vp = L.Vp;
  const SavedView sv = saved_view(saved ? saved : ws + L.saved, N);
  float* terms = term_loss ? term_loss : reinterpret_cast<float*>(ws + L.terms);
  float* seed = reinterpret_cast<float*>(ws + L.seed);
  const FwdBufs b{reinterpret_cast<float*>(ws + L.f_pz), reinterpret_cast<float*>(ws + L.f_pu),
                  k.stage_div ? reinterpret_cast<float*>(ws + L.f_p2) : nullptr,
                  reinterpret_cast<float*>(ws + L.f_zy), Nc, ws + L.tstat, nullptr};
  void* wt = L.wt_copy ? ws + L.f_wt : nullptr;
  void* ht = L.dw_copies ? ws + L.f_ht : nullptr;
  void* dz = ws + L.f_dz;
  float* zr = k.stage_div ? reinterpret_cast<float*>(ws + L.f_zr) : nullptr;
  float* ur = k.stage_div ? reinterpret_cast<float*>(ws + L.f_ur) : nullptr;
  void* dzt = L.dw_copies ? ws + L.f_dzt : nullptr;
  Tracer tr{p->trace, stream};

  TRY(launch_validity_for(p, k, sv, counts, tr, stream));
  TRY(launch_seed_for(p, sv, grad_loss, grad_mean, counts, seed, tr, stream));
  // aligned heads with divergences: the target statistics come per chunk
  if (L.shared_target && !(k.stage_div && heads_pass2(p, k)))
    TRY(target_prepass(p, L, b, tr, stream));
  if (dhidden && L.wt_copy)
    TRACED(tr, K_TRANSPOSE_W, 2.0 * Vp * H * L.es, launch_transpose(bf16, p->W, V, H, wt, Vp, Vp, stream));
  // label / argmax cross-entropies with the dW copies: pass 1 stages the
  // logit gradient in both layouts up to a per-row factor (ce_chunk_staged)
  // (not when w_lab + w_arg = 0: the row factor would vanish)
  const bool staged_ce = !k.stage_div && L.dw_copies &&
                         p->weights[SPECLOSS_CE_LABEL] + p->weights[SPECLOSS_CE_ARGMAX_P] != 0.0f;
  float* rscale = reinterpret_cast<float*>(ws + L.f_rs);
  SpanCarry carry;
  int chunk = 0;
  for (int64_t r0 = 0; r0 < N; r0 += Nc, ++chunk) {
    const int64_t rows = (N - r0) < Nc ? (N - r0) : Nc;
    void* htc = slot_cols(ht, L, chunk);
    void* dztc = slot_cols(dzt, L, chunk);
    if (staged_ce) {
      // with both gradients (bf16) the dh contraction writes dz^T from its
      // slabs of dz; otherwise pass 1 stores it
      const bool dzt_from_dh = dW && dhidden && bf16;
      TRY(ce_chunk_staged(p, k, L, b, sv, loss, terms, seed, r0, rows, dz,
                          dW && !dzt_from_dh ? dztc : nullptr, rscale, tr, stream));
      const void* hc = offset_rows(p->hidden_states, r0, H, L.es);
      if (dW)
        TRACED(tr, K_TRANSPOSE_H, 2.0 * Nc * H * L.es,
               launch_transpose(bf16, hc, rows, H, htc, Nc, L.ld_t, stream, rscale));
      if (dhidden)
        TRY(contract_dh(p, L, Nc, dz, wt, r0, rows, dhidden, dh_dtype, tr, stream, rscale,
                        reinterpret_cast<float*>(ws + L.f_dhp), dzt_from_dh ? dztc : nullptr,
                        L.ld_t));
      if (dW)
        TRY(dw_after_chunk(p, L, chunk, r0, rows, dz, dzt, ht, accumulate_dW, dW, tr, stream));
      continue;
    }
    if (k.stage_div) {
      RawRows rr{};
      TRY(div_chunk_raw(p, k, L, b, sv, loss, terms, r0, rows, zr, ur, rr, carry, tr, stream));
      TRY(dz_from_raw(p, L, rr, r0, rows, seed, sv, dz, dztc, tr, stream));
    } else {
      TRY(fwd_chunk(p, k, L, b, sv, loss, terms, r0, rows, dz, tr, stream));
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
      ds.dz = dz;
      ds.ld_dz = Vp;
      ds.dzt = dztc;
      ds.ld_dzt = L.ld_t;
      ds.row_blocks = (int32_t)(cdiv(rows, 256) * 4);
      TRACED(tr, K_DZ_STAGE, (double)ds.row_blocks * 64 * Vp * L.es * (2 + (dzt ? 1 : 0)),
             launch_dz_stage(bf16, ds, stream));
    }
    const void* hc = offset_rows(p->hidden_states, r0, H, L.es);
    if (dW && L.dw_copies)
      TRACED(tr, K_TRANSPOSE_H, 2.0 * Nc * H * L.es,
             launch_transpose(bf16, hc, rows, H, htc, Nc, L.ld_t, stream));
    if (dhidden)
      TRY(contract_dh(p, L, Nc, dz, wt, r0, rows, dhidden, dh_dtype, tr, stream, nullptr,
                      reinterpret_cast<float*>(ws + L.f_dhp)));
    if (dW)
      TRY(dw_after_chunk(p, L, chunk, r0, rows, dz, dzt, ht, accumulate_dW, dW, tr, stream));
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
    c1.target_absent = k.target ? 0 : 1;
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
  c1.target_absent = k.target ? 0 : 1;
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
      TRY(launch_pass2(p, k, L, b, sv, r0, rows, tr, stream));
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
                       SPECLOSS_F32, dW, accumulate_dW, sh->vocab_offset, true, stream);
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
