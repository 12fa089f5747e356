/*
 * libspecloss: streaming LM-head + loss for speculative draft-head training
 * on one AMD Instinct MI355X (gfx950).
 *
 * The operation (Nebius blog "Training speculative decoders: removing the
 * logits and attention bottlenecks", sections "The logits bottleneck..." and
 * "Streaming Cross Entropy"): hidden states -> LM head -> vocabulary logits ->
 * a per-token loss, computed tile by tile so that the [tokens, vocab] logits
 * tensor never exists in memory.  The losses are the language-model
 * cross-entropy against token labels and the target-vs-draft losses of the
 * vLLM speculators "Loss Functions" page ("Available Losses" table), alone or
 * as an unnormalised weighted sum ("Weighted Combinations").  The backward
 * ("Backward pass" section of the blog) recomputes logits tiles and returns
 * the gradients with respect to the hidden states and the LM-head weight.
 *
 * Notation: N aligned rows (tokens, or (head, position) pairs), hidden size
 * H, vocabulary V.  Draft logits z = W h with q = softmax(z); target logits
 * u = W_t g with p = softmax(u).  W and W_t are [V, H] row-major (one row
 * per vocabulary entry, the layout of a linear layer's weight), no bias.
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the
 *    library never allocates device memory.  Tensors are dense row-major.
 *    Floating tensors (hidden, W, target_hidden, W_t) and the gradient
 *    outputs (dhidden, dW) must be 16-byte aligned; every other pointer
 *    4-byte aligned (8 for counts).
 *  - Work is enqueued on `stream` (NULL = the null stream) and is
 *    asynchronous: outputs are valid once the stream has synchronised.
 *  - Every argument is checked on the host before anything is enqueued.
 *    Return value 0 = success, else a negative SPECLOSS_E_* code and
 *    nothing was enqueued.  An unsupported case is an error; there is no
 *    fallback to another implementation.  SPECLOSS_E_HIP is returned when
 *    a HIP launch fails (work enqueued before it may have run).
 *  - Labels, masks and row maps live on the device and are not inspected
 *    by the host: an unmasked row whose label (or target row) is out of
 *    range is treated as masked and counted in counts[1].
 *  - Results are deterministic: two calls with the same inputs, the same
 *    workspace size and the same device give bitwise-identical outputs.
 *  - Calls that share a workspace must not overlap in time.
 */
#ifndef SPECLOSS_H
#define SPECLOSS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Loss kinds.  Names (specloss_kind_name) follow the speculators page. */
typedef enum {
  SPECLOSS_CE_LABEL = 0,    /* "ce_label": -log q_y, y = given label (blog, "Streaming Cross Entropy") */
  SPECLOSS_CE_ARGMAX_P = 1, /* "ce": -log q_y, y = argmax p, lowest index on ties ("Available Losses", ce) */
  SPECLOSS_KL = 2,          /* "kl_div": KL(p || q) ("Available Losses", kl_div) */
  SPECLOSS_RKL = 3,         /* "rkl": KL(q || p) ("Available Losses", rkl) */
  SPECLOSS_JSD = 4,         /* "jsd": (KL(p||m) + KL(q||m)) / 2, m = (p+q)/2 ("Available Losses", jsd) */
  SPECLOSS_TV = 5,          /* "tv": 1 - alpha, alpha = sum_v min(p_v, q_v) ("Available Losses", tv) */
  SPECLOSS_NLA = 6,         /* "nla": -log alpha ("Available Losses", nla) */
  SPECLOSS_LK_HYBRID = 7,   /* "lk_hybrid": lam KL(p||q) + (1-lam)(1-alpha), lam = exp(-3 alpha)
                               held constant in the backward ("Available Losses", lk_hybrid) */
  SPECLOSS_NUM_KINDS = 8
} specloss_kind;

typedef enum { SPECLOSS_F32 = 0, SPECLOSS_BF16 = 1 } specloss_dtype;

/* Aligned draft heads a problem may declare (specloss_problem.n_heads). */
#define SPECLOSS_MAX_HEADS 4

enum {
  SPECLOSS_OK = 0,
  SPECLOSS_E_INVAL = -1,       /* null/inconsistent argument, bad size, no nonzero weight */
  SPECLOSS_E_UNSUPPORTED = -2, /* H not a multiple of 64, misaligned pointer, unknown dtype */
  SPECLOSS_E_WORKSPACE = -3,   /* workspace missing or smaller than the minimum */
  SPECLOSS_E_HIP = -4          /* a HIP launch failed */
};

#define SPECLOSS_IGNORE_INDEX (-100)

/*
 * Backward layout choice (specloss_problem.flags).  The two gradient
 * contractions read their operands either from transposed copies made in the
 * workspace (W^T for dhidden; the chunk's hidden rows and logit gradient
 * transposed for dW) or in place.  0: automatic (see
 * lmhead_loss_workspace_size).  SPECLOSS_FLAG_COPIES: always make every copy
 * (SPECLOSS_E_WORKSPACE if they do not fit).  SPECLOSS_FLAG_NO_WEIGHT_COPY:
 * the dW copies but no W^T (dhidden reads W in place).  SPECLOSS_FLAG_NO_COPIES:
 * no copy.  The last two are bf16 only (SPECLOSS_E_UNSUPPORTED for fp32).
 * Other values: SPECLOSS_E_INVAL.
 */
#define SPECLOSS_FLAG_COPIES 1
#define SPECLOSS_FLAG_NO_COPIES 2
#define SPECLOSS_FLAG_NO_WEIGHT_COPY 3

/*
 * Per-row state the forward saves for the backward: SPECLOSS_SAVED_FIELDS
 * arrays of N 4-byte values each (see specloss_saved_offset).  The fields a
 * caller may want to read are listed here; the others are internal.
 */
enum {
  SPECLOSS_SAVED_LSE_Q = 0,     /* fp32: logsumexp of the draft logits z */
  SPECLOSS_SAVED_LSE_P = 1,     /* fp32: logsumexp of the target logits u (0 without a target) */
  SPECLOSS_SAVED_Y_ARG = 3,     /* int32: argmax of u, lowest index on ties (-1 without a target) */
  SPECLOSS_SAVED_ALPHA = 4,     /* fp32: alpha = sum_v min(p_v, q_v) ("Available Losses",
                                   tv), written when tv, nla, lk_hybrid or jsd is on;
                                   1 otherwise (with kl_div and rkl as the only
                                   divergences no sum of min(p, q) is formed) */
  SPECLOSS_SAVED_VALID = 8,     /* int32: 1 on valid rows, 0 on masked or bad rows */
  SPECLOSS_SAVED_FLATNESS = 9,  /* fp32: flatness of the target distribution,
                                   cos(p, uniform) = 1 / (sqrt(V) |p|_2), in [1/sqrt(V), 1]
                                   ("Flatter Tokens are More Valuable for Speculative Draft
                                   Model Training", Approach: per-token flatness); written
                                   whenever a target is given, 0 on invalid rows */
  SPECLOSS_SAVED_FIELDS = 10
};

/* Opaque kernel trace (see specloss_trace_create). */
typedef struct specloss_trace specloss_trace;

/*
 * One loss problem.  Rows must already be aligned (blog, "Correctness:
 * alignment before chunking"): row r pairs hidden_states[r] with its label
 * and/or its target row; masks are per aligned row.
 *
 * A row is valid iff mask == NULL or mask[r] != 0, and, when the
 * SPECLOSS_CE_LABEL weight is nonzero, labels[r] != SPECLOSS_IGNORE_INDEX.
 * Invalid rows contribute exactly 0 to every loss and gradient.  The
 * number of valid rows is the loss denominator (blog, "Backward pass":
 * normalise by valid tokens, not by chunks).
 */
typedef struct {
  int64_t n_rows;              /* N > 0, < 2^30 */
  int64_t hidden;              /* H > 0, multiple of 64, < 2^30 */
  int64_t vocab;               /* V > 0, < 2^30 (SPECLOSS_E_UNSUPPORTED above) */
  int32_t in_dtype;            /* specloss_dtype of hidden_states, W, target_hidden, W_t */
  int32_t flags;               /* 0, or one of SPECLOSS_FLAG_* (backward layout choice) */
  const void* hidden_states;   /* [N, H] draft hidden states */
  const void* W;               /* [V, H] draft LM-head weight */
  const int32_t* labels;       /* [N] token labels, or NULL when no label kind is on */
  const void* target_hidden;   /* [n_target_rows, H] target hidden states, or NULL */
  int64_t n_target_rows;       /* rows of target_hidden */
  const void* W_t;             /* [V, H] target LM-head weight (may equal W), or NULL */
  const int32_t* target_row;   /* [N] row of target_hidden for each row, or NULL = identity;
                                  with a map, target_hidden must be smaller than 4 GiB */
  const uint8_t* mask;         /* [N] 0 = masked, or NULL = no mask */
  float weights[SPECLOSS_NUM_KINDS]; /* per-kind weight, used as given (not normalised); 0 = off */
  specloss_trace* trace;       /* NULL, or a trace that records every launch of the call */
  /* Aligned draft heads (blog, "Correctness: alignment before chunking"; the
   * layout specloss_align_heads writes): 0, or K in [1, SPECLOSS_MAX_HEADS]
   * when the rows are token-major heads, row T * K + k being head k at token
   * T, whose target row is T + head_shift[k].  n_rows must be a multiple of
   * K and target_row given; a row that is valid otherwise but has another
   * target row counts as bad.  With K = 2 or 3 (bf16) the second divergence
   * sweep computes each target tile once for the K rows it serves instead of
   * once per row.  Ignored when no kind needs the target side. */
  int32_t n_heads;
  int32_t head_shift[SPECLOSS_MAX_HEADS]; /* 0 <= shift <= 65536 */
} specloss_problem;

/*
 * Bytes of device workspace needed by any of the calls below.  The calls
 * process the rows in chunks (blog, "Streaming Cross Entropy" and "Backward
 * pass": per chunk, its logits, loss and gradients; only per-row statistics
 * outlive a chunk).  The single call and the backward stage a logit-gradient
 * chunk of about 2 x chunk x V elements in the input dtype, which is the
 * blog's streaming bound chunk x vocab x dtype x 2, plus (by default) a
 * transposed copy of W; for the divergences the single call also keeps the
 * chunk's two raw fp32 logit rows (draft and target), chunk x V x 4 x 2
 * bytes, so its chunks are smaller under the same limit.
 *   max_chunk_rows <= 0: the default policy.  The token set is streamed in
 *     at least four balanced chunks of at most 8192 rows, and the whole
 *     workspace stays strictly below N x V x (input element size) bytes, the
 *     size of the full logits tensor ("Backward pass": the streaming loss
 *     never stores the full logits).  Layouts are tried in the order every
 *     copy, no W^T copy, no copy (bf16), each with the largest chunk that
 *     fits; a layout is taken once its chunk reaches min(N, 1024) rows.  When
 *     no chunk fits below that size (tiny problems, whose W^T copy alone
 *     exceeds it), 256-row chunks with every copy are used.
 *   max_chunk_rows > 0: that many rows per chunk (rounded up to a multiple
 *     of 256, at most N rounded up), with every copy unless flags say
 *     otherwise.
 * The calls pick the largest chunk that fits the workspace they are given,
 * with every copy when that chunk reaches min(N, 1024) rows, otherwise
 * (bf16) without the W^T copy or without any copy if that allows a larger
 * chunk; lmhead_loss_chunk reports the choice.
 * dW groups: with the transposed copies (every copy, or no W^T copy), G = 2
 * to 4 consecutive chunks may share one dW contraction, each writing its
 * columns of a dz^T and h^T copy G chunks wide (dW is then read and written
 * once per G chunks).  The default policy and the calls take the group with
 * the fewest dW read-modify-writes among those that fit with a chunk of at
 * least min(N, 1024) rows, are at most 8192 rows deep and save at least two
 * dW contractions over the largest single chunk that would fit.
 * SPECLOSS_E_INVAL for a NULL `bytes` and as for the calls.
 */
int lmhead_loss_workspace_size(const specloss_problem* p, int64_t max_chunk_rows, size_t* bytes);

/*
 * The chunk the calls use with a workspace of ws_bytes: rows per chunk, the
 * backward layout (0 every copy, 1 no W^T copy, 2 no copy) and, when
 * dw_group is not NULL, the chunks per dW contraction (1 to 4; 1 for call 0),
 * for `call` 0 = lmhead_loss_fwd, 1 = lmhead_loss_bwd, 2 =
 * lmhead_loss_fwd_bwd.  Host only.  SPECLOSS_E_WORKSPACE when no chunk fits,
 * SPECLOSS_E_INVAL for a NULL chunk_rows or layout or an unknown call, and as
 * for the calls.
 */
int lmhead_loss_chunk(const specloss_problem* p, size_t ws_bytes, int32_t call,
                      int64_t* chunk_rows, int32_t* layout, int32_t* dw_group);

/*
 * Bytes of the `saved` buffer for n_rows rows (SPECLOSS_SAVED_FIELDS arrays of
 * n_rows 4-byte values, each 256-byte aligned); 0 for n_rows <= 0.  This is
 * the per-row state that outlives a chunk (blog, "Streaming Cross Entropy":
 * the loss of a token needs only its own logsumexp and label logit; the
 * target-vs-draft sums of "Available Losses" per row).  Host only.
 */
size_t specloss_saved_bytes(int64_t n_rows);

/*
 * Byte offset of saved field `field` (SPECLOSS_SAVED_*) inside a saved buffer
 * for n_rows rows; the field is n_rows 4-byte values from there.  Host only,
 * no device access.  SPECLOSS_E_INVAL for n_rows <= 0, an unknown field or
 * a NULL offset.
 */
int specloss_saved_offset(int64_t n_rows, int32_t field, size_t* offset);

/*
 * Forward (blog, "Streaming Cross Entropy": per chunk of tokens, the logits of
 * the chunk, the per-token losses and their sum; "Backward pass": the mean
 * divides by the valid tokens; speculators "Loss Functions", "Available
 * Losses" and "Weighted Combinations" for the kinds and their weights).
 * Outputs (device):
 *   loss      [N]    fp32, required: sum_k weights[k] * L_k(row), 0 on invalid rows.
 *   term_loss [K][N] fp32 or NULL: unweighted L_k(row) for every kind k
 *                    (rows of kinds that are off are left untouched); the
 *                    speculators page logs each term before its weight.
 *   lse_q     [N]    fp32 or NULL: logsumexp of the draft logits.
 *   saved            specloss_saved_bytes(N) bytes or NULL: state for the backward.
 *   counts    [2]    int64, required: n_valid, n_bad (unmasked rows with an
 *                    out-of-range label or target row; treated as masked).
 *   reduced   [1+K]  fp32 or NULL: sum(loss)/n_valid, then sum(L_k)/n_valid
 *                    for each kind (0 when n_valid == 0).
 * The divergences take a second sweep over the vocabulary after the
 * logsumexps, except when kl_div and rkl are the only ones and every row has
 * a target row of its own (no target_row map, or n_target_rows >= n_rows):
 * then one sweep computes both sides of a row together and forms
 * KL = E[log-ratio] - lse + lse from the same tiles.  When the workspace
 * holds the raw fp32 logit rows of both sides for min(N, 1024) rows, the
 * first sweep keeps them and the second reads them; otherwise the second
 * sweep recomputes both tiles.  Either way the results are the same bits
 * (lmhead_loss_chunk with call 0 gives the chunk).
 */
int lmhead_loss_fwd(const specloss_problem* p, void* workspace, size_t ws_bytes, float* loss,
                    float* term_loss, float* lse_q, void* saved, int64_t* counts, float* reduced,
                    hipStream_t stream);

/*
 * lmhead_loss_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight evaluation or
 * serving loops, harnesses that forbid allocation).  The call uses a
 * file-scope device array of SPECLOSS_NOALLOC_SCRATCH_BYTES bytes that the
 * library holds on each device it runs on until the process ends (its
 * address is looked up on the first call on a device); it calls no
 * hipMalloc or hipFree.  Outputs, their ownership and errors as for
 * lmhead_loss_fwd; SPECLOSS_E_WORKSPACE when the forward does not fit the
 * array even at its smallest chunk (roughly N * 90 bytes of per-row state,
 * less when term_loss and saved are given, plus 2 to 12 KiB of per-tile
 * partials per chunk row).  Every call on one device shares that device's
 * array: calls that overlap in time on one device race and must not be
 * made.  Nothing in the array needs clearing between calls (each call
 * writes every value it reads).
 */
#define SPECLOSS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int lmhead_loss_fwd_noalloc(const specloss_problem* p, float* loss, float* term_loss,
                            float* lse_q, void* saved, int64_t* counts, float* reduced,
                            hipStream_t stream);

/*
 * Backward (blog, "Backward pass": per chunk, the logits gradient, the
 * hidden-state gradient of the chunk, and the LM-head gradient accumulated
 * over chunks; the chunk's logits tiles are recomputed here from the saved
 * per-row state).  Gradient of sum_r seed_r * loss_r, with
 *   seed_r = (grad_loss ? grad_loss[r] : 0) + (grad_mean ? grad_mean[0] / n_valid : 0)
 * on valid rows and 0 elsewhere (grad_mean is the gradient of the mean
 * loss; counts and saved come from lmhead_loss_fwd on the same problem).
 * At least one of grad_loss, grad_mean is non-NULL.
 *   dhidden [N, H] in dh_dtype (fp32 or bf16), or NULL to skip.
 *   dW      [V, H] fp32, or NULL to skip.  accumulate_dW != 0 adds to its
 *           contents, else it is overwritten.  Gradients flow to the draft
 *           side only (no gradient for target_hidden or W_t).
 * For the divergences the recomputed logits go through raw fp32 rows of
 * both sides when the workspace holds them for min(N, 1024) rows (as in the
 * single call); otherwise the logit gradient is formed from the recomputed
 * tiles directly.  The two ways agree to fp32 rounding.
 */
int lmhead_loss_bwd(const specloss_problem* p, const float* grad_loss, const float* grad_mean,
                    const int64_t* counts, const void* saved, void* workspace, size_t ws_bytes,
                    void* dhidden, int32_t dh_dtype, float* dW, int accumulate_dW,
                    hipStream_t stream);

/*
 * Forward and backward in one call, for a loss that is the last node of the
 * graph (its upstream gradient is known before the forward runs): all the
 * outputs of lmhead_loss_fwd and of lmhead_loss_bwd for the seed
 *   seed_r = (grad_loss ? grad_loss[r] : 0) + (grad_mean ? grad_mean[0] / n_valid : 0)
 * on valid rows.  This is the per-chunk loop of the blog's "Backward pass"
 * section (logits, loss and gradients of one token chunk, LM-head gradient
 * accumulated over chunks), and the logits are never recomputed: for the
 * label and argmax-p cross-entropies the forward pass leaves exp(z - label
 * logit) of the chunk in the workspace (in the input dtype; its transposed
 * copy for the dW contraction is written by the dh contraction, or by the
 * forward pass when dhidden is NULL or the inputs are fp32);
 * with divergences the first forward pass keeps the raw fp32 logit rows of
 * both sides, from which the second sweep's sums and then the logit gradient
 * are formed.  `saved` may be NULL.  Errors as for the two calls.
 */
int lmhead_loss_fwd_bwd(const specloss_problem* p, void* workspace, size_t ws_bytes, float* loss,
                        float* term_loss, float* lse_q, void* saved, int64_t* counts,
                        float* reduced, const float* grad_loss, const float* grad_mean,
                        void* dhidden, int32_t dh_dtype, float* dW, int accumulate_dW,
                        hipStream_t stream);

/*
 * Alignment before chunking for draft heads (blog, "Correctness: alignment
 * before chunking"): head k predicts `shifts[k]` tokens ahead.  Rows are
 * token-major, row = (b * seq_len + t) * n_heads + k (a chunk of consecutive
 * rows holds every head of a run of tokens), and its target row is
 * b * seq_len + t + shifts[k] when that position is inside the sequence
 * and (if loss_mask != NULL) loss_mask of that position is nonzero; then
 * mask_out = 1, else mask_out = 0 and target_row_out = -1.
 *   shifts         host [n_heads], each >= 0
 *   loss_mask      device [batch * seq_len] or NULL
 *   target_row_out device int32 [n_heads * batch * seq_len]
 *   mask_out       device uint8 [n_heads * batch * seq_len]
 */
int specloss_align_heads(int64_t seq_len, int64_t batch, int32_t n_heads, const int32_t* shifts,
                         const uint8_t* loss_mask, int32_t* target_row_out, uint8_t* mask_out,
                         hipStream_t stream);

/*
 * Vocabulary-parallel variant (blog, "Backward pass": the loss is orthogonal
 * to the surrounding parallelism; the vocabulary split is the tensor-parallel
 * layout of the LM head).  Each of G shards owns rows
 * [vocab_offset, vocab_offset + p->vocab) of W (and of W_t): the problem
 * passed to the shard calls is the full problem with W / W_t pointing at the
 * shard's rows and `vocab` the shard's row count; labels stay global indices.
 * The shards exchange per-row records through `exchange`
 * (specloss_exchange_bytes(N, G) bytes, record g written only by shard g; on
 * several GPUs each would hold a copy filled by an all-gather).  Order:
 *   1. every shard: lmhead_shard_pass1   (its tiles -> record g, part 1)
 *   2. once:        lmhead_shard_merge1  (validity, lse_q, lse_p, argmax p,
 *                                         flatness into `saved`; counts)
 *   3. every shard: lmhead_shard_pass2   (label / argmax logits and the
 *                                         divergence sums of its tiles -> record g, part 2)
 *   4. once:        lmhead_shard_merge2  (per-row losses, means, saved alpha ...)
 *   5. every shard: lmhead_shard_bwd     (its dW rows; its fp32 partial of dh)
 *   6. once:        specloss_sum_partials over the G dh partials
 * Records are merged in shard order with the same fixed-order rules as the
 * tiles of one call, so the results equal lmhead_loss_fwd / _bwd on the whole
 * head up to the rounding of the merges.  Workspace: lmhead_loss_workspace_size
 * of the shard problem.  Errors: SPECLOSS_E_INVAL for an inconsistent shard
 * (offset or count out of range, vocab_offset + vocab > vocab_total), as for
 * the unsharded calls otherwise.
 */
typedef struct {
  int64_t vocab_offset;  /* first vocabulary row of this shard */
  int64_t vocab_total;   /* V of the whole head, < 2^31 */
  int32_t shard;         /* g in [0, n_shards) */
  int32_t n_shards;      /* G >= 1 */
  void* exchange;        /* device, specloss_exchange_bytes(N, G) bytes, 256-byte aligned */
} specloss_shard;

size_t specloss_exchange_bytes(int64_t n_rows, int32_t n_shards);

int lmhead_shard_pass1(const specloss_problem* p, const specloss_shard* sh, void* workspace,
                       size_t ws_bytes, hipStream_t stream);

/* saved: specloss_saved_bytes(N); counts [2] int64 as for lmhead_loss_fwd. */
int lmhead_shard_merge1(const specloss_problem* p, const specloss_shard* sh, void* saved,
                        int64_t* counts, hipStream_t stream);

int lmhead_shard_pass2(const specloss_problem* p, const specloss_shard* sh, const void* saved,
                       void* workspace, size_t ws_bytes, hipStream_t stream);

/* Outputs as for lmhead_loss_fwd (loss required; term_loss, lse_q, reduced optional). */
int lmhead_shard_merge2(const specloss_problem* p, const specloss_shard* sh, void* saved,
                        const int64_t* counts, float* loss, float* term_loss, float* lse_q,
                        float* reduced, hipStream_t stream);

/*
 * Backward of one shard for the seed of lmhead_loss_bwd: dW [vocab, H] fp32
 * of the shard's rows (accumulate_dW as there), and dh_partial [N, H] fp32
 * (overwritten, or NULL) = this shard's term of dhidden.
 */
int lmhead_shard_bwd(const specloss_problem* p, const specloss_shard* sh, const float* grad_loss,
                     const float* grad_mean, const int64_t* counts, const void* saved,
                     void* workspace, size_t ws_bytes, float* dh_partial, float* dW,
                     int accumulate_dW, hipStream_t stream);

/*
 * out[i] = sum over g of parts[g * n + i], g = 0 .. n_parts - 1 in order
 * (the dh reduction of the vocabulary-parallel backward).  parts: device fp32
 * [n_parts][n], 16-byte aligned, n a multiple of 4; out: device, out_dtype
 * fp32 or bf16.  SPECLOSS_E_UNSUPPORTED otherwise.
 */
int specloss_sum_partials(const float* parts, int64_t n, int32_t n_parts, void* out,
                          int32_t out_dtype, hipStream_t stream);

/*
 * Kernel trace for measurement.  specloss_trace_create makes `capacity`
 * pairs of HIP events on the current device (the only HIP objects the
 * library ever creates; NULL on failure).  While a problem's `trace` field
 * points at it, each kernel launch of lmhead_loss_fwd / lmhead_loss_bwd is
 * bracketed by an event pair recorded on the call's stream, together with
 * a kernel id (specloss_kernel_name) and its algorithmic work (flops for
 * the contractions, bytes moved for the row kernels).  Launches beyond the
 * capacity are counted but not recorded.  specloss_trace_read waits for the
 * recorded events and returns up to `max` entries (milliseconds per
 * launch); specloss_trace_reset forgets them.  A trace must not be used by
 * two calls at the same time.
 */
specloss_trace* specloss_trace_create(int32_t capacity);
void specloss_trace_destroy(specloss_trace* t);
void specloss_trace_reset(specloss_trace* t);
int specloss_trace_read(specloss_trace* t, int32_t max, int32_t* kernel_id, float* ms,
                        double* work, int32_t* count);
const char* specloss_kernel_name(int32_t id);

const char* specloss_strerror(int code);
const char* specloss_kind_name(int kind); /* "ce_label","ce","kl_div","rkl","jsd","tv","nla","lk_hybrid" */

#ifdef __cplusplus
}
#endif

#endif /* SPECLOSS_H */
