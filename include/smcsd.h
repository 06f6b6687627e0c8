/*
 * smcsd.h -- C ABI of libsmcsd.so: one round of Sequential Monte Carlo speculative decoding
 * (SMC-SD) on AMD Instinct MI355X (gfx950).
 *
 * The round follows "Faster LLM Inference via Sequential Monte Carlo", section 2
 * (Methodology). A request keeps N particles. The draft model has extended each particle by
 * K tokens, and one batched target pass has scored every position. This library takes those
 * logits. It weights every particle by importance instead of rejecting tokens, then evicts
 * low-weight particles and duplicates high-weight ones back to N. It draws the round's bonus
 * token from the target and shares the KV pages of duplicated particles by exchanging page
 * ids, never by copying KV tensors. Two by-products come from the same pass:
 *   - the per-position total-variation distance that the METASD page (section 2) uses as
 *     its block-divergence signal;
 *   - the bonus token itself, drawn with precomputed Gumbel noise as in the STAND page
 *     (method item 2: Gumbel-Top-K with cached noise, here k = 1).
 *
 * Conventions for every entry point:
 *  - Pointers are device memory owned by the caller (hipMalloc or a torch tensor) unless
 *    stated otherwise. The library allocates nothing, frees nothing and keeps no pointer
 *    after a call returns; all scratch lives in the caller's workspace.
 *  - Work is enqueued asynchronously on `stream` (NULL = the default stream). Results are
 *    valid once that stream has been synchronised. Calls on different streams with disjoint
 *    buffers may run concurrently. Two calls that share a workspace must not overlap.
 *  - Argument errors are found on the host, before any HIP call, and are returned
 *    synchronously; nothing is enqueued then. A failed launch returns SMCSD_ERR_DEVICE.
 *  - Device-side preconditions cannot be checked on the host: finite logits and noise,
 *    T > 0, u in [0,1), tokens in [0,V), page ids < num_pages, a consistent refcount.
 *    Kernels guard every index they use. They OR the bits below into *error_flags (when
 *    non-NULL, zeroed by the caller) instead of reading or writing out of bounds.
 *  - All results are deterministic: no floating-point atomics, fixed reduction orders.
 */
#ifndef SMCSD_H
#define SMCSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipStream_t / hipEvent_t handles, declared without the HIP headers. */
typedef struct ihipStream_t *smcsd_stream;
typedef struct ihipEvent_t *smcsd_event;

typedef enum smcsd_status {
    SMCSD_OK = 0,
    SMCSD_ERR_ARG = 1,         /* null, out-of-range or inconsistent argument */
    SMCSD_ERR_UNSUPPORTED = 2, /* valid request beyond the library's limits (see below) */
    SMCSD_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than smcsd_workspace_size() */
    SMCSD_ERR_DEVICE = 4,      /* a HIP launch or runtime call failed */
    SMCSD_ERR_SCRATCH = 5      /* smcsd_round_noalloc: more than SMCSD_NOALLOC_SCRATCH_BYTES */
} smcsd_status;

typedef enum smcsd_dtype { SMCSD_F32 = 0, SMCSD_BF16 = 1 } smcsd_dtype;

/* When to resample. ESS: iff ESS < ess_frac * N (strict). */
typedef enum smcsd_resample_mode {
    SMCSD_RESAMPLE_ALWAYS = 0,
    SMCSD_RESAMPLE_ESS = 1,
    SMCSD_RESAMPLE_NEVER = 2
} smcsd_resample_mode;

/* Device-side error bits OR-ed into *error_flags. */
#define SMCSD_DEVERR_TOKEN 1u     /* drafted token outside [0,V); its log-ratio counts as 0 */
#define SMCSD_DEVERR_ANCESTOR 2u  /* ancestor outside [0,N) given to remap; its row is skipped */
#define SMCSD_DEVERR_PAGE 4u      /* page id >= num_pages; its refcount update is skipped */
#define SMCSD_DEVERR_REFCOUNT 8u  /* a refcount went below zero (inconsistent input table) */
#define SMCSD_DEVERR_EXCHANGE 16u /* a TV slice exchange exceeded its time limit (results void).
                                     The limit is 4 s; the environment variable
                                     SMCSD_EXCHANGE_TIMEOUT_TICKS (ticks of the 100 MHz
                                     constant clock, read at each call) overrides it, e.g. to
                                     exercise this path */
#define SMCSD_DEVERR_POOL 32u     /* page free list ran dry (or its count was out of range): the
                                     entries it could not fill are left -1 */
#define SMCSD_DEVERR_LENGTH 64u   /* a request's lengths are not 0 <= before <= after <=
                                     P * page_size: its pages are left as they were */

/* Build limits. */
#define SMCSD_MAX_N 1024 /* particles per request */
#define SMCSD_MAX_K 256  /* drafted tokens per particle */
/* With TV on (tv != NULL), the S slices of a row pair exchange their partials within one
   wave, so S <= 64 and V is at most 64 slices x 512 lanes x 4 chunks x 8 (bf16) or x 4
   (fp32) elements. Larger V with TV returns SMCSD_ERR_UNSUPPORTED; without TV any V works. */
#define SMCSD_MAX_TV_V_BF16 1048576
#define SMCSD_MAX_TV_V_F32 524288

/*
 * Arguments of smcsd_round. Sizes first, then device pointers.
 * Row layout: every logits row and noise row is `ld` elements long, contiguous in v, and
 * only the first V elements are read. `ld` must be >= V and a multiple of 8 (bf16) or
 * 4 (f32), and the base pointers must be 16-byte aligned, so every row starts on a 16-byte
 * boundary. (Vocabularies that are not a multiple of 8 pad their rows; padding is ignored.)
 */
typedef struct smcsd_round_args {
    int32_t R;          /* requests in the batch (0 = nothing to do) */
    int32_t N;          /* particles per request, 1..SMCSD_MAX_N */
    int32_t K;          /* drafted tokens per particle, 1..SMCSD_MAX_K */
    int32_t V;          /* vocabulary size, >= 1 */
    int64_t ld;         /* row stride in elements of logits and noise rows */
    int32_t dtype;      /* smcsd_dtype of target_logits and draft_logits */
    int32_t mode;       /* smcsd_resample_mode */
    float ess_frac;     /* threshold for SMCSD_RESAMPLE_ESS, in (0, 1] */
    int32_t P;          /* page-table columns per particle (ignored if page_table_in NULL) */
    int32_t num_pages;  /* length of refcount */
    int32_t reserved0;  /* must be 0 */

    /* inputs */
    const void *target_logits;   /* [R][N][K+1][ld]: rows 0..K-1 score x_0..x_{K-1}, row K is
                                    the bonus position */
    const void *draft_logits;    /* [R][N][K][ld]: row k is the distribution x_k came from */
    const int32_t *draft_tokens; /* [R][N][K] drafted tokens x_k */
    const float *temperature;    /* [R] T_r > 0, divides target and draft logits */
    const float *gumbel;         /* [R][N][ld] f32 standard Gumbel noise for the bonus;
                                    NULL = no bonus in the round (bonus may be NULL, column K
                                    of out_tokens gets -1): for callers that draw it after
                                    resampling with smcsd_bonus_resampled */
    const float *uniform;        /* [R] u_r in [0,1) for systematic resampling */

    /* in/out */
    float *log_weights;          /* [R][N] normalised log-weights (LSE over N = 0);
                                    first round: -log N. Replaced by the new weights. */

    /* outputs */
    float *log_w_incr;           /* [R][N] sum_k log p(x_k) - log q(x_k), original particles */
    float *log_norm;             /* [R] logZ = LSE_i(log_weights_in + log_w_incr) */
    float *ess;                  /* [R] 1 / sum_i W_i^2 */
    int32_t *resampled;          /* [R] 1 if the request was resampled this round */
    int32_t *ancestors;          /* [R][N] source particle of each new slot (identity if not
                                    resampled) */
    int32_t *bonus;              /* [R][N] bonus token of each ORIGINAL particle */
    int32_t *out_tokens;         /* [R][N][K+1] tokens of each NEW slot: its ancestor's K
                                    drafted tokens and bonus; may be NULL */
    float *tv;                   /* [R][N][K] TV(p_k, q_k) per original particle; NULL = off */
    const int32_t *page_table_in;/* [R][N][P] page ids, negative = unused; NULL = no remap */
    int32_t *page_table_out;     /* [R][N][P] rows gathered through ancestors; must not alias
                                    page_table_in (swap the two buffers between rounds) */
    int32_t *refcount;           /* [num_pages] references from table entries; updated */
    int32_t *error_flags;        /* optional device int32, SMCSD_DEVERR_* bits OR-ed in */

    void *workspace;             /* device scratch, >= smcsd_workspace_size() bytes,
                                    256-byte aligned; contents need no initialisation */
    size_t workspace_bytes;

    smcsd_event timing_begin;    /* optional: recorded on `stream` right before and after */
    smcsd_event timing_end;      /* the logits pass (both of its kernels with TV on and the
                                    bonus drawn in the pass), for roofline timing */

    const float *log_potential;  /* optional [R][N]: log phi_i, added to particle i's
                                    incremental log weight (the tilted target p*phi of
                                    constrained or reward-weighted decoding, SMC-SD page,
                                    section 5). -inf removes a particle; at least one particle
                                    per request must stay finite. NULL = phi = 1. */
    smcsd_event timing_split;    /* optional: with TV on and the bonus drawn in the pass,
                                    recorded between the bonus-row kernel, which runs first,
                                    and the row-pair kernel (timing_split..timing_end then
                                    brackets the row pairs alone); otherwise recorded with
                                    timing_end */
} smcsd_round_args;

/*
 * One SMC-SD round for R independent requests ("Faster LLM Inference via Sequential Monte
 * Carlo", section 2: weight -> resample -> keep K+1 tokens -> share pages).
 * Per request r, particle i, position k < K, with a = target/T_r and b = draft/T_r:
 *   A_ik = LSE_v a[k,v],  B_ik = LSE_v b[k,v]                 (log-softmax normalisers)
 *   log_w_incr_i = sum_k (a[k,x_k] - A_ik) - (b[k,x_k] - B_ik) (importance weight p/q)
 *                  + log_potential_i                         (if given)
 *   tv_ik = 1/2 sum_v |exp(a[k,v]-A_ik) - exp(b[k,v]-B_ik)|    (METASD block divergence)
 *   bonus_i = argmax_v (target[K,v]/T_r + gumbel[v]), lowest v on equal keys
 *   l_i = log_weights_i + log_w_incr_i, logZ = LSE_i l_i, W_i = exp(l_i - logZ),
 *   ESS = 1/sum W_i^2; resample per `mode`.
 *   Resampled: C = inclusive prefix sum of W (double), U_j = (j+u_r)/N,
 *              ancestors_j = min{i : U_j < C_i} clamped to N-1; log_weights_i = -log N.
 *   Otherwise: ancestors_j = j; log_weights_i = l_i - logZ.
 *   page_table_out[j] = page_table_in[ancestors_j]; for each valid entry page of old row i
 *   with o_i = #{j : ancestors_j = i} != 1: refcount[page] += o_i - 1 (integer atomics).
 * Precision: logits widened exactly to f32, f32 accumulation over v, per-request weight
 * arithmetic and the prefix sum in f64. The bonus key is evaluated in binary32 as
 * fl32(fma(z, fl32(1/T), G)), at most 2^-24 (|z/T| + |key|) from the exact z/T + G; where
 * the exact top-2 keys of a row lie closer than twice that (< 1e-5 for |key| <= 64), the
 * token may be the runner-up.
 */
smcsd_status smcsd_round(const smcsd_round_args *args, smcsd_stream stream);

/*
 * smcsd_round for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments, definitions and
 * results (bit for bit) as smcsd_round, except that args->workspace must be NULL and
 * args->workspace_bytes 0: the workspace is a static device buffer inside the library,
 * SMCSD_NOALLOC_SCRATCH_BYTES on every GPU the library runs on, held until the process ends.
 * A request whose smcsd_workspace_size() exceeds that returns SMCSD_ERR_SCRATCH (validated
 * on the host, before anything is enqueued). The first call on a device looks up that
 * device's copy of the buffer (with the device current); no call allocates or frees memory.
 * Every call on one GPU uses the same buffer, and it keeps the last call's contents: nothing
 * in it needs to start at zero, because each round re-initialises what it reads (the TV
 * exchange slots by a fill kernel on the stream). Calls that overlap in time on one GPU
 * (different streams or host threads) race on the buffer; the caller must order them.
 */
#define SMCSD_NOALLOC_SCRATCH_BYTES (16u << 20)

smcsd_status smcsd_round_noalloc(const smcsd_round_args *args, smcsd_stream stream);

/*
 * Normalise, ESS, resample decision and systematic resampling alone, from given per-particle
 * log-weight increments (same definitions as in smcsd_round; "Faster LLM Inference via
 * Sequential Monte Carlo", section 2: evict and duplicate back to N).
 * log_w_incr [R][N] in; log_weights [R][N] in/out; uniform [R] in; log_norm, ess [R] out;
 * resampled [R] out; ancestors [R][N] out. No workspace is needed.
 */
smcsd_status smcsd_resample(int32_t R, int32_t N, const float *log_w_incr, float *log_weights,
                            const float *uniform, int32_t mode, float ess_frac,
                            float *log_norm, float *ess, int32_t *resampled,
                            int32_t *ancestors, smcsd_stream stream);

/*
 * Page-table remap by pointer exchange alone ("Faster LLM Inference via Sequential Monte
 * Carlo", section 2, KV-cache management: duplicated particles get a copy of the page
 * metadata and share the pages; KV tensors are untouched).
 * ancestors [R][N] in; page_table_in [R][N][P] in; page_table_out [R][N][P] out (must not
 * alias the input); refcount [num_pages] in/out; error_flags optional.
 * Definitions as in smcsd_round. Out-of-range ancestors skip their row, out-of-range page
 * ids skip their update, and both set a bit in *error_flags.
 */
smcsd_status smcsd_remap_pages(int32_t R, int32_t N, int32_t P, const int32_t *ancestors,
                               const int32_t *page_table_in, int32_t *page_table_out,
                               int32_t *refcount, int32_t num_pages, int32_t *error_flags,
                               smcsd_stream stream);

/*
 * Page lifecycle between rounds, the steps on either side of the remap ("Faster LLM
 * Inference via Sequential Monte Carlo", section 2, KV-cache management: duplicated
 * particles share KV pages through page metadata; the page leaves the pool itself open).
 * Readings, applied in this order:
 *  1. release: every page with refcount 0 goes on the free list, in increasing page id, and
 *     gets refcount -1 (the mark of a free page). free_ids[0 .. *n_free) is a stack: pushes
 *     go to free_ids[*n_free], pops take free_ids[*n_free - 1].
 *  2. copy-on-write: when len_before[r] is not a multiple of page_size, column
 *     c = (len_before[r] - 1) / page_size is partly filled and is written next. In that
 *     column the lowest particle naming a page keeps it; every later particle naming the same
 *     page pops a fresh page q, the KV bytes of the page are copied to q in every KV tensor,
 *     refcount[q] = 1 and the shared page's refcount drops by one.
 *  3. append: columns ceil(len_before/page_size) .. ceil(len_after/page_size) - 1 of every
 *     particle get fresh pages with refcount 1, particle by particle, column by column.
 *  Pops go request by request; within a request the copies (particle order) come before the
 *  appends. The result equals that sequential order exactly.
 * Arguments (device memory unless stated):
 *  len_before, len_after [R] int32: tokens held before and after the round, with
 *    0 <= len_before <= len_after <= P * page_size (else SMCSD_DEVERR_LENGTH and the request
 *    is left untouched);
 *  page_table [R][N][P] int32, in/out: page ids, -1 = unused; the entries appended to must
 *    be -1 on entry;
 *  refcount, free_ids [num_pages] int32, in/out; n_free [1] int32, in/out;
 *  kv: NULL (tables only) or kv_count KV tensors, tensor t's page p at byte
 *    kv + t * kv_stride + p * page_bytes; kv, page_bytes and kv_stride multiples of 16,
 *    kv_stride >= num_pages * page_bytes when kv_count > 1, page_bytes <= INT32_MAX;
 *  token_rows: 0 copies whole pages; nonzero declares token-major pages (page_size rows of
 *    page_bytes / page_size bytes, a multiple of 16, in token order, the layout of a token
 *    pool) and copies only the len_before mod page_size rows the tail holds; the other rows
 *    of the new page keep their bytes until the next round writes them;
 *  workspace of smcsd_pages_workspace_size(R, N, P, num_pages) bytes, 256-byte aligned;
 *  stats: NULL or [5] int32 out: pages released, pops served, pages copied, pops that found
 *    the free list empty, token rows the copies cover in each KV tensor (page_size per copy
 *    unless token_rows); error_flags optional.
 * A page must not be named by two requests' tables. If the free list runs dry, the
 * entries it cannot fill stay -1 and SMCSD_DEVERR_POOL is set.
 */
smcsd_status smcsd_pages_advance(int32_t R, int32_t N, int32_t P, int32_t page_size,
                                 const int32_t *len_before, const int32_t *len_after,
                                 int32_t *page_table, int32_t num_pages, int32_t *refcount,
                                 int32_t *free_ids, int32_t *n_free, void *kv,
                                 int64_t page_bytes, int32_t kv_count, int64_t kv_stride,
                                 int32_t token_rows, void *workspace, size_t workspace_bytes,
                                 int32_t *stats,
                                 int32_t *error_flags, smcsd_stream stream);

/* Workspace bytes smcsd_pages_advance needs (0 if the sizes are invalid). */
size_t smcsd_pages_workspace_size(int32_t R, int32_t N, int32_t P, int32_t num_pages);

/* Workspace bytes smcsd_round needs for these sizes (0 if the sizes are invalid). */
size_t smcsd_workspace_size(int32_t R, int32_t N, int32_t K, int32_t V, int32_t dtype,
                            int32_t tv_enabled);

/* Static, human-readable name of a status code ("unknown status" for any other value). */
const char *smcsd_status_string(int32_t status);

/* sizeof(smcsd_round_args) as compiled into the library (for bindings to check layout). */
size_t smcsd_round_args_size(void);

/*
 * Standard speculative-decoding verification of drafted blocks, on the same logits layout as
 * smcsd_round. It is the baseline the SMC-SD page compares against ("Faster LLM Inference via
 * Sequential Monte Carlo", section 1: the target verifies the draft, and the first rejection
 * discards the rest of the block), run here on every particle as an independent sequence.
 * Per request r, particle i (p_k, q_k the temperature-scaled softmaxes of row k):
 *   x_k is accepted iff accept_uniform[k] < min(1, p_k(x_k) / q_k(x_k)), for k = 0, 1, ...
 *   until the first rejection k*;
 *   n_accepted_i = k* (or K if all are accepted);
 *   next_token_i = the residual draw at k*: the first v (increasing) whose inclusive prefix
 *   sum of max(p_k* - q_k*, 0) exceeds residual_uniform * sum_v max(p_k* - q_k*, 0);
 *   or, if all K are accepted, the bonus argmax_v (target[K,v]/T + gumbel[v]) (keys in
 *   binary32 as in smcsd_round).
 * The residual mass is the position's TV, so the pass is the TV pass of smcsd_round plus a
 * short kernel that scans one slice of the rejected row per particle.
 * Decisions are taken on f32 logits with f64 per-particle arithmetic; a residual draw whose
 * uniform lies within 1e-5 of the residual mass from a cumulative-sum boundary may pick the
 * neighbouring token. Sizes, layouts, alignment and limits as for smcsd_round with TV on.
 */
typedef struct smcsd_verify_args {
    int32_t R, N, K, V;          /* as smcsd_round_args */
    int64_t ld;
    int32_t dtype;
    int32_t reserved0;           /* must be 0 */

    const void *target_logits;   /* [R][N][K+1][ld] */
    const void *draft_logits;    /* [R][N][K][ld] */
    const int32_t *draft_tokens; /* [R][N][K] */
    const float *temperature;    /* [R] */
    const float *gumbel;         /* [R][N][ld] bonus noise (used when a block is accepted) */
    const float *accept_uniform; /* [R][N][K] in [0,1) */
    const float *residual_uniform; /* [R][N] in [0,1) */

    int32_t *n_accepted;         /* [R][N] out: accepted drafted tokens, 0..K */
    int32_t *next_token;         /* [R][N] out: the token after the accepted ones */
    float *tv;                   /* [R][N][K] out, optional (NULL): TV(p_k, q_k) */
    int32_t *error_flags;        /* optional device int32, SMCSD_DEVERR_* bits OR-ed in */

    void *workspace;             /* >= smcsd_verify_workspace_size() bytes, 256-byte aligned */
    size_t workspace_bytes;

    smcsd_event timing_begin;    /* optional, around the logits pass as in smcsd_round */
    smcsd_event timing_end;
} smcsd_verify_args;

smcsd_status smcsd_sd_verify(const smcsd_verify_args *args, smcsd_stream stream);

/* Workspace bytes smcsd_sd_verify needs for these sizes (0 if the sizes are invalid). */
size_t smcsd_verify_workspace_size(int32_t R, int32_t N, int32_t K, int32_t V, int32_t dtype);

/* sizeof(smcsd_verify_args) as compiled into the library. */
size_t smcsd_verify_args_size(void);

/*
 * Gumbel-Top-K: k distinct tokens per row drawn without replacement from softmax(z/T) in one
 * step, as the STAND page describes for drafting (method item 2: add precomputed, cached
 * Gumbel noise to the log-probabilities and keep the indices of the k largest sums).
 *   key_v = logits[row][v] / temperature[row] + gumbel[row][v], evaluated in binary32 as
 *           fl32(fma(logits[row][v], fl32(1/temperature[row]), gumbel[row][v]))
 *   out_tokens[row][0..k-1] = the k largest keys' indices, by decreasing key, equal keys by
 *   increasing index; out_keys (optional, NULL) the keys themselves.
 * rows >= 0, 1 <= k <= min(V, SMCSD_MAX_TOPK), V <= SMCSD_MAX_TV_V_* for the dtype; ld and
 * alignment as for smcsd_round (logits and gumbel 16-byte aligned, ld a multiple of 8 for
 * bf16, 4 for f32). The slice and merge passes rank the same binary32 keys, so the result is
 * the exact ranking of those keys; each is at most 2^-24 (|z/T| + |key|) from the real key,
 * which bounds how far the order can differ from exact arithmetic in a near tie.
 */
#define SMCSD_MAX_TOPK 64

smcsd_status smcsd_gumbel_topk(int32_t rows, int32_t V, int64_t ld, int32_t dtype,
                               const void *logits, const float *temperature,
                               const float *gumbel, int32_t k, int32_t *out_tokens,
                               float *out_keys, void *workspace, size_t workspace_bytes,
                               smcsd_stream stream);

/* Workspace bytes smcsd_gumbel_topk needs (0 if the sizes are invalid). */
size_t smcsd_topk_workspace_size(int32_t rows, int32_t V, int32_t dtype, int32_t k);

/*
 * Bonus token drawn after resampling, one per NEW slot: the alternative to the in-pass bonus
 * of smcsd_round. The SMC-SD page ("Faster LLM Inference via Sequential Monte Carlo",
 * section 2) yields K + 1 tokens per particle and round without fixing when the last one is
 * drawn. Here slot j of request r takes the Gumbel-max (STAND page, method item 2, k = 1)
 * of its ancestor's bonus row with its own noise row:
 *   bonus[r][j] = argmax_v (target[r][a][K][v] / T_r + gumbel[r][j][v]),
 *   a = ancestors[r][j], lowest v on equal keys.
 * Run smcsd_round with gumbel = NULL first (it then skips its own bonus), then this call
 * with the round's ancestors and a fresh noise tensor.
 * target_logits [R][N][K+1][ld], temperature [R], ancestors [R][N] in; gumbel [R][N][ld]
 * f32 in; bonus [R][N] out; out_tokens NULL or [R][N][K+1] whose column K receives the
 * bonus. Sizes, dtype, ld and alignment as for smcsd_round. Workspace:
 * smcsd_bonus_workspace_size bytes, 256-byte aligned. An ancestor outside [0, N) gives -1 and
 * sets SMCSD_DEVERR_ANCESTOR. Keys in binary32 as for the in-pass bonus.
 */
smcsd_status smcsd_bonus_resampled(int32_t R, int32_t N, int32_t K, int32_t V, int64_t ld,
                                   int32_t dtype, const void *target_logits,
                                   const float *temperature, const int32_t *ancestors,
                                   const float *gumbel, int32_t *bonus, int32_t *out_tokens,
                                   void *workspace, size_t workspace_bytes,
                                   int32_t *error_flags, smcsd_stream stream);

/* Workspace bytes smcsd_bonus_resampled needs (0 if the sizes are invalid). */
size_t smcsd_bonus_workspace_size(int32_t R, int32_t N, int32_t V, int32_t dtype);

#ifdef __cplusplus
}
#endif

#endif /* SMCSD_H */
