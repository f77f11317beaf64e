/*
 * fp_prefill.h -- C ABI of the MI355X (gfx950) FlexPrefill sparse pre-filling
 * library, one attention layer's causal prefill on one GPU.
 *
 * Method (FlexPrefill, ICLR 2025 submission 1022): abstract on the OpenReview
 * and codewithpapers pages, "Approach" paragraph and ablation table of the
 * atlas.scime.ai summary page.  Per attention head:
 *   1. query-aware sparse pattern determination -- the last query block's
 *      exact attention over all keys, pooled per key block, is compared with
 *      the softmax of block-pooled queries x block-pooled keys by the square
 *      root of the Jensen-Shannon divergence; below tau the head is
 *      query-aware, otherwise vertical-slash;
 *   2. cumulative-attention index selection -- the smallest set of blocks
 *      (query-aware: the flattened estimated block map) or lines (vertical:
 *      key columns, slash: diagonals of the last block's attention) whose
 *      normalised attention reaches gamma, plus a minimum budget;
 *   3. causal attention restricted to the selected key blocks.
 * Steps 1-2 are fp_prefill_plan, step 3 is fp_prefill_attend.  Selection runs
 * in one fixed ("canonical") arithmetic, so plans are bit-reproducible.
 *
 * Conventions shared by every entry point
 *   Layouts (dense, row-major, device pointers; Q, K, V and O share one dtype):
 *     FP_LAYOUT_BHND  Q [B, Hq, N, d], K and V [B, Hkv, N, d], O like Q --
 *                     B sequences of N tokens (fp_prefill_plan[_ex],
 *                     fp_dense_attend);
 *     FP_LAYOUT_THD   packed sequences of different lengths, Q [T, Hq, d],
 *                     K and V [T, Hkv, d], O like Q; sequence b holds tokens
 *                     cu_seqlens[b] .. cu_seqlens[b+1]-1 (the *_varlen calls).
 *     Query head h reads key/value head h / (Hq / Hkv) (grouped-query
 *     attention).  Sequences are independent.
 *   Sequence lengths: any L >= 0.  A sequence has nb = ceil(L / block) query
 *     and key blocks; when L is not a multiple of the block, the last block
 *     holds the remaining L - (nb - 1) block tokens (its block mean averages
 *     those rows; the representative queries of step 1 are the last
 *     min(block, L) tokens).
 *   Supported shapes: d in {64, 128}; block in {64, 128}; nb <= 4096 per sequence;
 *     Hq a multiple of Hkv.  A problem without tokens or heads is empty:
 *     FP_OK, nothing is launched.
 *   Streams: `stream` is a hipStream_t (NULL = the legacy default stream).
 *     All device work is enqueued on it asynchronously; no call below blocks
 *     the host unless its comment says "synchronizes".
 *   Ownership: the caller owns q, k, v, o and keeps them alive until the
 *     enqueued work completes.  The library owns every plan buffer.
 *   Logging: with FP_LOG=1 in the environment every plan call synchronizes
 *     its stream and prints one line for the plan and one per head (pattern,
 *     square-root divergence, selected blocks and their share of the causal
 *     blocks) on stderr.
 *   Errors: every call returns an fp_status; nothing aborts or throws across
 *     the ABI.  Arguments are validated on the host before any HIP call, so
 *     validation errors need no GPU.  fp_last_error() describes the most
 *     recent failure of the calling thread.  Faults of already-enqueued
 *     kernels surface as FP_ERR_HIP from the next call that synchronizes.
 */
#ifndef FP_PREFILL_H
#define FP_PREFILL_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fp_status {
    FP_OK = 0,
    FP_ERR_INVALID_ARG = -1,   /* null pointer, gamma outside (0,1], tau < 0, ... */
    FP_ERR_UNSUPPORTED = -2,   /* d not 64/128, block not 64/128, unknown dtype */
    FP_ERR_SHAPE = -3,         /* Hq % Hkv != 0, more than 4096 blocks, sizes too large */
    FP_ERR_OOM = -4,           /* device allocation failed */
    FP_ERR_HIP = -5            /* a HIP runtime call failed */
} fp_status;

typedef enum fp_dtype { FP_BF16 = 0, FP_FP32 = 1 } fp_dtype;

/* Head pattern codes (fp_plan_copy_out `pattern`). */
enum { FP_PATTERN_VERTICAL_SLASH = 0, FP_PATTERN_QUERY_AWARE = 1 };

typedef enum fp_layout { FP_LAYOUT_BHND = 0, FP_LAYOUT_THD = 1 } fp_layout;

typedef struct fp_plan fp_plan;   /* opaque; device-resident block lists */

typedef struct fp_plan_info {
    int B, Hq, Hkv, N, d, block, nb;   /* B sequences; N = longest, nb = ceil(N / block) */
    fp_dtype dtype;
    float gamma, tau;
    int min_budget;
    long long total_blocks;            /* selected (query-block, key-block) pairs, all heads */
    long long dense_blocks;            /* causal blocks: sum over sequences of Hq * nb (nb + 1) / 2 */
    int query_aware_heads;             /* heads whose pattern is query-aware */
    int max_budget;                    /* tokens, 0 = uncapped */
    int qa_selection;                  /* fp_qa_selection */
    int layout;                        /* fp_layout */
    int vs_granularity;                /* fp_vs_granularity */
    long long tokens;                  /* B * N (BHND) or T (THD) */
    long long rows;                    /* query-block rows of all heads: sum over sequences of Hq * nb */
} fp_plan_info;

/* How a query-aware head selects its blocks from the estimated block map. */
typedef enum fp_qa_selection {
    FP_QA_FLATTENED = 0,   /* one list over the whole causal triangle (the method's default) */
    FP_QA_QUERYWISE = 1    /* every query-block row selects from its own row */
} fp_qa_selection;

/* How a vertical-slash head's selected key columns are attended. */
typedef enum fp_vs_granularity {
    FP_VS_BLOCK = 0,       /* whole key blocks touched by a selected column (the method's blocked kernel) */
    FP_VS_TOKEN = 1        /* each selected column on its own, gathered into dense key tiles */
} fp_vs_granularity;

/* Optional planning settings; a NULL pointer means all defaults (zeros). */
typedef struct fp_plan_options {
    int max_budget;        /* tokens per query-block row, 0 = uncapped */
    int qa_selection;      /* fp_qa_selection */
    int vs_granularity;    /* fp_vs_granularity */
} fp_plan_options;

/*
 * fp_prefill_plan -- steps 1 and 2 for every (batch, query head).
 *   q, k: device pointers, layout above, dtype `dtype`.
 *   gamma in (0, 1]: cumulative-attention threshold (pages: 0.95 default,
 *     0.9 and 0.85 tested); gamma == 1 selects every causal block.
 *   tau >= 0: divergence threshold; query-aware iff sqrt(JSD) < tau
 *     (pages: 0.1 default, 0 disables query-aware, 0.3 tested).
 *   min_budget >= 0 tokens: every query-block row keeps at least
 *     min(row + 1, max(1, ceil(min_budget / block))) blocks, the missing ones
 *     filled nearest-first from the diagonal (pages: 1024 default, 2048).
 *   On FP_OK *out receives a new plan (released with fp_plan_destroy).  The
 *   plan's buffers are one block of the library's device memory cache (see
 *   "Device memory" below), held until fp_plan_destroy; a transient
 *   workspace of B*Hq*block*ceil(N/256)*256*4 bytes is taken from the cache
 *   and given back within the call.
 */
fp_status fp_prefill_plan(const void* q, const void* k, fp_dtype dtype,
                          int B, int Hq, int Hkv, int N, int d, int block,
                          float gamma, float tau, int min_budget,
                          void* stream, fp_plan** out);

/*
 * fp_prefill_plan_ex -- fp_prefill_plan with optional settings (`options`
 *   may be NULL: identical to fp_prefill_plan).  Both variants come from the
 *   ablation table of the atlas.scime.ai summary page.
 *   options->max_budget > 0 (the table caps the computational budget at 8k
 *   or 32k tokens; uncapped is the method's default): every query-block row
 *   keeps at most ceil(max_budget / block) blocks -- after the
 *   minimum-budget fill, the row's blocks with the largest score stay, where
 *   the score is the estimated block attention for query-aware heads (and
 *   for gamma = 1) and the selected column plus diagonal line mass through
 *   the block for vertical-slash heads; ties keep the block nearer the
 *   diagonal.
 *   options->qa_selection = FP_QA_QUERYWISE (the table's alternative to
 *   selecting over the flattened estimated map): a query-aware head applies the cumulative rule to each estimated row on
 *   its own -- the minimal set of the row's key blocks, value descending
 *   then key block ascending, whose fixed-point mass reaches gamma of the
 *   row's total.  Vertical-slash heads are unaffected.
 *   options->vs_granularity = FP_VS_TOKEN (the Approach paragraph calls a
 *   vertical-slash selection a set of lines): a vertical-slash head attends
 *   each selected key column token by token -- every query j >= column sees
 *   it -- instead of computing every key block a column touches; the blocks
 *   its slash lines touch, the minimum-budget fill and the cap stay whole
 *   blocks (the block lists then hold only those).  fp_prefill_attend
 *   gathers the columns' K and V rows into dense 64-key tiles (a workspace
 *   of 2*B*Hq*nb*block*d elements).  Query-aware heads are unaffected.
 *   FP_ERR_INVALID_ARG if max_budget < 0, if it allows fewer blocks per row
 *   than min_budget asks for, or if qa_selection or vs_granularity is not a
 *   listed value.
 */
fp_status fp_prefill_plan_ex(const void* q, const void* k, fp_dtype dtype,
                             int B, int Hq, int Hkv, int N, int d, int block,
                             float gamma, float tau, int min_budget,
                             const fp_plan_options* options,
                             void* stream, fp_plan** out);

/*
 * fp_prefill_attend -- step 3: O = causal softmax(Q K^T / sqrt(d)) V with
 *   each query block attending only to the key blocks its plan selected.
 *   q must be the tensor the plan was built from (the plan stores lists,
 *   not values); k and v of the plan's shape and layout.  Every token row
 *   of o is written.  Uses a device workspace of V transposed, per
 *   sequence Hkv*d*nb*block elements, taken from the library's memory cache
 *   (see fp_workspace_trim).  `stream` may differ from the plan's
 *   stream: the call then waits for the planning kernels, and the plan's
 *   stream waits for this call's kernels (so fp_plan_destroy, ordered on the
 *   plan's stream, cannot free the lists under them).
 */
fp_status fp_prefill_attend(const fp_plan* plan, const void* q, const void* k,
                            const void* v, void* o, void* stream);

/*
 * fp_prefill_attend_noalloc -- fp_prefill_attend for callers that cannot
 *   allocate device memory (code under HIP graph capture, tight serving
 *   loops, harnesses that forbid allocation).  Same arguments, layouts and
 *   results as fp_prefill_attend; it calls no hipMalloc / hipFree and creates
 *   no events.  Its workspace (V transposed, Hkv*d*nb*block elements per
 *   sequence, plus 2*Hq*d*nb*block elements per sequence of gathered columns
 *   for FP_VS_TOKEN plans, each part rounded up to 256 bytes) lives in one
 *   static device array of 64 MiB per GPU, held until the process ends:
 *   FP_ERR_SHAPE (and nothing enqueued) if the plan needs more.  Every call
 *   on one GPU shares that array and overwrites what the previous call left
 *   there (every byte a call reads it has written first), so calls whose
 *   work overlaps on one GPU -- on different streams, or from different
 *   threads without ordering -- race; serialize them on one stream.  The
 *   measurement hooks do not time this call.
 */
fp_status fp_prefill_attend_noalloc(const fp_plan* plan, const void* q, const void* k,
                                    const void* v, void* o, void* stream);

/*
 * fp_prefill_plan_varlen -- fp_prefill_plan_ex for packed sequences of
 *   different lengths (FP_LAYOUT_THD): q [T, Hq, d], k [T, Hkv, d] with
 *   T = cu_seqlens[nseq].  cu_seqlens is a HOST array of nseq + 1 ints,
 *   cu_seqlens[0] = 0, non-decreasing (a zero-length sequence has no rows;
 *   its heads report pattern 0 and divergence 0).  Every sequence is planned
 *   exactly as fp_prefill_plan_ex would plan it alone, up to four sequences
 *   at once on streams of the library (forked from and joined back to
 *   `stream`); each of those streams takes one transient workspace of
 *   Hq*block*ceil(L/256)*256*4 bytes for the longest sequence L it plans.  The plan records the layout: fp_prefill_attend then takes
 *   packed q, k, v and o.
 *   FP_ERR_INVALID_ARG for a NULL or malformed cu_seqlens; FP_ERR_SHAPE for a
 *   sequence of more than 4096 blocks.
 */
fp_status fp_prefill_plan_varlen(const void* q, const void* k, fp_dtype dtype,
                                 int nseq, const int* cu_seqlens,
                                 int Hq, int Hkv, int d, int block,
                                 float gamma, float tau, int min_budget,
                                 const fp_plan_options* options,
                                 void* stream, fp_plan** out);

/*
 * fp_dense_attend -- full causal attention with the same tile kernel (every
 *   key block 0..row of every row); the baseline the sparse path is measured
 *   against (the pages compare with FlashAttention).  Same layout and
 *   support rules as above.
 */
fp_status fp_dense_attend(const void* q, const void* k, const void* v, void* o,
                          fp_dtype dtype, int B, int Hq, int Hkv, int N, int d,
                          int block, void* stream);

/* fp_dense_attend for packed sequences (FP_LAYOUT_THD, host cu_seqlens). */
fp_status fp_dense_attend_varlen(const void* q, const void* k, const void* v, void* o,
                                 fp_dtype dtype, int nseq, const int* cu_seqlens,
                                 int Hq, int Hkv, int d, int block, void* stream);

/* Plan summary.  Synchronizes the plan's stream. */
fp_status fp_plan_info_get(const fp_plan* plan, fp_plan_info* out);

/*
 * fp_plan_copy_out -- host copies of the plan (synchronizes `stream`).
 *   pattern [B*Hq]          FP_PATTERN_* per head        (may be NULL)
 *   djs     [B*Hq]          sqrt(JSD) per head            (may be NULL)
 *   row_ptr [rows + 1]      CSR row offsets, rows ordered (b, h, row); a
 *                           sequence contributes Hq * its nb rows
 *   col_idx [total_blocks]  key-block indices, ascending within a row
 *   row_ptr and col_idx may both be NULL; if one is given both must be.
 */
fp_status fp_plan_copy_out(const fp_plan* plan, unsigned char* pattern, double* djs,
                           int* row_ptr, int* col_idx, void* stream);

/*
 * fp_plan_copy_debug -- host copy of an intermediate of steps 1-2
 *   (synchronizes the plan's stream).  `bytes` must equal the item's size.
 *   Shapes for B sequences of N tokens; with packed sequences the arrays of
 *   the non-empty sequences follow one another, each with its own N and nb:
 *   FP_DBG_QBAR   float [B*Hq][nb][d]      block means of Q
 *   FP_DBG_KBAR   float [B*Hkv][nb][d]     block means of K
 *   FP_DBG_ROWMAX float [B*Hq][block]      last-block row maxima (scaled scores);
 *                                          rows i < block - min(block, N) do not
 *                                          exist and read 0
 *   FP_DBG_ROWSUM float [B*Hq][block]      last-block row sums of exp2 (same rows)
 *   FP_DBG_COLSUM float [B*Hq][N]          vertical line scores
 *   FP_DBG_DIAGSUM float [B*Hq][N]         slash line scores (offset i - j)
 *   FP_DBG_ATRUE  float [B*Hq][nb]         block-pooled true distribution
 *   FP_DBG_AHAT   float [B*Hq][nb(nb+1)/2] estimated map, causal triangle row-major
 *   FP_DBG_COUNTS int   [B*Hq][nb]         selected blocks per row
 *   FP_DBG_COLPTR int   [B*Hq][nb+1]       token-granular columns before each key
 *                                          block (FP_VS_TOKEN plans; 0 bytes otherwise)
 *   FP_DBG_COLIDX int   [B*Hq][N]          those columns ascending, the first
 *                                          colptr[nb] entries of each head valid
 *                                          (FP_VS_TOKEN plans; 0 bytes otherwise)
 */
enum {
    FP_DBG_QBAR = 0, FP_DBG_KBAR = 1, FP_DBG_ROWMAX = 2, FP_DBG_ROWSUM = 3,
    FP_DBG_COLSUM = 4, FP_DBG_DIAGSUM = 5, FP_DBG_ATRUE = 6, FP_DBG_AHAT = 7,
    FP_DBG_COUNTS = 8, FP_DBG_COLPTR = 9, FP_DBG_COLIDX = 10
};
fp_status fp_plan_copy_debug(const fp_plan* plan, int which, void* host_dst, size_t bytes);

/* Gives the plan's buffers back to the library's device memory cache without
 * waiting: they are reused only behind the plan's stream, which already
 * waits for every attend enqueued with the plan on another stream.  Work
 * using the plan must have been enqueued before this call. */
void fp_plan_destroy(fp_plan* plan);

/*
 * Device memory.  Plans, attends and dense attends take their device memory
 * (a plan's buffers, the score workspace of planning, the attention's V^T
 * workspace) from a cache kept by the library, and give it back when their
 * work is enqueued (a plan's buffers when it is destroyed).  A block given
 * back carries an event recorded on the stream of its last use; a later call
 * on any stream reuses it after making its stream wait on that event, so no
 * call waits on the host for earlier GPU work (an allocation from the
 * runtime's stream-ordered pool that reused memory freed earlier on a stream
 * made the host wait until the stream reached the free).  The cache holds at
 * most 16 GiB; beyond that its oldest blocks are freed once their last use
 * has completed.  Thread-safe.
 *
 * fp_workspace_trim -- frees every cached block (on every device), waiting on
 *   the host for the last use of each, and returns the runtime pool's unused
 *   memory to the device.  Blocks held by calls in flight on other threads
 *   and the buffers of live plans are not touched.  FP_ERR_HIP if a wait
 *   failed (the remaining blocks are still freed).
 */
fp_status fp_workspace_trim(void);

const char* fp_status_str(fp_status s);
const char* fp_last_error(void);

/*
 * Measurement hooks.  While enabled, fp_prefill_attend and fp_dense_attend
 * record HIP events around their attention kernel on the call's stream;
 * fp_profile_read synchronizes those events and returns the summed kernel
 * time in ms and the number of launches since the last reset.
 */
fp_status fp_profile_enable(int on);
fp_status fp_profile_read(double* sparse_ms, long long* sparse_launches,
                          double* dense_ms, long long* dense_launches, int reset);

/*
 * Canonical-arithmetic probes (host only, no GPU): the constants the
 * selection kernels use for head dim d -- exp2 Taylor coefficients e2[8]
 * (fp32 nearest to (ln 2)^k / k!), artanh series coefficients lnc[11]
 * (1 / (2k + 1)), ln 2, sqrt(1/2) and the score scale C = log2(e)/sqrt(d).
 */
fp_status fp_canonical_constants(int d, float* e2, double* lnc, double* ln2,
                                 double* sqrt_half, float* score_scale);

/* Device probes of the canonical exp2, ln and of the binary64 square root the
 * divergence uses, on n elements (device pointers, enqueued on `stream`). */
fp_status fp_probe_exp2(const float* x, float* y, long long n, void* stream);
fp_status fp_probe_ln(const double* x, double* y, long long n, void* stream);
fp_status fp_probe_sqrt(const double* x, double* y, long long n, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FP_PREFILL_H */
