/*
 * sampler.h -- C ABI of the MI355X (gfx950) batched logits sampler.
 *
 * One call post-processes a [batch, vocab] logits matrix, row by row:
 *
 *   1. repetition penalty over the row's history ids: a logit x of a token
 *      that appears in the history becomes x / rho when x > 0, else x * rho;
 *      each distinct id counts once, ids outside [0, vocab) are ignored
 *      (MiniMind generation chapter, sec. 10.7 "repetition penalty"; the C++
 *      post-processing blog, repetition_penalty);
 *   2. temperature: x / T (MiniMind sec. 10.4);  -0 is then written as +0;
 *   3. top-k: when the row's top-k bit is set and 1 <= k <= min(vocab, 1024),
 *      keep exactly the k largest logits, ties broken by the smaller vocab id;
 *      any other k skips the stage (Ascend torch_npu npu_top_k_top_p_sample
 *      page, topK section: valid range and Card(top_k_value) = top_k); with
 *      SAMPLER_TOPK_TIES, every logit equal to the k-th value is kept too
 *      (MiniMind sec. 10.5);
 *   4. softmax over the survivors (same page, topK/topP sections);
 *   5. top-p: when the row's top-p bit is set and p < 1, keep the shortest
 *      prefix of the survivors (in the order of step 3) whose probability
 *      mass reaches p; the first survivor is always kept; p >= 1 or NaN skips
 *      the stage (Ascend page topP section; MiniMind sec. 10.6);
 *   6. exponential sampling: with the sample bit set, the output token is the
 *      kept id i maximising softmax_K(x)_i / (q[row, i] + eps), lowest id on
 *      exact ties -- q is paired with candidates by vocabulary id; without it
 *      the output is the first kept token, i.e. the greedy argmax (Ascend
 *      page, Sample section; MiniMind sec. 10.8);
 *   6'. or, when the caller passes uniforms u instead, a multinomial draw
 *      from softmax_K made by inverse CDF: the kept token at which the
 *      cumulative probability, summed in the order of step 3, first reaches
 *      u[row] (MiniMind sec. 10.8, torch.multinomial over the filtered
 *      softmax);
 *   7. optional dense outputs: the filtered logits (x at kept ids, -inf
 *      elsewhere; the Ascend page's logits_top_kp_select) and the
 *      probabilities renormalised over the kept set (0 elsewhere);
 *   8. optional decode-step epilogue (MiniMind sec. 10.9, EOS batch
 *      handling): a row already marked finished outputs the EOS id instead
 *      of its draw, a row whose output is EOS becomes finished, the output
 *      is appended to the row's history (the sequence the penalty of the
 *      next step reads, sec. 10.7), and the rows still unfinished are
 *      counted so that the caller's loop can stop when none is left.
 *
 * Every step runs in hand-written HIP kernels on the caller's stream; the
 * library never copies data to the host and never synchronises in
 * sampler_run.
 */
#ifndef MI355X_SAMPLER_H
#define MI355X_SAMPLER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ------------------------------------------------------ */
#define SAMPLER_OK 0
#define SAMPLER_EINVAL (-1)   /* null / inconsistent argument               */
#define SAMPLER_ENOMEM (-2)   /* device workspace allocation failed         */
#define SAMPLER_EHIP (-3)     /* HIP runtime or kernel launch error         */

/* ---- logits storage types ---------------------------------------------- */
#define SAMPLER_F32 0
#define SAMPLER_BF16 1

/* ---- per-row stage bits (row_flags[b]) ----------------------------------- */
#define SAMPLER_ROW_TOPK 1u
#define SAMPLER_ROW_TOPP 2u
#define SAMPLER_ROW_SAMPLE 4u
#define SAMPLER_ROW_ALL 7u

/* ---- call flags (sampler_args.flags) ------------------------------------- */
#define SAMPLER_NEED_LOGITS 1u  /* write out_logits                          */
#define SAMPLER_NEED_PROBS 2u   /* write out_probs (debug; re-reads logits)  */
#define SAMPLER_TOPK_TIES 4u    /* top-k also keeps every logit equal to the
                                   k-th largest value (MiniMind sec. 10.5:
                                   only logits below the k-th value of topk
                                   are masked), so more than k may survive  */
#define SAMPLER_APPEND_HISTORY 8u /* step 8: append out_idx[b] to row b's
                                   history (needs penalty_len)              */
#define SAMPLER_PROFILE 256u    /* time each kernel with HIP events; read the
                                   averages with sampler_profile             */
#define SAMPLER_PROFILE_SLOTS 6

/* Largest k of the top-k stage and largest top-k guess. */
#define SAMPLER_TOPK_MAX 1024
/* Largest vocabulary the library accepts. */
#define SAMPLER_VOCAB_MAX (1 << 21)

typedef struct sampler_s sampler_t;

/* Tuning knobs.  None of them changes any result. */
typedef struct sampler_opts {
    /* Size G of the top-k guess used for top-p rows whose top-k stage is off
     * (Ascend page, topP section: the guess succeeds when the G most likely
     * tokens already hold mass >= p; otherwise a full-row cutoff search
     * runs).  0 = default (256); otherwise 1..1024. */
    int32_t topk_guess;
    /* Elements per tile of the streaming pass (one workgroup per tile; the
     * Ascend page's rolling top-k uses segments of 8192).  0 = automatic:
     * each call takes the shortest multiple of 1024 below 8192 for which
     * batch x tiles stays within 4 workgroups per compute unit and a row has
     * at most 64 tiles, else 8192 (small batches spread their rows over more
     * of the device); otherwise a multiple of 1024 in [1024, 32768]. */
    int32_t segment_len;
    /* Most rows per kernel launch: a call with more rows runs each kernel
     * over consecutive chunks of rows (in order, on the same stream).  0 =
     * automatic (as many as the launch limits allow); otherwise >= 1. */
    int32_t rows_per_launch;
} sampler_opts;

/*
 * Arguments of one call.  All array pointers are DEVICE pointers on the
 * handle's device; the caller owns every buffer.  Shapes use B = batch of
 * the call and V = the handle's vocab.
 */
typedef struct sampler_args {
    const void *logits;        /* [B, ld] row-major, SAMPLER_F32 or _BF16 */
    int64_t ld;                /* row stride of logits in elements, >= V   */
    const int32_t *top_k;      /* [B] or NULL (top-k off for every row)    */
    const float *top_p;        /* [B] or NULL (top-p off for every row)    */
    const float *q;            /* [B, V] fp32 sampling weights, row stride V
                                  (the Ascend page's q [batch, voc_size]);
                                  NULL = no exponential race in this call:
                                  rows with the sample bit then output their
                                  first kept token (greedy), unless u is
                                  given.  The per-row bits live in device
                                  memory, which the host does not read, so a
                                  sample bit without q cannot be an error;
                                  only row_flags == NULL (every row samples)
                                  with q and u both NULL is rejected.       */
    float eps;                 /* >= 0, added to q                         */
    float temperature;         /* > 0; 1 = stage off                        */
    float repetition_penalty;  /* > 0; 1 = stage off                        */
    int32_t *penalty_ids;      /* [nnz] history ids, or NULL; row b's slot is
                                  penalty_ids[offsets[b] .. offsets[b+1]).
                                  Written only with SAMPLER_APPEND_HISTORY */
    const int64_t *penalty_offsets; /* [B+1] CSR offsets into penalty_ids */
    const uint8_t *row_flags;  /* [B] SAMPLER_ROW_* bits, NULL = all on     */
    uint32_t flags;            /* SAMPLER_NEED_LOGITS | _NEED_PROBS | _TOPK_TIES |
                                  _APPEND_HISTORY | _PROFILE */
    int64_t *out_idx;          /* [B] sampled (or greedy) vocab id          */
    float *out_logits;         /* [B, V] row stride V; iff NEED_LOGITS      */
    float *out_probs;          /* [B, V] row stride V; iff NEED_PROBS       */
    const float *u;            /* [B] uniforms for inverse-CDF sampling, or
                                  NULL.  When given, rows with the sample bit
                                  draw the kept token whose inclusive
                                  cumulative probability (in the order of
                                  step 3) first reaches u[b] -- u <= 0 or NaN
                                  gives the first kept token, u beyond what
                                  rounding lets the sum reach gives the last
                                  -- and q is not read (it may be NULL).     */
    /* ---- step 8, the decode-step epilogue; every part optional ---------- */
    int32_t *penalty_len;      /* [B] or NULL.  Given: row b's history is the
                                  first n_b = clamp(penalty_len[b], 0, cap_b)
                                  ids of its slot (cap_b = offsets[b+1] -
                                  offsets[b]); NULL: the whole slot.  With
                                  SAMPLER_APPEND_HISTORY the call writes the
                                  output id at position n_b of the slot and
                                  sets penalty_len[b] = n_b + 1; a full slot
                                  (n_b >= cap_b) is left as it is and the row
                                  is counted in counts[1].                  */
    uint8_t *finished;         /* [B] in/out, or NULL (no EOS handling).  A
                                  row with finished[b] != 0 outputs eos_id;
                                  then finished[b] = 1 where the output is
                                  eos_id and finished[b] was 0 (a nonzero
                                  value is kept).  The draw and the dense
                                  outputs of a finished row are still made. */
    int64_t eos_id;            /* the EOS id, in [0, V) when finished is set */
    int32_t *counts;           /* [2] or NULL, written by every call with
                                  batch >= 1: [0] rows with finished[b] == 0
                                  after the call (batch when finished is
                                  NULL; 0 = every row has ended), [1] rows
                                  whose append found a full slot.            */
} sampler_args;

/*
 * Create a handle for batches of at most max_batch rows of vocab V logits of
 * the given storage type on the current HIP device (the Ascend page's
 * parameter list: logits [batch, voc_size] of float32 or bfloat16).  Allocates the device
 * workspace (about 80 KiB per row at 8192-element tiles).  opts
 * may be NULL.
 * Returns SAMPLER_OK and sets *h, SAMPLER_EINVAL for bad arguments
 * (max_batch < 1, V < 1 or > SAMPLER_VOCAB_MAX, unknown dtype, bad opts),
 * SAMPLER_ENOMEM or SAMPLER_EHIP.
 */
int sampler_create(sampler_t **h, int32_t max_batch, int32_t vocab, int32_t dtype,
                   const sampler_opts *opts);

/*
 * Check the arguments of a call without touching the GPU (the Ascend page's
 * parameter list and its value ranges: top_k in [1, min(voc_size, 1024)],
 * top_p, q, eps; MiniMind sec. 10.4 and 10.7: temperature and penalty
 * above 0).  Returns SAMPLER_OK
 * or SAMPLER_EINVAL: batch outside [0, max_batch], logits / out_idx NULL,
 * ld < V, temperature or penalty not finite and > 0, eps negative or not
 * finite, a requested dense output with a NULL buffer, exactly one of the
 * penalty arrays NULL, penalty_len without them, SAMPLER_APPEND_HISTORY
 * without all three, finished with eos_id outside [0, V), unknown flag bits,
 * or row_flags == NULL (every row samples) with both q and u NULL.
 * Per-row values are never errors: k outside [1, min(V, 1024)] skips top-k,
 * p >= 1 or NaN skips top-p, history ids outside [0, V) are ignored.
 */
int sampler_check(const sampler_t *h, int32_t batch, const sampler_args *a);

/*
 * Run one call on `stream` (a hipStream_t; NULL = the null stream): steps 1
 * to 8 above for every row (Ascend npu_top_k_top_p_sample page, calculation
 * formula: topK, topP and Sample sections; MiniMind ch. 10, sec. 10.4 to
 * 10.9).
 * Asynchronous: outputs are valid once the stream has completed.  Runs
 * sampler_check first.  The handle's workspace is reused by every call, so
 * calls with one handle must be ordered on one stream (not thread-safe).
 * Rows whose logits are NaN, or entirely -inf, are outside the contract.
 * A call with batch 0 launches nothing and writes nothing.
 * Returns SAMPLER_OK, SAMPLER_EINVAL or SAMPLER_EHIP (launch failure).
 */
int sampler_run(sampler_t *h, int32_t batch, const sampler_args *a, void *stream);

/*
 * (Measurement, no passage of the pages.)  Kernel times, in milliseconds,
 * averaged over the sampler_run calls made
 * with SAMPLER_PROFILE since the previous sampler_profile call (the last 64
 * of them if there were more), in launch order: [0] per-row planning (the
 * admission estimate of top-k / top-p rows), [1] the streaming pass over the
 * logits (every row), [2] row merge / cutoff / sample, [3] full-row search
 * (rows the pass could not settle, top-p rows whose guess failed, inverse-CDF
 * draws over whole rows), [4] dense outputs of filtered rows, [5] the
 * decode-step epilogue.  Each time runs from an event recorded
 * on the call's stream just before the kernel to one recorded just after
 * it.  Kernels that were not launched count 0.  Waits for the last profiled
 * call to finish, then forgets the calls it averaged.
 * Returns the number of entries written (<= n), or a negative error code
 * (SAMPLER_EINVAL when no profiled call is pending).
 */
int sampler_profile(sampler_t *h, float *ms, int32_t n);

/* Size of the library's static device workspace (per GPU), used by
 * sampler_run_static instead of a handle's allocation. */
#define SAMPLER_STATIC_SCRATCH_BYTES (32 << 20)

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as sampler_run, on batch rows of vocab V logits of the given storage
 * type with the given options (NULL = defaults), without a handle.  Nothing
 * is allocated: the workspace is a static device array of
 * SAMPLER_STATIC_SCRATCH_BYTES bytes per GPU, found once per device by its
 * symbol and held until the process ends.  The workspace of a call grows
 * with batch and with the number of tiles per row (about 78 KiB per row at
 * vocab 262144 and the default tile length: some 420 rows); a call that
 * does not fit returns SAMPLER_EINVAL, as do SAMPLER_PROFILE (no events are
 * made) and every argument sampler_run rejects.  Every call on one GPU
 * shares that GPU's workspace: calls that overlap in time on one GPU (other
 * streams, other threads) race and give wrong results; calls ordered on one
 * stream do not.  Nothing in the workspace has to start at zero (each call
 * writes what it reads).  Returns SAMPLER_OK, SAMPLER_EINVAL or
 * SAMPLER_EHIP.
 */
int sampler_run_static(int32_t batch, int32_t vocab, int32_t dtype, const sampler_opts *opts,
                       const sampler_args *a, void *stream);

/* Free the workspace and the handle (the ownership rule above: the handle owns
 * only its workspace).  NULL is accepted. */
int sampler_destroy(sampler_t *h);

/* Static description of a return code (SAMPLER_OK and the SAMPLER_E* codes
 * above). */
const char *sampler_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* MI355X_SAMPLER_H */
