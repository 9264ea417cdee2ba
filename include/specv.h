/*
 * libspecv: the speculative-sampling verify step on AMD Instinct MI355X
 * (gfx950).  C ABI: plain pointers and sizes, no framework types.
 *
 * The operation (one verification round per batch row) is the one defined in
 * "11.1 核心原理: Draft + Verify 与 Rejection Sampling", section 11.1.2 and
 * pseudo-code 10-1, and in "Fast Inference from Transformers via Speculative
 * Decoding" (speculative sampling):
 *
 *   for i = 0 .. gamma-1:   accept d_i with probability min(1, p_i(d_i) / q_i(d_i))
 *                            (uniform u: accept iff u * q_i(d_i) < p_i(d_i))
 *   at the first rejection:  emit t ~ norm(max(p_i - q_i, 0)) and stop
 *   if all were accepted:    emit the bonus t ~ p_gamma
 *   greedy rows:             accept while d_i == argmax p_i, emit the argmax
 *                            at the first mismatch (or as the bonus)
 *
 * p_i / q_i are the target / draft distributions after temperature, top-k and
 * top-p (11.1.2: both processed, q kept as the truncated distribution actually
 * sampled).  Emission stops after the first emitted EOS and after
 * max_new_tokens tokens; a correction or bonus token past the cap is not drawn
 * (remark after pseudo-code 10-1).
 *
 * Layouts (all device memory unless stated):
 *   target logits  [B, gamma+1, V]: row (b, i) starts at
 *                  target + b*t_stride_b + i*t_stride_pos (strides in
 *                  ELEMENTS); vocabulary contiguous.  Row i checks draft d_i;
 *                  row gamma is the bonus distribution (11.1.1 alignment).
 *   draft logits   [B, gamma, V] likewise; row (b, i) is q_i for d_i.
 *   draft tokens   int32 [B, gamma], contiguous.
 *   outputs        int32 num_accepted [B], out_tokens [B, gamma+1] (emitted
 *                  tokens then -1 padding), num_emitted [B], row_flags [B].
 *
 * Random numbers: Philox4x32-10 (Salmon et al., SC'11), key = seed (low word
 * first), counter = (b, i, purpose, step), u = (word0 >> 8) * 2^-24.
 * Purposes: 0 draft sample (specv_sample_draft), 1 accept test, 2 correction
 * sample, 3 bonus sample.  b is the row index within the call and i the
 * position within the round.
 *
 * Ownership: the caller owns every input and output buffer.  A handle owns a
 * device workspace allocated once by specv_create and freed by
 * specv_destroy; verify calls allocate nothing.  One handle serves one stream
 * at a time (calls on a handle must not overlap).  Calls enqueue one kernel
 * and nothing else (no memset, no host synchronisation), and may be captured
 * into a HIP graph and replayed.  The records a launch's workgroups exchange
 * are tagged with a call number: an eager call takes it from the handle (on
 * the host); a call made while its stream is being captured launches a
 * kernel that takes it on the device and advances it there (one closing
 * workgroup per launch), so every replay gets its own.  The two kinds keep
 * separate records in the handle and may be mixed freely.  A replay repeats
 * the captured arguments, seed and step included, and so draws the same
 * uniforms as the captured call on the same inputs.
 *
 * Errors: every argument error is reported synchronously, before anything is
 * enqueued, as a non-zero specv_status.  Calls are otherwise asynchronous on
 * the given stream; outputs are valid once the stream reaches them.  Data
 * faults found on the device never abort: they set row_flags bits and the row
 * takes the documented fallback.
 */
#ifndef SPECV_H
#define SPECV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef SPECV_API
#define SPECV_API __attribute__((visibility("default")))
#endif

typedef struct specv_ctx* specv_handle;

typedef enum {
    SPECV_OK = 0,
    SPECV_E_NULL = 1,      /* a required pointer is NULL                          */
    SPECV_E_SHAPE = 2,     /* B, gamma or V out of range, bad strides             */
    SPECV_E_DTYPE = 3,     /* dtype not one of specv_dtype                        */
    SPECV_E_ALIGN = 4,     /* output or token pointer not 4-byte aligned          */
    SPECV_E_CAPACITY = 5,  /* B, gamma or V above the handle's configured maximum */
    SPECV_E_PARAM = 6,     /* bad handle configuration                            */
    SPECV_E_NOMEM = 7,     /* workspace allocation failed (specv_create)          */
    SPECV_E_HIP = 8        /* a HIP runtime call failed                           */
} specv_status;

typedef enum { SPECV_F32 = 0, SPECV_BF16 = 1 } specv_dtype;

/* Row flag bits (row_flags[b]). */
#define SPECV_FLAG_TOKEN_OOR          (1 << 0) /* a draft token outside [0, V): row emits nothing   */
#define SPECV_FLAG_NONFINITE_ROW      (1 << 1) /* a consulted row has NaN/+inf or no finite value:
                                                  row emits nothing                                 */
#define SPECV_FLAG_Q_ZERO             (1 << 2) /* an accept test met d_i outside q_i's support
                                                  (accepted iff p_i(d_i) > 0)                       */
#define SPECV_FLAG_RESIDUAL_FALLBACK  (1 << 3) /* residual mass 0 / not finite: sampled from p_i    */
#define SPECV_FLAG_CAND_OVERFLOW      (1 << 4) /* reserved; never set: rows whose truncation the
                                                  candidate lists cannot settle (ties beyond the
                                                  lists, top-p alone on flat rows, top_k above
                                                  max_top_k) are truncated exactly over the
                                                  whole row                                         */
#define SPECV_FLAG_TOPP_NEAR          (1 << 5) /* a top-p cumulative mass was within 1e-5 of top_p  */
#define SPECV_FLAG_UNSUPPORTED        (1 << 6) /* a top-k / top-p row on a handle (or entry point)
                                                  without truncation workspace (max_top_k == 0):
                                                  the row emits nothing                             */

#define SPECV_FLAG_INTERNAL           (1 << 7) /* the sampling phase timed out waiting for the row's
                                                  decision (a launch without co-residency): the
                                                  row's outputs are not valid                      */

#define SPECV_MAX_GAMMA 31      /* one 64-bit status word holds a row's accept and stop bits */
#define SPECV_MAX_TOP_K 1024
#define SPECV_MAX_VOCAB 524288

typedef struct {
    int device;      /* HIP device ordinal the handle runs on                     */
    int max_batch;   /* largest B of any call                                     */
    int max_gamma;   /* largest gamma (0 .. SPECV_MAX_GAMMA)                      */
    int max_vocab;   /* largest V (at most SPECV_MAX_VOCAB)                       */
    int max_top_k;   /* candidates kept per 8192-entry chunk of truncated rows
                        (0 .. SPECV_MAX_TOP_K): rows with top_k <= max_top_k (and
                        top-p rows whose kept set the candidates hold) take the
                        candidate path; others, a larger top_k included, are
                        truncated exactly over the whole row (slower); 0 reserves
                        no candidate workspace: truncated rows are then flagged
                        SPECV_FLAG_UNSUPPORTED                                    */
} specv_config;

/* Per-row sampling parameters, device array [B] (16 bytes each). */
typedef struct {
    float temperature;      /* > 0: stochastic verify of z / T; == 0: greedy row        */
    int32_t top_k;          /* 0 < k < V keeps tokens >= the k-th largest logit (ties
                               kept); <= 0 or >= V: off                                  */
    float top_p;            /* < 1: keep the smallest value-ordered set with mass >=
                               top_p (ties kept); >= 1: off                              */
    int32_t max_new_tokens; /* >= 1: at most this many tokens emitted; <= 0: no cap      */
} specv_row_params;

/* Statistics of one processed draft row, written by specv_sample_draft and
 * read by specv_verify_sample_qstats (16 bytes).  With K the row's kept set
 * (every finite token without truncation; the top-k / top-p set otherwise):
 *   max        m = max_{v in K} z_v (the row maximum)
 *   sum        s = sum_{v in K} exp((z_v - m) / T), float32
 *   threshold  K = {v : z_v >= threshold}; -inf without truncation
 *   flags      SPECV_FLAG_* found while drawing (see specv_sample_draft)
 * so that q(v) = [z_v >= threshold] * exp((z_v - m) / T) / s.  max, sum and
 * threshold are NaN for greedy rows and rows without a draw. */
typedef struct {
    float max;
    float sum;
    float threshold;
    int32_t flags;
} specv_draft_stats;

/* Optional diagnostic outputs (device pointers, each may be NULL). */
typedef struct {
    float* p_at_draft;    /* [B, gamma]: p_i(d_i) for every accept test run, NaN otherwise */
    float* q_at_draft;    /* [B, gamma]: q_i(d_i) likewise                                */
    float* residual_sum;  /* [B]: sum_v max(p_n - q_n, 0) at the rejected position, else 0 */
} specv_diag;

/* Create a handle: selects cfg->device and allocates the workspace sized for
 * (max_batch, max_gamma, max_vocab).  *out is set on success only. */
SPECV_API specv_status specv_create(const specv_config* cfg, specv_handle* out);

/* Stochastic verification of B rows (rows whose temperature is 0 are verified
 * greedily).
 *   stream          hipStream_t (NULL = the null stream), as an opaque pointer
 *   target_logits   [B, gamma+1, V] of dtype, row strides t_stride_b / t_stride_pos
 *   draft_logits    [B, gamma, V] of dtype, row strides d_stride_b / d_stride_pos
 *                   (may be NULL when gamma == 0)
 *   draft_tokens    int32 [B, gamma] (may be NULL when gamma == 0)
 *   row_params      specv_row_params [B]
 *   seed, step      Philox key and the counter's step word
 *   eos_id          token that ends emission, or -1 for none
 *   out_*           see the layout above; out_row_flags may be NULL
 *   diag            host struct of optional device pointers, or NULL
 * B == 0 is a no-op.  1 <= V, 0 <= gamma <= SPECV_MAX_GAMMA. */
SPECV_API specv_status specv_verify_sample(specv_handle h, void* stream,
                                 const void* target_logits, int64_t t_stride_b, int64_t t_stride_pos,
                                 const void* draft_logits, int64_t d_stride_b, int64_t d_stride_pos,
                                 specv_dtype dtype, int B, int gamma, int V,
                                 const int32_t* draft_tokens, const specv_row_params* row_params,
                                 uint64_t seed, uint32_t step, int32_t eos_id,
                                 int32_t* out_num_accepted, int32_t* out_tokens,
                                 int32_t* out_num_emitted, int32_t* out_row_flags,
                                 const specv_diag* diag);

/* specv_verify_sample for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  No handle: the records the verify kernels exchange live in
 * one static device array of SPECV_NOALLOC_SCRATCH_BYTES per device (held
 * by each device the library runs on until the process ends), laid out for
 * B <= SPECV_NOALLOC_MAX_BATCH, gamma <= SPECV_NOALLOC_MAX_GAMMA and
 * V <= SPECV_NOALLOC_MAX_VOCAB; larger calls are rejected with
 * SPECV_E_CAPACITY before anything is enqueued.  Nothing is allocated by
 * this call or any other.  The array has no truncation candidates, so rows
 * with top-k / top-p are flagged SPECV_FLAG_UNSUPPORTED and emit nothing.
 *   device          HIP device ordinal the call runs on (the calling
 *                   thread's current device is restored on return); stream
 *                   must belong to it.  SPECV_E_PARAM if out of range.
 * Other arguments, layouts, outputs and errors as specv_verify_sample; the
 * outputs equal specv_verify_sample's on the same inputs.  The first call
 * on a device clears its array with a kernel on ``stream``.  Every call on
 * a device shares that device's array: calls that overlap on one device
 * (on other streams, or from host threads without stream order between
 * them) race, and their outputs are undefined.  Every call takes its call
 * number on the device (the array keeps no host state), so a call may be
 * captured into a HIP graph and replayed; when the captured call is the
 * device's first, the graph also holds the clearing kernel, and every
 * replay clears the array first (correct, only slower). */
#define SPECV_NOALLOC_MAX_BATCH 256
#define SPECV_NOALLOC_MAX_GAMMA 15
#define SPECV_NOALLOC_MAX_VOCAB 262144
#define SPECV_NOALLOC_SCRATCH_BYTES 11567872
SPECV_API specv_status specv_verify_sample_noalloc(int device, void* stream,
                                 const void* target_logits, int64_t t_stride_b, int64_t t_stride_pos,
                                 const void* draft_logits, int64_t d_stride_b, int64_t d_stride_pos,
                                 specv_dtype dtype, int B, int gamma, int V,
                                 const int32_t* draft_tokens, const specv_row_params* row_params,
                                 uint64_t seed, uint32_t step, int32_t eos_id,
                                 int32_t* out_num_accepted, int32_t* out_tokens,
                                 int32_t* out_num_emitted, int32_t* out_row_flags,
                                 const specv_diag* diag);

/* Stochastic verification against deterministic drafts: n-gram or
 * prompt-lookup proposals ("投机解码 Speculative Decoding" tutorial, sections
 * 2.1 and 4.2; the ICML summary's remark that the approximation model may be
 * an n-gram model or a context-repeat heuristic).  Such a draft proposes d_i
 * with probability one, so q_i is the point mass on d_i and the round above
 * reads: accept d_i with probability p_i(d_i); at the first rejection emit
 * t ~ p_i with d_i removed (norm(max(p_i - q_i, 0))); after full acceptance
 * the bonus t ~ p_gamma.  Temperature-0 rows are verified greedily.  No
 * draft logits are read; q_at_draft reports 1 for every test run.
 * Arguments, layouts, ownership and errors as specv_verify_sample without
 * the draft logits. */
SPECV_API specv_status specv_verify_point_mass(specv_handle h, void* stream,
                                 const void* target_logits, int64_t t_stride_b, int64_t t_stride_pos,
                                 specv_dtype dtype, int B, int gamma, int V,
                                 const int32_t* draft_tokens, const specv_row_params* row_params,
                                 uint64_t seed, uint32_t step, int32_t eos_id,
                                 int32_t* out_num_accepted, int32_t* out_tokens,
                                 int32_t* out_num_emitted, int32_t* out_row_flags,
                                 const specv_diag* diag);

/* Draft-side sampler: draws d_i ~ q_i for positions pos0 .. pos0+n_pos-1 of
 * B rows in one pass over the draft logits, and returns each row's
 * statistics for specv_verify_sample_qstats.  q_i is the draft distribution
 * after the row's temperature, top-k and top-p ("11.1 核心原理" 11.1.2: the
 * proposal is the distribution actually sampled; the "投机解码 Speculative
 * Decoding" tutorial, section 3.3, for the temperature); the draw is the
 * inverse CDF at the Philox uniform of purpose 0 with counter
 * (b, pos0 + i, 0, step): ascending token order, the first token whose
 * running mass exceeds u * W.  A drafter that produces one position at a
 * time calls this once per position (n_pos = 1, pos0 = the position).
 *   draft_logits    [B, n_pos, V] of dtype; row (b, i) is position pos0 + i
 *                   and starts at draft + b*d_stride_b + i*d_stride_pos
 *   row_params      specv_row_params [B] (max_new_tokens is not used)
 *   out_tokens      int32 [B, out_stride]: entry (b, pos0 + i) gets d_i, or -1
 *                   for a row without a draw (below)
 *   out_stats       specv_draft_stats [B, out_stride] or NULL: entry
 *                   (b, pos0 + i) gets the row's statistics and flags:
 *                   SPECV_FLAG_NONFINITE_ROW (NaN / +inf or no finite logit),
 *                   SPECV_FLAG_UNSUPPORTED (top-k / top-p on a handle without
 *                   truncation workspace): these rows get token -1;
 *                   SPECV_FLAG_INTERNAL (a bounded wait expired): the entry's
 *                   token and statistics are not valid (without out_stats
 *                   such a draw may leave its token unwritten);
 *                   SPECV_FLAG_TOPP_NEAR (the top-p decision was within 1e-5
 *                   of top_p) is informational
 * Rows with temperature 0 take the draft argmax (lowest index on ties).
 * Other entries of the outputs are left as they are.  0 <= pos0,
 * pos0 + n_pos <= out_stride, n_pos <= max(max_gamma, 1), B <= max_batch,
 * V <= max_vocab (SPECV_E_SHAPE / SPECV_E_CAPACITY); out_stats 16-byte
 * aligned; n_pos == 0 or B == 0 is a no-op.  Calls on a handle, sampler or
 * verify, must not overlap. */
SPECV_API specv_status specv_sample_draft(specv_handle h, void* stream,
                                 const void* draft_logits, int64_t d_stride_b, int64_t d_stride_pos,
                                 specv_dtype dtype, int B, int n_pos, int V, int pos0,
                                 const specv_row_params* row_params, uint64_t seed, uint32_t step,
                                 int32_t* out_tokens, specv_draft_stats* out_stats,
                                 int64_t out_stride);

/* Stochastic verification reusing the drafter's row statistics: the round of
 * specv_verify_sample, with draft_stats [B, s_stride_b] (entry (b, i) for
 * position i, as specv_sample_draft writes them) standing for the draft
 * distributions' normalisers and, for truncated rows, their kept sets.  No
 * draft row is streamed: the accept tests load q's entry at d_i, and the
 * draft row where the round stops is read for the correction draw (its
 * kept-list entries only, for truncated rows).  The statistics must come from
 * the same draft logits and row parameters as this call's; a row whose
 * statistics are marked non-finite (or are NaN, a zero sum, a max of -inf)
 * emits nothing with SPECV_FLAG_NONFINITE_ROW.  Greedy rows ignore them.
 * With statistics from specv_sample_draft the outputs equal
 * specv_verify_sample's bit for bit.  s_stride_b >= gamma; draft_stats
 * 16-byte aligned.  Other arguments, layouts, ownership and errors as
 * specv_verify_sample. */
SPECV_API specv_status specv_verify_sample_qstats(specv_handle h, void* stream,
                                 const void* target_logits, int64_t t_stride_b, int64_t t_stride_pos,
                                 const void* draft_logits, int64_t d_stride_b, int64_t d_stride_pos,
                                 const specv_draft_stats* draft_stats, int64_t s_stride_b,
                                 specv_dtype dtype, int B, int gamma, int V,
                                 const int32_t* draft_tokens, const specv_row_params* row_params,
                                 uint64_t seed, uint32_t step, int32_t eos_id,
                                 int32_t* out_num_accepted, int32_t* out_tokens,
                                 int32_t* out_num_emitted, int32_t* out_row_flags,
                                 const specv_diag* diag);

/* Greedy verification (11.1.2): accept while d_i == argmax of the raw target
 * logits (lowest index on ties), emit the argmax at the first mismatch or as
 * the bonus.  Draft logits are not read.
 *   max_new_tokens  int32 [B] caps (<= 0: no cap), or NULL for none. */
SPECV_API specv_status specv_verify_greedy(specv_handle h, void* stream,
                                 const void* target_logits, int64_t t_stride_b, int64_t t_stride_pos,
                                 specv_dtype dtype, int B, int gamma, int V,
                                 const int32_t* draft_tokens, const int32_t* max_new_tokens,
                                 int32_t eos_id,
                                 int32_t* out_num_accepted, int32_t* out_tokens,
                                 int32_t* out_num_emitted, int32_t* out_row_flags);

/* Kernel timing for measurement.  With enable != 0 every later call (verify
 * or sampler) records HIP events on its stream around its kernel (each call
 * is one kernel launch); the events are created here, not in the verify calls.
 * specv_get_profile waits for the recorded events and returns the number of
 * profiled calls and their summed kernel milliseconds since the last reset,
 * and resets the sums when reset != 0.  Errors: SPECV_E_NULL, SPECV_E_HIP. */
SPECV_API specv_status specv_set_profiling(specv_handle h, int enable);
SPECV_API specv_status specv_get_profile(specv_handle h, int reset, int* calls, double* ms_kernel);

/* The per-call kernel durations behind specv_get_profile: waits for the
 * recorded events, then copies the first min(max_samples, recorded) of the
 * per-call milliseconds since the last reset (at most 65536 are kept) to the
 * host array ms_out and their number to *n_out.  Does not reset.  Errors:
 * SPECV_E_NULL (h or n_out NULL, or ms_out NULL with max_samples > 0),
 * SPECV_E_HIP. */
SPECV_API specv_status specv_get_profile_samples(specv_handle h, int max_samples, float* ms_out,
                                                 int* n_out);

/* Measurement aid, no part of the verify step: one streaming read of the
 * device buffer buf (bytes, a multiple of 16, 16-byte aligned) by ``grid``
 * workgroups of 16-byte loads, the load shape of the verify kernels; each
 * workgroup writes the XOR of what it read to sink[blockIdx] (device,
 * uint32 [grid]) so that the read cannot be elided.  Timing it gives the
 * device's one-pass read rate, the ceiling the verify kernels are compared
 * with.  Asynchronous on ``stream``; allocates nothing.  Errors: SPECV_E_NULL,
 * SPECV_E_SHAPE (bytes < 16 or not a multiple of 16, grid < 1),
 * SPECV_E_ALIGN, SPECV_E_HIP. */
SPECV_API specv_status specv_read_ceiling(void* stream, const void* buf, int64_t bytes, int grid,
                                          uint32_t* sink);

/* For tests of failure handling only: sets how many polls every bounded wait
 * of the verify and draft-sampler kernels makes on ``device`` before it gives
 * up and flags its row SPECV_FLAG_INTERNAL (the outputs of such a row are not
 * valid; every other row's are).  polls = 0 restores the default (262144).
 * Process-wide for the device, for every handle; waits for the device first,
 * so no call is in flight when it changes.  The closing workgroup of a
 * graph-replayable launch keeps the default.  Errors: SPECV_E_PARAM
 * (polls < 0), SPECV_E_HIP. */
SPECV_API specv_status specv_debug_set_wait_limit(int device, int32_t polls);

/* Free the workspace and the handle.  Waits for the device first.  NULL is
 * accepted. */
SPECV_API specv_status specv_destroy(specv_handle h);

/* Static description of a status code. */
SPECV_API const char* specv_status_string(specv_status s);

#ifdef __cplusplus
}
#endif

#endif /* SPECV_H */
