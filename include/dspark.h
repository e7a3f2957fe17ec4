/*
 * dspark.h - C ABI of the confidence-scheduled ragged verify hot path on
 * AMD Instinct MI355X (gfx950).
 *
 * One speculative-decoding step of a batch of B requests, each with a drafted
 * block of gamma tokens, runs as:
 *   1. confidence head with per-position temperature  (dspark_confidence)
 *   2. survival curve, the running product of scores   (dspark_confidence)
 *   3. verify-length cut, per request or batch budget   (dspark_schedule; the
 *      per-request cutoffs may come from a cost table:  dspark_cost_cutoff)
 *   4. ragged compaction into a packed verify batch     (dspark_compact,
 *      and dspark_gather_rows for per-position activations)
 *   5. greedy acceptance against the target's argmax    (dspark_accept)
 *   6. bonus token                                      (dspark_accept)
 * or all six in one call (dspark_step). The verify modes of [P1, "The
 * confidence scheduler and verify modes"]: compact (the cut window, the
 * production path), static (DSPARK_CUT_STATIC, the full block) and cap-accept
 * (dspark_cap_accept over a static verify: commits the window, records the
 * full-verify acceptance for the utilisation audit).
 *
 * Sources (web pages): [P1] "DFlash to DSpark in SGLang: 4.3x faster decode,
 * and DeepSeek-V4 support" (yichizhang.dev tutorial); [P2] SGLang's DSpark
 * announcement (24vids.com repost). Each entry point names the section of the
 * page that defines its operation.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every array pointer is a DEVICE pointer to memory the caller allocated and
 *   owns. The library never allocates, frees or synchronises, keeps no state
 *   between calls (apart from cached per-device compute-unit counts and kernel
 *   occupancy figures, filled on first use and safe to share between threads)
 *   and does not retain any pointer after returning.
 * - Every call enqueues its kernels on `stream` (a hipStream_t passed as
 *   void*; NULL means the default stream) and returns without waiting. Results
 *   are ready when the stream reaches that point.
 * - Layouts are row-major with the last index contiguous. bf16 values are
 *   passed as their raw 16-bit patterns (dspark_bf16).
 * - The verify block of request b is tokens[b, 0..gamma]: column 0 is the last
 *   committed (root) token, columns 1..gamma are the drafts. Target-logit row j
 *   of request b (dense row b*(gamma+1)+j) scores the token that follows the
 *   root and j drafts, so it is compared with tokens[b, j+1]; row gamma only
 *   ever yields a bonus token.
 * - Packed outputs have capacity B*(gamma+1), the worst case, because the
 *   packed total is a device value. Entries at and after cu_seqlens[B] are
 *   left untouched.
 * - Host-side checks return a status synchronously and enqueue nothing:
 *     DSPARK_ERR_NULL   a required pointer is NULL;
 *     DSPARK_ERR_SHAPE  B < 1, gamma < 1, gamma > DSPARK_MAX_GAMMA, d < 1,
 *                       V < 1, or B*(gamma+1) above DSPARK_MAX_ROWS;
 *     DSPARK_ERR_ARG    a bad mode, a negative budget, a non-finite bias;
 *     DSPARK_ERR_ALIGN  a pointer misaligned for its element type
 *                       (2 bytes bf16, 4 bytes fp32/int32, 16 bytes ws);
 *     DSPARK_ERR_WORKSPACE  ws_bytes below dspark_workspace_bytes();
 *     DSPARK_ERR_HIP    a kernel launch failed (hipGetLastError).
 * - Device data is never validated on the host (that would need a sync).
 *   The kernels bound every index they use: lengths outside [0, gamma] are
 *   clamped, a cu_seqlens total above the capacity is clamped, and a
 *   packed_src_row entry outside the dense block gives packed_argmax = -1 for
 *   that row. Non-finite logits or hidden values give unspecified (but
 *   in-bounds) results; temperatures must be positive.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t dspark_bf16;

typedef enum dspark_status {
    DSPARK_OK = 0,
    DSPARK_ERR_NULL = 1,
    DSPARK_ERR_SHAPE = 2,
    DSPARK_ERR_ARG = 3,
    DSPARK_ERR_ALIGN = 4,
    DSPARK_ERR_WORKSPACE = 5,
    DSPARK_ERR_HIP = 6
} dspark_status;

typedef enum dspark_cut_mode {
    DSPARK_CUT_THRESHOLD = 0, /* per-request marginal cost cutoff[b] */
    DSPARK_CUT_BUDGET = 1,    /* batch-wide budget of `budget` drafted positions */
    DSPARK_CUT_STATIC = 2,    /* the full block: L_b = gamma (no-trim baseline) */
    DSPARK_CUT_COMBINED = 3   /* cutoff[b] and the budget together */
} dspark_cut_mode;

#define DSPARK_MAX_GAMMA 256
#define DSPARK_MAX_ROWS (1 << 24)

/*
 * Steps 1-2 [P1, "DSpark: a sequential head and a verify budget"]: the
 * score of each drafted position is a dot product of its drafter hidden
 * state with one weight vector plus a bias, divided by that position's
 * Sequential Temperature Scaling temperature and passed through the logistic
 * function; the block's survival curve multiplies those scores up to each
 * position.
 *   conf[b,i]     = 1 / (1 + exp(-(sum_k w[k]*hidden[b,i,k] + bias) / temps[i]))
 *   survival[b,i] = conf[b,0] * ... * conf[b,i]   (S_{i+1}; S_0 = 1 implicit)
 * hidden [B, gamma, d] bf16; w [d] bf16; bias host fp32; temps [gamma] fp32 (> 0).
 * conf, survival [B, gamma] fp32 outputs. Products of bf16 pairs are exact in
 * fp32; the dot product accumulates in fp32; survival is a sequential fp32
 * product, so it is non-increasing whenever every score is at most 1.
 */
dspark_status dspark_confidence(const dspark_bf16 *hidden, const dspark_bf16 *w, float bias,
                                const float *temps, int B, int gamma, int d,
                                float *conf, float *survival, void *stream);

/*
 * Step 3 [P1, "The confidence scheduler and verify modes" and "Zero-overhead
 * scheduling and kernels"; P2]: choose each request's verify length L_b in
 * [0, gamma] from its survival curve.
 *   DSPARK_CUT_THRESHOLD: L_b = #{k in 1..gamma : survival[b,k-1] >= cutoff[b]},
 *     the stopping point of a walk down a non-increasing curve that keeps a
 *     draft while its survival covers the request's marginal cost. A NaN
 *     cutoff gives 0. `budget` is ignored; cutoff is [B] fp32.
 *   DSPARK_CUT_BUDGET: rank all B*gamma (request, position) pairs by survival
 *     descending, ties by lower request then lower position, and keep the
 *     first min(budget, B*gamma); L_b counts request b's kept pairs. `cutoff`
 *     is ignored and may be NULL; budget >= 0.
 *   DSPARK_CUT_STATIC [P1, "The confidence scheduler and verify modes"]: the
 *     static verify mode, L_b = gamma for every request; survival is not read,
 *     `cutoff` and `budget` are ignored.
 *   DSPARK_CUT_COMBINED: a position is eligible when survival[b,k-1] >=
 *     cutoff[b]; the batch keeps the first min(budget, #eligible) eligible
 *     positions in the budget's ranking (survival descending, then lower
 *     request, then lower position). Eligibility is a prefix of each request,
 *     so L_b never exceeds its threshold length. cutoff [B] and budget >= 0.
 * survival [B, gamma] fp32 (finite); lengths [B] int32 output.
 */
dspark_status dspark_schedule(const float *survival, int B, int gamma, int mode,
                              const float *cutoff, long long budget, int32_t *lengths,
                              void *stream);

/*
 * Step 4 [P1, "Ragged verify under full CUDA graphs"; "Zero-overhead
 * scheduling and kernels" for the fused packing]: front-pack the scheduled
 * verify rows with no padding and mark segment starts.
 *   cu_seqlens[0] = 0, cu_seqlens[b+1] = cu_seqlens[b] + L_b + 1
 *   packed_tokens[cu_seqlens[b] + j]  = tokens[b, j]         (j = 0..L_b)
 *   packed_src_row[cu_seqlens[b] + j] = b*(gamma+1) + j
 *   packed_logits[cu_seqlens[b] + j, :] = logits[b, j, :]    (optional)
 * lengths [B] int32 (clamped to [0, gamma]); tokens [B, gamma+1] int32;
 * cu_seqlens [B+1]; packed_tokens, packed_src_row [B*(gamma+1)] int32.
 * logits [B, gamma+1, V] bf16 and packed_logits [B*(gamma+1), V] bf16 are
 * either both NULL (no row gather; V is then ignored) or both non-NULL.
 */
dspark_status dspark_compact(const int32_t *lengths, const int32_t *tokens, int B, int gamma,
                             int32_t *cu_seqlens, int32_t *packed_tokens,
                             int32_t *packed_src_row, const dspark_bf16 *logits, int V,
                             dspark_bf16 *packed_logits, void *stream);

/*
 * Graph tier [P1, "Ragged verify under full CUDA graphs"]: graphs are captured
 * for a ladder of packed sizes (tiers); a step runs the smallest tier that holds
 * its packed total, with the packed batch padded up to it.
 *   tiers [ntiers] int32 (device): the captured tier sizes, strictly
 *     ascending (not checked on the host; 1 <= ntiers <= 4096);
 *   tier_index[0]   = smallest t with tiers[t] >= cu_seqlens[B], or ntiers when
 *                     no tier holds the batch;
 *   padded_total[0] = tiers[tier_index], or cu_seqlens[B] when there is none.
 * Rows [cu_seqlens[B], min(padded_total, B*(gamma+1))) become padding:
 * packed_tokens = pad_token, packed_src_row = -1 (either array may be NULL).
 * Padding rows lie past cu_seqlens[B], so dspark_gather_rows and dspark_accept
 * never read them; a consumer that runs all padded_total rows sees source row
 * -1 there. Every launch shape of this library is independent of the packed
 * total, so this call, like every other entry point, can be captured in a HIP
 * graph together with the schedule and compaction and replayed for any total.
 */
dspark_status dspark_tier_select(const int32_t *cu_seqlens, int B, int gamma,
                                 const int32_t *tiers, int ntiers, int32_t pad_token,
                                 int32_t *padded_total, int32_t *tier_index,
                                 int32_t *packed_tokens, int32_t *packed_src_row, void *stream);

/*
 * Packed row gather [P1, "Ragged verify under full CUDA graphs"]: the
 * scheduled verify rows sit back to back, with no padding, in a single
 * buffer of total-tokens rows, which suits the target's row-wise matmuls. Gathers rows of
 * any width through the packed source rows of dspark_compact:
 *   dst[r, :] = src[packed_src_row[r], :]   for r < cu_seqlens[B]
 * src: B*(gamma+1) rows of row_bytes bytes (e.g. per-position activations
 * [B, gamma+1, hidden]); dst: capacity B*(gamma+1) rows of row_bytes. Rows at
 * and past cu_seqlens[B], and rows whose source index lies outside
 * [0, B*(gamma+1)), are left untouched. 16-byte accesses are used when
 * row_bytes and both pointers allow it, 4-byte or 1-byte otherwise.
 * DSPARK_ERR_SHAPE when row_bytes < 1 or B*(gamma+1)*row_bytes exceeds 2^48.
 */
dspark_status dspark_gather_rows(const void *src, const int32_t *packed_src_row,
                                 const int32_t *cu_seqlens, int B, int gamma, long long row_bytes,
                                 void *dst, void *stream);

/*
 * Cost-table cutoff [P1, "The confidence scheduler and verify modes"]: the
 * server stores the marginal cost of one more verify token per load level as
 * a cost table, and higher load tightens every window together.
 *   cutoff[b] = table[min(max(load[0], 0), n - 1)]   for b in [0, B)
 * table [n] fp32 (device): marginal costs in expected tokens, the unit the
 * survival values are compared in; load [1] int32 (device): the step's load
 * level, e.g. a bucket of the running batch, so the lookup stays on the
 * device with the rest of the step. cutoff [B] fp32 output, ready for
 * DSPARK_CUT_THRESHOLD or DSPARK_CUT_COMBINED.
 */
dspark_status dspark_cost_cutoff(const float *table, int n, const int32_t *load, int B,
                                 float *cutoff, void *stream);

/*
 * Steps 5-6 [P1, "Background"]: greedy verification commits the longest
 * prefix of drafts that agree with the target's own choices, plus one bonus
 * token from the first row that was not accepted.
 *   packed_argmax[r] = lowest index of the largest logit of packed row r
 *                      (-0 and +0 compare equal)
 *   accepted[b] = largest m <= L_b with packed_argmax[cu[b]+j] == tokens[b,j+1]
 *                 for all j < m, where L_b = cu[b+1] - cu[b] - 1
 *   bonus[b]    = packed_argmax[cu[b] + accepted[b]]
 * Packed row r reads dense row packed_src_row[r] of logits [B*(gamma+1), V];
 * when packed_src_row is NULL, logits is already packed (at least cu[B] rows
 * of V; the packed_logits output of dspark_compact has B*(gamma+1)) and row r
 * is read directly. Only packed rows are read. cu_seqlens [B+1] and
 * tokens [B, gamma+1] int32 inputs; packed_argmax [B*(gamma+1)], accepted
 * and bonus [B] int32 outputs. ws: scratch of at least
 * dspark_workspace_bytes(B, gamma, V) bytes, 16-byte aligned, zero-filled
 * before its first use (dspark_workspace_init): up to 4096 requests the call
 * counts each request's streamed rows on a per-request counter at bytes
 * [256 + 32 KiB, 256 + 64 KiB) of ws, which it returns to zero on completion.
 * Calls that share a workspace must not overlap in time.
 */
dspark_status dspark_accept(const dspark_bf16 *logits, const int32_t *packed_src_row,
                            const int32_t *cu_seqlens, const int32_t *tokens, int B, int gamma,
                            int V, int32_t *packed_argmax, int32_t *accepted, int32_t *bonus,
                            void *ws, size_t ws_bytes, void *stream);

/*
 * Steps 5b-6 in the cap-accept verify mode [P1, "The confidence scheduler and
 * verify modes"]: the audit arm pays the full (static) verify but commits only
 * the scheduled window, so its committed output equals the compact mode's
 * exactly while it logs the acceptance of the whole block beside it.
 *   packed_argmax_full [B*(gamma+1)] int32: the target's choice at every row
 *     of the full block, static packing (request b's row j at b*(gamma+1)+j),
 *     e.g. the packed_argmax of dspark_step in DSPARK_CUT_STATIC mode;
 *   tokens [B, gamma+1] int32; lengths [B] int32: the window L_b of the cut
 *     (clamped to [0, gamma]).
 *   accepted_full[b] = largest m <= gamma with
 *                      packed_argmax_full[b*(gamma+1)+j] == tokens[b,j+1], j < m
 *   accepted[b]      = min(accepted_full[b], L_b)
 *   bonus[b]         = packed_argmax_full[b*(gamma+1) + accepted[b]]
 *   sums (nullable) [2] int64: sum of accepted, sum of accepted_full; their
 *     ratio is the utilisation of the window against the full verify.
 * All outputs are device int32 [B] (sums int64 [2]).
 */
dspark_status dspark_cap_accept(const int32_t *packed_argmax_full, const int32_t *tokens,
                                const int32_t *lengths, int B, int gamma, int32_t *accepted,
                                int32_t *bonus, int32_t *accepted_full, long long *sums,
                                void *stream);

/*
 * Steps 1-6 fused, the production "compact" verify mode of [P1, "The
 * confidence scheduler and verify modes"]: the result equals dspark_confidence
 * -> dspark_schedule -> dspark_compact -> dspark_accept on the same inputs,
 * with the dense logits [B, gamma+1, V] read only at packed rows. With
 * DSPARK_CUT_STATIC it is the static mode (every row verified; its
 * packed_argmax and accepted feed dspark_cap_accept for the audit arm).
 * conf and survival may be NULL when the caller does not want them. ws must be
 * zero-filled before its first use with this entry point (dspark_workspace_init
 * does it on a stream): its first 256 bytes hold control words, followed by
 * 32 KiB of per-request counters of this entry point and 32 KiB of those of
 * dspark_accept, at the same offsets for every size, so one workspace serves
 * calls of any sizes it is large enough for. The rest is scratch. Calls that
 * share a workspace must not overlap in time. Batches above 4096 requests run
 * the same step through the stage kernels.
 *
 * Threshold and static cuts from 96 requests up run in one launch whose
 * workgroups wait once, for the verify lengths that its first workgroups
 * compute; the grid is sized to be resident on the device at once (otherwise,
 * and for smaller batches and budget or combined cuts, the step takes two
 * launches). The wait is bounded (about one second): a workgroup that gives up
 * leaves without streaming its share, and the 32-bit word at byte 192 of ws
 * becomes 1 and stays 1 until dspark_step_status reads it. The outputs of the
 * call that gave up are undefined; later calls on the same workspace are not
 * affected (every call starts its counters afresh), so no re-initialisation is
 * needed. A give-up does not happen while the device runs nothing else that
 * holds its compute units for that long. In either form, the wave that
 * finishes a request may re-read a key slot whose store, issued before the
 * count that made that wave the finisher, has not landed yet; that re-read has
 * the same bound and, should it give up, sets the same flag.
 */
dspark_status dspark_step(const dspark_bf16 *hidden, const dspark_bf16 *w, float bias,
                          const float *temps, const int32_t *tokens, const dspark_bf16 *logits,
                          int B, int gamma, int d, int V, int mode, const float *cutoff,
                          long long budget, float *conf, float *survival, int32_t *lengths,
                          int32_t *cu_seqlens, int32_t *packed_tokens, int32_t *packed_src_row,
                          int32_t *packed_argmax, int32_t *accepted, int32_t *bonus,
                          void *ws, size_t ws_bytes, void *stream);

/*
 * dspark_step with explicit controls, for measurement and testing. Results are
 * identical to dspark_step's for every value of the controls (bit for bit, and
 * whichever form runs); nothing is allocated.
 *   ev_start, ev_stop: hipEvent_t handles (as void*, created by the caller with
 *     timing enabled; either may be NULL), recorded on `stream` right before
 *     and right after the launch of the step's dominant kernel (in one launch,
 *     the whole step; in two, the stream over the draft rows, which also
 *     writes the acceptance), so the time between them is that kernel's.
 *   launches: 0 lets the library choose the form by size (as dspark_step
 *     does), 1 asks for the one-launch form where the cut allows it (threshold
 *     and static cuts, grid resident at once), 2 for two launches;
 *     DSPARK_ERR_ARG for any other value.
 *   wait_ticks: bound of the one-launch form's wait for the lengths (and of a
 *     finishing wave's re-read of a key slot), in ticks of the device's 100 MHz
 *     constant clock; 0 means the default (about one second). A bound too
 *     short for the lengths makes workgroups give up, as described under
 *     dspark_step; tests use it to drive that path.
 */
dspark_status dspark_step_ex(const dspark_bf16 *hidden, const dspark_bf16 *w, float bias,
                             const float *temps, const int32_t *tokens, const dspark_bf16 *logits,
                             int B, int gamma, int d, int V, int mode, const float *cutoff,
                             long long budget, float *conf, float *survival, int32_t *lengths,
                             int32_t *cu_seqlens, int32_t *packed_tokens,
                             int32_t *packed_src_row, int32_t *packed_argmax, int32_t *accepted,
                             int32_t *bonus, void *ws, size_t ws_bytes, void *stream,
                             void *ev_start, void *ev_stop, int launches,
                             unsigned long long wait_ticks);

/*
 * The fused step's give-up flag: enqueues on `stream` a read of the 32-bit word
 * at byte 192 of ws into status[0] (device int32: 0 when no workgroup of any
 * dspark_step / dspark_step_ex call since the last read gave up a bounded
 * wait, 1 otherwise) and clears the word, without synchronising. ws: the
 * workspace those calls used (16-byte aligned).
 */
dspark_status dspark_step_status(void *ws, int32_t *status, void *stream);

/*
 * dspark_step for callers that cannot allocate device memory at all: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc, where even a caller-owned workspace is unavailable. The
 * arguments and results are dspark_step's, without ws and ws_bytes: the
 * library's own scratch array in device memory (4 MiB per device, held until
 * the process ends) serves as the workspace. The first call on a device looks
 * the array up and zero-fills it on `stream`; later calls find its counters
 * back at zero. Nothing is allocated or freed by any call.
 *   status (nullable) [1] int32 device output: the call's give-up flag, read and
 *     cleared as dspark_step_status does (0 when every bounded wait ended).
 * DSPARK_ERR_WORKSPACE when dspark_workspace_bytes(B, gamma, V) exceeds the
 * 4 MiB array (about 240k verify rows B*(gamma+1)); the other checks are
 * dspark_step's. Every call on one device shares that device's array: calls
 * that overlap in time on one device (another stream, another thread) race and
 * give undefined results, so keep them ordered on one stream.
 */
dspark_status dspark_step_noalloc(const dspark_bf16 *hidden, const dspark_bf16 *w, float bias,
                                  const float *temps, const int32_t *tokens,
                                  const dspark_bf16 *logits, int B, int gamma, int d, int V,
                                  int mode, const float *cutoff, long long budget, float *conf,
                                  float *survival, int32_t *lengths, int32_t *cu_seqlens,
                                  int32_t *packed_tokens, int32_t *packed_src_row,
                                  int32_t *packed_argmax, int32_t *accepted, int32_t *bonus,
                                  int32_t *status, void *stream);

/* Scratch bytes needed by dspark_accept and dspark_step for these sizes
 * (independent of d); 0 for invalid sizes. */
size_t dspark_workspace_bytes(int B, int gamma, int V);

/* Zero-fill a workspace on `stream` with a kernel (no memset node, so it can
 * be captured in a graph). */
dspark_status dspark_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *dspark_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
