/*
 * dspark_oracle.c - plain fp64 CPU oracle of one confidence-scheduled ragged
 * verify step (confidence head, survival curve, verify-length cut, ragged
 * compaction, greedy acceptance, bonus token).
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load or call this file. The product path never does, and
 * this file shares no code, header, table or helper with it.
 *
 * Sources (web pages):
 *   [P1] "DFlash to DSpark in SGLang: 4.3x faster decode, and DeepSeek-V4
 *        support" (yichizhang.dev AI-Infra-Visualized tutorial).
 *   [P2] SGLang's DSpark announcement as reposted on 24vids.com.
 * Every function below names the section of [P1] whose definition it writes
 * out. The pages print no worked numbers, so each function is pinned by closed
 * forms, brute force, library cross-checks and invariants in the test suite.
 *
 * Arithmetic: every bf16 and fp32 input is widened exactly to double and all
 * arithmetic is done in double, in the plain order stated in each function.
 * The cut, the one decision that turns floating point into integers, compares
 * and ranks these double survival values as they are; the pages fix no other
 * precision for it. Readings of points the pages leave open are stated where
 * they are used.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum {
    ORACLE_OK = 0,
    ORACLE_ERR_SHAPE = 1,    /* a size is out of range */
    ORACLE_ERR_ARG = 2,      /* a scalar argument is invalid */
    ORACLE_ERR_NONFINITE = 3,/* an input value is NaN or infinite */
    ORACLE_ERR_RANGE = 4     /* an integer input or result is out of range */
};

/* A bf16 value is the upper 16 bits of an IEEE binary32 value; widening to
 * double is exact. */
static double bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Step 1, confidence head with STS [P1, "DSpark: a sequential head and a
 * verify budget"]: the head projects each drafted position's drafter hidden
 * state with a linear map and applies a sigmoid; Sequential Temperature
 * Scaling calibrates the score per position. Reading: the temperature T_i of
 * block position i divides the whole head logit, so
 *     z[b,i] = sum_{k=0}^{d-1} w[k] * hidden[b,i,k] + bias   (ascending k)
 *     conf[b,i] = 1 / (1 + exp(-z[b,i] / T_i)).
 * hidden is [B, gamma, d] row-major bf16 bits; w is [d]; temps is [gamma].
 * logit_out (nullable) receives z; conf_out receives the scores, [B, gamma].
 */
int oracle_confidence(const uint16_t *hidden, const uint16_t *w, float bias,
                      const float *temps, int B, int gamma, int d,
                      double *logit_out, double *conf_out)
{
    if (B < 1 || gamma < 1 || d < 1)
        return ORACLE_ERR_SHAPE;
    if (!isfinite(bias))
        return ORACLE_ERR_ARG;
    for (int i = 0; i < gamma; ++i)
        if (!isfinite(temps[i]) || !(temps[i] > 0.0f))
            return ORACLE_ERR_ARG;
    for (int b = 0; b < B; ++b) {
        for (int i = 0; i < gamma; ++i) {
            const uint16_t *h = hidden + ((size_t)b * gamma + i) * (size_t)d;
            double dot = 0.0;
            for (int k = 0; k < d; ++k) {
                double x = bf16_to_double(h[k]);
                double wk = bf16_to_double(w[k]);
                if (!isfinite(x) || !isfinite(wk))
                    return ORACLE_ERR_NONFINITE;
                dot += wk * x;
            }
            double z = dot + (double)bias;
            double p = 1.0 / (1.0 + exp(-z / (double)temps[i]));
            if (logit_out)
                logit_out[(size_t)b * gamma + i] = z;
            conf_out[(size_t)b * gamma + i] = p;
        }
    }
    return ORACLE_OK;
}

/*
 * Step 2, survival curve [P1, "DSpark: a sequential head and a verify
 * budget"]: the block's survival probability is the running product of the
 * per-position scores. S_0 = 1 is implicit; for k = 1..gamma,
 *     S_k = S_{k-1} * conf[b, k-1],
 * stored at surv[b*gamma + k-1]. S_k is the probability that the first k
 * drafts all survive verification.
 */
int oracle_survival(const double *conf, int B, int gamma, double *surv)
{
    if (B < 1 || gamma < 1)
        return ORACLE_ERR_SHAPE;
    for (int b = 0; b < B; ++b) {
        double s = 1.0;
        for (int k = 1; k <= gamma; ++k) {
            double p = conf[(size_t)b * gamma + (k - 1)];
            if (!isfinite(p))
                return ORACLE_ERR_NONFINITE;
            s = s * p;
            surv[(size_t)b * gamma + (k - 1)] = s;
        }
    }
    return ORACLE_OK;
}

/*
 * Step 3, per-request cut [P1, "DSpark: a sequential head and a verify
 * budget" and "The confidence scheduler and verify modes"]: the window
 * extends one position at a time along the survival curve for as long as the
 * tokens the next position is expected to add pay for its per-token cost c_b. Verifying draft k gains S_k expected
 * tokens, so draft k is kept while S_k >= c_b (reading: ">=" keeps a tie).
 * The verify length is the number of kept drafts,
 *     L_b = #{k in 1..gamma : S_k >= c_b},
 * which equals the walk's stopping point because S is non-increasing. A NaN
 * cutoff keeps nothing (every comparison is false). The cutoff is widened
 * exactly to double and compared with the double S_k.
 */
int oracle_cut_threshold(const double *surv, const float *cutoff, int B, int gamma,
                         int32_t *lengths)
{
    if (B < 1 || gamma < 1)
        return ORACLE_ERR_SHAPE;
    for (int b = 0; b < B; ++b) {
        double c = (double)cutoff[b];
        int32_t n = 0;
        for (int k = 1; k <= gamma; ++k) {
            double s = surv[(size_t)b * gamma + (k - 1)];
            if (!isfinite(s))
                return ORACLE_ERR_NONFINITE;
            if (s >= c)
                n += 1;
        }
        lengths[b] = n;
    }
    return ORACLE_OK;
}

/* One drafted position in the batch-wide ranking. */
typedef struct {
    double s;      /* survival S_k of the position */
    int64_t flat;  /* b * gamma + (k - 1): request-major, then position */
} oracle_rank_item;

/* Strict total order: larger survival first; on equal survival the lower
 * request, then the lower position (the lower flat index) first. */
static int oracle_rank_cmp(const void *pa, const void *pb)
{
    const oracle_rank_item *a = (const oracle_rank_item *)pa;
    const oracle_rank_item *b = (const oracle_rank_item *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    if (a->flat < b->flat) return -1;
    if (a->flat > b->flat) return 1;
    return 0;
}

/*
 * Step 3, batch-wide budget [P1, "Zero-overhead scheduling and kernels"
 * (the verify-length top-k schedule) and [P2] (dynamic budget against a fixed
 * one)]: the batch verifies at most T drafted positions, namely the T
 * positions with the largest survival values across all requests. Readings:
 * T counts drafted positions (root rows are always verified and are not
 * counted); T larger than B*gamma takes every position; equal survival values
 * are ranked by lower request, then lower position. L_b is the number of
 * request b's positions among the T picked. The double survival values are
 * ranked as they are: only exactly equal values tie.
 */
int oracle_cut_budget(const double *surv, int B, int gamma, long long budget,
                      int32_t *lengths)
{
    if (B < 1 || gamma < 1)
        return ORACLE_ERR_SHAPE;
    if (budget < 0)
        return ORACLE_ERR_ARG;
    int64_t n = (int64_t)B * gamma;
    int64_t t_eff = budget < n ? (int64_t)budget : n;
    oracle_rank_item *items = (oracle_rank_item *)malloc((size_t)n * sizeof *items);
    if (!items)
        return ORACLE_ERR_SHAPE;
    for (int64_t f = 0; f < n; ++f) {
        if (!isfinite(surv[f])) {
            free(items);
            return ORACLE_ERR_NONFINITE;
        }
        items[f].s = surv[f];
        items[f].flat = f;
    }
    qsort(items, (size_t)n, sizeof *items, oracle_rank_cmp);
    for (int b = 0; b < B; ++b)
        lengths[b] = 0;
    for (int64_t r = 0; r < t_eff; ++r)
        lengths[items[r].flat / gamma] += 1;
    free(items);
    return ORACLE_OK;
}

/*
 * Step 3, threshold and budget together [P1, "The confidence scheduler and
 * verify modes" (per-request marginal cost) with "Zero-overhead scheduling and
 * kernels" (batch-wide top-k budget)]. Reading: a drafted position is eligible
 * when it passes its request's cutoff, S_k >= c_b (in double, as in
 * oracle_cut_threshold), and the batch then verifies the T eligible positions
 * with the largest survival (ties by lower request, then lower position), or
 * every eligible position when there are at most T. Eligibility is a prefix of
 * each request and survival does not increase along it, so L_b is again the
 * count of request b's picks.
 */
int oracle_cut_combined(const double *surv, const float *cutoff, int B, int gamma,
                        long long budget, int32_t *lengths)
{
    if (B < 1 || gamma < 1)
        return ORACLE_ERR_SHAPE;
    if (budget < 0)
        return ORACLE_ERR_ARG;
    int64_t n = (int64_t)B * gamma;
    oracle_rank_item *items = (oracle_rank_item *)malloc((size_t)(n > 0 ? n : 1) * sizeof *items);
    if (!items)
        return ORACLE_ERR_SHAPE;
    int64_t m = 0;
    for (int64_t f = 0; f < n; ++f) {
        if (!isfinite(surv[f])) {
            free(items);
            return ORACLE_ERR_NONFINITE;
        }
        double s = surv[f];
        if (s >= (double)cutoff[f / gamma]) {
            items[m].s = s;
            items[m].flat = f;
            m += 1;
        }
    }
    qsort(items, (size_t)m, sizeof *items, oracle_rank_cmp);
    int64_t take = budget < m ? (int64_t)budget : m;
    for (int b = 0; b < B; ++b)
        lengths[b] = 0;
    for (int64_t r = 0; r < take; ++r)
        lengths[items[r].flat / gamma] += 1;
    free(items);
    return ORACLE_OK;
}

/*
 * Cost-table cutoff [P1, "The confidence scheduler and verify modes"]: the
 * server times the step cost of one more verify token at each load level
 * and keeps those figures as a cost table; under a heavier load each token
 * costs more, so all windows shrink at once. Reading: table[j] is the marginal
 * cost at load level j already expressed in expected tokens (the unit of the
 * survival values), and every request of the step gets the entry of the
 * step's load level, clamped to the table:
 *     cutoff[b] = table[min(max(load, 0), n - 1)].
 */
int oracle_cost_cutoff(const float *table, int n, int32_t load, int B, float *cutoff)
{
    if (n < 1 || B < 1)
        return ORACLE_ERR_SHAPE;
    int j = load < 0 ? 0 : (load > n - 1 ? n - 1 : load);
    for (int b = 0; b < B; ++b)
        cutoff[b] = table[j];
    return ORACLE_OK;
}

/*
 * Step 4, ragged compaction [P1, "Ragged verify under full CUDA graphs"]: the
 * scheduled verify rows of all requests are front-packed with no padding, and
 * cu_seqlens gives the first packed row of each request (and the total last). Request b
 * verifies L_b + 1 rows: its root row j = 0 plus drafts 1..L_b. With the dense
 * verify block laid out as [B, gamma+1] (column 0 = root token),
 *     cu[0] = 0,  cu[b+1] = cu[b] + L_b + 1,
 *     packed_tokens[cu[b] + j]  = tokens[b, j]          for j = 0..L_b,
 *     packed_src_row[cu[b] + j] = b * (gamma + 1) + j.
 * total_out receives cu[B]. Lengths outside [0, gamma] are rejected.
 */
int oracle_compact(const int32_t *lengths, const int32_t *tokens, int B, int gamma,
                   int32_t *cu_seqlens, int32_t *packed_tokens, int32_t *packed_src_row,
                   int64_t *total_out)
{
    if (B < 1 || gamma < 1)
        return ORACLE_ERR_SHAPE;
    int64_t cu = 0;
    cu_seqlens[0] = 0;
    for (int b = 0; b < B; ++b) {
        int32_t L = lengths[b];
        if (L < 0 || L > gamma)
            return ORACLE_ERR_RANGE;
        for (int32_t j = 0; j <= L; ++j) {
            packed_tokens[cu + j] = tokens[(size_t)b * (gamma + 1) + j];
            packed_src_row[cu + j] = (int32_t)((int64_t)b * (gamma + 1) + j);
        }
        cu += (int64_t)L + 1;
        if (cu > INT32_MAX)
            return ORACLE_ERR_RANGE;
        cu_seqlens[b + 1] = (int32_t)cu;
    }
    if (total_out)
        *total_out = cu;
    return ORACLE_OK;
}

/*
 * Packed row gather [P1, "Ragged verify under full CUDA graphs"]: the
 * per-row data of the scheduled verify tokens sits back to back, with no
 * padding, in a buffer of total-tokens rows. Row r < cu[B] of dst is a byte copy of row
 * packed_src_row[r] of src (rows of row_bytes bytes); later rows are left as
 * they are. A source row outside [0, B*(gamma+1)) is rejected.
 */
int oracle_gather_rows(const uint8_t *src, const int32_t *packed_src_row,
                       const int32_t *cu_seqlens, int B, int gamma, int64_t row_bytes,
                       uint8_t *dst)
{
    if (B < 1 || gamma < 1 || row_bytes < 1)
        return ORACLE_ERR_SHAPE;
    int64_t cap = (int64_t)B * (gamma + 1);
    int64_t total = cu_seqlens[B];
    if (total < 0 || total > cap)
        return ORACLE_ERR_RANGE;
    for (int64_t r = 0; r < total; ++r) {
        int64_t s = packed_src_row[r];
        if (s < 0 || s >= cap)
            return ORACLE_ERR_RANGE;
        for (int64_t k = 0; k < row_bytes; ++k)
            dst[r * row_bytes + k] = src[s * row_bytes + k];
    }
    return ORACLE_OK;
}

/*
 * Graph tier of a packed batch [P1, "Ragged verify under full CUDA graphs"]:
 * a batch runs the captured verify graph of the smallest tier that holds its
 * packed total, with its packed rows padded out to that tier's size.
 *   tier_index = smallest t with tiers[t] >= total (tiers ascending), or
 *                ntiers when no captured tier holds the batch;
 *   padded     = tiers[tier_index], or total when there is no such tier.
 * Rows [total, min(padded, B*(gamma+1))) of the packed arrays become padding:
 * packed_tokens = pad_token and packed_src_row = -1 (nullable arrays skipped).
 */
int oracle_tier_select(const int32_t *cu_seqlens, int B, int gamma, const int32_t *tiers,
                       int ntiers, int32_t pad_token, int32_t *padded_total,
                       int32_t *tier_index, int32_t *packed_tokens, int32_t *packed_src_row)
{
    if (B < 1 || gamma < 1 || ntiers < 1)
        return ORACLE_ERR_SHAPE;
    for (int t = 1; t < ntiers; ++t)
        if (tiers[t] <= tiers[t - 1])
            return ORACLE_ERR_ARG;
    int64_t cap = (int64_t)B * (gamma + 1);
    int64_t total = cu_seqlens[B];
    if (total < 0 || total > cap)
        return ORACLE_ERR_RANGE;
    int t = 0;
    while (t < ntiers && tiers[t] < total)
        t += 1;
    int64_t padded = t < ntiers ? tiers[t] : total;
    *tier_index = t;
    *padded_total = (int32_t)padded;
    int64_t end = padded < cap ? padded : cap;
    for (int64_t r = total; r < end; ++r) {
        if (packed_tokens)
            packed_tokens[r] = pad_token;
        if (packed_src_row)
            packed_src_row[r] = -1;
    }
    return ORACLE_OK;
}

/*
 * Step 5a, greedy target choice per verify row [P1, "Background"]: under
 * greedy verification the target's token at a row is the vocabulary entry with
 * the largest logit; among equal maxima the lowest index is taken (a later
 * entry replaces the best only when strictly larger, and -0 equals +0).
 * Row r of the output reads dense row src_row[r] of logits ([*, V] bf16 bits),
 * or row r itself when src_row is NULL.
 */
int oracle_argmax_rows(const uint16_t *logits, const int32_t *src_row, int64_t nrows,
                       int64_t V, int32_t *amax)
{
    if (nrows < 0 || V < 1 || V > INT32_MAX)
        return ORACLE_ERR_SHAPE;
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t src = src_row ? (int64_t)src_row[r] : r;
        if (src < 0)
            return ORACLE_ERR_RANGE;
        const uint16_t *row = logits + (size_t)src * (size_t)V;
        double best = bf16_to_double(row[0]);
        int64_t best_idx = 0;
        if (!isfinite(best))
            return ORACLE_ERR_NONFINITE;
        for (int64_t v = 1; v < V; ++v) {
            double x = bf16_to_double(row[v]);
            if (!isfinite(x))
                return ORACLE_ERR_NONFINITE;
            if (x > best) {
                best = x;
                best_idx = v;
            }
        }
        amax[r] = (int32_t)best_idx;
    }
    return ORACLE_OK;
}

/*
 * Steps 5b and 6, acceptance and bonus token [P1, "Background"]: the target
 * commits the longest prefix of drafts that agree with its own greedy choices,
 * and the verify forward yields one more token from the first row that was not
 * accepted. Packed row cu[b] + j holds the target's choice after the root and
 * j drafts, so it is compared with draft j + 1 = tokens[b, j + 1]. Only the
 * L_b verified drafts can be accepted (L_b = cu[b+1] - cu[b] - 1):
 *     a_b = max m <= L_b with amax[cu[b] + j] == tokens[b, j + 1] for j < m,
 *     bonus_b = amax[cu[b] + a_b].
 */
int oracle_accept(const int32_t *cu_seqlens, const int32_t *tokens, const int32_t *amax,
                  int B, int gamma, int32_t *accepted, int32_t *bonus)
{
    if (B < 1 || gamma < 1)
        return ORACLE_ERR_SHAPE;
    for (int b = 0; b < B; ++b) {
        int64_t start = cu_seqlens[b];
        int64_t L = (int64_t)cu_seqlens[b + 1] - start - 1;
        if (start < 0 || L < 0 || L > gamma)
            return ORACLE_ERR_RANGE;
        int64_t a = 0;
        while (a < L && amax[start + a] == tokens[(size_t)b * (gamma + 1) + a + 1])
            a += 1;
        accepted[b] = (int32_t)a;
        bonus[b] = amax[start + a];
    }
    return ORACLE_OK;
}

/*
 * Step 3 in the static verify mode [P1, "The confidence scheduler and verify
 * modes"]: the full drafted block is verified, L_b = gamma for every request.
 * Nothing is cut, so it is the reference the other modes are measured against.
 */
int oracle_cut_static(int B, int gamma, int32_t *lengths)
{
    if (B < 1 || gamma < 1)
        return ORACLE_ERR_SHAPE;
    for (int b = 0; b < B; ++b)
        lengths[b] = gamma;
    return ORACLE_OK;
}

/*
 * Steps 5b and 6 in the cap-accept verify mode [P1, "The confidence scheduler
 * and verify modes"]: the block was verified in full (static packing, request
 * b's rows at b*(gamma+1) + j), but only the scheduled window of L_b drafts may
 * be committed. The uncapped acceptance records what a full verify gives:
 *     a_full_b = max m <= gamma with amax[b*(gamma+1) + j] == tokens[b, j+1]
 *                for all j < m,
 * the committed count is a_b = min(a_full_b, L_b), and the bonus token is the
 * target's choice at the first row not committed, bonus_b = amax[b*(gamma+1)
 * + a_b]. Lengths outside [0, gamma] are rejected.
 */
int oracle_cap_accept(const int32_t *lengths, const int32_t *tokens, const int32_t *amax_full,
                      int B, int gamma, int32_t *accepted, int32_t *bonus,
                      int32_t *accepted_full)
{
    if (B < 1 || gamma < 1)
        return ORACLE_ERR_SHAPE;
    for (int b = 0; b < B; ++b) {
        int32_t L = lengths[b];
        if (L < 0 || L > gamma)
            return ORACLE_ERR_RANGE;
        const int32_t *row_am = amax_full + (size_t)b * (gamma + 1);
        const int32_t *tok = tokens + (size_t)b * (gamma + 1);
        int32_t a_full = 0;
        while (a_full < gamma && row_am[a_full] == tok[a_full + 1])
            a_full += 1;
        int32_t a = a_full < L ? a_full : L;
        accepted_full[b] = a_full;
        accepted[b] = a;
        bonus[b] = row_am[a];
    }
    return ORACLE_OK;
}

/*
 * One whole step in the pages' order: confidence -> survival -> cut ->
 * compaction -> argmax over the packed rows only -> acceptance and bonus.
 * mode 0 = per-request cutoffs (cutoff[B]); mode 1 = batch budget (budget);
 * mode 2 = static (the full block); mode 3 = cutoffs and budget together.
 * logits is the dense [B, gamma+1, V] block; only packed rows are read.
 * Output buffers: conf/surv [B*gamma]; lengths/accepted/bonus [B];
 * cu_seqlens [B+1]; packed_* [B*(gamma+1)] (entries past cu[B] untouched).
 */
int oracle_step(const uint16_t *hidden, const uint16_t *w, float bias, const float *temps,
                const int32_t *tokens, const uint16_t *logits,
                int B, int gamma, int d, int64_t V, int mode,
                const float *cutoff, long long budget,
                double *conf, double *surv, int32_t *lengths, int32_t *cu_seqlens,
                int32_t *packed_tokens, int32_t *packed_src_row, int32_t *packed_argmax,
                int32_t *accepted, int32_t *bonus)
{
    int rc = oracle_confidence(hidden, w, bias, temps, B, gamma, d, NULL, conf);
    if (rc) return rc;
    rc = oracle_survival(conf, B, gamma, surv);
    if (rc) return rc;
    if (mode == 0)
        rc = oracle_cut_threshold(surv, cutoff, B, gamma, lengths);
    else if (mode == 1)
        rc = oracle_cut_budget(surv, B, gamma, budget, lengths);
    else if (mode == 2)
        rc = oracle_cut_static(B, gamma, lengths);
    else if (mode == 3)
        rc = oracle_cut_combined(surv, cutoff, B, gamma, budget, lengths);
    else
        return ORACLE_ERR_ARG;
    if (rc) return rc;
    int64_t total = 0;
    rc = oracle_compact(lengths, tokens, B, gamma, cu_seqlens, packed_tokens,
                        packed_src_row, &total);
    if (rc) return rc;
    rc = oracle_argmax_rows(logits, packed_src_row, total, V, packed_argmax);
    if (rc) return rc;
    return oracle_accept(cu_seqlens, tokens, packed_argmax, B, gamma, accepted, bonus);
}
