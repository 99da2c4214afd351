/*
 * oracle.c -- plain, slow, fp64 CPU reference for grouped-query attention
 * with a per-head attention sink.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product calls this file: only the
 * tests, the smoke check and the CPU-baseline leg of the benchmark load it.
 * It shares no code, header, table or helper with the HIP library.
 *
 * What it computes follows "GPT-OSS on day 0" (Perplexity), section
 * "Kernels for GPT-OSS / Sink attention":
 *
 *   attn = softmax(q k^T * sm_scale + sink) V
 *
 * read as: each query head h owns one learned logit `sink_h` (natural-log
 * units, not multiplied by sm_scale) that joins the softmax denominator as an
 * extra entry whose value vector is zero.  The same section's statement that
 * the online softmax may start its running maximum at the head's sink (with
 * the running scale at 1) is exactly this extra entry: e^(sink - m) * 1 with
 * m = sink contributes 1 to the denominator and nothing to the numerator.
 *
 * Grouped-query attention ("Attention and MLP architecture": GQA with sinks):
 * query head h reads key/value head h / (Hq / Hkv).
 *
 * Causal masking is bottom-right aligned: with Lq queries over Lk keys, query
 * row i sits at key position Lk - Lq + i and sees keys 0 .. Lk - Lq + i.
 *
 * Four entry points:
 *   oracle_attention        the direct definition (max-shifted softmax over
 *                           the scores plus the sink, then the product with V)
 *   oracle_attention_split  the method as the section describes it: the keys
 *                           of each query are cut into blocks along the
 *                           sequence, each block runs the online softmax with
 *                           state (m, d, acc), m starting at the sink only in
 *                           the first block, and the block states are then
 *                           combined by log-sum-exp
 *   oracle_partials         the per-block states (m, d, acc) themselves
 *   oracle_split_row        one (query, head) over an arbitrary partition of
 *                           its keys (used to check partition invariance)
 *
 * All inputs are float32 arrays holding the exact values (bf16 inputs arrive
 * widened to float32, which is exact).  All arithmetic is double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2

/* ---- helpers that are plain index arithmetic ---------------------------- */

/* Number of keys query row i of a sequence can see (keys 0 .. n-1). */
static int64_t visible_keys(int causal, int64_t lq, int64_t lk, int64_t i)
{
    if (!causal)
        return lk;
    int64_t n = lk - lq + i + 1;
    if (n < 0)
        n = 0;
    if (n > lk)
        n = lk;
    return n;
}

/* Sequence that owns absolute query row `row` (cu_q is nondecreasing). */
static int owner_of_row(const int32_t *cu_q, int batch, int64_t row)
{
    for (int b = 0; b < batch; ++b)
        if (row >= cu_q[b] && row < cu_q[b + 1])
            return b;
    return -1;
}

/* s = sm_scale * <q, k>, in double. */
static double score(const float *q, const float *k, int d_head, double sm_scale)
{
    double acc = 0.0;
    for (int d = 0; d < d_head; ++d)
        acc += (double)q[d] * (double)k[d];
    return sm_scale * acc;
}

/* ---- the direct definition ---------------------------------------------- */

/*
 * One (query row, head): scores s_j over the visible keys, M = max(sink, s_j),
 * Z = e^(sink-M) + sum_j e^(s_j-M), out = sum_j e^(s_j-M) v_j / Z,
 * lse = M + ln Z.  With no visible keys and sink = -inf there is nothing to
 * normalise: out = 0, lse = -inf.
 */
static void direct_row(const float *qrow, const float *kbase, const float *vbase,
                       int64_t row_stride, int64_t n, int d_head, double sm_scale,
                       double sink, double *scratch, double *out, double *lse)
{
    double m = sink;
    for (int64_t j = 0; j < n; ++j) {
        scratch[j] = score(qrow, kbase + j * row_stride, d_head, sm_scale);
        if (scratch[j] > m)
            m = scratch[j];
    }
    for (int d = 0; d < d_head; ++d)
        out[d] = 0.0;
    if (m == -INFINITY) {
        *lse = -INFINITY;
        return;
    }
    double z = (sink == -INFINITY) ? 0.0 : exp(sink - m);
    for (int64_t j = 0; j < n; ++j) {
        double p = exp(scratch[j] - m);
        z += p;
        const float *vj = vbase + j * row_stride;
        for (int d = 0; d < d_head; ++d)
            out[d] += p * (double)vj[d];
    }
    for (int d = 0; d < d_head; ++d)
        out[d] /= z;
    *lse = m + log(z);
}

/*
 * q: [total_q, hq, d]   k, v: [total_k, hkv, d]   sinks: [hq]
 * cu_q, cu_k: [batch+1] absolute row offsets.
 * rows: optional list of absolute query rows to evaluate (NULL = all rows);
 * out: [nrows, hq, d] double, lse: [nrows, hq] double (nrows = total_q when
 * rows is NULL).
 */
int oracle_attention(const float *q, const float *k, const float *v, const float *sinks,
                     const int32_t *cu_q, const int32_t *cu_k, int batch, int hq, int hkv,
                     int d_head, double sm_scale, int causal, const int64_t *rows,
                     int64_t nrows, double *out, double *lse, int nthreads)
{
    if (batch < 1 || hq < 1 || hkv < 1 || d_head < 1 || hq % hkv != 0)
        return ORACLE_EINVAL;
    int64_t total_q = cu_q[batch] - cu_q[0];
    if (rows == NULL)
        nrows = total_q;
    int group = hq / hkv;
    int64_t max_lk = 0;
    for (int b = 0; b < batch; ++b)
        if (cu_k[b + 1] - cu_k[b] > max_lk)
            max_lk = cu_k[b + 1] - cu_k[b];
    int err = ORACLE_OK;
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel num_threads(nthreads)
    {
        double *scratch = (double *)malloc(sizeof(double) * (size_t)(max_lk > 0 ? max_lk : 1));
        if (scratch == NULL) {
#pragma omp atomic write
            err = ORACLE_ENOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < nrows * hq; ++t) {
            if (scratch == NULL)
                continue;
            int64_t r = t / hq;
            int h = (int)(t % hq);
            int64_t row = rows ? rows[r] : cu_q[0] + r;
            int b = owner_of_row(cu_q, batch, row);
            if (b < 0) {
#pragma omp atomic write
                err = ORACLE_EINVAL;
                continue;
            }
            int64_t lq = cu_q[b + 1] - cu_q[b], lk = cu_k[b + 1] - cu_k[b];
            int64_t n = visible_keys(causal, lq, lk, row - cu_q[b]);
            int g = h / group;
            const float *qrow = q + (row * hq + h) * d_head;
            const float *kbase = k + ((int64_t)cu_k[b] * hkv + g) * d_head;
            const float *vbase = v + ((int64_t)cu_k[b] * hkv + g) * d_head;
            direct_row(qrow, kbase, vbase, (int64_t)hkv * d_head, n, d_head, sm_scale,
                       (double)sinks[h], scratch, out + (r * hq + h) * d_head, lse + r * hq + h);
        }
        free(scratch);
    }
    return err;
}

/* ---- the method: blocks along the keys, online softmax, combine ---------- */

/*
 * Online softmax over keys [lo, hi) of one (query, head), starting from the
 * state (m, d, acc).  Each key updates m' = max(m, s), rescales the running
 * scale and accumulator by e^(m - m') and adds e^(s - m').  A state at
 * m = -inf carries no mass, so its rescale factor is 0.
 */
static void online_block(const float *qrow, const float *kbase, const float *vbase,
                         int64_t row_stride, int64_t lo, int64_t hi, int d_head,
                         double sm_scale, double *m, double *dsum, double *acc)
{
    for (int64_t j = lo; j < hi; ++j) {
        double s = score(qrow, kbase + j * row_stride, d_head, sm_scale);
        double m_new = (s > *m) ? s : *m;
        double alpha = (*m == -INFINITY) ? 0.0 : exp(*m - m_new);
        double p = exp(s - m_new);
        *dsum = alpha * (*dsum) + p;
        const float *vj = vbase + j * row_stride;
        for (int d = 0; d < d_head; ++d)
            acc[d] = alpha * acc[d] + p * (double)vj[d];
        *m = m_new;
    }
}

/* State of block c: m starts at the sink in block 0 only, the scale at 1. */
static void block_state(const float *qrow, const float *kbase, const float *vbase,
                        int64_t row_stride, int64_t lo, int64_t hi, int first, int d_head,
                        double sm_scale, double sink, double *m, double *dsum, double *acc)
{
    *m = first ? sink : -INFINITY;
    *dsum = 1.0;
    for (int d = 0; d < d_head; ++d)
        acc[d] = 0.0;
    online_block(qrow, kbase, vbase, row_stride, lo, hi, d_head, sm_scale, m, dsum, acc);
}

/*
 * Log-sum-exp combination of block states: M = max_c m_c, w_c = e^(m_c - M),
 * out = sum_c w_c acc_c / sum_c w_c d_c, lse = M + ln sum_c w_c d_c.  If every
 * block is at -inf there is no mass at all: out = 0, lse = -inf.
 */
static void combine(int nblocks, const double *ms, const double *ds, const double *accs,
                    int d_head, double *out, double *lse)
{
    double big = -INFINITY;
    for (int c = 0; c < nblocks; ++c)
        if (ms[c] > big)
            big = ms[c];
    for (int d = 0; d < d_head; ++d)
        out[d] = 0.0;
    if (big == -INFINITY) {
        *lse = -INFINITY;
        return;
    }
    double den = 0.0;
    for (int c = 0; c < nblocks; ++c) {
        if (ms[c] == -INFINITY)
            continue;
        double w = exp(ms[c] - big);
        den += w * ds[c];
        for (int d = 0; d < d_head; ++d)
            out[d] += w * accs[(int64_t)c * d_head + d];
    }
    for (int d = 0; d < d_head; ++d)
        out[d] /= den;
    *lse = big + log(den);
}

/*
 * One query row and head over an arbitrary partition of its n keys:
 * bounds[0] = 0 < bounds[1] < ... < bounds[nparts] = n (a single empty part
 * bounds = {0, 0} is allowed for n = 0).  q_row: [d], k, v: [n, d] rows with
 * stride row_stride floats.
 */
int oracle_split_row(const float *qrow, const float *k, const float *v, int64_t row_stride,
                     int64_t n, int d_head, double sm_scale, double sink,
                     const int64_t *bounds, int nparts, double *out, double *lse)
{
    if (nparts < 1 || bounds[0] != 0 || bounds[nparts] != n)
        return ORACLE_EINVAL;
    double *ms = (double *)malloc(sizeof(double) * (size_t)nparts);
    double *ds = (double *)malloc(sizeof(double) * (size_t)nparts);
    double *accs = (double *)malloc(sizeof(double) * (size_t)nparts * (size_t)d_head);
    if (!ms || !ds || !accs) {
        free(ms);
        free(ds);
        free(accs);
        return ORACLE_ENOMEM;
    }
    for (int c = 0; c < nparts; ++c)
        block_state(qrow, k, v, row_stride, bounds[c], bounds[c + 1], c == 0, d_head, sm_scale,
                    sink, &ms[c], &ds[c], &accs[(int64_t)c * d_head]);
    combine(nparts, ms, ds, accs, d_head, out, lse);
    free(ms);
    free(ds);
    free(accs);
    return ORACLE_OK;
}

/* Blocks of `chunk` keys: block c covers [c*chunk, min((c+1)*chunk, n)); at least one block. */
static int64_t num_blocks(int64_t n, int64_t chunk)
{
    int64_t nb = (n + chunk - 1) / chunk;
    return nb < 1 ? 1 : nb;
}

/* Same arguments as oracle_attention plus the block length along the keys. */
int oracle_attention_split(const float *q, const float *k, const float *v, const float *sinks,
                           const int32_t *cu_q, const int32_t *cu_k, int batch, int hq, int hkv,
                           int d_head, double sm_scale, int causal, int64_t chunk,
                           const int64_t *rows, int64_t nrows, double *out, double *lse,
                           int nthreads)
{
    if (batch < 1 || hq < 1 || hkv < 1 || d_head < 1 || hq % hkv != 0 || chunk < 1)
        return ORACLE_EINVAL;
    int64_t total_q = cu_q[batch] - cu_q[0];
    if (rows == NULL)
        nrows = total_q;
    int group = hq / hkv;
    int64_t max_lk = 0;
    for (int b = 0; b < batch; ++b)
        if (cu_k[b + 1] - cu_k[b] > max_lk)
            max_lk = cu_k[b + 1] - cu_k[b];
    int64_t max_blocks = num_blocks(max_lk, chunk);
    int err = ORACLE_OK;
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel num_threads(nthreads)
    {
        double *ms = (double *)malloc(sizeof(double) * (size_t)max_blocks);
        double *ds = (double *)malloc(sizeof(double) * (size_t)max_blocks);
        double *accs = (double *)malloc(sizeof(double) * (size_t)(max_blocks * d_head));
        if (!ms || !ds || !accs) {
#pragma omp atomic write
            err = ORACLE_ENOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < nrows * hq; ++t) {
            if (!ms || !ds || !accs)
                continue;
            int64_t r = t / hq;
            int h = (int)(t % hq);
            int64_t row = rows ? rows[r] : cu_q[0] + r;
            int b = owner_of_row(cu_q, batch, row);
            if (b < 0) {
#pragma omp atomic write
                err = ORACLE_EINVAL;
                continue;
            }
            int64_t lq = cu_q[b + 1] - cu_q[b], lk = cu_k[b + 1] - cu_k[b];
            int64_t n = visible_keys(causal, lq, lk, row - cu_q[b]);
            int g = h / group;
            const float *qrow = q + (row * hq + h) * d_head;
            const float *kbase = k + ((int64_t)cu_k[b] * hkv + g) * d_head;
            const float *vbase = v + ((int64_t)cu_k[b] * hkv + g) * d_head;
            int64_t nb = num_blocks(n, chunk);
            for (int64_t c = 0; c < nb; ++c) {
                int64_t lo = c * chunk, hi = (c + 1) * chunk < n ? (c + 1) * chunk : n;
                block_state(qrow, kbase, vbase, (int64_t)hkv * d_head, lo, hi, c == 0, d_head,
                            sm_scale, (double)sinks[h], &ms[c], &ds[c], &accs[c * d_head]);
            }
            combine((int)nb, ms, ds, accs, d_head, out + (r * hq + h) * d_head, lse + r * hq + h);
        }
        free(ms);
        free(ds);
        free(accs);
    }
    return err;
}

/*
 * Per-block states of single-query (decode) sequences.  q: [batch, hq, d];
 * block c of sequence b covers keys [c*chunk, min((c+1)*chunk, L_b)),
 * nblocks(b) = max(1, ceil(L_b / chunk)).  Writes, for c < nblocks(b):
 * part_m, part_d: [batch, hq, max_blocks], part_acc: [batch, hq, max_blocks, d]
 * (m in natural-log units, acc unnormalised).  Other slots are left as they are.
 */
int oracle_partials(const float *q, const float *k, const float *v, const float *sinks,
                    const int32_t *cu_k, int batch, int hq, int hkv, int d_head, double sm_scale,
                    int64_t chunk, int64_t max_blocks, double *part_m, double *part_d,
                    double *part_acc, int nthreads)
{
    if (batch < 1 || hq < 1 || hkv < 1 || d_head < 1 || hq % hkv != 0 || chunk < 1)
        return ORACLE_EINVAL;
    int group = hq / hkv;
    for (int b = 0; b < batch; ++b)
        if (num_blocks(cu_k[b + 1] - cu_k[b], chunk) > max_blocks)
            return ORACLE_EINVAL;
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
    for (int64_t t = 0; t < (int64_t)batch * hq; ++t) {
        int b = (int)(t / hq), h = (int)(t % hq);
        int64_t n = cu_k[b + 1] - cu_k[b];
        int g = h / group;
        const float *qrow = q + ((int64_t)b * hq + h) * d_head;
        const float *kbase = k + ((int64_t)cu_k[b] * hkv + g) * d_head;
        const float *vbase = v + ((int64_t)cu_k[b] * hkv + g) * d_head;
        int64_t nb = num_blocks(n, chunk);
        for (int64_t c = 0; c < nb; ++c) {
            int64_t lo = c * chunk, hi = (c + 1) * chunk < n ? (c + 1) * chunk : n;
            int64_t slot = t * max_blocks + c;
            block_state(qrow, kbase, vbase, (int64_t)hkv * d_head, lo, hi, c == 0, d_head,
                        sm_scale, (double)sinks[h], &part_m[slot], &part_d[slot],
                        &part_acc[slot * d_head]);
        }
    }
    return ORACLE_OK;
}
