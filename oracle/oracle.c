/*
 * Plain CPU oracle for DSA-style sparse attention over a paged latent KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; the two meet only through the
 * seeded input generator.  Everything here is written for clarity, not speed:
 * plain loops, fp32 indexer, a full sort for top-k, fp64 softmax attention.
 *
 * What is computed, per query row r that sits at position pos of sequence seq
 * (decode row b: seq = b, pos = ctx_b - 1; prefill row i: seq = 0,
 * pos = q_start + i):
 *
 *  1. Visible keys (causal limit): s = 0 .. pos, n = pos + 1.
 *     "Engineering Practices for Day-0 Adaptation of Million-Token Context
 *     Models on Domestic AI Chips", Four Key Layers item 1: each query attends
 *     to a small subset of the historical tokens.
 *  2. Paged addressing: token s lives in physical block block_table[seq][s/bs]
 *     at slot s % bs.  "Day-0 Adaptation: Running Trillion-Parameter Models on
 *     Domestic AI Accelerators", section 3.2 (block table maps logical blocks
 *     to physical ones) and section 3.1 (selection and attention share one
 *     block-mapping convention).
 *  3. Indexer score (fp32): d_j = sum_c iq[j][c] * ik[s][c] (increasing c),
 *     a_j = max(d_j, 0) when relu is on, score_s = sum_j w[j] * a_j
 *     (increasing j), then score_s + 0.0f folds -0 into +0.
 *     "Day-0 Adaptation for LLMs: Implementing Sparse Attention and
 *     Low-Precision Weights", section III.1 (a lightweight indexer scores every
 *     historical token; its matmul wants more precision than the attention).
 *     The ReLU-and-weighted-head-sum form is the lightning-indexer reading of
 *     that scoring network; the pages give no formula.
 *  4. Top-k: if n <= k every visible key is kept; otherwise the k keys that
 *     come first under (score descending, position ascending).  Emitted in
 *     ascending position order, padded with -1 to length k.
 *     Same page, section III.1 (top-k over long sequences) and the decode
 *     pseudocode (indexer -> topk -> gather -> attention).
 *  5. Attention (fp64): for every head h, l_s = scale * q[h] . kv[s][0:Dqk]
 *     over the kept s, p_s = exp(l_s - max l), o[h] = sum_s p_s kv[s][0:Dv] /
 *     sum_s p_s, lse[h] = max l + log(sum_s p_s).  K and V are the leading
 *     Dqk and Dv entries of one shared latent row.  With nothing kept
 *     (empty context) o = 0 and lse = -inf.
 *     Same page, section II (tile skeleton: gather by index, then a softmax
 *     reduction of q.k^T-weighted v; its literal accumulate-then-softmax
 *     order is not a softmax and is read as standard softmax attention) and the
 *     decode pseudocode.
 *
 * Appending (decode): before step 1 the current token of sequence b, position
 * ctx_b - 1, is written into the cache at its physical slot (step 2's
 * addressing): its latent row and its indexer key replace the slot's contents.
 * "Engineering Practices for Day-0 Adaptation of Million-Token Context Models
 * on Domestic AI Chips", Four Key Layers item 2 (block-level incremental cache
 * updates during decode) and item 3 (the update merged with the decode
 * attention).
 *
 * Precision: bf16 inputs are widened exactly; the indexer sums in fp32 with no
 * fused multiply-add (built with -ffp-contract=off); attention runs in double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static float bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static double now_seconds(void)
{
    struct timespec ts;
    clock_gettime(CLOCK_MONOTONIC, &ts);
    return (double)ts.tv_sec + 1e-9 * (double)ts.tv_nsec;
}

/* physical row of logical token s of sequence seq */
static int64_t physical_row(const int32_t *block_table, int64_t max_blocks, int64_t seq,
                            int64_t s, int64_t block_size)
{
    int64_t logical_block = s / block_size;
    int64_t physical_block = block_table[seq * max_blocks + logical_block];
    return physical_block * block_size + s % block_size;
}

typedef struct {
    int64_t num_heads, qk_dim, v_dim, idx_heads, idx_dim, block_size, topk;
    int relu;
    double scale;
    const uint16_t *kv;      /* [num_blocks][block_size][qk_dim] */
    const uint16_t *idx_k;   /* [num_blocks][block_size][idx_dim] */
    const int32_t *block_table;
    int64_t max_blocks;
} problem;

/* step 3 for keys 0..n-1 of one query row */
static void index_scores(const problem *p, int64_t seq, int64_t n, const uint16_t *iq,
                         const float *w, float *scores)
{
    int64_t s;
#pragma omp parallel for schedule(static)
    for (s = 0; s < n; s++) {
        const uint16_t *key = p->idx_k + physical_row(p->block_table, p->max_blocks, seq, s,
                                                      p->block_size) * p->idx_dim;
        float score = 0.0f;
        for (int64_t j = 0; j < p->idx_heads; j++) {
            float d = 0.0f;
            for (int64_t c = 0; c < p->idx_dim; c++) {
                float prod = bf16_to_float(iq[j * p->idx_dim + c]) * bf16_to_float(key[c]);
                d = d + prod;
            }
            float a = p->relu ? (d > 0.0f ? d : 0.0f) : d;
            float term = w[j] * a;
            score = score + term;
        }
        scores[s] = score + 0.0f;
    }
}

typedef struct {
    float score;
    int32_t pos;
} scored_key;

/* total order: higher score first, then lower position first */
static int by_score_then_position(const void *a, const void *b)
{
    const scored_key *x = (const scored_key *)a, *y = (const scored_key *)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->pos > y->pos) - (x->pos < y->pos);
}

static int ascending_int(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* step 4; returns the number of kept keys */
int64_t oracle_topk(const float *scores, int64_t n, int64_t k, int32_t *out)
{
    int64_t kept;
    if (n <= k) {
        for (int64_t s = 0; s < n; s++) out[s] = (int32_t)s;
        kept = n;
    } else {
        scored_key *all = (scored_key *)malloc((size_t)n * sizeof *all);
        if (!all) return -1;
        for (int64_t s = 0; s < n; s++) {
            all[s].score = scores[s];
            all[s].pos = (int32_t)s;
        }
        qsort(all, (size_t)n, sizeof *all, by_score_then_position);
        for (int64_t j = 0; j < k; j++) out[j] = all[j].pos;
        free(all);
        qsort(out, (size_t)k, sizeof *out, ascending_int);
        kept = k;
    }
    for (int64_t j = kept; j < k; j++) out[j] = -1;
    return kept;
}

/* step 5 for one query row over the kept positions sel[0..kept) */
static void attend(const problem *p, int64_t seq, const uint16_t *q, const int32_t *sel,
                   int64_t kept, double *o, double *lse)
{
    int64_t h;
#pragma omp parallel for schedule(static)
    for (h = 0; h < p->num_heads; h++) {
        double *orow = o + h * p->v_dim;
        for (int64_t v = 0; v < p->v_dim; v++) orow[v] = 0.0;
        if (kept == 0) {
            lse[h] = -INFINITY;
            continue;
        }
        double *logit = (double *)malloc((size_t)kept * sizeof(double));
        const uint16_t *qh = q + h * p->qk_dim;
        double m = -INFINITY;
        for (int64_t j = 0; j < kept; j++) {
            const uint16_t *row = p->kv + physical_row(p->block_table, p->max_blocks, seq, sel[j],
                                                       p->block_size) * p->qk_dim;
            double dot = 0.0;
            for (int64_t c = 0; c < p->qk_dim; c++)
                dot += (double)bf16_to_float(qh[c]) * (double)bf16_to_float(row[c]);
            logit[j] = p->scale * dot;
            if (logit[j] > m) m = logit[j];
        }
        double z = 0.0;
        for (int64_t j = 0; j < kept; j++) {
            const uint16_t *row = p->kv + physical_row(p->block_table, p->max_blocks, seq, sel[j],
                                                       p->block_size) * p->qk_dim;
            double e = exp(logit[j] - m);
            z += e;
            for (int64_t v = 0; v < p->v_dim; v++) orow[v] += e * (double)bf16_to_float(row[v]);
        }
        for (int64_t v = 0; v < p->v_dim; v++) orow[v] /= z;
        lse[h] = m + log(z);
        free(logit);
    }
}

/*
 * Run steps 1-5 for a list of query rows.
 *   mode 0 (decode): row r is query b = rows[r], sequence b, n = context_lens[b].
 *   mode 1 (prefill): row r is query i = rows[r], sequence 0, n = q_start + i + 1.
 * q: [T][num_heads][qk_dim] bf16, idx_q: [T][idx_heads][idx_dim] bf16, idx_w: [T][idx_heads].
 * Outputs per listed row: topk_out [nrows][topk], o [nrows][num_heads][v_dim] (double),
 * lse [nrows][num_heads] (double), and when scores_out is non-null the fp32 scores
 * [nrows][score_stride] (entries past n untouched).  stage_seconds (nullable, 3 entries)
 * accumulates wall time of scoring, selection and attention.
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_rows(int mode, int64_t num_heads, int64_t qk_dim, int64_t v_dim, int64_t idx_heads,
                int64_t idx_dim, int64_t block_size, int64_t topk, int relu, double scale,
                const uint16_t *kv, const uint16_t *idx_k, const int32_t *block_table,
                int64_t max_blocks, const int32_t *context_lens, int64_t q_start,
                const uint16_t *q, const uint16_t *idx_q, const float *idx_w,
                const int64_t *rows, int64_t nrows, int32_t *topk_out, double *o, double *lse,
                float *scores_out, int64_t score_stride, double *stage_seconds)
{
    if (topk < 1 || block_size < 1 || (mode != 0 && mode != 1)) return -1;
    problem p = {num_heads, qk_dim, v_dim, idx_heads, idx_dim, block_size, topk,
                 relu, scale, kv, idx_k, block_table, max_blocks};
    for (int64_t r = 0; r < nrows; r++) {
        int64_t row = rows[r];
        int64_t seq = mode == 0 ? row : 0;
        int64_t n = mode == 0 ? (int64_t)context_lens[row] : q_start + row + 1;
        float *scores = scores_out ? scores_out + r * score_stride
                                   : (float *)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
        if (!scores) return -1;
        double t0 = now_seconds();
        index_scores(&p, seq, n, idx_q + row * idx_heads * idx_dim, idx_w + row * idx_heads, scores);
        double t1 = now_seconds();
        int64_t kept = oracle_topk(scores, n, topk, topk_out + r * topk);
        double t2 = now_seconds();
        if (kept < 0) return -1;
        attend(&p, seq, q + row * num_heads * qk_dim, topk_out + r * topk, kept,
               o + r * num_heads * v_dim, lse + r * num_heads);
        double t3 = now_seconds();
        if (stage_seconds) {
            stage_seconds[0] += t1 - t0;
            stage_seconds[1] += t2 - t1;
            stage_seconds[2] += t3 - t2;
        }
        if (!scores_out) free(scores);
    }
    return 0;
}

/* Appends the current token of every decode sequence: for b with ctx[b] > 0,
 * position s = ctx[b] - 1 lives at physical slot block_table[b][s / bs] * bs +
 * s % bs; its kv row (qk_dim entries) and idx_k row (idx_dim entries) are
 * copied from new_kv[b] and new_idx_k[b].  A block-table entry outside
 * [0, num_blocks) appends nothing.  Returns the number of rows appended. */
int64_t oracle_append(int64_t batch, int64_t qk_dim, int64_t idx_dim, int64_t bs, int64_t num_blocks,
                      uint16_t *kv, uint16_t *idx_k, const int32_t *block_table, int64_t max_blocks,
                      const int32_t *ctx, const uint16_t *new_kv, const uint16_t *new_idx_k)
{
    int64_t appended = 0;
    for (int64_t b = 0; b < batch; ++b) {
        if (ctx[b] <= 0) continue;
        const int64_t s = ctx[b] - 1;
        const int64_t blk = block_table[b * max_blocks + s / bs];
        if (blk < 0 || blk >= num_blocks) continue;
        const int64_t slot = blk * bs + s % bs;
        for (int64_t c = 0; c < qk_dim; ++c) kv[slot * qk_dim + c] = new_kv[b * qk_dim + c];
        for (int64_t c = 0; c < idx_dim; ++c) idx_k[slot * idx_dim + c] = new_idx_k[b * idx_dim + c];
        ++appended;
    }
    return appended;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
