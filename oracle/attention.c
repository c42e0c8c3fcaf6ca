/*
 * CPU oracle for the attention forward pass. TEST INFRASTRUCTURE ONLY: it is
 * built and called by the tests, by the smoke check and by the bench's CPU
 * baseline leg, never by the library. It shares no code with the GPU path.
 *
 * What it computes is the plain definition, written out without tiling, online
 * rescaling, splitting or reduced precision:
 *
 *     O = softmax(scale * Q K^T + mask) V          (every value in double)
 *
 * The pages name this operation without printing it: "CUDA: fix FA occupancy,
 * optimize tile kernel" (llama.cpp, opening paragraph: the FlashAttention
 * kernels and their KQ accumulators) and "perf: FlashAttention-3 style MLA
 * PageAttention" (FlashInfer, change list item 4: MLA uses one ckv matrix as
 * both K and V). The mask is causal or not, aligned bottom-right (query i of Sq
 * sits at absolute position Skv - Sq + i); that is the reading under which a
 * 512-query microbatch attends to all prior keys, as in the llama.cpp
 * microbatch sweep ("Performance changes" table). Optionally an explicit
 * additive mask M[i][j] (finite or -infinity; the KQ mask that the llama.cpp
 * page's opening paragraph counts as memory traffic) is added to the scaled
 * scores, on top of the causal rule.
 *
 * Per query row (b, h, i):
 *   1. K/V head g = h / (Hq / Hkv)                  (grouped-query heads)
 *   2. visible keys J = { j : 0 <= j < Skv, and j <= i + Skv - Sq if causal }
 *   3. s_j = scale * sum_d q[d] * k_j[d] (+ M[i][j])   (ascending d)
 *   4. m = max_j s_j ; e_j = exp(s_j - m) ; l = sum_j e_j   (ascending j)
 *   5. o[d] = (sum_j e_j * v_j[d]) / l ; lse = m + log(l)   (natural log)
 *   6. no visible key (none in J, or M = -infinity on all of J): o = 0,
 *      lse = -infinity
 *
 * Threads split the rows; each row is computed by one thread, start to end.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q_rows;      /* [nrows, Dqk] */
    const int64_t *rb, *rh, *ri;  /* row coordinates (b, h, i) */
    int64_t nrows;
    const double *k;           /* [B, Skv, Hkv, Dqk] */
    const double *v;           /* [B, Skv, Hkv, Dv] */
    int64_t B, Hq, Hkv, Sq, Skv, Dqk, Dv;
    int causal;
    double scale;
    const double *mask;        /* additive mask, or NULL */
    int64_t mask_bstride, mask_stride;  /* elements between batches / rows */
    double *o_rows;            /* [nrows, Dv] */
    double *lse_rows;          /* [nrows] */
    int64_t next;              /* next row to take (guarded by lock) */
    pthread_mutex_t lock;
    int failed;
} oracle_job;

static void one_row(oracle_job *J, int64_t r, double *s) {
    const int64_t b = J->rb[r], h = J->rh[r], i = J->ri[r];
    const int64_t g = h / (J->Hq / J->Hkv);
    const double *q = J->q_rows + r * J->Dqk;
    double *o = J->o_rows + r * J->Dv;

    int64_t nvis = J->Skv;
    if (J->causal) {
        int64_t last = i + (J->Skv - J->Sq); /* last visible key index */
        if (last + 1 < nvis) nvis = last + 1;
    }
    if (nvis <= 0) {
        for (int64_t d = 0; d < J->Dv; ++d) o[d] = 0.0;
        J->lse_rows[r] = -INFINITY;
        return;
    }
    for (int64_t j = 0; j < nvis; ++j) {
        const double *kj = J->k + ((b * J->Skv + j) * J->Hkv + g) * J->Dqk;
        double acc = 0.0;
        for (int64_t d = 0; d < J->Dqk; ++d) acc += q[d] * kj[d];
        s[j] = J->scale * acc;
        if (J->mask) s[j] += J->mask[b * J->mask_bstride + i * J->mask_stride + j];
    }
    double m = s[0];
    for (int64_t j = 1; j < nvis; ++j)
        if (s[j] > m) m = s[j];
    if (m == -INFINITY) { /* every visible key masked out */
        for (int64_t d = 0; d < J->Dv; ++d) o[d] = 0.0;
        J->lse_rows[r] = -INFINITY;
        return;
    }
    double l = 0.0;
    for (int64_t j = 0; j < nvis; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (int64_t d = 0; d < J->Dv; ++d) o[d] = 0.0;
    for (int64_t j = 0; j < nvis; ++j) {
        const double *vj = J->v + ((b * J->Skv + j) * J->Hkv + g) * J->Dv;
        for (int64_t d = 0; d < J->Dv; ++d) o[d] += s[j] * vj[d];
    }
    for (int64_t d = 0; d < J->Dv; ++d) o[d] /= l;
    J->lse_rows[r] = m + log(l);
}

static void *worker(void *arg) {
    oracle_job *J = (oracle_job *)arg;
    double *s = (double *)malloc(sizeof(double) * (size_t)(J->Skv > 0 ? J->Skv : 1));
    if (!s) {
        pthread_mutex_lock(&J->lock);
        J->failed = 1;
        pthread_mutex_unlock(&J->lock);
        return NULL;
    }
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t r = J->next;
        J->next += 1;
        pthread_mutex_unlock(&J->lock);
        if (r >= J->nrows) break;
        one_row(J, r, s);
    }
    free(s);
    return NULL;
}

/*
 * Attention for an arbitrary list of query rows.
 *   q_rows  [nrows, Dqk]  the query vectors of the listed rows
 *   rb/rh/ri [nrows]      batch, query head and query index of each row
 *   k [B, Skv, Hkv, Dqk], v [B, Skv, Hkv, Dv]  (row-major, last index fastest)
 *   mask  additive mask element (b, i, j) at mask[b * mask_bstride + i * mask_stride + j],
 *         or NULL (mask_stride >= Skv; mask_bstride 0 shares one mask over the batch)
 *   o_rows [nrows, Dv], lse_rows [nrows]       outputs
 * Returns 0 on success, -1 on a bad argument, -2 when memory runs out.
 */
int oracle_attention_rows(const double *q_rows, const int64_t *rb, const int64_t *rh,
                          const int64_t *ri, int64_t nrows, const double *k, const double *v,
                          int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv,
                          int64_t Dqk, int64_t Dv, int causal, double scale,
                          const double *mask, int64_t mask_bstride, int64_t mask_stride,
                          double *o_rows, double *lse_rows, int nthreads) {
    if (nrows < 0 || B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || Sq < 0 || Skv < 0 ||
        Dqk <= 0 || Dv <= 0)
        return -1;
    if (mask && (mask_stride < Skv || mask_bstride < 0)) return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rb[r] < 0 || rb[r] >= B || rh[r] < 0 || rh[r] >= Hq || ri[r] < 0 || ri[r] >= Sq)
            return -1;
    oracle_job J;
    memset(&J, 0, sizeof(J));
    J.q_rows = q_rows; J.rb = rb; J.rh = rh; J.ri = ri; J.nrows = nrows;
    J.k = k; J.v = v;
    J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.Sq = Sq; J.Skv = Skv; J.Dqk = Dqk; J.Dv = Dv;
    J.causal = causal; J.scale = scale; J.o_rows = o_rows; J.lse_rows = lse_rows;
    J.mask = mask; J.mask_bstride = mask_bstride; J.mask_stride = mask_stride;
    pthread_mutex_init(&J.lock, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t tid[256];
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (pthread_create(&tid[t], NULL, worker, &J) != 0) break;
        ++started;
    }
    if (started == 0) worker(&J);
    for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
    pthread_mutex_destroy(&J.lock);
    return J.failed ? -2 : 0;
}
