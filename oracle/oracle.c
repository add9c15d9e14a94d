/*
 * CPU oracle for large-beam decode attention.  TEST INFRASTRUCTURE ONLY:
 * the tests, the smoke check and the benchmark's CPU-baseline leg are its
 * only callers; the library's compute path never links or calls it.
 *
 * What it computes (the plain definition, in fp64):
 *
 *   For request b, query row r of that request and query head h (KV head
 *   g = h / (Hq/Hkv)), the keys/values the row attends to are, in order,
 *     - every ContextKV token j < ctx_len[b]           (shared by all beams)
 *     - the BeamKV token beam_path[r][s] for s < beam_len[b]  (this beam only)
 *   and the result is ordinary softmax attention over that concatenation:
 *     z_j   = scale * <q[r,h,:], K_j>
 *     out   = sum_j exp(z_j - M) V_j / sum_j exp(z_j - M),   M = max_j z_j
 *     lse   = M + ln sum_j exp(z_j - M)        (natural log, scale included)
 *   With no keys at all, out = 0 and lse = -inf.
 *
 * Sources: GR-Inference blog (developer.nvidia.cn), sections on system design
 * (ContextKV kept once per request, BeamKV per beam, BeamPath index records)
 * and on kernel design (shared context, per-beam history along BeamPath, and
 * a log-sum-exp merge); xGR review (xllm-io), section "xAttention"
 * (shared / unshared / merging stages).  Splitting the keys into a shared
 * and an unshared part and merging by log-sum-exp reproduces exactly this
 * softmax (up to rounding), so the oracle is the unsplit definition: no
 * online rescaling, no tiling, no splitting; two plain passes per (row, head).
 *
 * Inputs are raw bf16 bit patterns (uint16), widened exactly to double.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

typedef struct {
    int B, R, Hq, Hkv, D, T_cap;
    int64_t ctx_cap, beam_cap;
    double scale;
    const uint16_t *q, *ctx_k, *ctx_v, *beam_k, *beam_v;
    const int32_t *ctx_len, *beam_len, *row_offset, *beam_path;
    const int32_t *rows;   /* rows to evaluate */
    int n_rows;
    double *out, *lse;     /* [n_rows][Hq][D], [n_rows][Hq] */
    int first, stride;     /* this worker evaluates rows first, first+stride, ... */
    int status;
} job_t;

/* request owning packed row r */
static int request_of_row(const job_t *J, int r)
{
    for (int b = 0; b < J->B; ++b)
        if (r >= J->row_offset[b] && r < J->row_offset[b + 1])
            return b;
    return -1;
}

/* pointer to the D-vector of token t, KV head g, request b in a [B][cap][Hkv][D] buffer */
static const uint16_t *kv_row(const uint16_t *buf, int64_t cap, int Hkv, int D,
                              int b, int64_t t, int g)
{
    return buf + (((int64_t)b * cap + t) * Hkv + g) * D;
}

static void one_row_head(const job_t *J, int b, int r, int h, double *z,
                         double *out, double *lse)
{
    const int D = J->D;
    const int g = h / (J->Hq / J->Hkv);
    const int L = J->ctx_len[b];
    const int T = J->beam_len[b];
    const int N = L + T;
    const uint16_t *qv = J->q + ((int64_t)r * J->Hq + h) * D;

    for (int d = 0; d < D; ++d)
        out[d] = 0.0;
    if (N == 0) {
        *lse = -INFINITY;
        return;
    }

    /* pass 1: scores of the concatenated key list, and their maximum */
    double M = -INFINITY;
    for (int j = 0; j < N; ++j) {
        const uint16_t *k;
        if (j < L)
            k = kv_row(J->ctx_k, J->ctx_cap, J->Hkv, D, b, j, g);
        else
            k = kv_row(J->beam_k, J->beam_cap, J->Hkv, D, b,
                       J->beam_path[(int64_t)r * J->T_cap + (j - L)], g);
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += bf16_to_double(qv[d]) * bf16_to_double(k[d]);
        z[j] = J->scale * dot;
        if (z[j] > M)
            M = z[j];
    }

    /* pass 2: softmax weights, their sum, and the weighted sum of values */
    double Z = 0.0;
    for (int j = 0; j < N; ++j) {
        const uint16_t *v;
        if (j < L)
            v = kv_row(J->ctx_v, J->ctx_cap, J->Hkv, D, b, j, g);
        else
            v = kv_row(J->beam_v, J->beam_cap, J->Hkv, D, b,
                       J->beam_path[(int64_t)r * J->T_cap + (j - L)], g);
        double p = exp(z[j] - M);
        Z += p;
        for (int d = 0; d < D; ++d)
            out[d] += p * bf16_to_double(v[d]);
    }
    for (int d = 0; d < D; ++d)
        out[d] /= Z;
    *lse = M + log(Z);
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    double *z = (double *)malloc(sizeof(double) * (size_t)(J->ctx_cap + J->T_cap + 1));
    if (!z) {
        J->status = -2;
        return NULL;
    }
    for (int i = J->first; i < J->n_rows; i += J->stride) {
        int r = J->rows ? J->rows[i] : i;
        int b = request_of_row(J, r);
        if (b < 0) {
            J->status = -3;
            break;
        }
        for (int h = 0; h < J->Hq; ++h)
            one_row_head(J, b, r, h, z,
                         J->out + ((int64_t)i * J->Hq + h) * J->D,
                         J->lse + (int64_t)i * J->Hq + h);
    }
    free(z);
    return NULL;
}

/*
 * Evaluate rows[0..n_rows) (all R rows when rows == NULL, n_rows = R) with
 * n_threads worker threads.  Returns 0, or a negative code on bad arguments
 * (-1), allocation failure (-2) or a row outside every request (-3).
 * Threads only split the rows; each (row, head) is computed the same way
 * whatever the thread count, so results do not depend on it.
 */
int oracle_decode_attn(int B, int R, int Hq, int Hkv, int D, int T_cap,
                       int64_t ctx_cap, int64_t beam_cap, double scale,
                       const uint16_t *q, const uint16_t *ctx_k, const uint16_t *ctx_v,
                       const int32_t *ctx_len, const uint16_t *beam_k,
                       const uint16_t *beam_v, const int32_t *beam_path,
                       const int32_t *beam_len, const int32_t *row_offset,
                       const int32_t *rows, int n_rows, double *out, double *lse,
                       int n_threads)
{
    if (B < 0 || R < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || T_cap < 0 ||
        !out || !lse || (!rows && n_rows != R))
        return -1;
    if (n_threads < 1)
        n_threads = 1;
    if (n_threads > n_rows)
        n_threads = n_rows > 0 ? n_rows : 1;

    job_t base = {B, R, Hq, Hkv, D, T_cap, ctx_cap, beam_cap, scale,
                  q, ctx_k, ctx_v, beam_k, beam_v, ctx_len, beam_len, row_offset,
                  beam_path, rows, n_rows, out, lse, 0, n_threads, 0};
    job_t *jobs = (job_t *)malloc(sizeof(job_t) * (size_t)n_threads);
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    if (!jobs || !tid) {
        free(jobs);
        free(tid);
        return -2;
    }
    char *created = (char *)calloc((size_t)n_threads, 1);
    if (!created) {
        free(jobs);
        free(tid);
        return -2;
    }
    for (int t = 0; t < n_threads; ++t) {
        jobs[t] = base;
        jobs[t].first = t;
    }
    for (int t = 1; t < n_threads; ++t)
        created[t] = pthread_create(&tid[t], NULL, worker, &jobs[t]) == 0;
    worker(&jobs[0]);
    for (int t = 1; t < n_threads; ++t) {
        if (created[t])
            pthread_join(tid[t], NULL);
        else
            worker(&jobs[t]);      /* no thread: evaluate its rows here */
    }
    int status = 0;
    for (int t = 0; t < n_threads; ++t)
        if (jobs[t].status && !status)
            status = jobs[t].status;
    free(created);
    free(jobs);
    free(tid);
    return status;
}

/*
 * One decode step of the per-beam state: BeamKV append and BeamPath update.
 *
 * Data model (GR-Inference blog, section on system design: BeamKV holds the
 * short per-beam history and BeamPath records how beams fork and reorder by
 * index, so the long context is never copied; SID-GR README, "Design
 * Highlights": BeamPath keeps the logical parent-child relation; xGR review,
 * section "xAttention": the unshared cache is managed per token and reached
 * by direct index, with no block copies).
 *
 * Request b had W_old = row_offset_old[b+1] - row_offset_old[b] beams whose
 * paths hold s = beam_len_old[b] tokens.  Beam selection gave it W_new =
 * row_offset_new[b+1] - row_offset_new[b] new beams; new beam k (packed row
 * r = row_offset_new[b] + k) descends from old beam parent[r] and its current
 * token is step s.  Then
 *   path_new[r][t]            = path_old[row_offset_old[b] + parent[r]][t],  t < s
 *   path_new[r][s]            = s * W_cap + k          (its own step-s slot)
 *   beam_k[b][s*W_cap + k][:] = new_k[r][:]            (all KV heads; same for V)
 *   beam_len_new[b]           = s + 1  if W_new > 0, else s
 * Path entries t > s of path_new and every other BeamKV slot are left as
 * they are.  The paths are rebuilt into a second table (path_new must not
 * be path_old): each new row reads only its parent's old row, so the update
 * has no read-before-write order to respect.
 *
 * A row whose slot or parent is out of range (s >= T_cap, k >= W_cap,
 * s*W_cap + k >= beam_cap, or s > 0 with parent outside [0, W_old)) writes
 * nothing; the return value counts such rows (>= 0), or is -1 on bad
 * arguments.  Plain loops; the data are copied as raw bits.
 */
int oracle_beam_step(int B, int Hkv, int D, int T_cap, int W_cap, int64_t beam_cap,
                     const int32_t *row_offset_old, const int32_t *row_offset_new,
                     const int32_t *parent, const int32_t *path_old,
                     const int32_t *beam_len_old, const uint16_t *new_k,
                     const uint16_t *new_v, int32_t *path_new, int32_t *beam_len_new,
                     uint16_t *beam_k, uint16_t *beam_v)
{
    if (B < 0 || Hkv <= 0 || D <= 0 || T_cap < 0 || W_cap < 0 || beam_cap < 0 ||
        !row_offset_old || !row_offset_new || !beam_len_old || !beam_len_new)
        return -1;
    const int64_t row_elems = (int64_t)Hkv * D;      /* one token, all KV heads */
    int skipped = 0;
    for (int b = 0; b < B; ++b) {
        const int s = beam_len_old[b];
        const int w_old = row_offset_old[b + 1] - row_offset_old[b];
        const int w_new = row_offset_new[b + 1] - row_offset_new[b];
        for (int k = 0; k < w_new; ++k) {
            const int r = row_offset_new[b] + k;
            const int64_t slot = (int64_t)s * W_cap + k;
            const int p = s > 0 ? parent[r] : 0;
            if (s < 0 || s >= T_cap || k >= W_cap || slot >= beam_cap ||
                (s > 0 && (p < 0 || p >= w_old))) {
                ++skipped;
                continue;
            }
            for (int t = 0; t < s; ++t)
                path_new[(int64_t)r * T_cap + t] =
                    path_old[(int64_t)(row_offset_old[b] + p) * T_cap + t];
            path_new[(int64_t)r * T_cap + s] = (int32_t)slot;
            for (int64_t e = 0; e < row_elems; ++e) {
                beam_k[((int64_t)b * beam_cap + slot) * row_elems + e] = new_k[(int64_t)r * row_elems + e];
                beam_v[((int64_t)b * beam_cap + slot) * row_elems + e] = new_v[(int64_t)r * row_elems + e];
            }
        }
        beam_len_new[b] = w_new > 0 ? s + 1 : s;
    }
    return skipped;
}
