/*
 * sse_oracle.c -- plain sequential fp64 reference for the Sparse State
 * Expansion (SSE) layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the HIP library and must never be used as a
 * fallback for it.
 *
 * Source of the method: the web page "Scaling Linear Attention with Sparse
 * State Expansion: 中文研读笔记" (study notes on arXiv 2507.16577v2).  Every
 * citation below names a section or equation of that page.
 *
 *   §2.3, eqs. (9)-(14): per token and head,
 *       e_t  = softmax over the N partitions of the router logits
 *       T_t  = indices of the k largest entries
 *       k_t  = softmax over the c key rows of the key logits
 *       S^i  = Lambda_t S^i + e^i k_t^T v_t   for i in T_t,
 *       S^i unchanged (no decay, no write)    for i not in T_t,
 *       o_t  = sum over i in T_t of e^i q_t S^i   (state read after the write)
 *   §2.1, eq. (6): the transition used by SSE is GLA-style, Lambda_t =
 *       diag(alpha_t), alpha_t in (0,1]^c scaling the c state rows.
 *   §2.3 (text under the equations): no renormalisation of e over T_t; the
 *       same e^i gates the write and the read.
 *   §2.5: one extra, always-selected shared partition, here with the same
 *       q, k, alpha and weight 1 on both write and read.
 *   §2.6 (closing paragraph): unselected partitions keep an identity
 *       transition; partition outputs are summed back per token.
 *
 * Readings taken where the page is silent (each is also listed in the design
 * notes of the repository):
 *   - top-k order is descending by logit, equal logits -> lower index first;
 *     the selection compares the logits themselves (softmax is monotone);
 *   - log_alpha is given per (token, head, row): alpha = exp(log_alpha);
 *   - no query scaling, no output normalisation;
 *   - states start at zero per sequence unless initial states are given.
 *
 * Precision: inputs arrive as fp32 or bf16 bit patterns and are converted to
 * fp64 exactly; everything after that is fp64.
 *
 * parity pins: see the tests (brute-force quadratic form, single-state GLA
 * reduction, identity of unselected states, the page's decay example, the
 * closed form of Appendix A Prop. 4 as summarised in §2.7, masked linear
 * attention at alpha = 1).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_MAX_N 256

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

/* Exact conversion of one stored input element to fp64. */
static double load_value(const void *base, int dtype, int64_t i)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Softmax over n values (max-subtracted). */
static void softmax(const double *x, int n, double *out)
{
    double m = x[0];
    for (int i = 1; i < n; i++)
        if (x[i] > m)
            m = x[i];
    double s = 0.0;
    for (int i = 0; i < n; i++) {
        out[i] = exp(x[i] - m);
        s += out[i];
    }
    for (int i = 0; i < n; i++)
        out[i] /= s;
}

/* TopKIndices of eq. (10): the k largest logits, descending; equal logits ->
 * lower index first (scan ascending, replace only on strictly greater). */
static void top_k(const double *z, int n, int k, int *sel)
{
    unsigned char taken[ORACLE_MAX_N];
    memset(taken, 0, sizeof taken);
    for (int r = 0; r < k; r++) {
        int best = -1;
        for (int i = 0; i < n; i++)
            if (!taken[i] && (best < 0 || z[i] > z[best]))
                best = i;
        taken[best] = 1;
        sel[r] = best;
    }
}

/*
 * One token of the recurrence for one head.
 *   z[N], q[c], kl[c], la[c], v[d]: this token's inputs (fp64)
 *   S: (N+1) states of c x d, row-major, partition N is the shared one
 *   o[d]: output; sel[k], esel[k]: chosen partitions and their router weights
 *   work: scratch of at least N + 2c doubles
 */
static void sse_token(int N, int k, int c, int d, const double *z, const double *q,
                      const double *kl, const double *la, const double *v, double *S,
                      double *o, int *sel, double *esel, double *work)
{
    double *e = work;           /* [N] router probabilities, eq. (9)       */
    double *kappa = work + N;   /* [c] softmax key, eq. (11)                */
    double *alpha = kappa + c;  /* [c] diagonal of Lambda_t, eq. (6)        */
    const int64_t cd = (int64_t)c * d;

    softmax(z, N, e);
    top_k(z, N, k, sel);
    softmax(kl, c, kappa);
    for (int j = 0; j < c; j++)
        alpha[j] = exp(la[j]);
    for (int m = 0; m < d; m++)
        o[m] = 0.0;

    /* k selected partitions (weight e^i on write and read) followed by the
     * shared partition (weight 1 on write and read). */
    for (int r = 0; r <= k; r++) {
        int part = (r < k) ? sel[r] : N;
        double w = (r < k) ? e[part] : 1.0;
        if (r < k)
            esel[r] = w;
        double *Sp = S + (int64_t)part * cd;
        /* eq. (12): S = diag(alpha) S + w k^T v */
        for (int j = 0; j < c; j++)
            for (int m = 0; m < d; m++)
                Sp[(int64_t)j * d + m] = alpha[j] * Sp[(int64_t)j * d + m] + w * kappa[j] * v[m];
        /* eq. (14): o += w q S (read after the write) */
        for (int m = 0; m < d; m++) {
            double acc = 0.0;
            for (int j = 0; j < c; j++)
                acc += q[j] * Sp[(int64_t)j * d + m];
            o[m] += w * acc;
        }
    }
}

/*
 * Run one (sequence, head) unit over tokens [t0, t1) of token-major inputs
 *   q, key_logits, log_alpha: [T_tot, H, c];  v: [T_tot, H, d];
 *   router_logits: [T_tot, H, N]
 * stored as fp32 or bf16 (dtype).
 *   S: [(N+1), c, d] fp64, in = initial state, out = final state
 *   o: [(t1-t0), d]; sel: [(t1-t0), k]; esel: [(t1-t0), k]
 * Returns 0, or -1 on bad arguments.
 */
int sse_oracle_unit(int dtype, const void *q, const void *key_logits, const void *v,
                    const void *log_alpha, const void *router_logits, int64_t t0, int64_t t1,
                    int h, int H, int c, int d, int N, int k, double *S, double *o,
                    int32_t *sel, double *esel)
{
    if (N < 1 || N > ORACLE_MAX_N || k < 1 || k > N || c < 1 || d < 1 || h < 0 || h >= H ||
        t1 < t0)
        return -1;
    double *buf = (double *)malloc(sizeof(double) * (size_t)(N + 3 * c + d + N + 2 * c));
    if (!buf)
        return -1;
    double *z = buf, *qq = z + N, *kk = qq + c, *ll = kk + c, *vv = ll + c, *work = vv + d;
    int selr[ORACLE_MAX_N];
    for (int64_t t = t0; t < t1; t++) {
        int64_t rc = (t * H + h) * (int64_t)c, rd = (t * H + h) * (int64_t)d,
                rn = (t * H + h) * (int64_t)N;
        for (int i = 0; i < N; i++)
            z[i] = load_value(router_logits, dtype, rn + i);
        for (int j = 0; j < c; j++) {
            qq[j] = load_value(q, dtype, rc + j);
            kk[j] = load_value(key_logits, dtype, rc + j);
            ll[j] = load_value(log_alpha, dtype, rc + j);
        }
        for (int m = 0; m < d; m++)
            vv[m] = load_value(v, dtype, rd + m);
        int64_t lt = t - t0;
        sse_token(N, k, c, d, z, qq, kk, ll, vv, S, o + lt * d, selr, esel + lt * k, work);
        for (int r = 0; r < k; r++)
            sel[lt * k + r] = selr[r];
    }
    free(buf);
    return 0;
}

/*
 * Whole varlen forward: sequences s = 0..num_seqs-1 occupy tokens
 * [cu_seqlens[s], cu_seqlens[s+1]).  Units (s, h) are independent and are
 * spread over n_threads threads (timing convenience only; each unit is
 * computed sequentially).
 *   init: [S, H, N+1, c, d] fp64 or NULL (zeros)
 *   o: [T_tot, H, d]; final_states: [S, H, N+1, c, d]
 *   topk_idx, topk_e: [T_tot, H, k]
 */
struct fwd_job {
    int dtype;
    const void *q, *kl, *v, *la, *z;
    const int32_t *cu;
    int num_seqs, H, c, d, N, k;
    const double *init;
    double *o, *fs, *e;
    int32_t *idx;
    int next_unit; /* shared counter, protected by mu */
    pthread_mutex_t mu;
    int status;
};

static void *fwd_worker(void *arg)
{
    struct fwd_job *J = (struct fwd_job *)arg;
    const int64_t cd = (int64_t)J->c * J->d, st = (int64_t)(J->N + 1) * cd;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int u = J->next_unit++;
        pthread_mutex_unlock(&J->mu);
        if (u >= J->num_seqs * J->H)
            break;
        int s = u / J->H, h = u % J->H;
        int64_t t0 = J->cu[s], t1 = J->cu[s + 1], L = t1 - t0;
        double *S = J->fs + (int64_t)u * st;
        if (J->init)
            memcpy(S, J->init + (int64_t)u * st, sizeof(double) * (size_t)st);
        else
            memset(S, 0, sizeof(double) * (size_t)st);
        double *o = (double *)malloc(sizeof(double) * (size_t)(L * J->d + 1));
        double *e = (double *)malloc(sizeof(double) * (size_t)(L * J->k + 1));
        int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(L * J->k + 1));
        int rc = (o && e && idx) ? sse_oracle_unit(J->dtype, J->q, J->kl, J->v, J->la, J->z, t0,
                                                   t1, h, J->H, J->c, J->d, J->N, J->k, S, o,
                                                   idx, e)
                                 : -1;
        if (rc == 0) {
            for (int64_t t = 0; t < L; t++) {
                int64_t g = (t0 + t) * J->H + h;
                memcpy(J->o + g * J->d, o + t * J->d, sizeof(double) * (size_t)J->d);
                memcpy(J->e + g * J->k, e + t * J->k, sizeof(double) * (size_t)J->k);
                memcpy(J->idx + g * J->k, idx + t * J->k, sizeof(int32_t) * (size_t)J->k);
            }
        } else {
            J->status = -1;
        }
        free(o);
        free(e);
        free(idx);
    }
    return NULL;
}

int sse_oracle_forward(int dtype, const void *q, const void *key_logits, const void *v,
                       const void *log_alpha, const void *router_logits,
                       const int32_t *cu_seqlens, int num_seqs, int H, int c, int d, int N,
                       int k, const double *init_states, double *o, double *final_states,
                       int32_t *topk_idx, double *topk_e, int n_threads)
{
    if (num_seqs < 0 || H < 1 || n_threads < 1)
        return -1;
    for (int s = 0; s < num_seqs; s++)
        if (cu_seqlens[s + 1] < cu_seqlens[s])
            return -1;
    struct fwd_job J;
    memset(&J, 0, sizeof J);
    J.dtype = dtype;
    J.q = q;
    J.kl = key_logits;
    J.v = v;
    J.la = log_alpha;
    J.z = router_logits;
    J.cu = cu_seqlens;
    J.num_seqs = num_seqs;
    J.H = H;
    J.c = c;
    J.d = d;
    J.N = N;
    J.k = k;
    J.init = init_states;
    J.o = o;
    J.fs = final_states;
    J.e = topk_e;
    J.idx = topk_idx;
    pthread_mutex_init(&J.mu, NULL);
    if (n_threads == 1) {
        fwd_worker(&J);
    } else {
        pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
        int started = 0;
        for (int i = 0; i < n_threads; i++)
            if (pthread_create(&th[i], NULL, fwd_worker, &J) == 0)
                started++;
            else
                break;
        if (started == 0)
            fwd_worker(&J);
        for (int i = 0; i < started; i++)
            pthread_join(th[i], NULL);
        free(th);
    }
    pthread_mutex_destroy(&J.mu);
    return J.status;
}

/*
 * One decode step (§2.6: decode recurs only on the selected states) for B
 * independent sequences x H heads, one token each.
 *   inputs: q, key_logits, log_alpha [B, H, c]; v [B, H, d]; router [B, H, N]
 *   states: [B, H, N+1, c, d] fp64, updated in place
 *   o: [B, H, d]; topk_idx, topk_e: [B, H, k]
 * It is the forward of a length-1 sequence per (b, h).
 */
int sse_oracle_decode_step(int dtype, const void *q, const void *key_logits, const void *v,
                           const void *log_alpha, const void *router_logits, int B, int H, int c,
                           int d, int N, int k, double *states, double *o, int32_t *topk_idx,
                           double *topk_e)
{
    const int64_t st = (int64_t)(N + 1) * c * d;
    for (int b = 0; b < B; b++)
        for (int h = 0; h < H; h++) {
            int64_t u = (int64_t)b * H + h;
            /* token b of a [B, H, .] array is row b of a token-major array */
            int rc = sse_oracle_unit(dtype, q, key_logits, v, log_alpha, router_logits, b, b + 1,
                                     h, H, c, d, N, k, states + u * st, o + u * d,
                                     topk_idx + u * k, topk_e + u * k);
            if (rc)
                return rc;
        }
    return 0;
}

/*
 * Varlen grouping (§2.6, varlen paragraph): records (token, slot) are
 * gathered per (sequence, head, partition) segment in time order.  Segment
 * id g = (s*H + h)*N + i.
 *   topk_idx: [T_tot, H, k]
 *   seg_offsets: [num_seqs*H*N + 1]; seg_tok, seg_slot: [T_tot*H*k]
 * Plain definition: for every segment in id order, scan its sequence in time
 * order and append every (t, j) whose j-th choice is the segment's partition.
 */
int sse_oracle_group(const int32_t *topk_idx, const int32_t *cu_seqlens, int num_seqs, int H,
                     int N, int k, int32_t *seg_offsets, int32_t *seg_tok, int32_t *seg_slot)
{
    int64_t pos = 0;
    for (int s = 0; s < num_seqs; s++)
        for (int h = 0; h < H; h++)
            for (int i = 0; i < N; i++) {
                seg_offsets[((int64_t)s * H + h) * N + i] = (int32_t)pos;
                for (int64_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; t++)
                    for (int j = 0; j < k; j++)
                        if (topk_idx[(t * H + h) * k + j] == i) {
                            seg_tok[pos] = (int32_t)t;
                            seg_slot[pos] = j;
                            pos++;
                        }
            }
    seg_offsets[(int64_t)num_seqs * H * N] = (int32_t)pos;
    return 0;
}

/*
 * Row-sparse key variant (§2.2, eqs. (7)-(8)): one state per head.  The key
 * keeps the k largest of the c key logits (descending, equal logits -> lower
 * row first) and is the softmax over those rows, zero on the others:
 *     kappa_j = exp(kl_j) / sum_{i in top} exp(kl_i)   (j in top), 0 otherwise.
 * The update is S = Lambda~ S + kappa^T v with Lambda~ = diag(alpha) on the
 * selected rows and, when identity_unselected is set, the identity on the
 * other rows (the "no forgetting of unselected rows" form the page says
 * needs an identity transition; otherwise every row decays, the plain
 * zeroed-key form).  o = q S, read after the write.
 *   S: [c, d] fp64, in = initial state, out = final state; o: [(t1-t0), d]
 */
int sse_oracle_rowsparse_unit(int dtype, const void *q, const void *key_logits, const void *v,
                              const void *log_alpha, int64_t t0, int64_t t1, int h, int H, int c,
                              int d, int k, int identity_unselected, double *S, double *o)
{
    if (k < 1 || k > c || c < 1 || d < 1 || h < 0 || h >= H || t1 < t0 || c > ORACLE_MAX_N)
        return -1;
    double qq[ORACLE_MAX_N], kk[ORACLE_MAX_N], ll[ORACLE_MAX_N], kappa[ORACLE_MAX_N];
    int top[ORACLE_MAX_N];
    unsigned char sel[ORACLE_MAX_N];
    double *vv = (double *)malloc(sizeof(double) * (size_t)d);
    if (!vv)
        return -1;
    for (int64_t t = t0; t < t1; t++) {
        int64_t rc = (t * H + h) * (int64_t)c, rd = (t * H + h) * (int64_t)d;
        for (int j = 0; j < c; j++) {
            qq[j] = load_value(q, dtype, rc + j);
            kk[j] = load_value(key_logits, dtype, rc + j);
            ll[j] = load_value(log_alpha, dtype, rc + j);
        }
        for (int m = 0; m < d; m++)
            vv[m] = load_value(v, dtype, rd + m);
        /* eq. (7): top-k of the key logits, then the softmax over them */
        top_k(kk, c, k, top);
        memset(sel, 0, sizeof sel);
        for (int r = 0; r < k; r++)
            sel[top[r]] = 1;
        double mx = kk[top[0]], z = 0.0;
        for (int r = 0; r < k; r++)
            z += exp(kk[top[r]] - mx);
        for (int j = 0; j < c; j++)
            kappa[j] = sel[j] ? exp(kk[j] - mx) / z : 0.0;
        /* eq. (8) with the transition of the selected rows only */
        for (int j = 0; j < c; j++) {
            double a = (sel[j] || !identity_unselected) ? exp(ll[j]) : 1.0;
            for (int m = 0; m < d; m++)
                S[(int64_t)j * d + m] = a * S[(int64_t)j * d + m] + kappa[j] * vv[m];
        }
        for (int m = 0; m < d; m++) {
            double acc = 0.0;
            for (int j = 0; j < c; j++)
                acc += qq[j] * S[(int64_t)j * d + m];
            o[(t - t0) * d + m] = acc;
        }
    }
    free(vv);
    return 0;
}

/* Varlen row-sparse forward over sequences [cu[s], cu[s+1]), every head.
 *   init: [S, H, c, d] or NULL (zeros); o: [T_tot, H, d]; fs: [S, H, c, d] */
int sse_oracle_rowsparse_forward(int dtype, const void *q, const void *key_logits, const void *v,
                                 const void *log_alpha, const int32_t *cu_seqlens, int num_seqs,
                                 int H, int c, int d, int k, int identity_unselected,
                                 const double *init, double *o, double *final_states)
{
    const int64_t cd = (int64_t)c * d;
    for (int s = 0; s < num_seqs; s++) {
        if (cu_seqlens[s + 1] < cu_seqlens[s])
            return -1;
        int64_t t0 = cu_seqlens[s], t1 = cu_seqlens[s + 1], L = t1 - t0;
        double *ou = (double *)malloc(sizeof(double) * (size_t)(L * d + 1));
        if (!ou)
            return -1;
        for (int h = 0; h < H; h++) {
            double *S = final_states + ((int64_t)s * H + h) * cd;
            if (init)
                memcpy(S, init + ((int64_t)s * H + h) * cd, sizeof(double) * (size_t)cd);
            else
                memset(S, 0, sizeof(double) * (size_t)cd);
            int rc = sse_oracle_rowsparse_unit(dtype, q, key_logits, v, log_alpha, t0, t1, h, H,
                                               c, d, k, identity_unselected, S, ou);
            if (rc) {
                free(ou);
                return rc;
            }
            for (int64_t t = 0; t < L; t++)
                memcpy(o + ((t0 + t) * H + h) * d, ou + t * d, sizeof(double) * (size_t)d);
        }
        free(ou);
    }
    return 0;
}

/*
 * General form (§2.5 and §2.3): the shared partition may have its own query
 * and key (the page gives it rank-64 LoRA projections of its own Q and K;
 * the projected rows are inputs here), and the partitions read may differ
 * from those written ("读写集合可以不同,默认相同": the read and write sets may
 * differ, the same by default).  Per token:
 *   write set W = top-k of the router logits z, weights e = softmax(z);
 *   read set  R = top-kr of the read logits zr, weights er = softmax(zr)
 *             (R = W and er = e when no read logits are given);
 *   for i in W: S^i = diag(alpha) S^i + e^i kappa^T v;  others unchanged;
 *   S^sh = diag(alpha) S^sh + kappa_sh^T v, kappa_sh = softmax(kl_sh);
 *   o = sum_{i in R} er^i q S^i + q_sh S^sh  (every read after the writes).
 * Reads of a partition not written at this token see its unchanged state.
 * Inputs of the optional pieces may be NULL: q_sh -> q, kl_sh -> kl,
 * zr -> none (kr ignored).  Outputs: o [(t1-t0), d]; wsel, rsel [(t1-t0), k]
 * and [(t1-t0), kr].
 */
int sse_oracle_unit_ex(int dtype, const void *q, const void *key_logits, const void *v,
                       const void *log_alpha, const void *router_logits, const void *q_sh,
                       const void *key_logits_sh, const void *read_logits, int kr, int64_t t0,
                       int64_t t1, int h, int H, int c, int d, int N, int k, double *S, double *o,
                       int32_t *wsel, int32_t *rsel)
{
    if (N < 1 || N > ORACLE_MAX_N || k < 1 || k > N || c < 1 || d < 1 || c > ORACLE_MAX_N ||
        h < 0 || h >= H || t1 < t0)
        return -1;
    if (read_logits && (kr < 1 || kr > N))
        return -1;
    const int krr = read_logits ? kr : k;
    const int64_t cd = (int64_t)c * d;
    double z[ORACLE_MAX_N], zr[ORACLE_MAX_N], e[ORACLE_MAX_N], er[ORACLE_MAX_N];
    double qq[ORACLE_MAX_N], qs[ORACLE_MAX_N], kk[ORACLE_MAX_N], ks[ORACLE_MAX_N];
    double ll[ORACLE_MAX_N], kap[ORACLE_MAX_N], kaps[ORACLE_MAX_N], alpha[ORACLE_MAX_N];
    int W[ORACLE_MAX_N], R[ORACLE_MAX_N];
    double *vv = (double *)malloc(sizeof(double) * (size_t)d);
    if (!vv)
        return -1;
    for (int64_t t = t0; t < t1; t++) {
        int64_t rc = (t * H + h) * (int64_t)c, rd = (t * H + h) * (int64_t)d,
                rn = (t * H + h) * (int64_t)N;
        for (int i = 0; i < N; i++) {
            z[i] = load_value(router_logits, dtype, rn + i);
            zr[i] = read_logits ? load_value(read_logits, dtype, rn + i) : z[i];
        }
        for (int j = 0; j < c; j++) {
            qq[j] = load_value(q, dtype, rc + j);
            qs[j] = q_sh ? load_value(q_sh, dtype, rc + j) : qq[j];
            kk[j] = load_value(key_logits, dtype, rc + j);
            ks[j] = key_logits_sh ? load_value(key_logits_sh, dtype, rc + j) : kk[j];
            ll[j] = load_value(log_alpha, dtype, rc + j);
        }
        for (int m = 0; m < d; m++)
            vv[m] = load_value(v, dtype, rd + m);
        softmax(z, N, e);                 /* eq. (9), write weights */
        top_k(z, N, k, W);                /* eq. (10), write set */
        softmax(zr, N, er);               /* read weights */
        top_k(zr, N, krr, R);             /* read set */
        softmax(kk, c, kap);              /* eq. (11) */
        softmax(ks, c, kaps);             /* the shared partition's own key */
        for (int j = 0; j < c; j++)
            alpha[j] = exp(ll[j]);
        /* writes: eq. (12) on the write set, the shared partition always */
        for (int r = 0; r < k + 1; r++) {
            const int part = (r < k) ? W[r] : N;
            const double ww = (r < k) ? e[part] : 1.0;
            const double *key = (r < k) ? kap : kaps;
            double *Sw = S + (int64_t)part * cd;
            for (int j = 0; j < c; j++)
                for (int m = 0; m < d; m++)
                    Sw[(int64_t)j * d + m] = alpha[j] * Sw[(int64_t)j * d + m] + ww * key[j] * vv[m];
        }
        /* reads: eq. (14) on the read set, plus the shared partition */
        int64_t lt = t - t0;
        for (int m = 0; m < d; m++)
            o[lt * d + m] = 0.0;
        for (int r = 0; r <= krr; r++) {
            int part = (r < krr) ? R[r] : N;
            double w = (r < krr) ? er[part] : 1.0;
            const double *qv = (r < krr) ? qq : qs;
            const double *Sp = S + (int64_t)part * cd;
            for (int m = 0; m < d; m++) {
                double acc = 0.0;
                for (int j = 0; j < c; j++)
                    acc += qv[j] * Sp[(int64_t)j * d + m];
                o[lt * d + m] += w * acc;
            }
        }
        for (int r = 0; r < k; r++)
            wsel[lt * k + r] = W[r];
        for (int r = 0; r < krr; r++)
            rsel[lt * krr + r] = R[r];
    }
    free(vv);
    return 0;
}

/* Varlen forward of the general form, sequence by sequence and head by
 * head.  init [S,H,N+1,c,d] or NULL; o [T,H,d]; fs [S,H,N+1,c,d];
 * wsel [T,H,k]; rsel [T,H,kr'] with kr' = kr (read logits given) or k. */
int sse_oracle_forward_ex(int dtype, const void *q, const void *key_logits, const void *v,
                          const void *log_alpha, const void *router_logits, const void *q_sh,
                          const void *key_logits_sh, const void *read_logits, int kr,
                          const int32_t *cu_seqlens, int num_seqs, int H, int c, int d, int N,
                          int k, const double *init, double *o, double *final_states,
                          int32_t *wsel, int32_t *rsel)
{
    const int64_t st = (int64_t)(N + 1) * c * d;
    const int krr = read_logits ? kr : k;
    for (int s = 0; s < num_seqs; s++) {
        if (cu_seqlens[s + 1] < cu_seqlens[s])
            return -1;
        int64_t t0 = cu_seqlens[s], t1 = cu_seqlens[s + 1], L = t1 - t0;
        double *ou = (double *)malloc(sizeof(double) * (size_t)(L * d + 1));
        int32_t *wu = (int32_t *)malloc(sizeof(int32_t) * (size_t)(L * k + 1));
        int32_t *ru = (int32_t *)malloc(sizeof(int32_t) * (size_t)(L * krr + 1));
        if (!ou || !wu || !ru) {
            free(ou);
            free(wu);
            free(ru);
            return -1;
        }
        for (int h = 0; h < H; h++) {
            double *Su = final_states + ((int64_t)s * H + h) * st;
            if (init)
                memcpy(Su, init + ((int64_t)s * H + h) * st, sizeof(double) * (size_t)st);
            else
                memset(Su, 0, sizeof(double) * (size_t)st);
            int rc = sse_oracle_unit_ex(dtype, q, key_logits, v, log_alpha, router_logits, q_sh,
                                        key_logits_sh, read_logits, kr, t0, t1, h, H, c, d, N, k,
                                        Su, ou, wu, ru);
            if (rc) {
                free(ou);
                free(wu);
                free(ru);
                return rc;
            }
            for (int64_t t = 0; t < L; t++) {
                int64_t g = (t0 + t) * H + h;
                memcpy(o + g * d, ou + t * d, sizeof(double) * (size_t)d);
                memcpy(wsel + g * k, wu + t * k, sizeof(int32_t) * (size_t)k);
                memcpy(rsel + g * krr, ru + t * krr, sizeof(int32_t) * (size_t)krr);
            }
        }
        free(ou);
        free(wu);
        free(ru);
    }
    return 0;
}

/*
 * Gradients of the forward (reverse mode over the definition above; the
 * page's §2.3 notes that the same e on write and read gives the router a
 * continuous gradient, while the discrete top-k indices carry none).  For
 * one (sequence, head) unit over tokens [t0, t1), with L = <do, o> +
 * <dS_final, S_final> as the scalar whose gradient is taken:
 *   forward: at each token, for every touched partition p (the k selected
 *     ones with w = e^p, then the shared one with w = 1) keep S_p before the
 *     write, write S_p = diag(alpha) S_p + w kappa^T v and keep y_p = q S_p;
 *   reverse: adjoints A_p start at dS_final[p]; for t = t1-1 .. t0 and each
 *     touched p (A_p is dL/dS_p after the write of token t):
 *       A_p += w q^T do_t                     (the read w q S_p)
 *       dq  += w S_p do_t                     (S_p after the write)
 *       dw  += y_p . do_t + kappa . (A_p v)   (read gate + write gate)
 *       dkappa += w A_p v;  dv += w kappa A_p
 *       dlog_alpha_j += alpha_j sum_m A_p[j,m] S_p_before[j,m]
 *       A_p = diag(alpha) A_p                 (dL/dS_p before the write)
 *     partitions not touched at t keep their adjoint (identity transition);
 *     dkey_logits = kappa * (dkappa - kappa . dkappa)  (softmax, eq. 11);
 *     drouter = e * (de - e . de), de_i = dw of selected partition i, 0
 *     otherwise (softmax over N, eq. 9).
 *   dS_init[p] = A_p at the end.
 * Buffers: S [N+1, c, d] in = initial state (consumed); dS [N+1, c, d] in =
 * dS_final or NULL (zeros), out = dS_init; do_ [(t1-t0), d]; outputs dq,
 * dkl, dla [(t1-t0), c], dv [(t1-t0), d], dz [(t1-t0), N].
 */
int sse_oracle_backward_unit(int dtype, const void *q, const void *key_logits, const void *v,
                             const void *log_alpha, const void *router_logits, int64_t t0,
                             int64_t t1, int h, int H, int c, int d, int N, int k, double *S,
                             const double *do_, double *dS, double *dq, double *dkl, double *dv,
                             double *dla, double *dz)
{
    if (N < 1 || N > ORACLE_MAX_N || k < 1 || k > N || c < 1 || d < 1 || c > ORACLE_MAX_N ||
        h < 0 || h >= H || t1 < t0)
        return -1;
    const int64_t L = t1 - t0, cd = (int64_t)c * d, np = k + 1;
    double *saved = (double *)malloc(sizeof(double) * (size_t)(L * np * cd + 1));
    double *ys = (double *)malloc(sizeof(double) * (size_t)(L * np * d + 1));
    double *vv = (double *)malloc(sizeof(double) * (size_t)(d + 1));
    int *selall = (int *)malloc(sizeof(int) * (size_t)(L * k + 1));
    if (!saved || !ys || !vv || !selall) {
        free(saved);
        free(ys);
        free(vv);
        free(selall);
        return -1;
    }
    double z[ORACLE_MAX_N], e[ORACLE_MAX_N], qq[ORACLE_MAX_N], kk[ORACLE_MAX_N],
        ll[ORACLE_MAX_N], kap[ORACLE_MAX_N], alpha[ORACLE_MAX_N], dkap[ORACLE_MAX_N],
        de[ORACLE_MAX_N];
    /* load one token's inputs, router and key */
#define LOAD_TOKEN(t)                                                                     \
    do {                                                                                  \
        int64_t rc_ = ((t)*H + h) * (int64_t)c, rd_ = ((t)*H + h) * (int64_t)d,           \
                rn_ = ((t)*H + h) * (int64_t)N;                                           \
        for (int i_ = 0; i_ < N; i_++)                                                    \
            z[i_] = load_value(router_logits, dtype, rn_ + i_);                           \
        for (int j_ = 0; j_ < c; j_++) {                                                  \
            qq[j_] = load_value(q, dtype, rc_ + j_);                                      \
            kk[j_] = load_value(key_logits, dtype, rc_ + j_);                             \
            ll[j_] = load_value(log_alpha, dtype, rc_ + j_);                              \
        }                                                                                 \
        for (int m_ = 0; m_ < d; m_++)                                                    \
            vv[m_] = load_value(v, dtype, rd_ + m_);                                      \
        softmax(z, N, e);                                                                 \
        softmax(kk, c, kap);                                                              \
        for (int j_ = 0; j_ < c; j_++)                                                    \
            alpha[j_] = exp(ll[j_]);                                                      \
    } while (0)

    /* forward, keeping the states before each write and the reads */
    for (int64_t t = t0; t < t1; t++) {
        const int64_t lt = t - t0;
        LOAD_TOKEN(t);
        int *sel = selall + lt * k;
        top_k(z, N, k, sel);
        for (int r = 0; r < np; r++) {
            const int p = (r < k) ? sel[r] : N;
            const double w = (r < k) ? e[p] : 1.0;
            double *St = S + (int64_t)p * cd;
            memcpy(saved + (lt * np + r) * cd, St, sizeof(double) * (size_t)cd);
            for (int j = 0; j < c; j++)
                for (int m = 0; m < d; m++)
                    St[(int64_t)j * d + m] = alpha[j] * St[(int64_t)j * d + m] + w * kap[j] * vv[m];
            double *y = ys + (lt * np + r) * d;
            for (int m = 0; m < d; m++) {
                double acc = 0.0;
                for (int j = 0; j < c; j++)
                    acc += qq[j] * St[(int64_t)j * d + m];
                y[m] = acc;
            }
        }
    }
    /* reverse */
    for (int64_t t = t1 - 1; t >= t0; t--) {
        const int64_t lt = t - t0;
        LOAD_TOKEN(t);
        const int *sel = selall + lt * k;
        const double *dot = do_ + lt * d;
        double *gq = dq + lt * c, *gk = dkl + lt * c, *gv = dv + lt * d, *gl = dla + lt * c;
        for (int j = 0; j < c; j++)
            gq[j] = gl[j] = dkap[j] = 0.0;
        for (int m = 0; m < d; m++)
            gv[m] = 0.0;
        for (int i = 0; i < N; i++)
            de[i] = 0.0;
        for (int r = 0; r < np; r++) {
            const int p = (r < k) ? sel[r] : N;
            const double w = (r < k) ? e[p] : 1.0;
            double *Ap = dS + (int64_t)p * cd;
            const double *Sb = saved + (lt * np + r) * cd;
            const double *y = ys + (lt * np + r) * d;
            /* the read: A += w q^T do */
            for (int j = 0; j < c; j++)
                for (int m = 0; m < d; m++)
                    Ap[(int64_t)j * d + m] += w * qq[j] * dot[m];
            double dw = 0.0;
            for (int m = 0; m < d; m++)
                dw += y[m] * dot[m];
            for (int j = 0; j < c; j++) {
                double sdo = 0.0, av = 0.0, as = 0.0;
                for (int m = 0; m < d; m++) {
                    const double snew = alpha[j] * Sb[(int64_t)j * d + m] + w * kap[j] * vv[m];
                    sdo += snew * dot[m];
                    av += Ap[(int64_t)j * d + m] * vv[m];
                    as += Ap[(int64_t)j * d + m] * Sb[(int64_t)j * d + m];
                }
                gq[j] += w * sdo;
                dkap[j] += w * av;
                dw += kap[j] * av;
                gl[j] += alpha[j] * as;
            }
            for (int m = 0; m < d; m++) {
                double ka = 0.0;
                for (int j = 0; j < c; j++)
                    ka += kap[j] * Ap[(int64_t)j * d + m];
                gv[m] += w * ka;
            }
            for (int j = 0; j < c; j++)
                for (int m = 0; m < d; m++)
                    Ap[(int64_t)j * d + m] *= alpha[j];
            if (r < k)
                de[p] = dw;
        }
        double kd = 0.0, ed = 0.0;
        for (int j = 0; j < c; j++)
            kd += kap[j] * dkap[j];
        for (int j = 0; j < c; j++)
            gk[j] = kap[j] * (dkap[j] - kd);
        for (int i = 0; i < N; i++)
            ed += e[i] * de[i];
        for (int i = 0; i < N; i++)
            dz[lt * N + i] = e[i] * (de[i] - ed);
    }
#undef LOAD_TOKEN
    free(saved);
    free(ys);
    free(vv);
    free(selall);
    return 0;
}

/* Varlen backward, (sequence, head) units over n_threads threads.
 *   init, dfinal: [S, H, N+1, c, d] or NULL (zeros); do_: [T, H, d]
 *   dq, dkl, dla: [T, H, c]; dv: [T, H, d]; dz: [T, H, N]; dinit: [S,H,N+1,c,d] */
struct bwd_job {
    int dtype;
    const void *q, *kl, *v, *la, *z;
    const int32_t *cu;
    int num_seqs, H, c, d, N, k;
    const double *init, *dfinal, *do_;
    double *dq, *dkl, *dv, *dla, *dz, *dinit;
    int next_unit;
    pthread_mutex_t mu;
    int status;
};

static void *bwd_worker(void *arg)
{
    struct bwd_job *J = (struct bwd_job *)arg;
    const int c = J->c, d = J->d, N = J->N, H = J->H;
    const int64_t cd = (int64_t)c * d, st = (int64_t)(N + 1) * cd;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int u = J->next_unit++;
        pthread_mutex_unlock(&J->mu);
        if (u >= J->num_seqs * H)
            break;
        int s = u / H, h = u % H;
        int64_t t0 = J->cu[s], t1 = J->cu[s + 1], L = t1 - t0;
        double *S0 = (double *)malloc(sizeof(double) * (size_t)st);
        double *dS = J->dinit + (int64_t)u * st;
        double *dob = (double *)malloc(sizeof(double) * (size_t)(L * d + 1));
        double *bq = (double *)malloc(sizeof(double) * (size_t)(L * c + 1));
        double *bk = (double *)malloc(sizeof(double) * (size_t)(L * c + 1));
        double *bl = (double *)malloc(sizeof(double) * (size_t)(L * c + 1));
        double *bv = (double *)malloc(sizeof(double) * (size_t)(L * d + 1));
        double *bz = (double *)malloc(sizeof(double) * (size_t)(L * N + 1));
        int rc = -1;
        if (S0 && dob && bq && bk && bl && bv && bz) {
            if (J->init)
                memcpy(S0, J->init + (int64_t)u * st, sizeof(double) * (size_t)st);
            else
                memset(S0, 0, sizeof(double) * (size_t)st);
            if (J->dfinal)
                memcpy(dS, J->dfinal + (int64_t)u * st, sizeof(double) * (size_t)st);
            else
                memset(dS, 0, sizeof(double) * (size_t)st);
            for (int64_t t = 0; t < L; t++)
                memcpy(dob + t * d, J->do_ + ((t0 + t) * H + h) * d, sizeof(double) * (size_t)d);
            rc = sse_oracle_backward_unit(J->dtype, J->q, J->kl, J->v, J->la, J->z, t0, t1, h, H,
                                          c, d, N, J->k, S0, dob, dS, bq, bk, bv, bl, bz);
        }
        if (rc == 0) {
            for (int64_t t = 0; t < L; t++) {
                const int64_t g = (t0 + t) * H + h;
                memcpy(J->dq + g * c, bq + t * c, sizeof(double) * (size_t)c);
                memcpy(J->dkl + g * c, bk + t * c, sizeof(double) * (size_t)c);
                memcpy(J->dla + g * c, bl + t * c, sizeof(double) * (size_t)c);
                memcpy(J->dv + g * d, bv + t * d, sizeof(double) * (size_t)d);
                memcpy(J->dz + g * N, bz + t * N, sizeof(double) * (size_t)N);
            }
        } else {
            J->status = -1;
        }
        free(S0);
        free(dob);
        free(bq);
        free(bk);
        free(bl);
        free(bv);
        free(bz);
    }
    return NULL;
}

int sse_oracle_backward(int dtype, const void *q, const void *key_logits, const void *v,
                        const void *log_alpha, const void *router_logits,
                        const int32_t *cu_seqlens, int num_seqs, int H, int c, int d, int N,
                        int k, const double *init, const double *do_, const double *dfinal,
                        double *dq, double *dkl, double *dv, double *dla, double *dz,
                        double *dinit, int n_threads)
{
    if (num_seqs < 0 || H < 1 || n_threads < 1)
        return -1;
    for (int s = 0; s < num_seqs; s++)
        if (cu_seqlens[s + 1] < cu_seqlens[s])
            return -1;
    struct bwd_job J;
    memset(&J, 0, sizeof J);
    J.dtype = dtype;
    J.q = q;
    J.kl = key_logits;
    J.v = v;
    J.la = log_alpha;
    J.z = router_logits;
    J.cu = cu_seqlens;
    J.num_seqs = num_seqs;
    J.H = H;
    J.c = c;
    J.d = d;
    J.N = N;
    J.k = k;
    J.init = init;
    J.dfinal = dfinal;
    J.do_ = do_;
    J.dq = dq;
    J.dkl = dkl;
    J.dv = dv;
    J.dla = dla;
    J.dz = dz;
    J.dinit = dinit;
    pthread_mutex_init(&J.mu, NULL);
    if (n_threads == 1) {
        bwd_worker(&J);
    } else {
        pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
        int started = 0;
        for (int i = 0; i < n_threads; i++)
            if (th && pthread_create(&th[i], NULL, bwd_worker, &J) == 0)
                started++;
            else
                break;
        if (started == 0)
            bwd_worker(&J);
        for (int i = 0; i < started; i++)
            pthread_join(th[i], NULL);
        free(th);
    }
    pthread_mutex_destroy(&J.mu);
    return J.status;
}
