/*
 * gdn_oracle.c -- plain fp64 CPU oracle of the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The product path (the
 * HIP library under hybrid_linear_attention_delta_amd/csrc) never calls it and
 * shares no code, header or constant with it.
 *
 * What it computes follows "Long-Context Aware Upcycling: A New Frontier for
 * Hybrid LLM Scaling" (arXiv:2604.24715), App. A.3 "GDN Layer Architecture",
 * Eqs. 16-19, per sequence and per head, one token at a time:
 *
 *   decay          S~_t  = e^{g_t} S_{t-1}                         (Eq. 16)
 *   delta          v'_t  = v_t - S~_t k_t                          (Eq. 17)
 *   write          S_t   = S~_t + beta_t v'_t k_t^T                (Eq. 18)
 *   read           o_t   = scale * S_t q_t                         (Eq. 19)
 *
 * The state is held as S[i][j] with i over the value dimension (d_v rows)
 * and j over the key dimension (d_k columns): the transpose of the paper's
 * d_k x d_v matrix, which is the same linear map.  Rows of S evolve
 * independently, which lets a caller ask for a subset of rows only.
 *
 * The paper sets the read scale to 1/sqrt(d_k) (Eq. 19); here it is an
 * argument.  q and k may be L2-normalised first (x / sqrt(sum x^2 + eps)); the
 * pages do not describe that step, it is a flag.
 *
 * Inputs are the stored values (fp64, fp32 or bf16) widened exactly to fp64;
 * all arithmetic is fp64 in the order written below.  No blocking, chunking
 * or reordering: chains (sequence, head) are independent and are spread over
 * POSIX threads, nothing else is parallel.
 *
 * The argument `mutation` plants one deliberate mistake (a misreading of the
 * equations) so that tests can show the oracle's pins detect it.  It is 0 in
 * every real use.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F64 = 0, OR_F32 = 1, OR_BF16 = 2 };

enum {
    MUT_NONE = 0,
    MUT_RETRIEVE_UNDECAYED = 1, /* Eq. 17 retrieves from S_{t-1} instead of S~_t   */
    MUT_READ_BEFORE_WRITE = 2,  /* Eq. 19 reads the state before the Eq. 18 write  */
    MUT_DELTA_SIGN = 3,         /* v'_t = v_t + S~_t k_t                             */
    MUT_NO_BETA_WRITE = 4,      /* Eq. 18 writes v'_t k_t^T without beta            */
    MUT_DECAY_AFTER_WRITE = 5,  /* decay applied after the rank-1 write             */
    MUT_Q_UNNORMALISED = 6,     /* L2 normalisation applied to k only              */
    MUT_OUTPUT_USES_K = 7,      /* o_t = S_t k_t                                    */
    MUT_NUM = 8
};

static double load_val(const void* p, int dt, int64_t i)
{
    if (dt == OR_F64) return ((const double*)p)[i];
    if (dt == OR_F32) return (double)((const float*)p)[i];
    /* bf16: the upper 16 bits of an IEEE binary32 */
    uint32_t bits = ((uint32_t)((const uint16_t*)p)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

typedef struct {
    const void *q, *k, *v;
    int qkv_dt;
    const void *g, *beta;
    int gate_dt;
    const void* init_state;
    int state_dt;
    const int64_t* cu_seqlens;
    int32_t N;
    int32_t H, dk, dv;
    double scale;
    int32_t qk_l2norm;
    double eps;
    const int32_t* rows;
    int32_t n_rows;
    double* o;
    double* final_state;
    int32_t n_threads;
    int32_t mutation;
    int32_t tid;
} job_t;

/* x <- x / sqrt(sum x^2 + eps) */
static void l2_normalise(double* x, int32_t n, double eps)
{
    double ss = 0.0;
    for (int32_t j = 0; j < n; ++j) ss += x[j] * x[j];
    double r = 1.0 / sqrt(ss + eps);
    for (int32_t j = 0; j < n; ++j) x[j] *= r;
}

/* One (sequence n, head h) chain, sequential over its tokens. */
static void run_chain(const job_t* a, int32_t n, int32_t h, double* S, double* qh, double* kh)
{
    const int32_t H = a->H, dk = a->dk, dv = a->dv;
    const int32_t nr = a->rows ? a->n_rows : dv;

    /* initial state rows */
    for (int32_t ri = 0; ri < nr; ++ri) {
        int32_t i = a->rows ? a->rows[ri] : ri;
        for (int32_t j = 0; j < dk; ++j) {
            int64_t idx = (((int64_t)n * H + h) * dv + i) * dk + j;
            S[(int64_t)ri * dk + j] = a->init_state ? load_val(a->init_state, a->state_dt, idx) : 0.0;
        }
    }

    for (int64_t t = a->cu_seqlens[n]; t < a->cu_seqlens[n + 1]; ++t) {
        const int64_t th = t * H + h;
        for (int32_t j = 0; j < dk; ++j) {
            qh[j] = load_val(a->q, a->qkv_dt, th * dk + j);
            kh[j] = load_val(a->k, a->qkv_dt, th * dk + j);
        }
        if (a->qk_l2norm) {
            if (a->mutation != MUT_Q_UNNORMALISED) l2_normalise(qh, dk, a->eps);
            l2_normalise(kh, dk, a->eps);
        }
        const double alpha = exp(load_val(a->g, a->gate_dt, th)); /* forget gate e^{g_t} */
        const double b = load_val(a->beta, a->gate_dt, th);       /* write strength      */
        const double* rd = (a->mutation == MUT_OUTPUT_USES_K) ? kh : qh;

        for (int32_t ri = 0; ri < nr; ++ri) {
            const int32_t i = a->rows ? a->rows[ri] : ri;
            double* s = S + (int64_t)ri * dk;
            const double vi = load_val(a->v, a->qkv_dt, th * dv + i);

            double sk = 0.0; /* (S_{t-1} k_t)_i */
            for (int32_t j = 0; j < dk; ++j) sk += s[j] * kh[j];
            double o_before = 0.0;
            if (a->mutation == MUT_READ_BEFORE_WRITE)
                for (int32_t j = 0; j < dk; ++j) o_before += alpha * s[j] * rd[j];

            /* Eq. 17: retrieval uses the decayed state S~_t = alpha S_{t-1} */
            double retrieved = (a->mutation == MUT_RETRIEVE_UNDECAYED) ? sk : alpha * sk;
            double vprime = (a->mutation == MUT_DELTA_SIGN) ? vi + retrieved : vi - retrieved;
            double w = (a->mutation == MUT_NO_BETA_WRITE) ? vprime : b * vprime;

            if (a->mutation == MUT_DECAY_AFTER_WRITE) {
                for (int32_t j = 0; j < dk; ++j) s[j] = alpha * (s[j] + w * kh[j]);
            } else {
                /* Eq. 16 + Eq. 18: S_t = alpha S_{t-1} + beta v'_t k_t^T */
                for (int32_t j = 0; j < dk; ++j) s[j] = alpha * s[j] + w * kh[j];
            }

            /* Eq. 19: read the updated state */
            double acc = 0.0;
            for (int32_t j = 0; j < dk; ++j) acc += s[j] * rd[j];
            if (a->mutation == MUT_READ_BEFORE_WRITE) acc = o_before;
            a->o[th * dv + i] = a->scale * acc;
        }
    }

    if (a->final_state) {
        for (int32_t ri = 0; ri < nr; ++ri) {
            int32_t i = a->rows ? a->rows[ri] : ri;
            for (int32_t j = 0; j < dk; ++j)
                a->final_state[(((int64_t)n * H + h) * dv + i) * dk + j] = S[(int64_t)ri * dk + j];
        }
    }
}

static void* worker(void* p)
{
    const job_t* a = (const job_t*)p;
    const int32_t nr = a->rows ? a->n_rows : a->dv;
    double* S = (double*)malloc(sizeof(double) * ((size_t)nr * a->dk + 2 * (size_t)a->dk));
    if (!S) return (void*)1;
    double* qh = S + (size_t)nr * a->dk;
    double* kh = qh + a->dk;
    const int64_t chains = (int64_t)a->N * a->H;
    for (int64_t c = a->tid; c < chains; c += a->n_threads)
        run_chain(a, (int32_t)(c / a->H), (int32_t)(c % a->H), S, qh, kh);
    free(S);
    return NULL;
}

/*
 * Prefill over packed sequences: tokens of sequence n are rows
 * [cu_seqlens[n], cu_seqlens[n+1]) of q [T,H,dk], k [T,H,dk], v [T,H,dv],
 * g [T,H], beta [T,H].  init_state / final_state are [N,H,dv,dk] (init may be
 * NULL = zeros, final may be NULL).  o is [T,H,dv] fp64.  rows (length n_rows)
 * selects the state rows to evaluate; NULL = all d_v rows.  Entries of o and
 * final_state outside the selected rows are left untouched.
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_prefill_f64(const void* q, const void* k, const void* v, int qkv_dt,
                       const void* g, const void* beta, int gate_dt,
                       const void* init_state, int state_dt,
                       const int64_t* cu_seqlens, int32_t N,
                       int32_t H, int32_t dk, int32_t dv,
                       double scale, int32_t qk_l2norm, double eps,
                       const int32_t* rows, int32_t n_rows,
                       double* o, double* final_state,
                       int32_t n_threads, int32_t mutation)
{
    if (!q || !k || !v || !g || !beta || !cu_seqlens || !o || N < 0 || H <= 0 || dk <= 0 || dv <= 0)
        return -1;
    if (mutation < 0 || mutation >= MUT_NUM) return -1;
    for (int32_t n = 0; n < N; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    if (rows)
        for (int32_t r = 0; r < n_rows; ++r)
            if (rows[r] < 0 || rows[r] >= dv) return -1;

    job_t base;
    memset(&base, 0, sizeof base);
    base.q = q; base.k = k; base.v = v; base.qkv_dt = qkv_dt;
    base.g = g; base.beta = beta; base.gate_dt = gate_dt;
    base.init_state = init_state; base.state_dt = state_dt;
    base.cu_seqlens = cu_seqlens; base.N = N;
    base.H = H; base.dk = dk; base.dv = dv;
    base.scale = scale; base.qk_l2norm = qk_l2norm; base.eps = eps;
    base.rows = rows; base.n_rows = n_rows;
    base.o = o; base.final_state = final_state;
    base.mutation = mutation;

    int64_t chains = (int64_t)N * H;
    int32_t nt = n_threads > 0 ? n_threads : 1;
    if (nt > chains) nt = (int32_t)(chains > 0 ? chains : 1);
    base.n_threads = nt;

    job_t* jobs = (job_t*)malloc(sizeof(job_t) * (size_t)nt);
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
    if (!jobs || !th) { free(jobs); free(th); return -1; }
    int rc = 0;
    for (int32_t i = 0; i < nt; ++i) {
        jobs[i] = base;
        jobs[i].tid = i;
    }
    if (nt == 1) {
        rc = worker(&jobs[0]) ? -1 : 0;
    } else {
        int32_t started = 0;
        for (; started < nt; ++started)
            if (pthread_create(&th[started], NULL, worker, &jobs[started]) != 0) { rc = -1; break; }
        for (int32_t i = 0; i < started; ++i) {
            void* ret = NULL;
            pthread_join(th[i], &ret);
            if (ret) rc = -1;
        }
    }
    free(jobs);
    free(th);
    return rc;
}

/*
 * One recurrent decode step for N independent sequences: each (n, h) takes
 * one token q/k [N,H,dk], v [N,H,dv], g/beta [N,H] and updates its state
 * [N,H,dv,dk] (fp64, in place).  o is [N,H,dv].  This is the same per-token
 * update as the prefill, applied to sequences of length one.
 */
int oracle_decode_f64(const void* q, const void* k, const void* v, int qkv_dt,
                      const void* g, const void* beta, int gate_dt,
                      double* state, int32_t N, int32_t H, int32_t dk, int32_t dv,
                      double scale, int32_t qk_l2norm, double eps,
                      double* o, int32_t n_threads)
{
    if (N < 0) return -1;
    int64_t* cu = (int64_t*)malloc(sizeof(int64_t) * ((size_t)N + 1));
    if (!cu) return -1;
    for (int32_t n = 0; n <= N; ++n) cu[n] = n;
    int rc = oracle_prefill_f64(q, k, v, qkv_dt, g, beta, gate_dt, state, OR_F64, cu, N, H, dk, dv,
                                scale, qk_l2norm, eps, NULL, 0, o, state, n_threads, MUT_NONE);
    free(cu);
    return rc;
}
