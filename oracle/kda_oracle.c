/*
 * KDA fp64 CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The product path (the HIP library) never links,
 * loads or calls it, and this file shares no code, header, table or helper
 * with that path.
 *
 * What it computes: the token-by-token KDA recurrence, in double precision,
 * exactly as the pages state it (no chunking, no reordering):
 *
 *   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *   o_t = S_t^T q_t
 *
 *   - "Hybrid Linear Attention Architectures: Breaking Through the
 *     Long-Context Engineering Bottleneck in LLMs", section "Core Module
 *     Design", Stage 3 (KDA's fused design).
 *   - "Linear Attention KDA Gating in a 3:1 Hybrid Architecture", section 2,
 *     item 5 (KDA: the channel-wise decay is applied first, then the
 *     key-direction overwrite).
 *   - "Designing and Deploying Hybrid MLA and Linear Attention
 *     Architectures for LLMs", section 2, Step 3.
 *
 * Readings taken where the pages are garbled:
 *   - The pages print the write term as beta v k^T.  With the state as a
 *     d_k x d_v matrix acted on from the left by the d_k x d_k erase and
 *     decay operators, the only well-typed write is beta k v^T, and the
 *     read-out is o = S^T q.  This is also the convention of the scalar
 *     gated form "S += k (outer) v, y = q . S" in "Linear Attention +
 *     Sparse Attention: The Hybrid Architecture Trade-off for Large Models",
 *     section 2, item 2.
 *   - The output of token t is read AFTER its own write (the causal mask
 *     includes the diagonal: token i sees j <= i; "Linear Attention KDA
 *     Gating...", section 3.2).
 *   - No query scaling is applied.
 *
 * Arithmetic: Diag(alpha) S decays the rows (key channels) of S.  The rank-1
 * erase-and-write is expanded as
 *     S <- S~ + beta k (v - S~^T k)^T,   S~ = Diag(alpha) S,
 * which is the same matrix as (I - beta k k^T) S~ + beta k v^T term by term
 * (distributivity only).  The tests pin this against the literal matrix
 * product.
 *
 * Backward (kda_oracle_bwd): reverse-mode differentiation of the same
 * recurrence for the loss  L = sum(dO * o) + sum(dS_T * S_T), i.e. the
 * vector-Jacobian product a training backward needs (the pages present the
 * chunk algorithm as the training form: "Hybrid Linear Attention
 * Architectures...", Hardware-Aware Chunkwise Parallelism).  Each token's
 * step is differentiated by the chain rule, in reverse token order.  States
 * are kept at every SEG-th token and the states inside a segment are
 * recomputed from its checkpoint with the same forward step before that
 * segment is differentiated, so every state the backward uses is bit-equal
 * to the forward's.
 *
 * Layouts (row-major, contiguous):
 *   q, k     [rows, H, Dk]     rows = B*T tokens (batch-major) or packed
 *   v, o     [rows, H, Dv]
 *   alpha    [rows, H, Dk]
 *   beta     [rows, H]
 *   state    [N, H, Dk, Dv]    N = number of sequences
 *   cu_seqlens (int64) [N+1]   NULL => N = B sequences of length T
 */
#define _GNU_SOURCE
#include <pthread.h>
#include <sched.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v, *alpha, *beta, *s0;
    double *o, *sT;
    /* backward only: upstream gradients and the gradients produced */
    const double *dout, *dsT;
    double *dq, *dk, *dv, *dalpha, *dbeta, *ds0;
    int backward;
    const int64_t *cu;
    int64_t B, T;
    int N, H, Dk, Dv;
    int64_t next;              /* next (seq, head) pair to take; atomic */
    int err;
} job_t;

static void seq_bounds(const job_t *J, int n, int64_t *t0, int64_t *t1)
{
    if (J->cu) {
        *t0 = J->cu[n];
        *t1 = J->cu[n + 1];
    } else {
        *t0 = (int64_t)n * J->T;
        *t1 = *t0 + J->T;
    }
}

/* One token of the recurrence: S (Dk x Dv) is advanced in place from S_{t-1}
 * to S_t; p is scratch of Dv doubles; o_t = S_t^T q_t is written to ot when
 * ot is not NULL. */
static void step_token(int Dk, int Dv, double *S, double *p, const double *qt,
                       const double *kt, const double *vt, const double *at, double bt,
                       double *ot)
{
    /* S~ = Diag(alpha_t) S : decay every key channel (row) first. */
    for (int c = 0; c < Dk; ++c) {
        double *row = S + (size_t)c * Dv;
        const double a = at[c];
        for (int j = 0; j < Dv; ++j) row[j] *= a;
    }
    /* p = S~^T k_t : the value the decayed memory predicts for k_t. */
    for (int j = 0; j < Dv; ++j) p[j] = 0.0;
    for (int c = 0; c < Dk; ++c) {
        const double *row = S + (size_t)c * Dv;
        const double kc = kt[c];
        for (int j = 0; j < Dv; ++j) p[j] += kc * row[j];
    }
    /* e = beta_t (v_t - p);  S <- S~ + k_t e^T  (erase along k_t, write v_t). */
    for (int j = 0; j < Dv; ++j) p[j] = bt * (vt[j] - p[j]);
    for (int c = 0; c < Dk; ++c) {
        double *row = S + (size_t)c * Dv;
        const double kc = kt[c];
        for (int j = 0; j < Dv; ++j) row[j] += kc * p[j];
    }
    if (!ot) return;
    /* o_t = S_t^T q_t, read after this token's write. */
    for (int j = 0; j < Dv; ++j) ot[j] = 0.0;
    for (int c = 0; c < Dk; ++c) {
        const double *row = S + (size_t)c * Dv;
        const double qc = qt[c];
        for (int j = 0; j < Dv; ++j) ot[j] += qc * row[j];
    }
}

/* Run the recurrence for one (sequence, head) pair.  S and p are scratch of
 * Dk*Dv and Dv doubles. */
static void run_pair(const job_t *J, int n, int h, double *S, double *p)
{
    const int H = J->H, Dk = J->Dk, Dv = J->Dv;
    int64_t t0, t1;
    seq_bounds(J, n, &t0, &t1);

    const size_t ssz = (size_t)Dk * Dv;
    if (J->s0)
        memcpy(S, J->s0 + ((size_t)n * H + h) * ssz, ssz * sizeof(double));
    else
        memset(S, 0, ssz * sizeof(double));

    for (int64_t t = t0; t < t1; ++t) {
        const size_t rk = ((size_t)t * H + h) * Dk;
        const size_t rv = ((size_t)t * H + h) * Dv;
        step_token(Dk, Dv, S, p, J->q + rk, J->k + rk, J->v + rv, J->alpha + rk,
                   J->beta[(size_t)t * H + h], J->o + rv);
    }
    if (J->sT)
        memcpy(J->sT + ((size_t)n * H + h) * ssz, S, ssz * sizeof(double));
}

#define SEG 64

/* Reverse-mode step of token t.  Sp = S_{t-1} (unchanged), dS = dL/dS_t on
 * entry and dL/dS_{t-1} on exit.  St (Dk*Dv), e, de (Dv) and ge (Dk) are
 * scratch.  Writes the token's dq, dk, dv, dalpha, dbeta. */
static void back_token(const job_t *J, int64_t t, int h, const double *Sp, double *dS,
                       double *St, double *e, double *de, double *ge)
{
    const int H = J->H, Dk = J->Dk, Dv = J->Dv;
    const size_t rk = ((size_t)t * H + h) * Dk;
    const size_t rv = ((size_t)t * H + h) * Dv;
    const double *qt = J->q + rk, *kt = J->k + rk, *at = J->alpha + rk;
    const double *vt = J->v + rv, *got = J->dout + rv;
    const double bt = J->beta[(size_t)t * H + h];
    double *dqt = J->dq + rk, *dkt = J->dk + rk, *dat = J->dalpha + rk, *dvt = J->dv + rv;

    /* Forward quantities of this token: S~ = Diag(alpha) S_{t-1} (in St) and
     * the innovation e = v - S~^T k, so that S_t = S~ + beta k e^T. */
    for (int c = 0; c < Dk; ++c)
        for (int j = 0; j < Dv; ++j) St[(size_t)c * Dv + j] = at[c] * Sp[(size_t)c * Dv + j];
    for (int j = 0; j < Dv; ++j) e[j] = vt[j];
    for (int c = 0; c < Dk; ++c)
        for (int j = 0; j < Dv; ++j) e[j] -= kt[c] * St[(size_t)c * Dv + j];

    /* o_t = S_t^T q_t:  dq = S_t dO = S~ dO + beta k (e . dO);  dS_t += q dO^T. */
    double edo = 0.0;
    for (int j = 0; j < Dv; ++j) edo += e[j] * got[j];
    for (int c = 0; c < Dk; ++c) {
        double acc = 0.0;
        for (int j = 0; j < Dv; ++j) acc += St[(size_t)c * Dv + j] * got[j];
        dqt[c] = acc + bt * kt[c] * edo;
    }
    for (int c = 0; c < Dk; ++c)
        for (int j = 0; j < Dv; ++j) dS[(size_t)c * Dv + j] += qt[c] * got[j];

    /* S_t = S~ + beta k e^T, with G = dL/dS_t:
     *   dbeta = k^T G e,  dk = beta G e,  de = beta G^T k,  dS~ = G. */
    for (int c = 0; c < Dk; ++c) {
        double acc = 0.0;
        for (int j = 0; j < Dv; ++j) acc += dS[(size_t)c * Dv + j] * e[j];
        ge[c] = acc;
    }
    double db = 0.0;
    for (int c = 0; c < Dk; ++c) db += kt[c] * ge[c];
    J->dbeta[(size_t)t * H + h] = db;
    for (int c = 0; c < Dk; ++c) dkt[c] = bt * ge[c];
    for (int j = 0; j < Dv; ++j) de[j] = 0.0;
    for (int c = 0; c < Dk; ++c)
        for (int j = 0; j < Dv; ++j) de[j] += dS[(size_t)c * Dv + j] * kt[c];
    for (int j = 0; j < Dv; ++j) de[j] *= bt;

    /* e = v - S~^T k:  dv = de,  dS~ -= k de^T,  dk -= S~ de. */
    for (int j = 0; j < Dv; ++j) dvt[j] = de[j];
    for (int c = 0; c < Dk; ++c) {
        double acc = 0.0;
        for (int j = 0; j < Dv; ++j) acc += St[(size_t)c * Dv + j] * de[j];
        dkt[c] -= acc;
        for (int j = 0; j < Dv; ++j) dS[(size_t)c * Dv + j] -= kt[c] * de[j];
    }

    /* S~ = Diag(alpha) S_{t-1}:  dalpha_c = sum_j dS~[c,j] S_{t-1}[c,j];
     * dS_{t-1} = Diag(alpha) dS~. */
    for (int c = 0; c < Dk; ++c) {
        double acc = 0.0;
        for (int j = 0; j < Dv; ++j) {
            acc += dS[(size_t)c * Dv + j] * Sp[(size_t)c * Dv + j];
            dS[(size_t)c * Dv + j] *= at[c];
        }
        dat[c] = acc;
    }
}

/* Backward of one (sequence, head) pair.  Returns 0, or -2 when scratch could
 * not be allocated. */
static int run_pair_bwd(const job_t *J, int n, int h)
{
    const int H = J->H, Dk = J->Dk, Dv = J->Dv;
    int64_t t0, t1;
    seq_bounds(J, n, &t0, &t1);
    const int64_t len = t1 - t0;
    const int64_t nseg = (len + SEG - 1) / SEG;
    const size_t ssz = (size_t)Dk * Dv;

    /* ck: state entering each segment; seg: state entering each token of the
     * segment being differentiated; S, dS, St: working matrices. */
    double *ck = (double *)malloc(sizeof(double) * ssz * (size_t)(nseg + 1));
    double *seg = (double *)malloc(sizeof(double) * ssz * SEG);
    double *S = (double *)malloc(sizeof(double) * (3 * ssz + 3 * (size_t)Dv + Dk));
    if (!ck || !seg || !S) {
        free(ck); free(seg); free(S);
        return -2;
    }
    double *dS = S + ssz, *St = dS + ssz, *p = St + ssz, *de = p + Dv, *e2 = de + Dv,
           *ge = e2 + Dv;

    if (J->s0)
        memcpy(S, J->s0 + ((size_t)n * H + h) * ssz, ssz * sizeof(double));
    else
        memset(S, 0, ssz * sizeof(double));
    for (int64_t g = 0; g < nseg; ++g) {
        memcpy(ck + (size_t)g * ssz, S, ssz * sizeof(double));
        const int64_t te = t0 + (g + 1) * SEG < t1 ? t0 + (g + 1) * SEG : t1;
        for (int64_t t = t0 + g * SEG; t < te; ++t) {
            const size_t rk = ((size_t)t * H + h) * Dk;
            step_token(Dk, Dv, S, p, J->q + rk, J->k + rk, J->v + ((size_t)t * H + h) * Dv,
                       J->alpha + rk, J->beta[(size_t)t * H + h], NULL);
        }
    }

    if (J->dsT)
        memcpy(dS, J->dsT + ((size_t)n * H + h) * ssz, ssz * sizeof(double));
    else
        memset(dS, 0, ssz * sizeof(double));
    for (int64_t g = nseg - 1; g >= 0; --g) {
        const int64_t ts = t0 + g * SEG;
        const int64_t te = ts + SEG < t1 ? ts + SEG : t1;
        memcpy(S, ck + (size_t)g * ssz, ssz * sizeof(double));
        for (int64_t t = ts; t < te; ++t) {
            memcpy(seg + (size_t)(t - ts) * ssz, S, ssz * sizeof(double));
            const size_t rk = ((size_t)t * H + h) * Dk;
            step_token(Dk, Dv, S, p, J->q + rk, J->k + rk, J->v + ((size_t)t * H + h) * Dv,
                       J->alpha + rk, J->beta[(size_t)t * H + h], NULL);
        }
        for (int64_t t = te - 1; t >= ts; --t)
            back_token(J, t, h, seg + (size_t)(t - ts) * ssz, dS, St, e2, de, ge);
    }
    if (J->ds0)
        memcpy(J->ds0 + ((size_t)n * H + h) * ssz, dS, ssz * sizeof(double));
    free(ck); free(seg); free(S);
    return 0;
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    double *S = (double *)malloc(sizeof(double) * ((size_t)J->Dk * J->Dv + J->Dv));
    if (!S) {
        __atomic_store_n(&J->err, 1, __ATOMIC_RELAXED);
        return NULL;
    }
    double *p = S + (size_t)J->Dk * J->Dv;
    const int64_t pairs = (int64_t)J->N * J->H;
    for (;;) {
        const int64_t i = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
        if (i >= pairs) break;
        if (J->backward) {
            if (run_pair_bwd(J, (int)(i / J->H), (int)(i % J->H)) != 0)
                __atomic_store_n(&J->err, 1, __ATOMIC_RELAXED);
        } else {
            run_pair(J, (int)(i / J->H), (int)(i % J->H), S, p);
        }
    }
    free(S);
    return NULL;
}

static int default_threads(void)
{
    cpu_set_t set;
    if (sched_getaffinity(0, sizeof(set), &set) == 0) {
        int n = CPU_COUNT(&set);
        if (n > 0) return n;
    }
    return 1;
}

static int run_jobs(job_t *J, int nthreads)
{
    const int64_t pairs = (int64_t)J->N * J->H;
    if (nthreads <= 0) nthreads = default_threads();
    if (nthreads > pairs) nthreads = (int)(pairs > 0 ? pairs : 1);
    if (nthreads > 256) nthreads = 256;
    pthread_t tid[256];
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&tid[i], NULL, worker, J) != 0) break;
        started = i;
    }
    worker(J);
    for (int i = 1; i <= started; ++i) pthread_join(tid[i], NULL);
    return J->err ? -2 : 0;
}

/* Full-sequence forward.  Returns 0 on success, -1 on bad arguments,
 * -2 if scratch could not be allocated.  Returns the number of threads used
 * through *threads_used when that pointer is non-NULL. */
int kda_oracle_fwd(const double *q, const double *k, const double *v,
                   const double *alpha, const double *beta,
                   const double *initial_state, double *final_state,
                   const int64_t *cu_seqlens, int num_seqs,
                   double *o, int64_t B, int64_t T, int H, int Dk, int Dv,
                   int nthreads, int *threads_used)
{
    if (!q || !k || !v || !alpha || !beta || !o) return -1;
    if (B < 0 || T < 0 || H <= 0 || Dk <= 0 || Dv <= 0) return -1;
    job_t J;
    memset(&J, 0, sizeof(J));
    J.q = q; J.k = k; J.v = v; J.alpha = alpha; J.beta = beta;
    J.s0 = initial_state; J.sT = final_state; J.o = o;
    J.cu = cu_seqlens; J.B = B; J.T = T;
    J.H = H; J.Dk = Dk; J.Dv = Dv;
    if (cu_seqlens) {
        if (B != 1 || num_seqs < 0) return -1;
        J.N = num_seqs;
    } else {
        J.N = (int)B;
    }
    int nt = nthreads <= 0 ? default_threads() : nthreads;
    const int64_t pairs = (int64_t)J.N * H;
    if (nt > pairs) nt = (int)(pairs > 0 ? pairs : 1);
    if (nt > 256) nt = 256;
    if (threads_used) *threads_used = nt;
    return run_jobs(&J, nt);
}

/* One recurrent (decode) step for N sequences: q,k [N,H,Dk], v,o [N,H,Dv],
 * alpha [N,H,Dk], beta [N,H], state [N,H,Dk,Dv] updated in place. */
int kda_oracle_step(const double *q, const double *k, const double *v,
                    const double *alpha, const double *beta, double *state,
                    double *o, int N, int H, int Dk, int Dv, int nthreads,
                    int *threads_used)
{
    if (!q || !k || !v || !alpha || !beta || !state || !o) return -1;
    if (N < 0 || H <= 0 || Dk <= 0 || Dv <= 0) return -1;
    /* A step is the fixed-length forward with T = 1, B = N, in-place state. */
    return kda_oracle_fwd(q, k, v, alpha, beta, state, state, NULL, 0, o,
                          (int64_t)N, 1, H, Dk, Dv, nthreads, threads_used);
}

/* Backward of the full-sequence forward: given dout = dL/do [rows,H,Dv] and
 * dfinal_state = dL/dS_T [N,H,Dk,Dv] (NULL = zeros), writes dq, dk, dalpha
 * [rows,H,Dk], dv [rows,H,Dv], dbeta [rows,H] and, when dinitial_state is not
 * NULL, dL/dS_0 [N,H,Dk,Dv].  Every token of every sequence is written.
 * Return codes as kda_oracle_fwd. */
int kda_oracle_bwd(const double *q, const double *k, const double *v,
                   const double *alpha, const double *beta, const double *initial_state,
                   const int64_t *cu_seqlens, int num_seqs, const double *dout,
                   const double *dfinal_state, double *dq, double *dk, double *dv,
                   double *dalpha, double *dbeta, double *dinitial_state,
                   int64_t B, int64_t T, int H, int Dk, int Dv, int nthreads,
                   int *threads_used)
{
    if (!q || !k || !v || !alpha || !beta || !dout || !dq || !dk || !dv || !dalpha || !dbeta)
        return -1;
    if (B < 0 || T < 0 || H <= 0 || Dk <= 0 || Dv <= 0) return -1;
    job_t J;
    memset(&J, 0, sizeof(J));
    J.q = q; J.k = k; J.v = v; J.alpha = alpha; J.beta = beta; J.s0 = initial_state;
    J.dout = dout; J.dsT = dfinal_state;
    J.dq = dq; J.dk = dk; J.dv = dv; J.dalpha = dalpha; J.dbeta = dbeta;
    J.ds0 = dinitial_state; J.backward = 1;
    J.cu = cu_seqlens; J.B = B; J.T = T;
    J.H = H; J.Dk = Dk; J.Dv = Dv;
    if (cu_seqlens) {
        if (B != 1 || num_seqs < 0) return -1;
        J.N = num_seqs;
    } else {
        J.N = (int)B;
    }
    int nt = nthreads <= 0 ? default_threads() : nthreads;
    const int64_t pairs = (int64_t)J.N * H;
    if (nt > pairs) nt = (int)(pairs > 0 ? pairs : 1);
    if (nt > 256) nt = 256;
    if (threads_used) *threads_used = nt;
    return run_jobs(&J, nt);
}
