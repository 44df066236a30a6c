/*
 * Double-precision CPU oracle for the gated delta rule (GDN) — TEST
 * INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the CPU
 * baseline leg of bench.py may load this library.  It shares no code, header
 * or constant with the HIP library under gated_delta_rule_85_amd/.
 *
 * What it computes.  The FlashQLA pages ("FlashQLA - A high-performance
 * linear attention operator library", section "Main functions"; the PyPI
 * README, section "Usage / High-level API") name the operator
 * chunk_gated_delta_rule(q, k, v, g, beta, scale, initial_state,
 * output_final_state, cu_seqlens) for the Gated Delta Network, with shapes
 * q, k [B,T,H_q,K], v [B,T,H_v,V], g, beta [B,T,H_v], state [B,H_v,K,V].
 * The pages do not print the recurrence.  Its plainest reading is the gated
 * delta rule
 *     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = scale * S_t q_t,
 * with S a V x K matrix.  The state is stored K x V (h = S^T) because the
 * README's state shape is [.., K, V].  Written for h, one token is
 *     h   <- exp(g_t) h                      (gate / decay)
 *     u   <- beta_t (v_t - h^T k_t)          (delta-rule prediction error)
 *     h   <- h + k_t u^T                     (rank-one write)
 *     o_t <- scale * h^T q_t.
 * q/k head hq serves v heads hv with hv / (H_v/H_q) == hq (contiguous
 * groups).  Variable-length batches (README "High-level API", cu_seqlens)
 * are packed token spans, each with its own state.
 *
 * Everything is evaluated token by token in double precision; the inputs
 * are the exact values the GPU receives, widened to double by the caller.
 * One (sequence, v-head) unit per OpenMP iteration.  No blocking, chunking or reordering of the recurrence:
 * the chunk length only decides where chunk-start states are recorded.
 *
 * Layouts (row-major, packed token axis of length Ttot):
 *   q, k  [Ttot, Hq, K]     v   [Ttot, Hv, V]     g, beta  [Ttot, Hv]
 *   h0    [nseq, Hv, K, V]  (NULL = zeros)        o  [Ttot, Hv, V]
 *   hT    [nseq, Hv, K, V]  (NULL = not wanted)
 *   hchunks [nchunks_total, Hv, K, V], chunk n of sequence j at index
 *          chunk_base(j) + n, where chunk_base(j) = sum_{i<j} ceil(len_i/C).
 * seq_off has nseq+1 entries: sequence j is tokens [seq_off[j], seq_off[j+1]).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int64_t nseq;
    const int64_t *seq_off;
    int64_t Hq, Hv, K, V, C;
    const double *q, *k, *v, *g, *beta;
    double scale;
} problem;

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

static int64_t chunk_base(const problem *p, int64_t j) {
    int64_t base = 0;
    for (int64_t i = 0; i < j; ++i) base += ceil_div(p->seq_off[i + 1] - p->seq_off[i], p->C);
    return base;
}

/* One token of the recurrence for head hv at packed token t.  h is K x V,
   work holds V doubles.  If o_row is non-NULL the output row is written. */
static void token_step(const problem *p, int64_t t, int64_t hv, double *h, double *work,
                       double *o_row) {
    const int64_t K = p->K, V = p->V, G = p->Hv / p->Hq, hq = hv / G;
    const double *kt = p->k + (t * p->Hq + hq) * K;
    const double *vt = p->v + (t * p->Hv + hv) * V;
    const double decay = exp(p->g[t * p->Hv + hv]);
    const double b = p->beta[t * p->Hv + hv];

    for (int64_t i = 0; i < K * V; ++i) h[i] *= decay;
    for (int64_t j = 0; j < V; ++j) work[j] = 0.0;
    for (int64_t i = 0; i < K; ++i)
        for (int64_t j = 0; j < V; ++j) work[j] += h[i * V + j] * kt[i];
    for (int64_t j = 0; j < V; ++j) work[j] = b * (vt[j] - work[j]);
    for (int64_t i = 0; i < K; ++i)
        for (int64_t j = 0; j < V; ++j) h[i * V + j] += kt[i] * work[j];
    if (o_row) {
        const double *qt = p->q + (t * p->Hq + hq) * K;
        for (int64_t j = 0; j < V; ++j) o_row[j] = 0.0;
        for (int64_t i = 0; i < K; ++i)
            for (int64_t j = 0; j < V; ++j) o_row[j] += h[i * V + j] * qt[i];
        for (int64_t j = 0; j < V; ++j) o_row[j] *= p->scale;
    }
}

static void load_state(double *h, const double *src, int64_t n) {
    if (src)
        for (int64_t i = 0; i < n; ++i) h[i] = src[i];
    else
        memset(h, 0, sizeof(double) * (size_t)n);
}

static int set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* Exact forward.  Returns the number of threads used. */
int gdr_oracle_fwd(int64_t nseq, const int64_t *seq_off, int64_t Hq, int64_t Hv, int64_t K,
                   int64_t V, int64_t C, const double *q, const double *k, const double *v,
                   const double *g, const double *beta, double scale, const double *h0, double *o,
                   double *hT, double *hchunks, int nthreads) {
    problem p = {nseq, seq_off, Hq, Hv, K, V, C, q, k, v, g, beta, scale};
    const int used = set_threads(nthreads);
    const int64_t nunits = nseq * Hv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < nunits; ++u) {
        const int64_t j = u / Hv, hv = u % Hv;
        double *h = (double *)malloc(sizeof(double) * (size_t)(K * V));
        double *work = (double *)malloc(sizeof(double) * (size_t)V);
        load_state(h, h0 ? h0 + (j * Hv + hv) * K * V : NULL, K * V);
        const int64_t t0 = seq_off[j], t1 = seq_off[j + 1];
        const int64_t cb = hchunks ? chunk_base(&p, j) : 0;
        for (int64_t t = t0; t < t1; ++t) {
            if (hchunks && (t - t0) % C == 0)
                memcpy(hchunks + ((cb + (t - t0) / C) * Hv + hv) * K * V, h,
                       sizeof(double) * (size_t)(K * V));
            token_step(&p, t, hv, h, work, o + (t * Hv + hv) * V);
        }
        if (hT) memcpy(hT + (j * Hv + hv) * K * V, h, sizeof(double) * (size_t)(K * V));
        free(h);
        free(work);
    }
    return used;
}

/*
 * Sequence-split forward with a sliding-window warm-up (the AutoCP mode of
 * the FlashQLA pages: "Technical Principles" / "Core advantages" on the
 * aiboss88 page, and section "1. Gate-Driven Automatic Intra-Card Context
 * Parallelism" of the efeozkan blog).  Each sequence's chunks are cut into
 * segments of seg_chunks chunks.  Segment s starts at chunk c_s = s*seg_chunks.
 * Its start state is obtained by running the recurrence over the warm_chunks
 * chunks before c_s from a zero state, instead of the exact carried state;
 * when that window reaches chunk 0 it starts from the true initial state,
 * which makes that segment exact.  The segment then runs its own chunks,
 * writing outputs and chunk-start states.  The last segment's end state is
 * the final state.  Same layouts as gdr_oracle_fwd.
 */
int gdr_oracle_fwd_split(int64_t nseq, const int64_t *seq_off, int64_t Hq, int64_t Hv,
                         int64_t K, int64_t V, int64_t C, const double *q, const double *k,
                         const double *v, const double *g, const double *beta, double scale,
                         const double *h0, double *o, double *hT, double *hchunks,
                         int64_t seg_chunks, int64_t warm_chunks, int nthreads) {
    problem p = {nseq, seq_off, Hq, Hv, K, V, C, q, k, v, g, beta, scale};
    const int used = set_threads(nthreads);
    const int64_t nunits = nseq * Hv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < nunits; ++u) {
        const int64_t j = u / Hv, hv = u % Hv;
        double *h = (double *)malloc(sizeof(double) * (size_t)(K * V));
        double *work = (double *)malloc(sizeof(double) * (size_t)V);
        const double *h0u = h0 ? h0 + (j * Hv + hv) * K * V : NULL;
        const int64_t t0 = seq_off[j], t1 = seq_off[j + 1];
        const int64_t nch = ceil_div(t1 - t0, C);
        const int64_t cb = hchunks ? chunk_base(&p, j) : 0;
        if (nch == 0) load_state(h, h0u, K * V);
        for (int64_t cs = 0; cs < nch; cs += seg_chunks) {
            const int64_t w0 = cs - warm_chunks;
            if (w0 <= 0) {
                load_state(h, h0u, K * V);
                for (int64_t t = t0; t < t0 + cs * C; ++t) token_step(&p, t, hv, h, work, NULL);
            } else {
                memset(h, 0, sizeof(double) * (size_t)(K * V));
                for (int64_t t = t0 + w0 * C; t < t0 + cs * C; ++t) token_step(&p, t, hv, h, work, NULL);
            }
            int64_t ce = cs + seg_chunks;
            if (ce > nch) ce = nch;
            for (int64_t t = t0 + cs * C; t < t0 + ce * C && t < t1; ++t) {
                if (hchunks && (t - t0) % C == 0)
                    memcpy(hchunks + ((cb + (t - t0) / C) * Hv + hv) * K * V, h,
                           sizeof(double) * (size_t)(K * V));
                token_step(&p, t, hv, h, work, o + (t * Hv + hv) * V);
            }
        }
        if (hT) memcpy(hT + (j * Hv + hv) * K * V, h, sizeof(double) * (size_t)(K * V));
        free(h);
        free(work);
    }
    return used;
}

/*
 * Backward (the README's chunk_gated_delta_rule_bwd returns dq, dk, dv,
 * dbeta, dg, dh0).  Reverse-mode differentiation of the token recurrence
 * above, one unit at a time: the forward is re-run storing the state at
 * every chunk start; the reverse sweep re-runs each chunk forward from its
 * stored state, then walks its tokens backwards applying the chain rule to
 *     a = exp(g_t);  hd = a h_{t-1};  p = hd^T k;  u = beta (v - p);
 *     h_t = hd + k u^T;  o_t = scale h_t^T q.
 * Gradients: dg is with respect to the per-token log-gate g, dbeta with
 * respect to beta itself; dq and dk are summed over the v heads that share
 * the q/k head.  dht (NULL = zeros) is the gradient reaching the final state.
 * Outputs: dq, dk [Ttot, Hq, K]; dv [Ttot, Hv, V]; dbeta, dg [Ttot, Hv];
 * dh0 [nseq, Hv, K, V] (NULL = not wanted).
 */
int gdr_oracle_bwd(int64_t nseq, const int64_t *seq_off, int64_t Hq, int64_t Hv, int64_t K,
                   int64_t V, int64_t C, const double *q, const double *k, const double *v,
                   const double *g, const double *beta, double scale, const double *h0,
                   const double *dout, const double *dht, double *dq, double *dk, double *dv,
                   double *dbeta, double *dg, double *dh0, int nthreads) {
    problem p = {nseq, seq_off, Hq, Hv, K, V, C, q, k, v, g, beta, scale};
    const int used = set_threads(nthreads);
    const int64_t G = Hv / Hq, nunits = nseq * Hv, Ttot = seq_off[nseq];
    /* per-v-head partials of dq, dk; summed over each head group at the end */
    double *dqv = (double *)calloc((size_t)(Ttot * Hv * K), sizeof(double));
    double *dkv = (double *)calloc((size_t)(Ttot * Hv * K), sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < nunits; ++u) {
        const int64_t j = u / Hv, hv = u % Hv, hq = hv / G;
        const int64_t t0 = seq_off[j], t1 = seq_off[j + 1];
        const int64_t nch = ceil_div(t1 - t0, C), KV = K * V;
        double *ckpt = (double *)malloc(sizeof(double) * (size_t)((nch + 1) * KV));
        double *hs = (double *)malloc(sizeof(double) * (size_t)((C + 1) * KV));
        double *Gb = (double *)malloc(sizeof(double) * (size_t)KV);
        double *work = (double *)malloc(sizeof(double) * (size_t)V);
        double *uu = (double *)malloc(sizeof(double) * (size_t)V);
        double *pp = (double *)malloc(sizeof(double) * (size_t)V);
        double *du = (double *)malloc(sizeof(double) * (size_t)V);
        double *dp = (double *)malloc(sizeof(double) * (size_t)V);
        /* forward with a state checkpoint at every chunk start */
        load_state(ckpt, h0 ? h0 + (j * Hv + hv) * KV : NULL, KV);
        for (int64_t c = 0; c < nch; ++c) {
            memcpy(ckpt + (c + 1) * KV, ckpt + c * KV, sizeof(double) * (size_t)KV);
            for (int64_t t = t0 + c * C; t < t0 + (c + 1) * C && t < t1; ++t)
                token_step(&p, t, hv, ckpt + (c + 1) * KV, work, NULL);
        }
        load_state(Gb, dht ? dht + (j * Hv + hv) * KV : NULL, KV);
        for (int64_t c = nch - 1; c >= 0; --c) {
            const int64_t ts = t0 + c * C;
            const int64_t te = (ts + C < t1) ? ts + C : t1;
            memcpy(hs, ckpt + c * KV, sizeof(double) * (size_t)KV);
            for (int64_t t = ts; t < te; ++t) {
                memcpy(hs + (t - ts + 1) * KV, hs + (t - ts) * KV, sizeof(double) * (size_t)KV);
                token_step(&p, t, hv, hs + (t - ts + 1) * KV, work, NULL);
            }
            for (int64_t t = te - 1; t >= ts; --t) {
                const double *hprev = hs + (t - ts) * KV, *hcur = hs + (t - ts + 1) * KV;
                const double *qt = q + (t * Hq + hq) * K, *kt = k + (t * Hq + hq) * K;
                const double *vt = v + (t * Hv + hv) * V, *dot = dout + (t * Hv + hv) * V;
                const double a = exp(g[t * Hv + hv]), b = beta[t * Hv + hv];
                double *dq_t = dqv + (t * Hv + hv) * K, *dk_t = dkv + (t * Hv + hv) * K;
                /* o_t = scale h_t^T q_t */
                for (int64_t i = 0; i < K; ++i) {
                    double s = 0.0;
                    for (int64_t jj = 0; jj < V; ++jj) s += hcur[i * V + jj] * dot[jj];
                    dq_t[i] = scale * s;
                }
                for (int64_t i = 0; i < K; ++i)
                    for (int64_t jj = 0; jj < V; ++jj)
                        Gb[i * V + jj] += scale * qt[i] * dot[jj];
                /* recompute p = (a h_{t-1})^T k and u = beta (v - p) */
                for (int64_t jj = 0; jj < V; ++jj) pp[jj] = 0.0;
                for (int64_t i = 0; i < K; ++i)
                    for (int64_t jj = 0; jj < V; ++jj) pp[jj] += a * hprev[i * V + jj] * kt[i];
                for (int64_t jj = 0; jj < V; ++jj) uu[jj] = b * (vt[jj] - pp[jj]);
                /* h_t = hd + k u^T:  dhd = Gb, dk += Gb u, du = Gb^T k */
                for (int64_t i = 0; i < K; ++i) {
                    double s = 0.0;
                    for (int64_t jj = 0; jj < V; ++jj) s += Gb[i * V + jj] * uu[jj];
                    dk_t[i] = s;
                }
                for (int64_t jj = 0; jj < V; ++jj) du[jj] = 0.0;
                for (int64_t i = 0; i < K; ++i)
                    for (int64_t jj = 0; jj < V; ++jj) du[jj] += Gb[i * V + jj] * kt[i];
                /* u = beta (v - p) */
                double db = 0.0;
                for (int64_t jj = 0; jj < V; ++jj) db += du[jj] * (vt[jj] - pp[jj]);
                dbeta[t * Hv + hv] = db;
                for (int64_t jj = 0; jj < V; ++jj) dv[(t * Hv + hv) * V + jj] = b * du[jj];
                for (int64_t jj = 0; jj < V; ++jj) dp[jj] = -b * du[jj];
                /* p = hd^T k:  dhd += k dp^T,  dk += hd dp */
                for (int64_t i = 0; i < K; ++i) {
                    double s = 0.0;
                    for (int64_t jj = 0; jj < V; ++jj) s += a * hprev[i * V + jj] * dp[jj];
                    dk_t[i] += s;
                }
                for (int64_t i = 0; i < K; ++i)
                    for (int64_t jj = 0; jj < V; ++jj) Gb[i * V + jj] += kt[i] * dp[jj];
                /* hd = a h_{t-1}:  dg = a <dhd, h_{t-1}>,  dh_{t-1} = a dhd */
                double dga = 0.0;
                for (int64_t i = 0; i < KV; ++i) dga += Gb[i] * hprev[i];
                dg[t * Hv + hv] = a * dga;
                for (int64_t i = 0; i < KV; ++i) Gb[i] *= a;
            }
        }
        if (dh0) memcpy(dh0 + (j * Hv + hv) * KV, Gb, sizeof(double) * (size_t)KV);
        free(ckpt); free(hs); free(Gb); free(work); free(uu); free(pp); free(du); free(dp);
    }
    /* sum the per-v-head partials of dq, dk over each q/k head's group */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < Ttot; ++t)
        for (int64_t hq = 0; hq < Hq; ++hq)
            for (int64_t i = 0; i < K; ++i) {
                double sq = 0.0, sk = 0.0;
                for (int64_t r = 0; r < G; ++r) {
                    sq += dqv[(t * Hv + hq * G + r) * K + i];
                    sk += dkv[(t * Hv + hq * G + r) * K + i];
                }
                dq[(t * Hq + hq) * K + i] = sq;
                dk[(t * Hq + hq) * K + i] = sk;
            }
    free(dqv);
    free(dkv);
    return used;
}
