/*
 * kda_oracle.c -- plain, slow fp64 CPU reference for Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's CPU
 * baseline may load this library.  It shares no code with the GPU library.
 *
 * What it computes.  KDA is a delta-rule linear attention with a channel-wise
 * forget gate, evaluated as a recursive state update in which the gate decides
 * what is kept (blog.csdn.net article on the Kimi K3 report, section 一.1
 * "KimiDelta Attention"; "Kimi K3 深度解析" on bbs.huaweicloud.com, section 3.1).
 * The pages do not print the update, so this file takes the standard gated
 * delta-rule form: per head, with state S (dk x dv) and token t,
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t                     (output reads the updated state)
 *
 * alpha_t = exp(log_alpha_t) is a dk-vector (one gate per key channel), beta_t a
 * scalar.  The update is evaluated as written, token by token, in fp64:
 *     1. D = Diag(alpha_t) S            (scale row i of S by alpha_t[i])
 *     2. u = D^T k_t                    (dv-vector)
 *     3. delta = beta_t (v_t - u)
 *     4. S = D + k_t delta^T            (= (I - b k k^T) D + b k v^T)
 *     5. o_t = S^T q_t
 * No chunking, no blocking, no reordering: the chunk-parallel GPU evaluation is
 * only a faster way to the same numbers (myzaker "Kimi K3 开源日来了", section
 * "FlashKDA": parallel inside a chunk, serial across chunks).
 *
 * Segment decomposition ("Kimi K3 开源日来了", section "针对适配的 Infra", the
 * KDA context-parallel paragraph): a segment's end state is what it produces from
 * a zero start plus its linear action on the incoming state.  The oracle gets
 * both by running the same recurrence: once from S = 0 with the segment's v, and
 * once from S = I (dk x dk) with v = 0, which yields the transfer map
 * M = A_T ... A_1 with A_t = (I - beta_t k_t k_t^T) Diag(alpha_t).  The merge
 * is the plain definition S <- M_i S + S0_end_i over the segments in order.
 *
 * State snapshots (same page and section, the prefix-cache paragraph): the KDA
 * state of a request has a fixed size and is kept only at a sparse subset of the
 * 512-token block boundaries used for prefix matching.  The oracle records the
 * state after every `interval` tokens while running the same recurrence.
 *
 * Gradients (for training; the K3 report credits FlashKDA with faster training
 * as well as inference, "Kimi K3 开源日来了", section "FlashKDA").  For a loss
 * L with dL/do_t = dO_t and dL/dS_T = dS_T, the oracle runs the same token
 * steps backwards, applying the chain rule to each of steps 1-5 in reverse
 * order (reverse-mode differentiation of the recurrence as written):
 *     5. dq_t = S_t dO_t;             dS += q_t dO_t^T
 *     4. dk_t = dS delta;             d_delta = dS^T k_t;   dD = dS
 *     3. dbeta_t = d_delta . (v_t - u);  dv_t = beta_t d_delta;  du = -beta_t d_delta
 *     2. dk_t += D du;                dD += k_t du^T
 *     1. dlog_alpha_t[i] = sum_j D[i][j] dD[i][j];   dS = Diag(alpha_t) dD
 * and dS0 is the dS left after token 0.  The forward states are recomputed by
 * a forward pass that stores the state before every token (T dk dv doubles per
 * head: sized for test inputs).
 *
 * Layouts: row-major, [B][H][T][D] for per-token tensors, [B][H][T] for beta,
 * [B][H][dk][dv] for states, [B][n_snap][H][dk][dv] for snapshots.  All arrays
 * are fp64.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Planted-mistake builds for the oracle's own pin tests (never set in the
 * normal build): 1 drops the decay, 2 flips the sign of the delta correction,
 * 3 reads the output from the pre-update state, 4 uses k for q in the output,
 * 5 applies the decay after the delta correction, 6 transposes the state read
 * in step 2 (uses row j instead of column j), 7 records each snapshot one token
 * late; in the gradients, 8 drops the output's term q dO^T from dS, 9 flips the
 * sign of du, 10 takes dlog_alpha from the state before the decay, 11 passes dD
 * back without the decay. */
#ifndef KDA_ORACLE_MUTANT
#define KDA_ORACLE_MUTANT 0
#endif

/* One head, T tokens.  S (dk x dv) is updated in place.  o may be NULL.
 * u is scratch of length dv (>= dk when mutant 6 is built). */
static void kda_head(int T, int dk, int dv, const double* q, const double* k, const double* v,
                     const double* la, const double* beta, double* S, double* o, double* u) {
    for (int t = 0; t < T; ++t) {
        const double* qt = q ? q + (size_t)t * dk : NULL;
        const double* kt = k + (size_t)t * dk;
        const double* vt = v ? v + (size_t)t * dv : NULL;
        const double* lat = la + (size_t)t * dk;
        const double bt = beta[t];

        if (KDA_ORACLE_MUTANT != 5 && KDA_ORACLE_MUTANT != 1) {
            for (int i = 0; i < dk; ++i) {
                const double a = exp(lat[i]);
                for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a;
            }
        }
        if (KDA_ORACLE_MUTANT == 3 && o) {
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * qt[i];
                o[(size_t)t * dv + j] = acc;
            }
        }
        for (int j = 0; j < dv; ++j) u[j] = 0.0;
        if (KDA_ORACLE_MUTANT == 6 && dk == dv) {
            for (int j = 0; j < dv; ++j)
                for (int i = 0; i < dk; ++i) u[j] += S[(size_t)j * dv + i] * kt[i];
        } else {
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) u[j] += S[(size_t)i * dv + j] * kt[i];
        }
        for (int j = 0; j < dv; ++j) {
            const double vj = vt ? vt[j] : 0.0;
            u[j] = (KDA_ORACLE_MUTANT == 2) ? bt * (vj + u[j]) : bt * (vj - u[j]);
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += kt[i] * u[j];
        if (KDA_ORACLE_MUTANT == 5) {
            for (int i = 0; i < dk; ++i) {
                const double a = exp(lat[i]);
                for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a;
            }
        }
        if (o && KDA_ORACLE_MUTANT != 3) {
            const double* qq = (KDA_ORACLE_MUTANT == 4) ? kt : qt;
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * qq[i];
                o[(size_t)t * dv + j] = acc;
            }
        }
    }
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int kda_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Prefill: o [B,H,T,dv] (may be NULL), S_T [B,H,dk,dv]; S0 [B,H,dk,dv] or NULL (= 0). */
int kda_oracle_prefill(int B, int H, int T, int dk, int dv, const double* q, const double* k,
                       const double* v, const double* la, const double* beta, const double* S0,
                       double* o, double* S_T, int nthreads) {
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0) return 1;
    set_threads(nthreads);
    const int BH = B * H;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < BH; ++bh) {
        double* u = (double*)malloc(sizeof(double) * (size_t)(dv > dk ? dv : dk));
        if (!u) { err = 2; continue; }
        double* S = S_T + (size_t)bh * dk * dv;
        if (S0) memcpy(S, S0 + (size_t)bh * dk * dv, sizeof(double) * (size_t)dk * dv);
        else memset(S, 0, sizeof(double) * (size_t)dk * dv);
        const size_t tk = (size_t)bh * T * dk, tv = (size_t)bh * T * dv;
        kda_head(T, dk, dv, q + tk, k + tk, v + tv, la + tk, beta + (size_t)bh * T, S,
                 o ? o + tv : NULL, u);
        free(u);
    }
    return err;
}

/* Prefill with snapshots: as kda_oracle_prefill, and snap [B, T/interval, H, dk, dv]
 * (n_snap = floor(T / interval)) receives the state after the first (j+1)*interval
 * tokens in entry j.  interval >= 1. */
int kda_oracle_prefill_snap(int B, int H, int T, int dk, int dv, const double* q, const double* k,
                            const double* v, const double* la, const double* beta, const double* S0,
                            double* o, double* S_T, double* snap, int interval, int nthreads) {
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0 || interval < 1) return 1;
    set_threads(nthreads);
    const int BH = B * H;
    const int nsnap = T / interval;
    const size_t nS = (size_t)dk * dv;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < BH; ++bh) {
        double* u = (double*)malloc(sizeof(double) * (size_t)(dv > dk ? dv : dk));
        if (!u) { err = 2; continue; }
        const int b = bh / H, h = bh % H;
        double* S = S_T + (size_t)bh * nS;
        if (S0) memcpy(S, S0 + (size_t)bh * nS, sizeof(double) * nS);
        else memset(S, 0, sizeof(double) * nS);
        const size_t tk = (size_t)bh * T * dk, tv = (size_t)bh * T * dv;
        /* tokens [t0, t1) per piece; a snapshot closes every full piece */
        int t0 = 0;
        for (int j = 0; j <= nsnap; ++j) {
            int t1 = j < nsnap ? (j + 1) * interval : T;
            if (KDA_ORACLE_MUTANT == 7 && j < nsnap && t1 < T) t1 += 1;
            kda_head(t1 - t0, dk, dv, q + tk + (size_t)t0 * dk, k + tk + (size_t)t0 * dk,
                     v + tv + (size_t)t0 * dv, la + tk + (size_t)t0 * dk, beta + (size_t)bh * T + t0,
                     S, o ? o + tv + (size_t)t0 * dv : NULL, u);
            if (j < nsnap)
                memcpy(snap + (((size_t)b * nsnap + j) * H + h) * nS, S, sizeof(double) * nS);
            t0 = t1;
        }
        free(u);
    }
    return err;
}

/* Segment pass: the sequence of each (b,h) is G segments of Tseg tokens.
 * S_zero_end [G,B,H,dk,dv]: each segment's end state from a zero start.
 * M [G,B,H,dk,dk]: each segment's transfer map (S_end = M S_start + S_zero_end). */
int kda_oracle_segments(int B, int H, int G, int Tseg, int dk, int dv, const double* k,
                        const double* v, const double* la, const double* beta,
                        double* S_zero_end, double* M, int nthreads) {
    if (B < 0 || H < 0 || G < 0 || Tseg < 0 || dk <= 0 || dv <= 0) return 1;
    set_threads(nthreads);
    const int BH = B * H;
    const size_t T = (size_t)G * Tseg;
    int err = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int gi = 0; gi < G; ++gi) {
        for (int bh = 0; bh < BH; ++bh) {
            double* u = (double*)malloc(sizeof(double) * (size_t)(dv > dk ? dv : dk));
            if (!u) { err = 2; continue; }
            const size_t t0 = (size_t)gi * Tseg;
            const double* kk = k + ((size_t)bh * T + t0) * dk;
            const double* vv = v + ((size_t)bh * T + t0) * dv;
            const double* ll = la + ((size_t)bh * T + t0) * dk;
            const double* bb = beta + (size_t)bh * T + t0;
            double* S = S_zero_end + ((size_t)gi * BH + bh) * dk * dv;
            memset(S, 0, sizeof(double) * (size_t)dk * dv);
            kda_head(Tseg, dk, dv, NULL, kk, vv, ll, bb, S, NULL, u);
            double* Mm = M + ((size_t)gi * BH + bh) * dk * dk;
            memset(Mm, 0, sizeof(double) * (size_t)dk * dk);
            for (int i = 0; i < dk; ++i) Mm[(size_t)i * dk + i] = 1.0;
            kda_head(Tseg, dk, dk, NULL, kk, NULL, ll, bb, Mm, NULL, u);
            free(u);
        }
    }
    return err;
}

/* Merge: per (b,h), S = S_in (or 0); for i in 0..G-1: S_start[i] = S; S = M_i S + S0_end_i.
 * S_start [G,B,H,dk,dv] may be NULL; S_T [B,H,dk,dv]. */
int kda_oracle_merge(int B, int H, int G, int dk, int dv, const double* S_in,
                     const double* S_zero_end, const double* M, double* S_start, double* S_T) {
    if (B < 0 || H < 0 || G < 0 || dk <= 0 || dv <= 0) return 1;
    const int BH = B * H;
    const size_t nS = (size_t)dk * dv;
    double* tmp = (double*)malloc(sizeof(double) * nS);
    if (!tmp) return 2;
    for (int bh = 0; bh < BH; ++bh) {
        double* S = S_T + (size_t)bh * nS;
        if (S_in) memcpy(S, S_in + (size_t)bh * nS, sizeof(double) * nS);
        else memset(S, 0, sizeof(double) * nS);
        for (int gi = 0; gi < G; ++gi) {
            if (S_start) memcpy(S_start + ((size_t)gi * BH + bh) * nS, S, sizeof(double) * nS);
            const double* Mi = M + ((size_t)gi * BH + bh) * dk * dk;
            const double* Zi = S_zero_end + ((size_t)gi * BH + bh) * nS;
            for (int r = 0; r < dk; ++r)
                for (int c = 0; c < dv; ++c) {
                    double acc = Zi[(size_t)r * dv + c];
                    for (int m = 0; m < dk; ++m) acc += Mi[(size_t)r * dk + m] * S[(size_t)m * dv + c];
                    tmp[(size_t)r * dv + c] = acc;
                }
            memcpy(S, tmp, sizeof(double) * nS);
        }
    }
    free(tmp);
    return 0;
}

/* One decode step for N*H independent heads: S [N,H,dk,dv] in place, o [N,H,dv].
 * q, k, la [N,H,dk]; v [N,H,dv]; beta [N,H]. */
int kda_oracle_decode_step(int N, int H, int dk, int dv, const double* q, const double* k,
                           const double* v, const double* la, const double* beta, double* S,
                           double* o, int nthreads) {
    if (N < 0 || H < 0 || dk <= 0 || dv <= 0) return 1;
    set_threads(nthreads);
    const int NH = N * H;
    int err = 0;
#pragma omp parallel for schedule(static)
    for (int nh = 0; nh < NH; ++nh) {
        double* u = (double*)malloc(sizeof(double) * (size_t)(dv > dk ? dv : dk));
        if (!u) { err = 2; continue; }
        kda_head(1, dk, dv, q + (size_t)nh * dk, k + (size_t)nh * dk, v + (size_t)nh * dv,
                 la + (size_t)nh * dk, beta + nh, S + (size_t)nh * dk * dv, o + (size_t)nh * dv, u);
        free(u);
    }
    return err;
}

/* Gradients of L = sum(dO * o) + sum(dS_T * S_T) with respect to every input of
 * kda_oracle_prefill.  dO [B,H,T,dv] or NULL (= 0), dS_T [B,H,dk,dv] or NULL
 * (= 0).  Outputs dq, dk, dla [B,H,T,dk], dv [B,H,T,dv], dbeta [B,H,T],
 * dS0 [B,H,dk,dv]; every output must be given.  S0 NULL means a zero start. */
int kda_oracle_backward(int B, int H, int T, int dk, int dv, const double* q, const double* k,
                        const double* v, const double* la, const double* beta, const double* S0,
                        const double* dO, const double* dS_T, double* dq, double* dkk, double* dvv,
                        double* dla, double* dbeta, double* dS0, int nthreads) {
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0) return 1;
    if (!dq || !dkk || !dvv || !dla || !dbeta || !dS0) return 1;
    set_threads(nthreads);
    const int BH = B * H;
    const size_t nS = (size_t)dk * dv;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < BH; ++bh) {
        double* hist = (double*)malloc(sizeof(double) * nS * (size_t)(T > 0 ? T : 1));
        double* S = (double*)malloc(sizeof(double) * nS);
        double* D = (double*)malloc(sizeof(double) * nS);
        double* dS = (double*)malloc(sizeof(double) * nS);
        double* u = (double*)malloc(sizeof(double) * (size_t)(dv > dk ? dv : dk));
        double* del = (double*)malloc(sizeof(double) * (size_t)dv);
        double* ddel = (double*)malloc(sizeof(double) * (size_t)dv);
        if (!hist || !S || !D || !dS || !u || !del || !ddel) {
            err = 2;
            free(hist); free(S); free(D); free(dS); free(u); free(del); free(ddel);
            continue;
        }
        const size_t tk = (size_t)bh * T * dk, tv = (size_t)bh * T * dv;
        const double* qh = q + tk; const double* kh = k + tk; const double* vh = v + tv;
        const double* lh = la + tk; const double* bh_ = beta + (size_t)bh * T;

        /* forward, keeping the state before every token */
        if (S0) memcpy(S, S0 + (size_t)bh * nS, sizeof(double) * nS);
        else memset(S, 0, sizeof(double) * nS);
        for (int t = 0; t < T; ++t) {
            memcpy(hist + (size_t)t * nS, S, sizeof(double) * nS);
            kda_head(1, dk, dv, NULL, kh + (size_t)t * dk, vh + (size_t)t * dv, lh + (size_t)t * dk,
                     bh_ + t, S, NULL, u);
        }

        /* backward */
        if (dS_T) memcpy(dS, dS_T + (size_t)bh * nS, sizeof(double) * nS);
        else memset(dS, 0, sizeof(double) * nS);
        for (int t = T - 1; t >= 0; --t) {
            const double* qt = qh + (size_t)t * dk;
            const double* kt = kh + (size_t)t * dk;
            const double* vt = vh + (size_t)t * dv;
            const double* lat = lh + (size_t)t * dk;
            const double bt = bh_[t];
            const double* dot = dO ? dO + tv + (size_t)t * dv : NULL;
            const double* Sprev = hist + (size_t)t * nS;
            double* dqt = dq + tk + (size_t)t * dk;
            double* dkt = dkk + tk + (size_t)t * dk;
            double* dvt = dvv + tv + (size_t)t * dv;
            double* dlat = dla + tk + (size_t)t * dk;

            /* recompute step 1-4: D, u, delta and the updated state S */
            for (int i = 0; i < dk; ++i) {
                const double a = exp(lat[i]);
                for (int j = 0; j < dv; ++j) D[(size_t)i * dv + j] = a * Sprev[(size_t)i * dv + j];
            }
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += D[(size_t)i * dv + j] * kt[i];
                u[j] = acc;
                del[j] = bt * (vt[j] - acc);
            }
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] = D[(size_t)i * dv + j] + kt[i] * del[j];

            /* 5. o_t = S^T q_t */
            for (int i = 0; i < dk; ++i) {
                double acc = 0.0;
                if (dot)
                    for (int j = 0; j < dv; ++j) acc += S[(size_t)i * dv + j] * dot[j];
                dqt[i] = acc;
            }
            if (dot && KDA_ORACLE_MUTANT != 8)
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) dS[(size_t)i * dv + j] += qt[i] * dot[j];

            /* 4. S = D + k delta^T  (dS now stands for dD) */
            for (int i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int j = 0; j < dv; ++j) acc += dS[(size_t)i * dv + j] * del[j];
                dkt[i] = acc;
            }
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += dS[(size_t)i * dv + j] * kt[i];
                ddel[j] = acc;
            }

            /* 3. delta = beta (v - u) */
            double db = 0.0;
            for (int j = 0; j < dv; ++j) {
                db += ddel[j] * (vt[j] - u[j]);
                dvt[j] = bt * ddel[j];
                ddel[j] = (KDA_ORACLE_MUTANT == 9) ? bt * ddel[j] : -bt * ddel[j];  /* now du */
            }
            dbeta[(size_t)bh * T + t] = db;

            /* 2. u = D^T k */
            for (int i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int j = 0; j < dv; ++j) acc += D[(size_t)i * dv + j] * ddel[j];
                dkt[i] += acc;
            }
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) dS[(size_t)i * dv + j] += kt[i] * ddel[j];

            /* 1. D = Diag(alpha) S_prev */
            for (int i = 0; i < dk; ++i) {
                const double a = exp(lat[i]);
                const double* src = (KDA_ORACLE_MUTANT == 10) ? Sprev : D;
                double acc = 0.0;
                for (int j = 0; j < dv; ++j) acc += src[(size_t)i * dv + j] * dS[(size_t)i * dv + j];
                dlat[i] = acc;
                if (KDA_ORACLE_MUTANT != 11)
                    for (int j = 0; j < dv; ++j) dS[(size_t)i * dv + j] *= a;
            }
        }
        memcpy(dS0 + (size_t)bh * nS, dS, sizeof(double) * nS);
        free(hist); free(S); free(D); free(dS); free(u); free(del); free(ddel);
    }
    return err;
}
