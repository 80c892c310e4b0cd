/*
 * MoBA causal prefill: plain, slow, fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check
 * and the bench's CPU-baseline leg load this library.  It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * calls it.
 *
 * What is computed, and where the pages state it:
 *   - MoBA ("Mixture of Block Attention") splits the context into blocks and
 *     routes each query token to a few of them with a parameter-free top-k
 *     gate (tech-report write-up "MoBA: Mixture of Block Attention", section
 *     "MoBA：將MoE原理應用于注意力機制", the list of MoBA's parts).
 *   - The gate scores a query against an aggregated representation of each
 *     block's keys and keeps the highest-scoring blocks; the block holding
 *     the query is always kept, and no token attends to a future position
 *     (Taiwan AI overview of MoBA, section "技術細節與優勢").
 *   - Attention then runs over the tokens of the kept blocks only; the
 *     outputs of the current block and several history blocks are combined
 *     by an online softmax (write-up, same section, the five implementation
 *     steps), which is exact: the result equals one softmax over the union.
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes): the aggregation is the mean over the block's tokens (over the
 * tokens present for a short tail block); the gate score is the plain inner
 * product, unscaled; top-k counts the own block (the 95.31% sparsity of the
 * 1M model at block 4096 / top-k 12 is 1 - 12/256); ties go to the smaller
 * block index; the attention logit scale is 1/sqrt(d); query head h uses KV
 * head h / (Hq/Hkv).
 *
 * Storage codes: 0 = bf16 held as uint16 bit patterns, 1 = fp32.  Every
 * element is decoded exactly to double; all arithmetic is double.
 * Row lists are int64 triples (b, h, t).
 *
 * Return codes: 0 ok, 1 bad argument, 2 bad selection entry, 3 out of memory.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_abi_version(void) { return 1; }

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static double load_elem(const void *p, int code, size_t i) {
    if (code == 1) return (double)((const float *)p)[i];
    uint32_t u = ((uint32_t)((const uint16_t *)p)[i]) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int n_blocks(int S, int block) { return (S + block - 1) / block; }

/* K̄[b][g][j][:] = (1 / |block j|) * sum of K[b][t][g][:] over t in block j. */
int oracle_pool(const void *k, int code, int batch, int S, int hkv, int d, int block,
                double *kbar) {
    if (!k || !kbar || batch <= 0 || S <= 0 || hkv <= 0 || d <= 0 || block <= 0) return 1;
    const int n = n_blocks(S, block);
    const long long items = (long long)batch * hkv * n;
#pragma omp parallel for schedule(static)
    for (long long it = 0; it < items; ++it) {
        const int j = (int)(it % n);
        const int g = (int)((it / n) % hkv);
        const int b = (int)(it / ((long long)n * hkv));
        const int t0 = j * block;
        const int t1 = (t0 + block < S) ? t0 + block : S;
        double *dst = kbar + (size_t)it * d;
        for (int i = 0; i < d; ++i) dst[i] = 0.0;
        for (int t = t0; t < t1; ++t) {
            const size_t base = (((size_t)b * S + t) * hkv + g) * d;
            for (int i = 0; i < d; ++i) dst[i] += load_elem(k, code, base + i);
        }
        for (int i = 0; i < d; ++i) dst[i] /= (double)(t1 - t0);
    }
    return 0;
}

static int check_dims(int batch, int S, int hq, int hkv, int d, int block, int topk) {
    if (batch <= 0 || S <= 0 || hq <= 0 || hkv <= 0 || d <= 0 || block <= 0 || topk <= 0) return 1;
    if (hq % hkv != 0) return 1;
    return 0;
}

/*
 * Gate and causal top-k for the listed rows.
 *   idx_out    [R][topk]: selected blocks ascending, own block included, -1 padded.
 *   margin_out [R]: lowest selected past score minus highest unselected past
 *                   score; +inf where no choice exists (every causal block is
 *                   selected, or topk == 1).
 *   scores_out [R][n] (optional): s_j for j < blk(t), NaN elsewhere.
 */
int oracle_gate(const void *q, int code, const double *kbar, int batch, int S, int hq, int hkv,
                int d, int block, int topk, long long R, const long long *rows,
                int *idx_out, double *margin_out, double *scores_out) {
    if (!q || !kbar || !rows || !idx_out || !margin_out) return 1;
    if (check_dims(batch, S, hq, hkv, d, block, topk)) return 1;
    const int n = n_blocks(S, block);
    const int group = hq / hkv;
    int err = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)n);
        char *picked = (char *)malloc((size_t)n);
        if (!s || !picked) {
#pragma omp atomic write
            err = 3;
        }
#pragma omp for schedule(dynamic, 64)
        for (long long r = 0; r < R; ++r) {
            if (!s || !picked) continue;
            const long long b = rows[3 * r], h = rows[3 * r + 1], t = rows[3 * r + 2];
            if (b < 0 || b >= batch || h < 0 || h >= hq || t < 0 || t >= S) {
#pragma omp atomic write
                err = 1;
                continue;
            }
            const int g = (int)(h / group);
            const int own = (int)(t / block);
            const size_t qbase = (((size_t)b * S + t) * hq + h) * d;
            /* scores for the past blocks only */
            for (int j = 0; j < own; ++j) {
                const double *kb = kbar + (((size_t)b * hkv + g) * n + j) * d;
                double acc = 0.0;
                for (int i = 0; i < d; ++i) acc += load_elem(q, code, qbase + i) * kb[i];
                s[j] = acc;
                picked[j] = 0;
            }
            const int npast = (topk - 1 < own) ? topk - 1 : own;
            /* repeated arg-max; strict '>' keeps the smaller index on ties */
            for (int c = 0; c < npast; ++c) {
                int best = -1;
                for (int j = 0; j < own; ++j)
                    if (!picked[j] && (best < 0 || s[j] > s[best])) best = j;
                picked[best] = 1;
            }
            int *dst = idx_out + (size_t)r * topk;
            int w = 0;
            for (int j = 0; j < own; ++j)
                if (picked[j]) dst[w++] = j;
            dst[w++] = own;
            for (; w < topk; ++w) dst[w] = -1;
            double margin = INFINITY;
            if (npast < own && npast > 0) {
                double lo_sel = INFINITY, hi_rest = -INFINITY;
                for (int j = 0; j < own; ++j) {
                    if (picked[j]) { if (s[j] < lo_sel) lo_sel = s[j]; }
                    else if (s[j] > hi_rest) hi_rest = s[j];
                }
                margin = lo_sel - hi_rest;
            }
            margin_out[r] = margin;
            if (scores_out) {
                double *so = scores_out + (size_t)r * n;
                for (int j = 0; j < n; ++j) so[j] = (j < own) ? s[j] : NAN;
            }
        }
        free(s);
        free(picked);
    }
    return err;
}

/* Mark the blocks of one row's selection; returns 0, or 2 on an entry that is
 * neither -1 nor a block in [0, own]. */
static int mark_selection(const int *sel, int topk, int own, char *flag, int n) {
    for (int j = 0; j < n; ++j) flag[j] = 0;
    for (int c = 0; c < topk; ++c) {
        const int j = sel[c];
        if (j == -1) continue;
        if (j < 0 || j > own) return 2;
        flag[j] = 1;
    }
    return 0;
}

/*
 * Dense masked softmax attention for the listed rows under the supplied
 * selection: keys t' <= t whose block is selected, logits q.k / sqrt(d).
 *   out [R][d], lse [R] = log of the softmax normaliser (natural log, logits scaled).
 */
int oracle_attend(const void *q, const void *k, const void *v, int code, int batch, int S,
                  int hq, int hkv, int d, int block, int topk, long long R,
                  const long long *rows, const int *idx, double *out, double *lse) {
    if (!q || !k || !v || !rows || !idx || !out || !lse) return 1;
    if (check_dims(batch, S, hq, hkv, d, block, topk)) return 1;
    const int n = n_blocks(S, block);
    const int group = hq / hkv;
    const double scale = 1.0 / sqrt((double)d);
    int err = 0;
#pragma omp parallel
    {
        char *flag = (char *)malloc((size_t)n);
        double *z = (double *)malloc(sizeof(double) * (size_t)S);
        double *qv = (double *)malloc(sizeof(double) * (size_t)d);
        if (!flag || !z || !qv) {
#pragma omp atomic write
            err = 3;
        }
#pragma omp for schedule(dynamic, 4)
        for (long long r = 0; r < R; ++r) {
            if (!flag || !z || !qv) continue;
            const long long b = rows[3 * r], h = rows[3 * r + 1], t = rows[3 * r + 2];
            if (b < 0 || b >= batch || h < 0 || h >= hq || t < 0 || t >= S) {
#pragma omp atomic write
                err = 1;
                continue;
            }
            const int g = (int)(h / group);
            const int own = (int)(t / block);
            if (mark_selection(idx + (size_t)r * topk, topk, own, flag, n)) {
#pragma omp atomic write
                err = 2;
                continue;
            }
            const size_t qbase = (((size_t)b * S + t) * hq + h) * d;
            for (int i = 0; i < d; ++i) qv[i] = load_elem(q, code, qbase + i);
            double m = -INFINITY;
            for (long long tp = 0; tp <= t; ++tp) {
                if (!flag[tp / block]) continue;
                const size_t kbase = (((size_t)b * S + tp) * hkv + g) * d;
                double acc = 0.0;
                for (int i = 0; i < d; ++i) acc += qv[i] * load_elem(k, code, kbase + i);
                z[tp] = acc * scale;
                if (z[tp] > m) m = z[tp];
            }
            double l = 0.0;
            double *o = out + (size_t)r * d;
            for (int i = 0; i < d; ++i) o[i] = 0.0;
            for (long long tp = 0; tp <= t; ++tp) {
                if (!flag[tp / block]) continue;
                const double p = exp(z[tp] - m);
                l += p;
                const size_t vbase = (((size_t)b * S + tp) * hkv + g) * d;
                for (int i = 0; i < d; ++i) o[i] += p * load_elem(v, code, vbase + i);
            }
            for (int i = 0; i < d; ++i) o[i] /= l;
            lse[r] = m + log(l);
        }
        free(flag);
        free(z);
        free(qv);
    }
    return err;
}

/*
 * The same quantity reached the way the pages describe the merge: one softmax
 * per selected block (its own max, normaliser and normalised output), then the
 * per-block outputs combined with weights exp(lse_j - L), L = log sum_j exp(lse_j).
 * Exact in real arithmetic, so it must agree with oracle_attend to rounding.
 */
int oracle_attend_merged(const void *q, const void *k, const void *v, int code, int batch,
                         int S, int hq, int hkv, int d, int block, int topk, long long R,
                         const long long *rows, const int *idx, double *out, double *lse) {
    if (!q || !k || !v || !rows || !idx || !out || !lse) return 1;
    if (check_dims(batch, S, hq, hkv, d, block, topk)) return 1;
    const int n = n_blocks(S, block);
    const int group = hq / hkv;
    const double scale = 1.0 / sqrt((double)d);
    int err = 0;
#pragma omp parallel
    {
        char *flag = (char *)malloc((size_t)n);
        double *z = (double *)malloc(sizeof(double) * (size_t)block);
        double *qv = (double *)malloc(sizeof(double) * (size_t)d);
        double *po = (double *)malloc(sizeof(double) * (size_t)topk * d);
        double *pl = (double *)malloc(sizeof(double) * (size_t)topk);
        if (!flag || !z || !qv || !po || !pl) {
#pragma omp atomic write
            err = 3;
        }
#pragma omp for schedule(dynamic, 4)
        for (long long r = 0; r < R; ++r) {
            if (!flag || !z || !qv || !po || !pl) continue;
            const long long b = rows[3 * r], h = rows[3 * r + 1], t = rows[3 * r + 2];
            if (b < 0 || b >= batch || h < 0 || h >= hq || t < 0 || t >= S) {
#pragma omp atomic write
                err = 1;
                continue;
            }
            const int g = (int)(h / group);
            const int own = (int)(t / block);
            if (mark_selection(idx + (size_t)r * topk, topk, own, flag, n)) {
#pragma omp atomic write
                err = 2;
                continue;
            }
            const size_t qbase = (((size_t)b * S + t) * hq + h) * d;
            for (int i = 0; i < d; ++i) qv[i] = load_elem(q, code, qbase + i);
            int np = 0;
            for (int j = 0; j <= own; ++j) {
                if (!flag[j]) continue;
                const long long t0 = (long long)j * block;
                long long t1 = t0 + block - 1;
                if (t1 > t) t1 = t;
                double m = -INFINITY;
                for (long long tp = t0; tp <= t1; ++tp) {
                    const size_t kbase = (((size_t)b * S + tp) * hkv + g) * d;
                    double acc = 0.0;
                    for (int i = 0; i < d; ++i) acc += qv[i] * load_elem(k, code, kbase + i);
                    z[tp - t0] = acc * scale;
                    if (z[tp - t0] > m) m = z[tp - t0];
                }
                double l = 0.0;
                double *o = po + (size_t)np * d;
                for (int i = 0; i < d; ++i) o[i] = 0.0;
                for (long long tp = t0; tp <= t1; ++tp) {
                    const double p = exp(z[tp - t0] - m);
                    l += p;
                    const size_t vbase = (((size_t)b * S + tp) * hkv + g) * d;
                    for (int i = 0; i < d; ++i) o[i] += p * load_elem(v, code, vbase + i);
                }
                for (int i = 0; i < d; ++i) o[i] /= l;
                pl[np] = m + log(l);
                ++np;
            }
            double mx = -INFINITY;
            for (int c = 0; c < np; ++c)
                if (pl[c] > mx) mx = pl[c];
            double sum = 0.0;
            for (int c = 0; c < np; ++c) sum += exp(pl[c] - mx);
            const double L = mx + log(sum);
            double *o = out + (size_t)r * d;
            for (int i = 0; i < d; ++i) o[i] = 0.0;
            for (int c = 0; c < np; ++c) {
                const double w = exp(pl[c] - L);
                for (int i = 0; i < d; ++i) o[i] += w * po[(size_t)c * d + i];
            }
            lse[r] = L;
        }
        free(flag);
        free(z);
        free(qv);
        free(po);
        free(pl);
    }
    return err;
}

/*
 * Check a supplied selection against the fp64 gate scores of its row.
 *   valid_out [R]: 1 if the row's entries are the own block plus
 *                  min(topk-1, blk(t)) distinct past blocks, ascending, then
 *                  -1 padding; 0 otherwise.
 *   gap_out   [R]: lowest score among the selected past blocks minus the
 *                  highest score among the unselected past blocks (+inf when
 *                  either set is empty).  A selection is a correct top-k up
 *                  to eps exactly when gap >= -eps.
 */
int oracle_selection_gap(const void *q, int code, const double *kbar, int batch, int S, int hq,
                         int hkv, int d, int block, int topk, long long R,
                         const long long *rows, const int *idx, int *valid_out,
                         double *gap_out) {
    if (!q || !kbar || !rows || !idx || !valid_out || !gap_out) return 1;
    if (check_dims(batch, S, hq, hkv, d, block, topk)) return 1;
    const int n = n_blocks(S, block);
    const int group = hq / hkv;
    int err = 0;
#pragma omp parallel
    {
        char *flag = (char *)malloc((size_t)n);
        if (!flag) {
#pragma omp atomic write
            err = 3;
        }
#pragma omp for schedule(dynamic, 64)
        for (long long r = 0; r < R; ++r) {
            if (!flag) continue;
            const long long b = rows[3 * r], h = rows[3 * r + 1], t = rows[3 * r + 2];
            if (b < 0 || b >= batch || h < 0 || h >= hq || t < 0 || t >= S) {
#pragma omp atomic write
                err = 1;
                continue;
            }
            const int g = (int)(h / group);
            const int own = (int)(t / block);
            const int npast = (topk - 1 < own) ? topk - 1 : own;
            const int *sel = idx + (size_t)r * topk;
            int ok = 1;
            for (int j = 0; j < n; ++j) flag[j] = 0;
            for (int c = 0; c < npast; ++c) {
                if (sel[c] < 0 || sel[c] >= own) ok = 0;
                else if (c > 0 && sel[c] <= sel[c - 1]) ok = 0;
                else flag[sel[c]] = 1;
            }
            if (sel[npast] != own) ok = 0;
            for (int c = npast + 1; c < topk; ++c)
                if (sel[c] != -1) ok = 0;
            valid_out[r] = ok;
            double lo_sel = INFINITY, hi_rest = -INFINITY;
            if (ok) {
                const size_t qbase = (((size_t)b * S + t) * hq + h) * d;
                for (int j = 0; j < own; ++j) {
                    const double *kb = kbar + (((size_t)b * hkv + g) * n + j) * d;
                    double acc = 0.0;
                    for (int i = 0; i < d; ++i) acc += load_elem(q, code, qbase + i) * kb[i];
                    if (flag[j]) { if (acc < lo_sel) lo_sel = acc; }
                    else if (acc > hi_rest) hi_rest = acc;
                }
            }
            gap_out[r] = (lo_sel == INFINITY || hi_rest == -INFINITY) ? INFINITY : lo_sel - hi_rest;
        }
        free(flag);
    }
    return err;
}

/*
 * Gradients of the attention under a supplied selection, for every row.
 * The write-up trains with MoBA (its continual pre-training and fine-tuning
 * runs), so the attention has a backward; the selection itself gets none:
 * the top-k is piecewise constant and the gate has no parameters of its own.
 * With p_ts the softmax weights over T(t) (as in oracle_attend) and dout the
 * upstream gradient of out:
 *   dv_s   = sum over rows (t, h) with s in T(t) of p_ts dout_t
 *   dp_ts  = dout_t . v_s,   delta_t = sum_s p_ts dp_ts
 *   ds_ts  = p_ts (dp_ts - delta_t)
 *   dq_t   = sum_s ds_ts k_s / sqrt(d),   dk_s = sum over rows of ds_ts q_t / sqrt(d)
 * idx: [batch][hq][S][topk], the layout of the GPU's block_idx.
 * dout, dq: [batch][S][hq][d]; dk, dv: [batch][S][hkv][d]; all double.
 * Only rows t >= t_lo contribute (0: every row).  Causality makes dq of rows
 * t >= t_lo and dk, dv of keys s >= t_lo exact all the same: no earlier row
 * attends a later key.
 * Parallel over (batch, KV head): each owns its dk / dv rows, so no races.
 */
int oracle_backward(const void *q, const void *k, const void *v, int code, const double *dout,
                    int batch, int S, int hq, int hkv, int d, int block, int topk,
                    const int *idx, int t_lo, double *dq, double *dk, double *dv) {
    if (!q || !k || !v || !dout || !idx || !dq || !dk || !dv || t_lo < 0) return 1;
    if (check_dims(batch, S, hq, hkv, d, block, topk)) return 1;
    const int n = n_blocks(S, block);
    const int group = hq / hkv;
    const double scale = 1.0 / sqrt((double)d);
    memset(dq, 0, sizeof(double) * (size_t)batch * S * hq * d);
    memset(dk, 0, sizeof(double) * (size_t)batch * S * hkv * d);
    memset(dv, 0, sizeof(double) * (size_t)batch * S * hkv * d);
    int err = 0;
#pragma omp parallel
    {
        char *flag = (char *)malloc((size_t)n);
        double *p = (double *)malloc(sizeof(double) * (size_t)S);
        double *dp = (double *)malloc(sizeof(double) * (size_t)S);
        double *qv = (double *)malloc(sizeof(double) * (size_t)d);
        if (!flag || !p || !dp || !qv) {
#pragma omp atomic write
            err = 3;
        }
#pragma omp for schedule(dynamic, 1)
        for (long long bg = 0; bg < (long long)batch * hkv; ++bg) {
            if (!flag || !p || !dp || !qv) continue;
            const int b = (int)(bg / hkv), g = (int)(bg % hkv);
            for (int h = g * group; h < (g + 1) * group; ++h) {
                for (int t = t_lo; t < S; ++t) {
                    const int own = t / block;
                    const int *sel = idx + (((size_t)b * hq + h) * S + t) * topk;
                    if (mark_selection(sel, topk, own, flag, n)) {
#pragma omp atomic write
                        err = 2;
                        continue;
                    }
                    const size_t qbase = (((size_t)b * S + t) * hq + h) * d;
                    for (int i = 0; i < d; ++i) qv[i] = load_elem(q, code, qbase + i);
                    const double *go = dout + qbase;
                    /* softmax weights over T(t) */
                    double m = -INFINITY;
                    for (int s = 0; s <= t; ++s) {
                        if (!flag[s / block]) continue;
                        const size_t kb = (((size_t)b * S + s) * hkv + g) * d;
                        double acc = 0.0;
                        for (int i = 0; i < d; ++i) acc += qv[i] * load_elem(k, code, kb + i);
                        p[s] = acc * scale;
                        if (p[s] > m) m = p[s];
                    }
                    double l = 0.0;
                    for (int s = 0; s <= t; ++s)
                        if (flag[s / block]) {
                            p[s] = exp(p[s] - m);
                            l += p[s];
                        }
                    /* dp and delta */
                    double delta = 0.0;
                    for (int s = 0; s <= t; ++s) {
                        if (!flag[s / block]) continue;
                        p[s] /= l;
                        const size_t vb = (((size_t)b * S + s) * hkv + g) * d;
                        double acc = 0.0;
                        for (int i = 0; i < d; ++i) acc += go[i] * load_elem(v, code, vb + i);
                        dp[s] = acc;
                        delta += p[s] * acc;
                    }
                    double *gq = dq + qbase;
                    for (int s = 0; s <= t; ++s) {
                        if (!flag[s / block]) continue;
                        const size_t kb = (((size_t)b * S + s) * hkv + g) * d;
                        const double ds = p[s] * (dp[s] - delta);
                        for (int i = 0; i < d; ++i) {
                            gq[i] += ds * load_elem(k, code, kb + i) * scale;
                            dk[kb + i] += ds * qv[i] * scale;
                            dv[kb + i] += p[s] * go[i];
                        }
                    }
                }
            }
        }
        free(flag);
        free(p);
        free(dp);
        free(qv);
    }
    return err;
}
