/*
 * dropkv_oracle.c -- plain, slow, float64 CPU reference for DropKV scoring,
 * selection and compaction.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path
 * (libdropkv, HIP kernels) never calls it, and the two share no code.
 *
 * What it follows (DropKV: Decoupling Residual-Output Perturbation for
 * Near-Optimal KV-Cache Eviction, arXiv 2610.22130, as described on the four
 * pages studied):
 *   - Section 3.1 / Appendix C.2: deleting token j from one query's softmax
 *     changes the output a = sum_j p_j v_j by  Delta_j = p_j/(1-p_j) (a - v_j).
 *   - Section 3.3 and the third-party notes' "Core equation": the score of token j
 *     is  s_j = sum over the tail-window queries t of ||Delta_j^(t)||^2.
 *   - The third-party notes' description of "Algorithm 1": query heads that share
 *     a physical KV head are averaged; MaxPool1D smooths the scores; the recent
 *     observation window is set to +inf; the smallest scores are evicted; a
 *     probability that rounds to 1 is rejected rather than epsilon-patched.
 *   - Section 2.2: eviction removes the tokens from the resident cache
 *     (compaction keeps the surviving rows).
 *   - "paper tables", Table 14 (SnapKV row) and "paper digest", App. B: the
 *     attention-only score the pages compare against (oracle_attention_*).
 *
 * Readings taken where the pages leave a step open (all listed in the design doc):
 *   - q-head h uses KV head g = h / G, G = Hq / Hkv (contiguous groups).
 *   - aggregation: sum over the w window queries, arithmetic mean over the G
 *     heads of a group.
 *   - causality is tail-aligned: window query t sits at position n-w+t and sees
 *     keys j <= n-w+t (itself included).
 *   - logits are q.k / sqrt(d), d = head dimension; inputs are already
 *     position-encoded.
 *   - MaxPool1D has stride 1, window `pool` (odd), radius r=(pool-1)/2, and
 *     ignores out-of-range neighbours; it runs over all n raw scores, window
 *     positions included, and the +inf protection of positions >= n-w comes after.
 *   - the budget b counts kept tokens per KV head including the window;
 *     k = n - b are evicted by ascending (score, index), so among equal scores
 *     the older token goes first; kept indices are listed in ascending order.
 *   - singular rows: only a row's arg-max j* can have p > 1/2; its probability
 *     p* = 1/(1 + S_excl) (S_excl = sum over j != j* of exp(l_j - l_j*)) rounds to
 *     1.0 in binary64 exactly when S_excl <= 2^-53.  Any such row rejects the
 *     whole call (ORC_ESINGULAR).
 *   - for j*, the algebraically identical form Delta_j* = p*(abar - v_j*) with
 *     abar the output over the other tokens is used, which stays accurate as
 *     p* -> 1; every other token has p_j <= 1/2 and uses the closed form.
 *   - non-finite inputs reject the call (ENONFINITE); then an input element of
 *     magnitude 2^48 or more rejects it with ERANGE (the input contract: below
 *     it no score, and no fp32 intermediate a scorer forms, can exceed
 *     FLT_MAX); a finite score above FLT_MAX, which the fp32 output cannot
 *     hold, would also be ERANGE (unreachable inside the contract).
 *
 * Inputs are bf16 bit patterns (uint16), widened exactly to double.
 * Layouts: q [Hq][w][d], k and v [Hkv][n][d], scores [Hkv][n].
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL 1
#define ORC_ESINGULAR 2
#define ORC_ENONFINITE 3
#define ORC_ERANGE 4
#define ORC_ENOMEM 6

static double bf16_to_double(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int bf16_is_finite(uint16_t b) { return (b & 0x7F80u) != 0x7F80u; }
/* Input contract (reading R-11): |x| < 2^48, i.e. the bits without the sign
 * below those of 2^48 (exponent 127 + 48). */
static int bf16_in_range(uint16_t b) { return (b & 0x7FFFu) < 0x5780u; }

static int check_shapes(int64_t n, int w, int hq, int hkv, int d) {
    if (n < 1 || w < 1 || w > n || hq < 1 || hkv < 1 || d < 1) return ORC_EINVAL;
    if (hq % hkv != 0) return ORC_EINVAL;
    return ORC_OK;
}

/*
 * One window query (one row): softmax over the keys it sees, its output a, and
 * the per-token contributions ||Delta_j||^2 added into raw[0..P].
 * Returns ORC_ESINGULAR if p* rounds to 1.
 */
static int score_one_row(const double *q, const double *K, const double *V, int64_t P, int d,
                         double *l, double *a, double *abar, double *raw) {
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    /* logits l_j = q . k_j / sqrt(d), j = 0..P */
    for (int64_t j = 0; j <= P; ++j) {
        double s = 0.0;
        for (int i = 0; i < d; ++i) s += q[i] * K[j * d + i];
        l[j] = s * inv_sqrt_d;
    }
    /* maximum and its first position j* */
    int64_t jstar = 0;
    for (int64_t j = 1; j <= P; ++j)
        if (l[j] > l[jstar]) jstar = j;
    const double m = l[jstar];
    /* e_j = exp(l_j - m); S = sum e_j; S_excl = sum over j != j* (e_j* = 1) */
    double S = 0.0, S_excl = 0.0;
    for (int64_t j = 0; j <= P; ++j) {
        l[j] = exp(l[j] - m); /* l now holds e_j */
        S += l[j];
        if (j != jstar) S_excl += l[j];
    }
    if (S_excl <= ldexp(1.0, -53)) return ORC_ESINGULAR;
    /* a = sum_j p_j v_j ;  abar = sum_{j != j*} e_j v_j / S_excl */
    for (int i = 0; i < d; ++i) { a[i] = 0.0; abar[i] = 0.0; }
    for (int64_t j = 0; j <= P; ++j) {
        const double pj = l[j] / S;
        for (int i = 0; i < d; ++i) a[i] += pj * V[j * d + i];
        if (j != jstar) {
            const double wj = l[j] / S_excl;
            for (int i = 0; i < d; ++i) abar[i] += wj * V[j * d + i];
        }
    }
    /* ||Delta_j||^2 for every visible token */
    for (int64_t j = 0; j <= P; ++j) {
        const double pj = l[j] / S;
        double dist2 = 0.0, c;
        if (j == jstar) {
            /* Delta_j* = p* (abar - v_j*) */
            for (int i = 0; i < d; ++i) {
                const double r = abar[i] - V[j * d + i];
                dist2 += r * r;
            }
            c = pj * pj * dist2;
        } else {
            /* Delta_j = p_j / (1 - p_j) (a - v_j), with 1 - p_j = (S - e_j) / S */
            const double one_minus = (S - l[j]) / S;
            const double odds = pj / one_minus;
            for (int i = 0; i < d; ++i) {
                const double r = a[i] - V[j * d + i];
                dist2 += r * r;
            }
            c = odds * odds * dist2;
        }
        raw[j] += c;
    }
    return ORC_OK;
}

/*
 * Raw (un-pooled, un-protected) head-averaged scores:
 *   raw[g][j] = (1/G) * sum_{h in group g} sum_{t} ||Delta_j^(h,t)||^2,
 * with Delta = 0 for keys a query does not see.
 */
int oracle_raw_scores(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t n, int w,
                      int hq, int hkv, int d, int nthreads, double *raw) {
    int rc = check_shapes(n, w, hq, hkv, d);
    if (rc) return rc;
    const int G = hq / hkv;
    /* non-finite inputs reject the call */
    for (int64_t i = 0; i < (int64_t)hq * w * d; ++i)
        if (!bf16_is_finite(q[i])) return ORC_ENONFINITE;
    for (int64_t i = 0; i < (int64_t)hkv * n * d; ++i)
        if (!bf16_is_finite(k[i]) || !bf16_is_finite(v[i])) return ORC_ENONFINITE;
    /* then elements outside the contract reject it with ERANGE */
    for (int64_t i = 0; i < (int64_t)hq * w * d; ++i)
        if (!bf16_in_range(q[i])) return ORC_ERANGE;
    for (int64_t i = 0; i < (int64_t)hkv * n * d; ++i)
        if (!bf16_in_range(k[i]) || !bf16_in_range(v[i])) return ORC_ERANGE;

    /* Work is spread over the window rows (h, t) of every KV head: each row
     * writes its contributions to a buffer of its own, and each head's rows are
     * then added in (h, t) order -- the order a single thread walking the rows
     * would add them in, so the result does not depend on the thread count. */
    if (nthreads < 1) nthreads = 1;
    const int M = G * w;                      /* window rows per KV head */
    const int64_t units = (int64_t)hkv * M;
    double *Kd = malloc(sizeof(double) * (size_t)hkv * n * d);
    double *Vd = malloc(sizeof(double) * (size_t)hkv * n * d);
    double *rows = malloc(sizeof(double) * (size_t)units * n);
    int status = (Kd && Vd && rows) ? ORC_OK : ORC_ENOMEM;
    if (status == ORC_OK) {
#pragma omp parallel for schedule(static) num_threads(nthreads)
        for (int g = 0; g < hkv; ++g)
            for (int64_t i = 0; i < n * d; ++i) {
                Kd[(size_t)g * n * d + i] = bf16_to_double(k[(size_t)g * n * d + i]);
                Vd[(size_t)g * n * d + i] = bf16_to_double(v[(size_t)g * n * d + i]);
            }
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
        for (int64_t u = 0; u < units; ++u) {
            const int g = (int)(u / M), row = (int)(u % M);
            const int h = g * G + row / w, t = row % w;
            double *l = malloc(sizeof(double) * (size_t)n);
            double *a = malloc(sizeof(double) * (size_t)d);
            double *abar = malloc(sizeof(double) * (size_t)d);
            double *qq = malloc(sizeof(double) * (size_t)d);
            double *ru = rows + (size_t)u * n;
            int local = ORC_OK;
            if (!l || !a || !abar || !qq) local = ORC_ENOMEM;
            if (local == ORC_OK) {
                for (int64_t j = 0; j < n; ++j) ru[j] = 0.0;
                for (int i = 0; i < d; ++i) qq[i] = bf16_to_double(q[((size_t)h * w + t) * d + i]);
                const int64_t P = n - w + t; /* last key this query sees */
                local = score_one_row(qq, Kd + (size_t)g * n * d, Vd + (size_t)g * n * d, P, d, l,
                                      a, abar, ru);
            }
            free(l); free(a); free(abar); free(qq);
            if (local != ORC_OK) {
#pragma omp critical
                { if (local > status) status = local; }
            }
        }
    }
    if (status == ORC_OK) {
        /* raw[g][j] = (1/G) * sum over the group's rows in (h, t) order */
#pragma omp parallel for schedule(static) num_threads(nthreads)
        for (int g = 0; g < hkv; ++g) {
            double *rg = raw + (size_t)g * n;
            for (int64_t j = 0; j < n; ++j) rg[j] = 0.0;
            for (int row = 0; row < M; ++row) {
                const double *ru = rows + ((size_t)g * M + row) * n;
                for (int64_t j = 0; j < n; ++j) rg[j] += ru[j];
            }
            for (int64_t j = 0; j < n; ++j) rg[j] /= (double)G;
        }
    }
    free(Kd); free(Vd); free(rows);
    return status;
}

/* MaxPool1D (stride 1, odd window, out-of-range neighbours ignored), then +inf
 * on the last w positions of every head.  ERANGE if a raw score exceeds FLT_MAX. */
int oracle_pool_protect(const double *raw, int64_t n, int hkv, int w, int pool, double *scores) {
    if (n < 1 || hkv < 1 || w < 1 || w > n || pool < 1 || pool % 2 == 0) return ORC_EINVAL;
    const int64_t r = (pool - 1) / 2;
    for (int64_t i = 0; i < (int64_t)hkv * n; ++i)
        if (raw[i] > (double)FLT_MAX) return ORC_ERANGE;
    for (int g = 0; g < hkv; ++g) {
        const double *x = raw + (size_t)g * n;
        double *y = scores + (size_t)g * n;
        for (int64_t j = 0; j < n; ++j) {
            const int64_t lo = j - r < 0 ? 0 : j - r;
            const int64_t hi = j + r > n - 1 ? n - 1 : j + r;
            double mx = x[lo];
            for (int64_t i = lo + 1; i <= hi; ++i)
                if (x[i] > mx) mx = x[i];
            y[j] = (j >= n - w) ? INFINITY : mx;
        }
    }
    return ORC_OK;
}

/* Full scoring: raw scores, pooling, protection. */
int oracle_score(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t n, int w, int hq,
                 int hkv, int d, int pool, int nthreads, double *scores) {
    if (pool < 1 || pool % 2 == 0) return ORC_EINVAL;
    double *raw = malloc(sizeof(double) * (size_t)hkv * n);
    if (!raw) return ORC_ENOMEM;
    int rc = oracle_raw_scores(q, k, v, n, w, hq, hkv, d, nthreads, raw);
    if (rc == ORC_OK) rc = oracle_pool_protect(raw, n, hkv, w, pool, scores);
    free(raw);
    return rc;
}

/* ---- selection: evict the k = n - budget smallest by (score, index) ---- */
typedef struct { double s; int64_t j; } keyed;

static int keyed_cmp(const void *x, const void *y) {
    const keyed *a = x, *b = y;
    if (a->s < b->s) return -1;
    if (a->s > b->s) return 1;
    return (a->j > b->j) - (a->j < b->j);
}

static int index_cmp(const void *x, const void *y) {
    const int32_t a = *(const int32_t *)x, b = *(const int32_t *)y;
    return (a > b) - (a < b);
}

/* keep[g][0..budget) = indices that survive, ascending.  Scores must not be NaN. */
int oracle_select(const double *scores, int hkv, int64_t n, int64_t budget, int32_t *keep) {
    if (hkv < 1 || n < 1 || budget < 0 || budget > n) return ORC_EINVAL;
    keyed *tmp = malloc(sizeof(keyed) * (size_t)n);
    if (!tmp) return ORC_ENOMEM;
    const int64_t evict = n - budget;
    for (int g = 0; g < hkv; ++g) {
        for (int64_t j = 0; j < n; ++j) {
            tmp[j].s = scores[(size_t)g * n + j];
            if (tmp[j].s != tmp[j].s) { free(tmp); return ORC_ENONFINITE; }
            tmp[j].j = j;
        }
        qsort(tmp, (size_t)n, sizeof(keyed), keyed_cmp);
        int32_t *kg = keep + (size_t)g * budget;
        for (int64_t i = evict; i < n; ++i) kg[i - evict] = (int32_t)tmp[i].j;
        qsort(kg, (size_t)budget, sizeof(int32_t), index_cmp);
    }
    free(tmp);
    return ORC_OK;
}

/*
 * Layer-wide selection (cross-head budgets; "paper digest" §5.3 pairs DropKV
 * scores with an adaptive head-budget allocation whose rule the pages do not
 * give -- reading: one selection over the whole layer).  Evict the
 * hkv*n - budget smallest scores over all heads by (score, head, index)
 * ascending; keep[] lists the survivors as flat indices g*n + j in ascending
 * order and counts[g] how many of them belong to head g.
 */
int oracle_select_layer(const double *scores, int hkv, int64_t n, int64_t budget, int32_t *keep,
                        int32_t *counts) {
    const int64_t total = (int64_t)hkv * n;
    if (hkv < 1 || n < 1 || total >= ((int64_t)1 << 31) || budget < 0 || budget > total)
        return ORC_EINVAL;
    /* the flat [hkv][n] array is one sequence whose index order is (head, index) */
    int rc = oracle_select(scores, 1, total, budget, keep);
    if (rc != ORC_OK) return rc;
    for (int g = 0; g < hkv; ++g) counts[g] = 0;
    for (int64_t r = 0; r < budget; ++r) counts[keep[r] / n] += 1;
    return ORC_OK;
}

/* Compaction: out[g][r][:] = in[g][keep[g][r]][:] as exact bit copies. */
int oracle_compact(const uint16_t *in, int hkv, int64_t n, int d, const int32_t *keep,
                   int64_t budget, uint16_t *out) {
    for (int g = 0; g < hkv; ++g)
        for (int64_t r = 0; r < budget; ++r) {
            const int64_t j = keep[(size_t)g * budget + r];
            if (j < 0 || j >= n) return ORC_EINVAL;
            memcpy(out + ((size_t)g * budget + r) * d, in + ((size_t)g * n + j) * d,
                   sizeof(uint16_t) * (size_t)d);
        }
    return ORC_OK;
}

/*
 * In-place compaction of a resident cache [hkv][cap][d] (Section 2.2: eviction
 * removes tokens from the resident cache).  For every head, row r becomes old
 * row keep[g][r], r = 0 .. budget-1, copied one row at a time in ascending r.
 * The list must be strictly ascending inside [0, n_valid): then keep[r] >= r,
 * so every source row is read before a later copy can overwrite it.  All lists
 * are checked first; an invalid one returns ORC_ERANGE with nothing moved.
 */
int oracle_compact_inplace(uint16_t *cache, int hkv, int64_t cap, int64_t n_valid, int d,
                           const int32_t *keep, int64_t budget) {
    if (hkv < 1 || cap < 1 || n_valid < 1 || n_valid > cap || d < 1 || budget < 0 ||
        budget > n_valid)
        return ORC_EINVAL;
    for (int g = 0; g < hkv; ++g)
        for (int64_t r = 0; r < budget; ++r) {
            const int64_t j = keep[(size_t)g * budget + r];
            const int64_t prev = r > 0 ? keep[(size_t)g * budget + r - 1] : -1;
            if (j < 0 || j >= n_valid || j <= prev) return ORC_ERANGE;
        }
    for (int g = 0; g < hkv; ++g) {
        uint16_t *base = cache + (size_t)g * cap * d;
        for (int64_t r = 0; r < budget; ++r) {
            const int64_t j = keep[(size_t)g * budget + r];
            if (j != r) memcpy(base + (size_t)r * d, base + (size_t)j * d, sizeof(uint16_t) * (size_t)d);
        }
    }
    return ORC_OK;
}

/*
 * Decode-time rescoring of a resident cache ("paper digest" §6 leaves a
 * decode-time kernel as future work; reading: the n_valid resident rows of
 * every head, kept tokens then appended decode tokens, are scored exactly as a
 * prefill cache of n_valid tokens whose window is the last w rows).  k and v are
 * [hkv][cap][d] with rows n_valid .. cap-1 ignored; the resident rows are
 * gathered into [hkv][n_valid][d] and scored by oracle_score.
 */
int oracle_rescore(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t cap,
                   int64_t n_valid, int w, int hq, int hkv, int d, int pool, int nthreads,
                   double *scores) {
    if (cap < 1 || n_valid < 1 || n_valid > cap || hkv < 1 || d < 1) return ORC_EINVAL;
    uint16_t *kr = malloc(sizeof(uint16_t) * (size_t)hkv * n_valid * d);
    uint16_t *vr = malloc(sizeof(uint16_t) * (size_t)hkv * n_valid * d);
    int rc = (kr && vr) ? ORC_OK : ORC_ENOMEM;
    if (rc == ORC_OK) {
        for (int g = 0; g < hkv; ++g) {
            memcpy(kr + (size_t)g * n_valid * d, k + (size_t)g * cap * d,
                   sizeof(uint16_t) * (size_t)n_valid * d);
            memcpy(vr + (size_t)g * n_valid * d, v + (size_t)g * cap * d,
                   sizeof(uint16_t) * (size_t)n_valid * d);
        }
        rc = oracle_score(q, kr, vr, n_valid, w, hq, hkv, d, pool, nthreads, scores);
    }
    free(kr); free(vr);
    return rc;
}

/*
 * Log-sum-exp of every window query's logits over the keys it sees (natural
 * log): lse[h][t] = log sum_{j <= n-w+t} exp(q.k_j / sqrt(d)).  With the output a
 * of oracle_window_attention, this is what pass 1 can hand back to the caller
 * (the pages' result object returns the query output alongside the scores).
 */
int oracle_window_lse(const uint16_t *q, const uint16_t *k, int64_t n, int w, int hq, int hkv,
                      int d, double *lse) {
    int rc = check_shapes(n, w, hq, hkv, d);
    if (rc) return rc;
    const int G = hq / hkv;
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    double *lg = malloc(sizeof(double) * (size_t)n);
    if (!lg) return ORC_ENOMEM;
    for (int h = 0; h < hq; ++h) {
        const int g = h / G;
        for (int t = 0; t < w; ++t) {
            const int64_t last = n - w + t;
            const uint16_t *qr = q + ((size_t)h * w + t) * d;
            double mx = -INFINITY;
            for (int64_t j = 0; j <= last; ++j) {
                double acc = 0.0;
                for (int i = 0; i < d; ++i)
                    acc += bf16_to_double(qr[i]) * bf16_to_double(k[((size_t)g * n + j) * d + i]);
                lg[j] = acc * inv_sqrt_d;
                if (lg[j] > mx) mx = lg[j];
            }
            double sum = 0.0;
            for (int64_t j = 0; j <= last; ++j) sum += exp(lg[j] - mx);
            lse[(size_t)h * w + t] = mx + log(sum);
        }
    }
    free(lg);
    return ORC_OK;
}

/*
 * Attention-only scores (the pages' negative control; "paper tables", Table 14,
 * SnapKV row: MaxPool1d over the window-summed attention weights, kept large;
 * "paper digest", App. B: the same observation window and pooling kernel as
 * DropKV, the scores differing only by the value-residual factor).  Reading:
 * heads of a group are averaged as for DropKV, and the same protection and
 * eviction of the smallest follow.
 *   raw[g][j] = (1/G) * sum_{h in group g} sum_t p_j^(h,t),  p = 0 for unseen keys.
 * Only K is read.
 */
int oracle_attention_raw(const uint16_t *q, const uint16_t *k, int64_t n, int w, int hq, int hkv,
                         int d, int nthreads, double *raw) {
    int rc = check_shapes(n, w, hq, hkv, d);
    if (rc) return rc;
    const int G = hq / hkv;
    for (int64_t i = 0; i < (int64_t)hq * w * d; ++i)
        if (!bf16_is_finite(q[i])) return ORC_ENONFINITE;
    for (int64_t i = 0; i < (int64_t)hkv * n * d; ++i)
        if (!bf16_is_finite(k[i])) return ORC_ENONFINITE;
    for (int64_t i = 0; i < (int64_t)hq * w * d; ++i)
        if (!bf16_in_range(q[i])) return ORC_ERANGE;
    for (int64_t i = 0; i < (int64_t)hkv * n * d; ++i)
        if (!bf16_in_range(k[i])) return ORC_ERANGE;
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    int status = ORC_OK;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int g = 0; g < hkv; ++g) {
        double *l = malloc(sizeof(double) * (size_t)n);
        double *rg = raw + (size_t)g * n;
        if (!l) {
#pragma omp critical
            { status = ORC_ENOMEM; }
            continue;
        }
        for (int64_t j = 0; j < n; ++j) rg[j] = 0.0;
        for (int h = g * G; h < (g + 1) * G; ++h) {
            for (int t = 0; t < w; ++t) {
                const int64_t Pt = n - w + t; /* query t's last visible key */
                const uint16_t *qr = q + ((size_t)h * w + t) * d;
                double m = -INFINITY;
                for (int64_t j = 0; j <= Pt; ++j) {
                    double s = 0.0;
                    for (int i = 0; i < d; ++i)
                        s += bf16_to_double(qr[i]) * bf16_to_double(k[((size_t)g * n + j) * d + i]);
                    l[j] = inv_sqrt_d * s;
                    if (l[j] > m) m = l[j];
                }
                double S = 0.0;
                for (int64_t j = 0; j <= Pt; ++j) {
                    l[j] = exp(l[j] - m);
                    S += l[j];
                }
                for (int64_t j = 0; j <= Pt; ++j) rg[j] += l[j] / S;
            }
        }
        for (int64_t j = 0; j < n; ++j) rg[j] = rg[j] / (double)G;
        free(l);
    }
    return status;
}

/* Attention-only scoring: raw attention sums, pooling, protection. */
int oracle_attention_score(const uint16_t *q, const uint16_t *k, int64_t n, int w, int hq, int hkv,
                           int d, int pool, int nthreads, double *scores) {
    if (pool < 1 || pool % 2 == 0) return ORC_EINVAL;
    double *raw = malloc(sizeof(double) * (size_t)hkv * n);
    if (!raw) return ORC_ENOMEM;
    int rc = oracle_attention_raw(q, k, n, w, hq, hkv, d, nthreads, raw);
    if (rc == ORC_OK) rc = oracle_pool_protect(raw, n, hkv, w, pool, scores);
    free(raw);
    return rc;
}

/*
 * Diagnostics for the tests: per window query (h, t), the probabilities over
 * keys (zero for unseen keys), the output a and S_excl.
 * p [hq][w][n], a [hq][w][d], s_excl [hq][w].
 */
int oracle_window_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t n,
                            int w, int hq, int hkv, int d, double *p, double *a, double *s_excl) {
    int rc = check_shapes(n, w, hq, hkv, d);
    if (rc) return rc;
    const int G = hq / hkv;
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    double *l = malloc(sizeof(double) * (size_t)n);
    if (!l) return ORC_ENOMEM;
    for (int h = 0; h < hq; ++h) {
        const int g = h / G;
        for (int t = 0; t < w; ++t) {
            const int64_t P = n - w + t;
            const uint16_t *qr = q + ((size_t)h * w + t) * d;
            for (int64_t j = 0; j <= P; ++j) {
                double s = 0.0;
                for (int i = 0; i < d; ++i)
                    s += bf16_to_double(qr[i]) * bf16_to_double(k[((size_t)g * n + j) * d + i]);
                l[j] = s * inv_sqrt_d;
            }
            int64_t jstar = 0;
            for (int64_t j = 1; j <= P; ++j)
                if (l[j] > l[jstar]) jstar = j;
            const double m = l[jstar];
            double S = 0.0, Sx = 0.0;
            for (int64_t j = 0; j <= P; ++j) {
                l[j] = exp(l[j] - m);
                S += l[j];
                if (j != jstar) Sx += l[j];
            }
            double *pr = p + ((size_t)h * w + t) * n;
            double *ar = a + ((size_t)h * w + t) * d;
            for (int i = 0; i < d; ++i) ar[i] = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                pr[j] = j <= P ? l[j] / S : 0.0;
                if (j <= P)
                    for (int i = 0; i < d; ++i)
                        ar[i] += pr[j] * bf16_to_double(v[((size_t)g * n + j) * d + i]);
            }
            s_excl[(size_t)h * w + t] = Sx;
        }
    }
    free(l);
    return ORC_OK;
}
