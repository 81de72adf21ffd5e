/*
 * piattn_oracle.c -- plain, slow, fp64 CPU oracle for pi-Attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke entry point and the CPU
 * baseline leg of bench.py may load this library.  It shares no code, header
 * or constant with the HIP library under sparse_long_context_piattn_amd/.
 *
 * What it computes (pi-Attention, arXiv 2511.10696, as summarised on
 * gist.science "pi-Attention: Periodic Sparse Transformers ...", section 2
 * "Methodology", items "Ring-Local Attention", "pi-Skip Attention" and
 * "Dynamic Adaptive Fusion"; the Dutch summary, section 2 "Methodologie"):
 *
 *   For query i of a sequence of length n:
 *     local set  L(i) = { j : 0 <= j < n, |i - j| <= k, and j <= i unless
 *                         the pattern is bidirectional }
 *     skip set   S(i) = { j = i - m*pi (and i + m*pi when bidirectional) :
 *                         1 <= m <= M, 0 <= j < n, j not in L(i) }
 *     alpha_i = sigmoid(g_i)
 *     logit_j = scale * <q_i, k_j> + log(alpha_i)      for j in L(i)
 *             = scale * <q_i, k_j> + log(1 - alpha_i)  for j in S(i)
 *     (when S(i) is empty the prior is a constant shift and is left out)
 *     o_i = sum_j softmax(logit)_j v_j      one softmax over L(i) u S(i)
 *
 * Skip schedules (the hierarchical skip schedules the Dutch summary names as
 * future work, section 5 "Betekenis en Conclusie"): a list of levels
 * (pi_r, M_r); S(i) is the union over the levels of the single-period skip
 * sets, each key once, all with the skip prior.  One level is the pattern
 * above.
 *
 * The set definitions are written as membership tests; the sets are built
 * by testing candidates and then sorted ascending.  Inputs are read exactly
 * (bf16 bits are widened to fp32 and then to fp64) and all arithmetic is
 * fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F64 = 0, OR_F32 = 1, OR_BF16 = 2 };
enum { KIND_LOCAL = 1, KIND_SKIP = 2 };

static double load_elem(const void *base, int64_t idx, int dt)
{
    if (dt == OR_F64)
        return ((const double *)base)[idx];
    if (dt == OR_F32)
        return (double)((const float *)base)[idx];
    {
        uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
}

/* Membership test for the ring-local window of query i. */
static int is_local(int n, int k, int bidir, int i, int j)
{
    if (j < 0 || j >= n)
        return 0;
    if (!bidir && j > i)
        return 0;
    return abs(i - j) <= k;
}

/* Membership test for the periodic skip set of query i. */
static int is_skip(int n, int k, int pi, int M, int bidir, int i, int j)
{
    int dist;
    if (j < 0 || j >= n || j == i)
        return 0;
    if (!bidir && j > i)
        return 0;
    if (is_local(n, k, bidir, i, j))
        return 0;
    dist = abs(i - j);
    if (dist % pi != 0)
        return 0;
    return dist / pi >= 1 && dist / pi <= M;
}

/* Membership test for the skip set of a schedule: a skip of some level. */
static int is_skip_levels(int n, int k, int nlev, const int *lpi, const int *lM,
                          int bidir, int i, int j)
{
    int r;
    for (r = 0; r < nlev; ++r)
        if (is_skip(n, k, lpi[r], lM[r], bidir, i, j))
            return 1;
    return 0;
}

static int in_list(const int32_t *idx, int cnt, int32_t j)
{
    int a;
    for (a = 0; a < cnt; ++a)
        if (idx[a] == j)
            return 1;
    return 0;
}

/*
 * Neighbour list of query i under a schedule of nlev levels (ascending key
 * index, kind 1 = local, 2 = skip; a key reached by several levels appears
 * once).  idx/kind must hold at least (2k + 1) + 2 sum(M_r) entries.
 * Returns the count.
 */
int oracle_neighbors_levels(int n, int k, int nlev, const int *lpi,
                            const int *lM, int bidir, int i, int32_t *idx,
                            int8_t *kind)
{
    int cnt = 0, a, b, m, r;
    /* candidates: the window offsets and the multiples of each period */
    for (a = -k; a <= k; ++a) {
        int j = i + a;
        if (is_local(n, k, bidir, i, j)) {
            idx[cnt] = j;
            kind[cnt] = KIND_LOCAL;
            ++cnt;
        }
    }
    for (r = 0; r < nlev; ++r) {
        for (m = 1; m <= lM[r]; ++m) {
            int64_t jb = (int64_t)i - (int64_t)m * lpi[r];
            int64_t jf = (int64_t)i + (int64_t)m * lpi[r];
            if (jb >= 0 && is_skip_levels(n, k, nlev, lpi, lM, bidir, i, (int)jb) &&
                !in_list(idx, cnt, (int32_t)jb)) {
                idx[cnt] = (int32_t)jb;
                kind[cnt] = KIND_SKIP;
                ++cnt;
            }
            if (bidir && jf < n && is_skip_levels(n, k, nlev, lpi, lM, bidir, i, (int)jf) &&
                !in_list(idx, cnt, (int32_t)jf)) {
                idx[cnt] = (int32_t)jf;
                kind[cnt] = KIND_SKIP;
                ++cnt;
            }
        }
    }
    /* insertion sort by key index (lists are short) */
    for (a = 1; a < cnt; ++a) {
        int32_t ti = idx[a];
        int8_t tk = kind[a];
        b = a - 1;
        while (b >= 0 && idx[b] > ti) {
            idx[b + 1] = idx[b];
            kind[b + 1] = kind[b];
            --b;
        }
        idx[b + 1] = ti;
        kind[b + 1] = tk;
    }
    return cnt;
}

/* The single-period pattern: one level (pi, M).  Capacity (2k + 1) + 2M. */
int oracle_neighbors(int n, int k, int pi, int M, int bidir, int i,
                     int32_t *idx, int8_t *kind)
{
    return oracle_neighbors_levels(n, k, 1, &pi, &M, bidir, i, idx, kind);
}

/* log(sigmoid(x)) without overflow; log(1 - sigmoid(x)) = log(sigmoid(-x)). */
static double log_sigmoid(double x)
{
    if (x >= 0)
        return -log1p(exp(-x));
    return x - log1p(exp(x));
}

/*
 * One attention row.  q_row: d elements (dtype dt).  Key/value row j lives
 * at element offset kv_base + j * kv_tok_stride in k / v.
 */
static void attend_row(int n, int i, int d, const void *q, int64_t q_off,
                       const void *kk, const void *vv, int64_t kv_base,
                       int64_t kv_tok_stride, int dt, double g, int kw,
                       int nlev, const int *lpi, const int *lM, int bidir,
                       double scale, int32_t *idx, int8_t *kind, double *sc,
                       double *out, double *lse)
{
    int cnt = oracle_neighbors_levels(n, kw, nlev, lpi, lM, bidir, i, idx, kind);
    int has_skip = 0, a, c;
    double prior_local = log_sigmoid(g), prior_skip = log_sigmoid(-g);
    double mx = -INFINITY, z = 0.0;

    for (a = 0; a < cnt; ++a)
        if (kind[a] == KIND_SKIP)
            has_skip = 1;
    for (a = 0; a < cnt; ++a) {
        int64_t kb = kv_base + (int64_t)idx[a] * kv_tok_stride;
        double dot = 0.0;
        for (c = 0; c < d; ++c)
            dot += load_elem(q, q_off + c, dt) * load_elem(kk, kb + c, dt);
        sc[a] = scale * dot;
        if (has_skip)
            sc[a] += (kind[a] == KIND_LOCAL) ? prior_local : prior_skip;
        if (sc[a] > mx)
            mx = sc[a];
    }
    for (c = 0; c < d; ++c)
        out[c] = 0.0;
    for (a = 0; a < cnt; ++a) {
        int64_t vb = kv_base + (int64_t)idx[a] * kv_tok_stride;
        double w = exp(sc[a] - mx);
        z += w;
        for (c = 0; c < d; ++c)
            out[c] += w * load_elem(vv, vb + c, dt);
    }
    for (c = 0; c < d; ++c)
        out[c] /= z;
    if (lse)
        *lse = mx + log(z);
}

static int list_cap(int k, int nlev, const int *lM)
{
    int r, c = 2 * k + 1;
    for (r = 0; r < nlev; ++r)
        c += 2 * lM[r];
    return c;
}

/*
 * Forward (prefill) over a packed batch.
 *   nseq sequences, token offsets cu[0..nseq] (int64), heads H, head dim d.
 *   q, k, v: [T, H, d] contiguous, element type dt.  g: [T, H] fp64 gate logits.
 *   rows: nrows flat row ids (token * H + head), or NULL for all T*H rows.
 *   out: [nrows, d] fp64; lse: [nrows] fp64 or NULL.
 */
void oracle_fwd_levels(int nseq, const int64_t *cu, int H, int d,
                       const void *q, const void *kk, const void *vv, int dt,
                       const double *g, int kw, int nlev, const int *lpi,
                       const int *lM, int bidir, double scale, int64_t nrows,
                       const int64_t *rows, double *out, double *lse,
                       int nthreads)
{
    int64_t total = cu[nseq] * (int64_t)H;
    int64_t count = rows ? nrows : total;
    int cap = list_cap(kw, nlev, lM);
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * cap);
        int8_t *kind = (int8_t *)malloc((size_t)cap);
        double *sc = (double *)malloc(sizeof(double) * cap);
        int64_t r;
#pragma omp for schedule(dynamic, 64)
        for (r = 0; r < count; ++r) {
            int64_t row = rows ? rows[r] : r;
            int64_t tok = row / H;
            int h = (int)(row % H);
            int lo = 0, hi = nseq - 1, s, n, i;
            while (lo < hi) { /* sequence holding tok */
                int mid = (lo + hi + 1) / 2;
                if (cu[mid] <= tok)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            s = lo;
            n = (int)(cu[s + 1] - cu[s]);
            i = (int)(tok - cu[s]);
            attend_row(n, i, d, q, (tok * H + h) * (int64_t)d, kk, vv,
                       (cu[s] * H + h) * (int64_t)d, (int64_t)H * d, dt,
                       g[tok * H + h], kw, nlev, lpi, lM, bidir, scale, idx,
                       kind, sc, out + r * (int64_t)d, lse ? lse + r : NULL);
        }
        free(idx);
        free(kind);
        free(sc);
    }
}

void oracle_fwd(int nseq, const int64_t *cu, int H, int d, const void *q,
                const void *kk, const void *vv, int dt, const double *g,
                int kw, int pi, int M, int bidir, double scale, int64_t nrows,
                const int64_t *rows, double *out, double *lse, int nthreads)
{
    oracle_fwd_levels(nseq, cu, H, d, q, kk, vv, dt, g, kw, 1, &pi, &M, bidir,
                      scale, nrows, rows, out, lse, nthreads);
}

/*
 * Decode: one query per (sequence, head) at position len-1 of its cache
 * (the new token's own key/value already appended), causal pattern.
 *   q: [S, H, d]; kc, vc: caches addressed as s*cs[0] + h*cs[1] + t*cs[2]
 *   (elements, last dim contiguous); lens: [S]; g: [S, H] fp64.
 *   out: [S, H, d] fp64; lse: [S, H] or NULL.
 */
void oracle_decode_levels(int S, int H, int d, const void *q, const void *kc,
                          const void *vc, int dt, const int64_t *cs,
                          const int32_t *lens, const double *g, int kw,
                          int nlev, const int *lpi, const int *lM, double scale,
                          double *out, double *lse, int nthreads)
{
    int cap = list_cap(kw, nlev, lM);
    int64_t total = (int64_t)S * H;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * cap);
        int8_t *kind = (int8_t *)malloc((size_t)cap);
        double *sc = (double *)malloc(sizeof(double) * cap);
        int64_t r;
#pragma omp for schedule(dynamic, 4)
        for (r = 0; r < total; ++r) {
            int s = (int)(r / H), h = (int)(r % H);
            int n = lens[s];
            attend_row(n, n - 1, d, q, r * (int64_t)d, kc, vc,
                       (int64_t)s * cs[0] + (int64_t)h * cs[1], cs[2], dt,
                       g[r], kw, nlev, lpi, lM, 0, scale, idx, kind, sc,
                       out + r * (int64_t)d, lse ? lse + r : NULL);
        }
        free(idx);
        free(kind);
        free(sc);
    }
}

void oracle_decode(int S, int H, int d, const void *q, const void *kc,
                   const void *vc, int dt, const int64_t *cs,
                   const int32_t *lens, const double *g, int kw, int pi, int M,
                   double scale, double *out, double *lse, int nthreads)
{
    oracle_decode_levels(S, H, d, q, kc, vc, dt, cs, lens, g, kw, 1, &pi, &M,
                         scale, out, lse, nthreads);
}

/*
 * Backward of the prefill over a packed batch (every row).  The key-side
 * gradients are scattered within a (sequence, head), so the pairs run in
 * parallel (OpenMP) and the rows of one pair in order: every sum is taken in
 * the same order as in a serial run.  dout [T, H, d] (element
 * type dtd) is the gradient of the loss with respect to out; the results are
 * the gradients with respect to q, k, v ([T, H, d] fp64, zeroed here) and
 * the gate logits g ([T, H] fp64).  It is the chain rule through the one
 * softmax of each row, with the row's logits recomputed:
 *   P_a      = softmax(logit)_a over the row's neighbours j_a
 *   dP_a     = <dout_i, v_{j_a}>,   D = sum_a P_a dP_a   (= <dout_i, out_i>)
 *   dlogit_a = P_a (dP_a - D)
 *   dq_i    += scale dlogit_a k_{j_a}
 *   dk_{j_a}+= scale dlogit_a q_i
 *   dv_{j_a}+= P_a dout_i
 *   dg_i    += dlogit_a * d prior_a / d g_i: d log(sigmoid(g)) / dg =
 *              1 - sigmoid(g) for a local key, d log(1 - sigmoid(g)) / dg =
 *              -sigmoid(g) for a skip key, and no term when the row has no
 *              skip key (it has no prior).
 */
void oracle_bwd_levels(int nseq, const int64_t *cu, int H, int d,
                       const void *q, const void *kk, const void *vv, int dt,
                       const double *g, const void *dout, int dtd, int kw,
                       int nlev, const int *lpi, const int *lM, int bidir,
                       double scale, double *dq, double *dk, double *dv,
                       double *dg)
{
    int64_t T = cu[nseq];
    int cap = list_cap(kw, nlev, lM);
    int64_t pair;

    memset(dq, 0, sizeof(double) * (size_t)(T * H * d));
    memset(dk, 0, sizeof(double) * (size_t)(T * H * d));
    memset(dv, 0, sizeof(double) * (size_t)(T * H * d));
    memset(dg, 0, sizeof(double) * (size_t)(T * H));
#pragma omp parallel
    {
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * cap);
    int8_t *kind = (int8_t *)malloc((size_t)cap);
    double *sc = (double *)malloc(sizeof(double) * cap);
    double *dp = (double *)malloc(sizeof(double) * cap);
#pragma omp for schedule(dynamic, 1)
    for (pair = 0; pair < (int64_t)nseq * H; ++pair) {
        int s = (int)(pair / H), h = (int)(pair % H), i, a, c;
        int n = (int)(cu[s + 1] - cu[s]);
        {
            int64_t base = (cu[s] * H + h) * (int64_t)d; /* token 0 of this (sequence, head) */
            int64_t ts = (int64_t)H * d;                 /* token stride */
            for (i = 0; i < n; ++i) {
                int64_t qo = base + i * ts, go = (cu[s] + i) * H + h;
                int cnt = oracle_neighbors_levels(n, kw, nlev, lpi, lM, bidir, i, idx, kind);
                int has_skip = 0;
                double ga = g[go], mx = -INFINITY, z = 0.0, D = 0.0;
                double alpha = 1.0 / (1.0 + exp(-ga));
                for (a = 0; a < cnt; ++a)
                    if (kind[a] == KIND_SKIP)
                        has_skip = 1;
                for (a = 0; a < cnt; ++a) {
                    int64_t ko = base + idx[a] * ts;
                    double dot = 0.0, dpa = 0.0;
                    for (c = 0; c < d; ++c) {
                        dot += load_elem(q, qo + c, dt) * load_elem(kk, ko + c, dt);
                        dpa += load_elem(dout, qo + c, dtd) * load_elem(vv, ko + c, dt);
                    }
                    sc[a] = dot * scale;
                    if (has_skip)
                        sc[a] += (kind[a] == KIND_LOCAL) ? log_sigmoid(ga) : log_sigmoid(-ga);
                    dp[a] = dpa;
                    if (sc[a] > mx)
                        mx = sc[a];
                }
                for (a = 0; a < cnt; ++a)
                    z += exp(sc[a] - mx);
                for (a = 0; a < cnt; ++a) {
                    sc[a] = exp(sc[a] - mx) / z; /* now P_a */
                    D += sc[a] * dp[a];
                }
                for (a = 0; a < cnt; ++a) {
                    int64_t ko = base + idx[a] * ts;
                    double ds = sc[a] * (dp[a] - D);
                    for (c = 0; c < d; ++c) {
                        dq[qo + c] += scale * ds * load_elem(kk, ko + c, dt);
                        dk[ko + c] += scale * ds * load_elem(q, qo + c, dt);
                        dv[ko + c] += sc[a] * load_elem(dout, qo + c, dtd);
                    }
                    if (has_skip)
                        dg[go] += ds * ((kind[a] == KIND_LOCAL) ? (1.0 - alpha) : -alpha);
                }
            }
        }
    }
    free(idx);
    free(kind);
    free(sc);
    free(dp);
    }
}

void oracle_bwd(int nseq, const int64_t *cu, int H, int d, const void *q,
                const void *kk, const void *vv, int dt, const double *g,
                const void *dout, int dtd, int kw, int pi, int M, int bidir,
                double scale, double *dq, double *dk, double *dv, double *dg)
{
    oracle_bwd_levels(nseq, cu, H, d, q, kk, vv, dt, g, dout, dtd, kw, 1, &pi,
                      &M, bidir, scale, dq, dk, dv, dg);
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Neighbour lists of queries q_begin .. q_begin+q_count-1 as a padded table:
 * idx [q_count, cap] (-1 padding), kind [q_count, cap] (0 padding),
 * count [q_count].  Returns 0, or -1 if some list does not fit in cap.
 */
int oracle_neighbor_table_levels(int n, int k, int nlev, const int *lpi,
                                 const int *lM, int bidir, int q_begin,
                                 int q_count, int cap, int32_t *idx,
                                 int8_t *kind, int32_t *count)
{
    int bad = 0;
    int full = list_cap(k, nlev, lM);
#pragma omp parallel
    {
        int32_t *ti = (int32_t *)malloc(sizeof(int32_t) * full);
        int8_t *tk = (int8_t *)malloc((size_t)full);
        int r;
#pragma omp for schedule(static)
        for (r = 0; r < q_count; ++r) {
            int c = oracle_neighbors_levels(n, k, nlev, lpi, lM, bidir, q_begin + r, ti, tk);
            int a;
            if (c > cap) {
#pragma omp atomic write
                bad = 1;
                c = cap;
            }
            for (a = 0; a < cap; ++a) {
                idx[(int64_t)r * cap + a] = a < c ? ti[a] : -1;
                kind[(int64_t)r * cap + a] = a < c ? tk[a] : 0;
            }
            count[r] = c;
        }
        free(ti);
        free(tk);
    }
    return bad ? -1 : 0;
}

int oracle_neighbor_table(int n, int k, int pi, int M, int bidir, int q_begin,
                          int q_count, int cap, int32_t *idx, int8_t *kind,
                          int32_t *count)
{
    return oracle_neighbor_table_levels(n, k, 1, &pi, &M, bidir, q_begin,
                                        q_count, cap, idx, kind, count);
}
