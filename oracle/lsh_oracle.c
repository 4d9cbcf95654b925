/*
 * lsh_oracle.c -- plain fp64 CPU oracle for shared-QK LSH attention,
 * forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the correctness reference that the GPU
 * library is checked against.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg load it; the library never does, and it shares
 * no code, header or table with the library.
 *
 * Source of the method: "Reformer: The Efficient Transformer" (Kitaev, Kaiser,
 * Levskaya, arXiv:2001.04451v2), as summarised on its paperlayer.ai page, and
 * the authors' remark about gradients quoted in Hacker News thread 22095523.
 * Each function names the passage it follows.  Everything is computed in fp64
 * on the exact values of the (possibly bf16- or fp32-rounded) inputs, one
 * (batch, head) slice at a time, with plain loops and no blocking.
 *
 * Readings where the pages leave a step open (the plainest reading that the
 * rest supports):
 *   - [xR; -xR] is the concatenation: entry j < nb/2 is +y_j, entry nb/2+j is
 *     -y_j; ties go to the smallest index.
 *   - one rotation per round, shared by all (batch, head) slices; rotation
 *     is [n_hashes][d][n_buckets/2].
 *   - keys are the L2-normalised queries (shared-QK); logits are
 *     scale * q_i . k_j.
 *   - sort order per round is ascending (bucket, position); chunk of a
 *     position is floor(sorted index / m); m divides L.
 *   - round-r attended set of query i (self included):
 *       A_i^r = { j : h_r(j) = h_r(i), j <= i, chunk_r(i) - chunk_r(j) in {0,1} }.
 *     Every attention entry point takes a `causal` flag; with causal = 0
 *     (encoder self-attention, which the pages do not spell out) the
 *     condition j <= i is dropped and nothing else changes: same bucket,
 *     own chunk or the one before (no look-ahead to the next chunk, and the
 *     first chunk has no chunk before it: no wrap-around).
 *     And a `bucket_mask` flag: with bucket_mask = 0 the condition
 *     h_r(j) = h_r(i) is dropped (the alternative reading in which the
 *     chunks of the sorted order alone restrict attention), nothing else
 *     changes.
 *   - duplicate correction: by default every member of the union counts
 *     once.  With `dup_by_bucket` (forward, backward), the count N_ij that
 *     divides a pair is the number of rounds in which j shares i's bucket,
 *     whether or not the round's chunks let i attend to j; a member that
 *     i attends to in k_ij rounds then carries weight k_ij / N_ij (the two
 *     readings agree when no bucket is cut by the chunk window).
 *   - the query attends to the union U_i of its round sets, each key once
 *     (duplicate correction); self is dropped from the union unless nothing
 *     else is in it, in which case o_i = v_i and lse_i = scale * q_i . k_i.
 *   - no gradient through hashing or sorting; gradient does flow through
 *     the key normalisation.
 *
 * All entry points return 0 on success and 1 on invalid arguments.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

int lsh_oracle_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------- */
/* Hashing.  §2 "Locality-Sensitive Hashing Attention": random projections,
 * h(x) = argmax([xR; -xR]).  Hashing q or q/|q| gives the same argmax, so the
 * raw query is projected.                                                    */

static int argmax_concat(const double *y, int half)
{
    int best = 0;
    double bv = y[0];
    for (int j = 1; j < 2 * half; ++j) {
        double z = (j < half) ? y[j] : -y[j - half];
        if (z > bv) {
            bv = z;
            best = j;
        }
    }
    return best;
}

int lsh_oracle_hash(int L, int d, int nh, int nb, const double *q, const double *rot,
                    int32_t *buckets /* [nh][L] */)
{
    if (L <= 0 || d <= 0 || nh <= 0 || nb < 2 || (nb & 1))
        return 1;
    const int half = nb / 2;
#pragma omp parallel
    {
        double *y = (double *)malloc(sizeof(double) * (size_t)half);
#pragma omp for collapse(2) schedule(static)
        for (int r = 0; r < nh; ++r)
            for (int t = 0; t < L; ++t) {
                for (int j = 0; j < half; ++j) {
                    double s = 0.0;
                    for (int k = 0; k < d; ++k)
                        s += q[(size_t)t * d + k] * rot[((size_t)r * d + k) * half + j];
                    y[j] = s;
                }
                buckets[(size_t)r * L + t] = argmax_concat(y, half);
            }
        free(y);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Sorting.  §2: sorting queries/keys by bucket clusters same-bucket pairs;
 * ties by position.  The composite key bucket*L + pos is unique, so the
 * ascending order of the keys is the stable sort by bucket.                  */

static int cmp_i64(const void *a, const void *b)
{
    int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x > y) - (x < y);
}

/* Round-r attended-set predicate (self included), §2 and App. A:
 * same bucket (unless bucket_mask is 0), not in the future (causal only),
 * and in the own chunk or the one before. */
static int in_round_set(int L, int m, int causal, int bucket_mask, const int32_t *bk, const int32_t *inv, int i,
                        int j)
{
    (void)L;
    if ((bucket_mask && bk[j] != bk[i]) || (causal && j > i))
        return 0;
    int ci = inv[i] / m, cj = inv[j] / m;
    return (ci - cj == 0) || (ci - cj == 1);
}

int lsh_oracle_sort(int L, int nh, int m, const int32_t *buckets, int32_t *perm, int32_t *inv,
                    int32_t *win_lo)
{
    if (L <= 0 || nh <= 0 || m <= 0 || L % m)
        return 1;
    int64_t *key = (int64_t *)malloc(sizeof(int64_t) * (size_t)L);
    for (int r = 0; r < nh; ++r) {
        const int32_t *bk = buckets + (size_t)r * L;
        int32_t *pr = perm + (size_t)r * L, *iv = inv + (size_t)r * L, *wl = win_lo + (size_t)r * L;
        for (int t = 0; t < L; ++t)
            key[t] = (int64_t)bk[t] * L + t;
        qsort(key, (size_t)L, sizeof(int64_t), cmp_i64);
        for (int s = 0; s < L; ++s) {
            pr[s] = (int32_t)(key[s] % L);
            iv[pr[s]] = s;
        }
        /* win_lo(t): the smallest sorted index of any member of A_t^r,
         * found by scanning the chunk window of t.  The causal set is used;
         * the non-causal set adds only members after t in sorted order, so
         * its smallest sorted index is the same. */
#pragma omp parallel for schedule(static)
        for (int t = 0; t < L; ++t) {
            int c = iv[t] / m;
            int lo = (c - 1) * m < 0 ? 0 : (c - 1) * m;
            int hi = (c + 1) * m > L ? L : (c + 1) * m;
            int best = iv[t];
            for (int s = lo; s < hi; ++s)
                if (in_round_set(L, m, 1, 1, bk, iv, t, pr[s]) && s < best)
                    best = s;
            wl[t] = best;
        }
    }
    free(key);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Attended sets.  App. A: a query attends to the union of its round sets; the
 * duplicate correction makes each member count once.  Candidates are the
 * members of the chunk window (own chunk and one back) of every round.
 * Writes the members of U_i \ {i} to list (capacity nh*2m) and returns their
 * number; stamp is a per-thread scratch array of L ints.                     */

static int union_set(int L, int nh, int m, int causal, int bucket_mask, const int32_t *buckets, const int32_t *perm,
                     const int32_t *inv, int i, int *stamp, int stamp_val, int32_t *list)
{
    int n = 0;
    for (int r = 0; r < nh; ++r) {
        const int32_t *bk = buckets + (size_t)r * L, *pr = perm + (size_t)r * L, *iv = inv + (size_t)r * L;
        int c = iv[i] / m;
        int lo = (c - 1) * m < 0 ? 0 : (c - 1) * m;
        int hi = (c + 1) * m > L ? L : (c + 1) * m;
        for (int s = lo; s < hi; ++s) {
            int j = pr[s];
            if (j != i && stamp[j] != stamp_val && in_round_set(L, m, causal, bucket_mask, bk, iv, i, j)) {
                stamp[j] = stamp_val;
                list[n++] = j;
            }
        }
    }
    return n;
}

/* Dense membership of U_i (self included), for tiny problems. */
int lsh_oracle_union_mask(int L, int nh, int m, int causal, int bucket_mask, const int32_t *buckets,
                          const int32_t *perm,
                          const int32_t *inv, uint8_t *mask /* [L][L] */)
{
    if (L <= 0 || nh <= 0 || m <= 0 || L % m)
        return 1;
    int *stamp = (int *)calloc((size_t)L, sizeof(int));
    int32_t *list = (int32_t *)malloc(sizeof(int32_t) * (size_t)(2 * m * nh + 1));
    memset(mask, 0, (size_t)L * L);
    for (int i = 0; i < L; ++i) {
        int n = union_set(L, nh, m, causal, bucket_mask, buckets, perm, inv, i, stamp, i + 1, list);
        mask[(size_t)i * L + i] = 1;
        for (int a = 0; a < n; ++a)
            mask[(size_t)i * L + list[a]] = 1;
    }
    free(list);
    free(stamp);
    return 0;
}

/* Weight of member j of U_i under the duplicate correction (App. A): 1, or
 * with dup_by_bucket k_ij / N_ij, k_ij = rounds whose set holds j, N_ij =
 * rounds in which j is in i's bucket. */
static double dup_weight(int L, int nh, int m, int causal, int bucket_mask, int dup_by_bucket,
                         const int32_t *buckets, const int32_t *inv, int i, int j)
{
    if (!dup_by_bucket)
        return 1.0;
    int k = 0, n = 0;
    for (int r = 0; r < nh; ++r) {
        const int32_t *bk = buckets + (size_t)r * L, *iv = inv + (size_t)r * L;
        k += in_round_set(L, m, causal, bucket_mask, bk, iv, i, j);
        n += bk[i] == bk[j];
    }
    return (double)k / (double)n;
}

static double dot(const double *a, const double *b, int d)
{
    double s = 0.0;
    for (int k = 0; k < d; ++k)
        s += a[k] * b[k];
    return s;
}

/* Keys: shared-QK attention uses k = q / |q| (§2 causal-masking bullet,
 * §5 "Shared query-key space"). */
static void make_keys(int L, int d, const double *q, double *k, double *qnorm)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < L; ++t) {
        double n = sqrt(dot(q + (size_t)t * d, q + (size_t)t * d, d));
        qnorm[t] = n;
        for (int c = 0; c < d; ++c)
            k[(size_t)t * d + c] = q[(size_t)t * d + c] / n;
    }
}

/* ------------------------------------------------------------------------- */
/* Forward.  Softmax attention of each query over U_i \ {i}; a query with an
 * empty set attends only to itself (§2 causal-masking bullet, App. A masking
 * bullet: the first token attends only to itself).                           */

int lsh_oracle_forward(int L, int d, int nh, int m, int causal, int bucket_mask, int dup_by_bucket, double scale,
                       const double *q, const double *v,
                       const int32_t *buckets, const int32_t *perm, const int32_t *inv,
                       double *out /* [L][d] */, double *lse /* [L] */)
{
    if (L <= 0 || d <= 0 || nh <= 0 || m <= 0 || L % m)
        return 1;
    double *k = (double *)malloc(sizeof(double) * (size_t)L * d);
    double *qn = (double *)malloc(sizeof(double) * (size_t)L);
    make_keys(L, d, q, k, qn);
    const int cap = 2 * m * nh + 1;
#pragma omp parallel
    {
        int *stamp = (int *)calloc((size_t)L, sizeof(int));
        int32_t *list = (int32_t *)malloc(sizeof(int32_t) * (size_t)cap);
        double *logit = (double *)malloc(sizeof(double) * (size_t)cap);
#pragma omp for schedule(dynamic, 64)
        for (int i = 0; i < L; ++i) {
            const double *qi = q + (size_t)i * d;
            double *oi = out + (size_t)i * d;
            int n = union_set(L, nh, m, causal, bucket_mask, buckets, perm, inv, i, stamp, i + 1, list);
            if (n == 0) {
                for (int c = 0; c < d; ++c)
                    oi[c] = v[(size_t)i * d + c];
                lse[i] = scale * dot(qi, k + (size_t)i * d, d);
                continue;
            }
            double mx = -INFINITY;
            for (int a = 0; a < n; ++a) {
                logit[a] = scale * dot(qi, k + (size_t)list[a] * d, d) +
                           log(dup_weight(L, nh, m, causal, bucket_mask, dup_by_bucket, buckets, inv, i, list[a]));
                if (logit[a] > mx)
                    mx = logit[a];
            }
            double den = 0.0;
            for (int a = 0; a < n; ++a)
                den += exp(logit[a] - mx);
            for (int c = 0; c < d; ++c)
                oi[c] = 0.0;
            for (int a = 0; a < n; ++a) {
                double p = exp(logit[a] - mx) / den;
                const double *vj = v + (size_t)list[a] * d;
                for (int c = 0; c < d; ++c)
                    oi[c] += p * vj[c];
            }
            lse[i] = mx + log(den);
        }
        free(logit);
        free(list);
        free(stamp);
    }
    free(qn);
    free(k);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Backward with the attended sets held fixed: no gradient through the bucket
 * assignment or the sort order (the authors, quoted in Hacker News thread
 * 22095523).  Gradient of softmax attention over U_i \ {i} with respect to q
 * (through both the query and the normalised key) and v.
 *   p_ij = exp(l_ij - lse_i), D_i = dO_i . o_i,
 *   dv_j += p_ij dO_i,   g_ij = p_ij (dO_i . v_j - D_i),
 *   dq_i += scale g_ij k_j,   dk_j += scale g_ij q_i,
 *   dQ_t = dq_t + (dk_t - k_t (k_t . dk_t)) / |q_t|,   dV = dv.
 * A query with an empty set has o_i = v_i, so dv_i += dO_i.
 * Query-side sums run over each query's set; key-side sums run over the
 * queries whose set contains the key, found through the same predicate.     */

static int in_union(int L, int nh, int m, int causal, int bucket_mask, const int32_t *buckets, const int32_t *inv,
                    int i, int j)
{
    for (int r = 0; r < nh; ++r)
        if (in_round_set(L, m, causal, bucket_mask, buckets + (size_t)r * L, inv + (size_t)r * L, i, j))
            return 1;
    return 0;
}

int lsh_oracle_backward(int L, int d, int nh, int m, int causal, int bucket_mask, int dup_by_bucket, double scale,
                        const double *q, const double *v,
                        const double *dout, const int32_t *buckets, const int32_t *perm,
                        const int32_t *inv, const double *out, const double *lse,
                        double *dq_out /* [L][d] */, double *dv_out /* [L][d] */)
{
    if (L <= 0 || d <= 0 || nh <= 0 || m <= 0 || L % m)
        return 1;
    double *k = (double *)malloc(sizeof(double) * (size_t)L * d);
    double *qn = (double *)malloc(sizeof(double) * (size_t)L);
    double *D = (double *)malloc(sizeof(double) * (size_t)L);
    uint8_t *alone = (uint8_t *)malloc((size_t)L);
    double *dk = (double *)calloc((size_t)L * d, sizeof(double));
    make_keys(L, d, q, k, qn);
    const int cap = 2 * m * nh + 1;

    /* query side: D_i, dq_i, and whether the set is empty */
#pragma omp parallel
    {
        int *stamp = (int *)calloc((size_t)L, sizeof(int));
        int32_t *list = (int32_t *)malloc(sizeof(int32_t) * (size_t)cap);
#pragma omp for schedule(dynamic, 64)
        for (int i = 0; i < L; ++i) {
            const double *qi = q + (size_t)i * d, *doi = dout + (size_t)i * d;
            double *dqi = dq_out + (size_t)i * d;
            D[i] = dot(doi, out + (size_t)i * d, d);
            for (int c = 0; c < d; ++c)
                dqi[c] = 0.0;
            int n = union_set(L, nh, m, causal, bucket_mask, buckets, perm, inv, i, stamp, i + 1, list);
            alone[i] = (uint8_t)(n == 0);
            for (int a = 0; a < n; ++a) {
                int j = list[a];
                double p = exp(scale * dot(qi, k + (size_t)j * d, d) - lse[i]) *
                           dup_weight(L, nh, m, causal, bucket_mask, dup_by_bucket, buckets, inv, i, j);
                double g = p * (dot(doi, v + (size_t)j * d, d) - D[i]);
                for (int c = 0; c < d; ++c)
                    dqi[c] += scale * g * k[(size_t)j * d + c];
            }
        }
        free(list);
        free(stamp);
    }

    /* key side: dv_j and dk_j over the queries that attend to j.  A query i
     * with j in A_i^r lies in the chunk window of j shifted forward (own
     * chunk or the next one) in round r, in either mode; every candidate is
     * re-tested with the union predicate and counted once. */
#pragma omp parallel
    {
        int *stamp = (int *)calloc((size_t)L, sizeof(int));
#pragma omp for schedule(dynamic, 64)
        for (int j = 0; j < L; ++j) {
            double *dvj = dv_out + (size_t)j * d, *dkj = dk + (size_t)j * d;
            const double *kj = k + (size_t)j * d, *vj = v + (size_t)j * d;
            for (int c = 0; c < d; ++c)
                dvj[c] = alone[j] ? dout[(size_t)j * d + c] : 0.0;
            for (int r = 0; r < nh; ++r) {
                const int32_t *pr = perm + (size_t)r * L, *iv = inv + (size_t)r * L;
                int c = iv[j] / m;
                int lo = c * m;
                int hi = (c + 2) * m > L ? L : (c + 2) * m;
                for (int s = lo; s < hi; ++s) {
                    int i = pr[s];
                    if (i == j || stamp[i] == j + 1 || !in_union(L, nh, m, causal, bucket_mask, buckets, inv, i, j))
                        continue;
                    stamp[i] = j + 1;
                    const double *qi = q + (size_t)i * d, *doi = dout + (size_t)i * d;
                    double p = exp(scale * dot(qi, kj, d) - lse[i]) *
                               dup_weight(L, nh, m, causal, bucket_mask, dup_by_bucket, buckets, inv, i, j);
                    double g = p * (dot(doi, vj, d) - D[i]);
                    for (int cc = 0; cc < d; ++cc) {
                        dvj[cc] += p * doi[cc];
                        dkj[cc] += scale * g * qi[cc];
                    }
                }
            }
        }
        free(stamp);
    }

    /* through the normalisation k = q / |q| */
#pragma omp parallel for schedule(static)
    for (int t = 0; t < L; ++t) {
        const double *kt = k + (size_t)t * d, *dkt = dk + (size_t)t * d;
        double kd = dot(kt, dkt, d);
        for (int c = 0; c < d; ++c)
            dq_out[(size_t)t * d + c] += (dkt[c] - kt[c] * kd) / qn[t];
    }
    free(dk);
    free(alone);
    free(D);
    free(qn);
    free(k);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* One (batch, head) slice end to end: hash, sort, forward and (when dout is
 * not NULL) backward.  Any output pointer may be NULL except those the later
 * stages need internally, which are then allocated here.                    */

int lsh_oracle_head(int L, int d, int nh, int nb, int m, int causal, int bucket_mask, int dup_by_bucket, double scale,
                    const double *q,
                    const double *v, const double *rot, const double *dout, int32_t *buckets,
                    int32_t *perm, int32_t *inv, int32_t *win_lo, double *out, double *lse,
                    double *dq, double *dv)
{
    if (L <= 0 || d <= 0 || nh <= 0 || nb < 2 || (nb & 1) || m <= 0 || L % m)
        return 1;
    size_t n = (size_t)nh * L;
    int32_t *bk = buckets ? buckets : (int32_t *)malloc(n * sizeof(int32_t));
    int32_t *pr = perm ? perm : (int32_t *)malloc(n * sizeof(int32_t));
    int32_t *iv = inv ? inv : (int32_t *)malloc(n * sizeof(int32_t));
    int32_t *wl = win_lo ? win_lo : (int32_t *)malloc(n * sizeof(int32_t));
    double *o = out ? out : (double *)malloc(sizeof(double) * (size_t)L * d);
    double *ls = lse ? lse : (double *)malloc(sizeof(double) * (size_t)L);
    int rc = lsh_oracle_hash(L, d, nh, nb, q, rot, bk);
    if (!rc)
        rc = lsh_oracle_sort(L, nh, m, bk, pr, iv, wl);
    if (!rc)
        rc = lsh_oracle_forward(L, d, nh, m, causal, bucket_mask, dup_by_bucket, scale, q, v, bk, pr, iv, o, ls);
    if (!rc && dout && dq && dv)
        rc = lsh_oracle_backward(L, d, nh, m, causal, bucket_mask, dup_by_bucket, scale, q, v, dout, bk, pr, iv, o,
                                 ls, dq, dv);
    if (!buckets) free(bk);
    if (!perm) free(pr);
    if (!inv) free(iv);
    if (!win_lo) free(wl);
    if (!out) free(o);
    if (!lse) free(ls);
    return rc;
}
