/*
 * oracle.c -- plain, slow, obviously-correct CPU oracle for the Split-KV
 * per-device hot path.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the package's smoke check and
 * the CPU-baseline leg of the benchmark load this library. The product path
 * never calls it, and this file shares no code, header or constant with the
 * HIP library.
 *
 * Source: "Split-KV: Efficient Context Parallelism for Training Diffusion
 * Drafters" (arXiv 2611.05926v1):
 *   Eq. 1/Eq. 2 (§3.3)  causal and anchor load profiles c(x)
 *   Eq. 3 (§4.1)        per-rank masked partial attention and its LSE
 *   Eq. 4 (§4.1)        exact LSE merge of the partials
 *   Algorithm 1 (§4.1)  backward: AttnBwd_p after MERGE_BWD
 *   Eq. 6 (§4.2)        chunk cost; the cost-aware LPT rule with J per rank
 *   §4.2 (balance)      D = (N/P) B^2, W_p = C_p + D, rho = max W / mean W
 *   §3.3, Figure 5(b)   Zigzag: 2P chunks per sample, rank p gets p and 2P-1-p
 *   §4.1, Algorithm 1   MERGE in per-rank form: LSE reduction, then rescaling
 *   §3.1, Figure 1      a valid anchor window lies inside the packed context
 *   §4.2 (placement)    locality matching of the LPT bundles to physical ranks
 *
 * Floating point is fp64 throughout, inputs included: the tests widen the exact
 * bf16/fp32 values the GPU consumed to fp64 before calling in.
 * Integer work is int64. OpenMP parallelises independent outputs only; every
 * output is computed by one plain sequential loop.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define EXPORT __attribute__((visibility("default")))

/* Threads the parallel loops below use (1 without OpenMP). */
EXPORT int oracle_omp_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int64_t max64(int64_t x, int64_t y) { return x > y ? x : y; }
static int64_t min64(int64_t x, int64_t y) { return x < y ? x : y; }

/* ------------------------------------------------------------------------- */
/* §3.1, Figure 1: block i's rows see the context window [s_i, a_i) of their   */
/* sample, a sub-interval of the packed context [0, S) (empty allowed).        */
/* out = {number of blocks violating 0 <= s_i <= a_i <= S, first such i or -1}. */
/* ------------------------------------------------------------------------- */
EXPORT void oracle_validate_anchors(int64_t n_blocks, const int64_t* s, const int64_t* a,
                                    int64_t S, int64_t* out) {
    int64_t bad = 0, first = -1;
    for (int64_t i = 0; i < n_blocks; ++i) {
        int ok = 0 <= s[i] && s[i] <= a[i] && a[i] <= S;
        if (!ok) {
            if (first < 0) first = i;
            bad += 1;
        }
    }
    out[0] = bad;
    out[1] = first;
}

/* ------------------------------------------------------------------------- */
/* Eq. 2: c(x) = B * #{ i : s_i <= x < a_i }, x in [0, S). Brute force.       */
/* ------------------------------------------------------------------------- */
EXPORT void oracle_anchor_profile(int64_t n_blocks, const int64_t* s, const int64_t* a,
                                  int64_t B, int64_t S, int64_t* prof) {
#pragma omp parallel for schedule(static)
    for (int64_t x = 0; x < S; ++x) {
        int64_t cnt = 0;
        for (int64_t i = 0; i < n_blocks; ++i)
            if (s[i] <= x && x < a[i]) cnt += 1;
        prof[x] = B * cnt;
    }
}

/* ------------------------------------------------------------------------- */
/* Eq. 6: c_j = B * sum_i ( min(a_i, lam_j + m) - max(s_i, lam_j) )^+,       */
/* with lam_j = j*m the left boundary of global chunk j.                     */
/* ------------------------------------------------------------------------- */
EXPORT void oracle_chunk_costs(int64_t n_blocks, const int64_t* s, const int64_t* a,
                               int64_t B, int64_t n_chunks, int64_t m, int64_t* cost) {
    for (int64_t j = 0; j < n_chunks; ++j) {
        int64_t lam = j * m, total = 0;
        for (int64_t i = 0; i < n_blocks; ++i) {
            int64_t overlap = min64(a[i], lam + m) - max64(s[i], lam);
            if (overlap > 0) total += overlap;
        }
        cost[j] = B * total;
    }
}

/* Second form of Eq. 6 through the cumulative load
 * C(y) = B * sum_i ( min(a_i, y) - s_i )^+ = sum_{x<y} c(x) (for s_i <= a_i):
 * c_j = C(lam_j + m) - C(lam_j). Must agree with the direct form bit-exactly. */
static int64_t cumulative_load(int64_t n_blocks, const int64_t* s, const int64_t* a,
                               int64_t B, int64_t y) {
    int64_t total = 0;
    for (int64_t i = 0; i < n_blocks; ++i) {
        int64_t len = min64(a[i], y) - s[i];
        if (len > 0) total += len;
    }
    return B * total;
}

EXPORT void oracle_chunk_costs_prefix(int64_t n_blocks, const int64_t* s, const int64_t* a,
                                      int64_t B, int64_t n_chunks, int64_t m, int64_t* cost) {
    for (int64_t j = 0; j < n_chunks; ++j)
        cost[j] = cumulative_load(n_blocks, s, a, B, (j + 1) * m) -
                  cumulative_load(n_blocks, s, a, B, j * m);
}

/* ------------------------------------------------------------------------- */
/* §4.2 cost-aware LPT: sort chunks by cost (highest first); repeatedly give  */
/* the costliest remaining chunk to the least-loaded rank holding fewer than  */
/* J chunks. Ties: equal costs go in ascending chunk index; equal loads go to  */
/* the lowest rank index. bundles[p] lists rank p's chunks in ascending index. */
/* Returns 0, or -1 if n_chunks != P*J.                                       */
/* ------------------------------------------------------------------------- */
static const int64_t* g_sort_cost; /* qsort has no context argument */

static int by_cost_desc(const void* x, const void* y) {
    int64_t i = *(const int64_t*)x, j = *(const int64_t*)y;
    if (g_sort_cost[i] != g_sort_cost[j]) return g_sort_cost[i] > g_sort_cost[j] ? -1 : 1;
    return i < j ? -1 : (i > j ? 1 : 0);
}

EXPORT int oracle_lpt(int64_t n_chunks, const int64_t* cost, int32_t P, int32_t J,
                      int32_t* owner, int32_t* bundles, int64_t* load) {
    if (P <= 0 || J <= 0 || n_chunks != (int64_t)P * J) return -1;
    int64_t* order = (int64_t*)malloc(sizeof(int64_t) * n_chunks);
    int32_t* count = (int32_t*)calloc(P, sizeof(int32_t));
    for (int64_t j = 0; j < n_chunks; ++j) order[j] = j;
    g_sort_cost = cost;
    qsort(order, n_chunks, sizeof(int64_t), by_cost_desc);
    for (int32_t p = 0; p < P; ++p) load[p] = 0;

    for (int64_t t = 0; t < n_chunks; ++t) {
        int64_t j = order[t];
        int32_t best = -1;
        for (int32_t p = 0; p < P; ++p) {
            if (count[p] >= J) continue;
            if (best < 0 || load[p] < load[best]) best = p;
        }
        owner[j] = best;
        load[best] += cost[j];
        count[best] += 1;
    }
    for (int32_t p = 0; p < P; ++p) count[p] = 0;
    for (int64_t j = 0; j < n_chunks; ++j) {
        int32_t p = owner[j];
        bundles[(int64_t)p * J + count[p]] = (int32_t)j;
        count[p] += 1;
    }
    free(order);
    free(count);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Locality matching (§4.2): the LPT bundles are placed on physical ranks     */
/* without changing their loads, keeping as many context rows in place as     */
/* possible. Reading: before the step's all-to-all, physical rank r holds the */
/* r-th of P equal contiguous parts of [0, S), S = P*J*m, so chunk j starts   */
/* on rank j / J. keep[b][r] = m * #{ chunks j of bundle b : j / J == r }.    */
/* The placement maximises sum_b keep[b][perm[b]]: a linear assignment       */
/* problem, solved exactly by the Hungarian method with row and column        */
/* potentials on the cost J*m - keep >= 0 (rows = bundles, columns = ranks;   */
/* the constant leaves the best placement unchanged; each row                 */
/* enters by a shortest augmenting path; of equal reduced costs the lowest    */
/* column is taken). Outputs: perm[b] = physical rank of bundle b; send[src*P */
/* + dst] = rows rank src sends to rank dst (m per chunk of the bundle placed */
/* on dst whose home is src != dst); kept_moved = {rows in place, S - kept}.  */
/* Chunk ids outside [0, P*J) count as neither kept nor sent.                 */
/* ------------------------------------------------------------------------- */
static int64_t keep_rows(const int32_t* bundles, int32_t J, int64_t m, int32_t PJ, int32_t b,
                         int32_t r) {
    int64_t n = 0;
    for (int32_t k = 0; k < J; ++k) {
        int32_t j = bundles[(int64_t)b * J + k];
        if (j >= 0 && j < PJ && j / J == r) n += 1;
    }
    return n * m;
}

/* The all-to-all of one placement (any permutation perm: bundle b runs on   */
/* physical rank perm[b]), by the definition: every chunk j of bundle b lives  */
/* on rank j / J before the step and on rank perm[b] after it, so its m rows   */
/* stay in place when the two agree and are sent from j / J to perm[b]        */
/* otherwise. send[src*P + dst] = rows sent from src to dst (zero diagonal);   */
/* kept_moved = {rows in place, P*J*m - rows in place}. Chunk ids outside     */
/* [0, P*J) count as neither kept nor sent. Returns -1 when perm is not a     */
/* permutation of 0 .. P-1.                                                   */
EXPORT int oracle_placement_rows(const int32_t* bundles, int32_t P, int32_t J, int64_t m,
                                 const int32_t* perm, int64_t* send, int64_t* kept_moved) {
    if (P <= 0 || J <= 0 || m <= 0) return -1;
    char* seen = (char*)calloc(P, 1);
    for (int32_t b = 0; b < P; ++b) {
        if (perm[b] < 0 || perm[b] >= P || seen[perm[b]]) { free(seen); return -1; }
        seen[perm[b]] = 1;
    }
    free(seen);
    const int32_t PJ = P * J;
    for (int64_t x = 0; x < (int64_t)P * P; ++x) send[x] = 0;
    int64_t kept = 0;
    for (int32_t b = 0; b < P; ++b) {
        int32_t dst = perm[b];
        for (int32_t k = 0; k < J; ++k) {
            int32_t j = bundles[(int64_t)b * J + k];
            if (j < 0 || j >= PJ) continue;
            int32_t src = j / J;
            if (src == dst) kept += m;
            else send[(int64_t)src * P + dst] += m;
        }
    }
    kept_moved[0] = kept;
    kept_moved[1] = (int64_t)PJ * m - kept;
    return 0;
}

EXPORT int oracle_locality_match(const int32_t* bundles, int32_t P, int32_t J, int64_t m,
                                 int32_t* perm, int64_t* send, int64_t* kept_moved) {
    if (P <= 0 || J <= 0 || m <= 0) return -1;
    const int32_t PJ = P * J;
    const int64_t INF = INT64_MAX / 4;
    int64_t* u = (int64_t*)calloc(P + 1, sizeof(int64_t));
    int64_t* v = (int64_t*)calloc(P + 1, sizeof(int64_t));
    int64_t* minv = (int64_t*)malloc(sizeof(int64_t) * (P + 1));
    int32_t* match = (int32_t*)calloc(P + 1, sizeof(int32_t)); /* column -> row, 0 = free */
    int32_t* way = (int32_t*)calloc(P + 1, sizeof(int32_t));
    char* used = (char*)malloc(P + 1);
    for (int32_t i = 1; i <= P; ++i) {
        match[0] = i;
        int32_t j0 = 0;
        for (int32_t j = 0; j <= P; ++j) { minv[j] = INF; used[j] = 0; }
        do {
            used[j0] = 1;
            int32_t i0 = match[j0], j1 = 0;
            int64_t delta = INF;
            for (int32_t j = 1; j <= P; ++j) {
                if (used[j]) continue;
                int64_t cur = (int64_t)J * m - keep_rows(bundles, J, m, PJ, i0 - 1, j - 1) - u[i0] - v[j];
                if (cur < minv[j]) { minv[j] = cur; way[j] = j0; }
                if (minv[j] < delta) { delta = minv[j]; j1 = j; }
            }
            for (int32_t j = 0; j <= P; ++j) {
                if (used[j]) { u[match[j]] += delta; v[j] -= delta; }
                else minv[j] -= delta;
            }
            j0 = j1;
        } while (match[j0] != 0);
        do {
            int32_t j1 = way[j0];
            match[j0] = match[j1];
            j0 = j1;
        } while (j0 != 0);
    }
    for (int32_t j = 1; j <= P; ++j) perm[match[j] - 1] = j - 1;
    free(u); free(v); free(minv); free(match); free(way); free(used);
    return oracle_placement_rows(bundles, P, J, m, perm, send, kept_moved);
}

/* ------------------------------------------------------------------------- */
/* Comparators (§3.3, Figure 5(b); §5.3 "No balance")                         */
/* ------------------------------------------------------------------------- */
/* Zigzag: each sample u (start st_u, length len_u, divisible by 2P) is cut   */
/* into 2P equal chunks; rank p receives chunks p and 2P-1-p of every sample. */
/* load_p = sum of the profile over those positions. Returns -1 if a length   */
/* is not divisible by 2P.                                                    */
EXPORT int oracle_zigzag_loads(int64_t n_samples, const int64_t* st, const int64_t* len,
                               const int64_t* prof, int32_t P, int64_t* load) {
    for (int32_t p = 0; p < P; ++p) load[p] = 0;
    for (int64_t u = 0; u < n_samples; ++u) {
        if (len[u] % (2 * P) != 0) return -1;
        int64_t w = len[u] / (2 * P);
        for (int32_t p = 0; p < P; ++p) {
            int64_t first = st[u] + (int64_t)p * w;
            int64_t second = st[u] + (int64_t)(2 * P - 1 - p) * w;
            for (int64_t x = 0; x < w; ++x) load[p] += prof[first + x] + prof[second + x];
        }
    }
    return 0;
}

/* No balance: rank p receives the contiguous range [p*S/P, (p+1)*S/P). */
EXPORT int oracle_contiguous_loads(int64_t S, const int64_t* prof, int32_t P, int64_t* load) {
    if (S % P != 0) return -1;
    int64_t w = S / P;
    for (int32_t p = 0; p < P; ++p) {
        load[p] = 0;
        for (int64_t x = 0; x < w; ++x) load[p] += prof[(int64_t)p * w + x];
    }
    return 0;
}

/* Both comparators as explicit ranges, in the order the product reports them */
/* (strategy 0 = No balance, 1 = Zigzag):                                    */
/*   No balance: range p = [p*S/P, (p+1)*S/P) owned by rank p, S = sum len.   */
/*   Zigzag: range u*2P + c = chunk c of sample u, owned by rank c if c < P,  */
/*   else by rank 2P-1-c.                                                     */
/* A range's cost is the sum of the profile over its positions; a rank's     */
/* load is the sum of its ranges' costs. The samples are packed in order     */
/* (st[u] = sum of the earlier lengths). Returns the number of ranges R, or  */
/* -1 if a length does not divide.                                           */
EXPORT int64_t oracle_baseline_plan(int32_t strategy, int64_t n_samples, const int64_t* st,
                                    const int64_t* len, const int64_t* prof, int32_t P,
                                    int64_t* range_cost, int64_t* load) {
    int64_t S = 0;
    for (int64_t u = 0; u < n_samples; ++u) S += len[u];
    for (int32_t p = 0; p < P; ++p) load[p] = 0;
    if (strategy == 0) {
        if (S % P != 0) return -1;
        int64_t w = S / P;
        for (int32_t p = 0; p < P; ++p) {
            int64_t c = 0;
            for (int64_t x = (int64_t)p * w; x < (int64_t)(p + 1) * w; ++x) c += prof[x];
            range_cost[p] = c;
            load[p] += c;
        }
        return P;
    }
    for (int64_t u = 0; u < n_samples; ++u)
        if (len[u] % (2 * P) != 0) return -1;
    for (int64_t u = 0; u < n_samples; ++u) {
        int64_t w = len[u] / (2 * P);
        for (int32_t c = 0; c < 2 * P; ++c) {
            int32_t owner = c < P ? c : 2 * P - 1 - c;
            int64_t lo = st[u] + (int64_t)c * w, cost = 0;
            for (int64_t x = lo; x < lo + w; ++x) cost += prof[x];
            range_cost[u * 2 * P + c] = cost;
            load[owner] += cost;
        }
    }
    return 2 * (int64_t)P * n_samples;
}

/* §4.2: W_p = C_p + D with D = (N/P) B^2; rho = max_p W_p / mean_p W_p. */
EXPORT double oracle_imbalance(int32_t P, const int64_t* ctx_load, int64_t n_blocks, int64_t B) {
    double D = (double)n_blocks / (double)P * (double)(B * B);
    double mx = -INFINITY, sum = 0.0;
    for (int32_t p = 0; p < P; ++p) {
        double w = (double)ctx_load[p] + D;
        if (w > mx) mx = w;
        sum += w;
    }
    return mx / (sum / (double)P);
}

/* ------------------------------------------------------------------------- */
/* Eq. 3: partial attention of selected query rows against a key set.         */
/*                                                                            */
/* rows[n_sel]: packed query-row indices; row r belongs to block r / B, whose */
/*   window is [s_i, a_i). q_sel [n_sel, hq, d] holds those rows' queries.    */
/* key_pos[n_keys]: global context position of each key row of k, v          */
/*   ([n_keys, hkv, d]). Query head h reads key/value head h / (hq/hkv).      */
/* For each (row, h): live keys X = { x : s_i <= key_pos[x] < a_i }.          */
/*   X empty -> o = 0, lse = -inf.                                            */
/*   else z_x = scale * <q, k_x>, lse = log sum_x exp(z_x),                   */
/*        o = sum_x exp(z_x - lse) v_x.                                       */
/* Outputs o [n_sel, hq, d], lse [n_sel, hq] in fp64.                         */
/* ------------------------------------------------------------------------- */
EXPORT void oracle_partial_attn(int64_t n_sel, const int64_t* rows, int64_t B,
                                const int64_t* s, const int64_t* a,
                                int32_t hq, int32_t hkv, int32_t d, double scale,
                                const double* q_sel, int64_t n_keys, const int64_t* key_pos,
                                const double* k, const double* v, double* o, double* lse) {
    int32_t group = hq / hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t t = 0; t < n_sel; ++t) {
        for (int32_t h = 0; h < hq; ++h) {
            int64_t blk = rows[t] / B;
            int64_t lo = s[blk], hi = a[blk];
            int32_t g = h / group;
            const double* qv = q_sel + (t * hq + h) * (int64_t)d;
            double* ov = o + (t * hq + h) * (int64_t)d;
            double* z = (double*)malloc(sizeof(double) * (n_keys > 0 ? n_keys : 1));
            double zmax = -INFINITY;
            int64_t live = 0;
            for (int64_t x = 0; x < n_keys; ++x) {
                if (key_pos[x] < lo || key_pos[x] >= hi) continue;
                const double* kv = k + (x * hkv + g) * (int64_t)d;
                double dot = 0.0;
                for (int32_t c = 0; c < d; ++c) dot += qv[c] * kv[c];
                z[x] = dot * scale;
                if (z[x] > zmax) zmax = z[x];
                live += 1;
            }
            for (int32_t c = 0; c < d; ++c) ov[c] = 0.0;
            if (live == 0) {
                lse[t * hq + h] = -INFINITY;
                free(z);
                continue;
            }
            double sum = 0.0;
            for (int64_t x = 0; x < n_keys; ++x)
                if (key_pos[x] >= lo && key_pos[x] < hi) sum += exp(z[x] - zmax);
            double l = zmax + log(sum);
            for (int64_t x = 0; x < n_keys; ++x) {
                if (key_pos[x] < lo || key_pos[x] >= hi) continue;
                double p = exp(z[x] - l);
                const double* vv = v + (x * hkv + g) * (int64_t)d;
                for (int32_t c = 0; c < d; ++c) ov[c] += p * vv[c];
            }
            lse[t * hq + h] = l;
            free(z);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Eq. 4: l = log sum_p exp(l_p); o = sum_p exp(l_p - l) o_p.                 */
/* o_parts [P, rows, d], lse_parts [P, rows]. Partials with l_p = -inf        */
/* contribute nothing; if every partial of a row is empty -> (0, -inf).       */
/* ------------------------------------------------------------------------- */
EXPORT void oracle_merge(int32_t P, int64_t rows, int32_t d, const double* o_parts,
                         const double* lse_parts, double* o, double* lse) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double mx = -INFINITY;
        for (int32_t p = 0; p < P; ++p)
            if (lse_parts[(int64_t)p * rows + r] > mx) mx = lse_parts[(int64_t)p * rows + r];
        double* orow = o + r * d;
        for (int32_t c = 0; c < d; ++c) orow[c] = 0.0;
        if (mx == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double sum = 0.0;
        for (int32_t p = 0; p < P; ++p) {
            double lp = lse_parts[(int64_t)p * rows + r];
            if (lp != -INFINITY) sum += exp(lp - mx);
        }
        double l = mx + log(sum);
        for (int32_t p = 0; p < P; ++p) {
            double lp = lse_parts[(int64_t)p * rows + r];
            if (lp == -INFINITY) continue;
            double w = exp(lp - l);
            const double* op = o_parts + ((int64_t)p * rows + r) * d;
            for (int32_t c = 0; c < d; ++c) orow[c] += w * op[c];
        }
        lse[r] = l;
    }
}

/* ------------------------------------------------------------------------- */
/* Algorithm 1, MERGE_BWD: the global per-(row, head) statistic               */
/* Delta = <do, o> with o the merged (globally normalised) output.            */
/* ------------------------------------------------------------------------- */
/* ------------------------------------------------------------------------- */
/* Eq. 4 in the two halves each rank applies in Algorithm 1's MERGE when the  */
/* partials live on different devices: the LSE statistics are reduced first   */
/* (lse = log sum_p exp lse_p, all -inf gives -inf), then each rank rescales  */
/* its own partial, o_bar_p = exp(lse_p - lse) o_p (0 where lse_p = -inf).    */
/* Summed over p, the o_bar_p are the merged output.                          */
/* ------------------------------------------------------------------------- */
EXPORT void oracle_lse_reduce(int32_t P, int64_t rows, const double* lse_parts, double* lse) {
    for (int64_t r = 0; r < rows; ++r) {
        double mx = -INFINITY;
        for (int32_t p = 0; p < P; ++p)
            if (lse_parts[(int64_t)p * rows + r] > mx) mx = lse_parts[(int64_t)p * rows + r];
        if (mx == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double sum = 0.0;
        for (int32_t p = 0; p < P; ++p) sum += exp(lse_parts[(int64_t)p * rows + r] - mx);
        lse[r] = mx + log(sum);
    }
}

EXPORT void oracle_lse_rescale(int64_t rows, int32_t d, const double* o_part,
                               const double* lse_part, const double* lse, double* o_bar) {
    for (int64_t r = 0; r < rows; ++r) {
        double w = lse_part[r] == -INFINITY ? 0.0 : exp(lse_part[r] - lse[r]);
        for (int32_t c = 0; c < d; ++c) o_bar[r * d + c] = w * o_part[r * d + c];
    }
}

EXPORT void oracle_delta(int64_t rows, int32_t hq, int32_t d, const double* o,
                         const double* dout, double* delta) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows * hq; ++r) {
        double acc = 0.0;
        for (int32_t c = 0; c < d; ++c) acc += o[r * d + c] * dout[r * d + c];
        delta[r] = acc;
    }
}

/* ------------------------------------------------------------------------- */
/* Algorithm 1, AttnBwd_p: gradient of the masked attention restricted to the */
/* local keys, given the global lse and Delta. For a live pair (row r, head h,*/
/* key x, kv head g = h / (hq/hkv)):                                          */
/*   z = scale <q, k_x>;  P = exp(z - lse[r,h]);                              */
/*   dv_x += P * do;  dp = <do, v_x>;  ds = P * (dp - Delta[r,h]);            */
/*   dq_r += scale * ds * k_x;  dk_x += scale * ds * q_r.                     */
/* Rows with lse = -inf contribute nothing.                                   */
/*                                                                            */
/* q, dout: [Q, hq, d] for ALL rows; lse, delta: [Q, hq]; k, v: [n_keys, hkv,  */
/* d] with key_pos as in oracle_partial_attn. dq is produced for the rows     */
/* listed in dq_rows ([n_dq, hq, d]); dk, dv for the keys listed in dkv_keys  */
/* ([n_dkv, hkv, d]).                                                         */
/* ------------------------------------------------------------------------- */
EXPORT void oracle_attn_bwd(int64_t Q, int64_t B, const int64_t* s, const int64_t* a,
                            int32_t hq, int32_t hkv, int32_t d, double scale,
                            const double* q, const double* dout, const double* lse,
                            const double* delta, int64_t n_keys, const int64_t* key_pos,
                            const double* k, const double* v,
                            int64_t n_dq, const int64_t* dq_rows, double* dq,
                            int64_t n_dkv, const int64_t* dkv_keys, double* dk, double* dv) {
    int32_t group = hq / hkv;
    /* dq for the selected rows: sum over live local keys. */
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t t = 0; t < n_dq; ++t) {
        for (int32_t h = 0; h < hq; ++h) {
            int64_t r = dq_rows[t];
            int64_t blk = r / B;
            int32_t g = h / group;
            double* out = dq + (t * hq + h) * (int64_t)d;
            for (int32_t c = 0; c < d; ++c) out[c] = 0.0;
            double l = lse[r * hq + h];
            if (l == -INFINITY) continue;
            const double* qv = q + (r * hq + h) * (int64_t)d;
            const double* gv = dout + (r * hq + h) * (int64_t)d;
            for (int64_t x = 0; x < n_keys; ++x) {
                if (key_pos[x] < s[blk] || key_pos[x] >= a[blk]) continue;
                const double* kv = k + (x * hkv + g) * (int64_t)d;
                const double* vv = v + (x * hkv + g) * (int64_t)d;
                double dot = 0.0, dp = 0.0;
                for (int32_t c = 0; c < d; ++c) {
                    dot += qv[c] * kv[c];
                    dp += gv[c] * vv[c];
                }
                double P = exp(dot * scale - l);
                double ds = P * (dp - delta[r * hq + h]);
                for (int32_t c = 0; c < d; ++c) out[c] += scale * ds * kv[c];
            }
        }
    }
    /* dk, dv for the selected keys: sum over all rows and heads that read them. */
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t t = 0; t < n_dkv; ++t) {
        for (int32_t g = 0; g < hkv; ++g) {
            int64_t x = dkv_keys[t];
            const double* kv = k + (x * hkv + g) * (int64_t)d;
            const double* vv = v + (x * hkv + g) * (int64_t)d;
            double* dko = dk + (t * hkv + g) * (int64_t)d;
            double* dvo = dv + (t * hkv + g) * (int64_t)d;
            for (int32_t c = 0; c < d; ++c) dko[c] = dvo[c] = 0.0;
            for (int64_t r = 0; r < Q; ++r) {
                int64_t blk = r / B;
                if (key_pos[x] < s[blk] || key_pos[x] >= a[blk]) continue;
                for (int32_t h = g * group; h < (g + 1) * group; ++h) {
                    double l = lse[r * hq + h];
                    if (l == -INFINITY) continue;
                    const double* qv = q + (r * hq + h) * (int64_t)d;
                    const double* gv = dout + (r * hq + h) * (int64_t)d;
                    double dot = 0.0, dp = 0.0;
                    for (int32_t c = 0; c < d; ++c) {
                        dot += qv[c] * kv[c];
                        dp += gv[c] * vv[c];
                    }
                    double P = exp(dot * scale - l);
                    double ds = P * (dp - delta[r * hq + h]);
                    for (int32_t c = 0; c < d; ++c) {
                        dvo[c] += P * gv[c];
                        dko[c] += scale * ds * qv[c];
                    }
                }
            }
        }
    }
}
