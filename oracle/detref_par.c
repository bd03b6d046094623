/*
 * detref_par.c -- the oracle of detref.c run over independent units on several threads.
 *
 * TEST INFRASTRUCTURE, under the same rules as detref.c: only the test suite and the
 * benchmark's CPU-baseline leg may load it; the GPU library never links, loads or calls it.
 *
 * This file includes detref.c, so every value is computed by the oracle's own functions
 * (oref_pw, tile_local, pw_pairs, segop); only which thread evaluates a unit changes, and the
 * units are independent by the readings detref.c states:
 *  - sum: PW over aligned chunks of 2^20 elements, then PW over the chunk values.  Each
 *    aligned power-of-two chunk is a subtree of PW(x) (R1: padding with more identity leaves
 *    changes nothing), so this is PW(x) itself.
 *  - scatter-add: the stable grouping by destination as a counting sort over contiguous
 *    slices of the sources (members of a destination slice by slice, which keeps ascending
 *    source index), then each destination's PW and its addition to out_init on any thread
 *    (R4: destinations share nothing).
 *  - scan: the local part of every tile on any thread, the anchor values (interval totals,
 *    super-interval carries) in order on one thread, then every tile's combine on any thread
 *    (R5: a tile's outputs depend only on its own local part and the anchor values).
 * The threads are OpenMP's (OMP_NUM_THREADS); the results are the single-threaded oracle's
 * bits, which the tests check.
 */
#include <omp.h>

#include "detref.c"

/* Number of threads an OpenMP parallel region would use here. */
int FN(opar_threads)(void) { return omp_get_max_threads(); }

/* ---------------------------------------------------------------- sum */

DET_T FN(opar_sum)(const DET_T* x, int64_t n) {
    if (n <= 0) return (DET_T)0.0; /* +0.0, as oref_sum */
    const int64_t C = (int64_t)1 << 20;
    if (n <= C) return FN(oref_pw)(x, n);
    const int64_t nc = (n + C - 1) / C;
    DET_T* v = (DET_T*)malloc((size_t)nc * sizeof(DET_T));
    if (!v) abort();
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < nc; ++c) {
        const int64_t len = (n - c * C < C) ? n - c * C : C;
        v[c] = FN(oref_pw)(x + c * C, len);
    }
    DET_T r = FN(oref_pw)(v, nc);
    free(v);
    return r;
}

/* ---------------------------------------------------------------- scatter-add */

/* As oref_scatter_add without prev: out updated in place; returns the skipped count or a
 * negative error code. */
int64_t FN(opar_scatter_add)(const DET_T* values, const int32_t* index, int64_t n,
                             int64_t row_len, DET_T* out, int64_t num_out) {
    if (n < 0 || row_len < 1 || num_out < 0) return OREF_BAD_ARG;
    /* The stable grouping as a counting sort over contiguous slices of the sources, one per
     * thread: members of destination b from slice 0 first, then slice 1, ..., each slice in
     * ascending source index, which is ascending source index overall. */
    const int nt = omp_get_max_threads();
    int64_t* start = (int64_t*)calloc((size_t)num_out + 1, sizeof(int64_t));
    int64_t* cnt = (int64_t*)calloc((size_t)nt * (size_t)(num_out > 0 ? num_out : 1),
                                    sizeof(int64_t));
    int64_t* skip = (int64_t*)calloc((size_t)nt, sizeof(int64_t));
    if (!start || !cnt || !skip) { free(start); free(cnt); free(skip); return OREF_NO_MEM; }
    const int64_t slice = (n + nt - 1) / (nt > 0 ? nt : 1);
#pragma omp parallel num_threads(nt)
    {
        const int t = omp_get_thread_num();
        int64_t* c = cnt + (int64_t)t * num_out;
        const int64_t i0 = t * slice, i1 = (i0 + slice < n) ? i0 + slice : n;
        for (int64_t i = i0; i < i1; ++i) {
            int64_t b = index[i];
            if (b < 0 || b >= num_out) { ++skip[t]; continue; }
            c[b] += 1;
        }
    }
    int64_t skipped = 0;
    for (int t = 0; t < nt; ++t) skipped += skip[t];
    /* cnt[t][b] becomes where slice t's members of b start; start[b] where b starts */
    int64_t run = 0;
    for (int64_t b = 0; b < num_out; ++b) {
        start[b] = run;
        for (int t = 0; t < nt; ++t) {
            const int64_t v = cnt[(int64_t)t * num_out + b];
            cnt[(int64_t)t * num_out + b] = run;
            run += v;
        }
    }
    start[num_out] = run;
    int64_t valid = n - skipped;
    int64_t* order = (int64_t*)malloc((size_t)(valid > 0 ? valid : 1) * sizeof(int64_t));
    if (!order) { free(start); free(cnt); free(skip); return OREF_NO_MEM; }
#pragma omp parallel num_threads(nt)
    {
        const int t = omp_get_thread_num();
        int64_t* fill = cnt + (int64_t)t * num_out;
        const int64_t i0 = t * slice, i1 = (i0 + slice < n) ? i0 + slice : n;
        for (int64_t i = i0; i < i1; ++i) {
            int64_t b = index[i];
            if (b < 0 || b >= num_out) continue;
            order[fill[b]++] = i;
        }
    }
    free(cnt); free(skip);
    int64_t maxm = 0;
    for (int64_t b = 0; b < num_out; ++b)
        if (start[b + 1] - start[b] > maxm) maxm = start[b + 1] - start[b];
    int failed = 0;
#pragma omp parallel
    {
        DET_T* col = (DET_T*)malloc((size_t)(maxm > 0 ? maxm : 1) * sizeof(DET_T));
        if (!col) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 64)
        for (int64_t b = 0; b < num_out; ++b) {
            int64_t m = start[b + 1] - start[b];
            if (m == 0 || !col) continue; /* untouched */
            for (int64_t c = 0; c < row_len; ++c) {
                for (int64_t k = 0; k < m; ++k) col[k] = values[order[start[b] + k] * row_len + c];
                out[b * row_len + c] = out[b * row_len + c] + FN(oref_pw)(col, m);
            }
        }
        free(col);
    }
    free(start); free(order);
    return failed ? OREF_NO_MEM : skipped;
}

/* ---------------------------------------------------------------- scan */

/* scan_forward_inclusive of detref.c with the tiles spread over threads. */
static int scan_forward_inclusive_par(const DET_T* x, const unsigned char* h, int64_t n,
                                      int64_t V, int64_t W, int64_t NW, int64_t A, int64_t A2,
                                      DET_T* y) {
    if (n == 0) return OREF_OK;
    const int64_t L = W * NW;
    const int64_t T = V * L;
    const int64_t nt = (n + T - 1) / T;
    const int64_t nq = (nt + A - 1) / A;
    const int64_t nQ = (nq + A2 - 1) / A2;
    const int64_t big = L > NW ? L : NW;
    pair_t* agg = (pair_t*)malloc((size_t)nt * sizeof(pair_t));
    pair_t* g = (pair_t*)malloc((size_t)nq * sizeof(pair_t));
    pair_t* cc = (pair_t*)malloc((size_t)(nQ + 1) * sizeof(pair_t));
    if (!agg || !g || !cc) { free(agg); free(g); free(cc); return OREF_NO_MEM; }
    int failed = 0;
    /* the local part of every tile: its total */
#pragma omp parallel
    {
        pair_t* s = (pair_t*)malloc((size_t)T * sizeof(pair_t));
        pair_t* u = (pair_t*)malloc((size_t)L * sizeof(pair_t));
        pair_t* tmp = (pair_t*)malloc((size_t)big * sizeof(pair_t));
        pair_t* p = (pair_t*)malloc((size_t)L * sizeof(pair_t));
        pair_t* om = (pair_t*)malloc((size_t)NW * sizeof(pair_t));
        pair_t* pw = (pair_t*)malloc((size_t)NW * sizeof(pair_t));
        const int ok = s && u && tmp && p && om && pw;
        if (!ok) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t j = 0; j < nt; ++j)
            if (ok) tile_local(x, h, n, j, V, W, NW, s, u, tmp, p, om, pw, &agg[j]);
        free(s); free(u); free(tmp); free(p); free(om); free(pw);
    }
    if (failed) { free(agg); free(g); free(cc); return OREF_NO_MEM; }
    /* the anchor values, in order */
    for (int64_t q = 0; q < nq; ++q) {
        int64_t cnt = (nt - q * A < A) ? nt - q * A : A;
        g[q] = pw_pairs(agg + q * A, cnt);
    }
    cc[0] = pair_identity();
    for (int64_t Q = 0; Q < nQ; ++Q) {
        int64_t cnt = (nq - Q * A2 < A2) ? nq - Q * A2 : A2;
        cc[Q + 1] = segop(cc[Q], pw_pairs(g + Q * A2, cnt));
    }
    /* every tile's combine */
#pragma omp parallel
    {
        pair_t* s = (pair_t*)malloc((size_t)T * sizeof(pair_t));
        pair_t* u = (pair_t*)malloc((size_t)L * sizeof(pair_t));
        pair_t* tmp = (pair_t*)malloc((size_t)big * sizeof(pair_t));
        pair_t* p = (pair_t*)malloc((size_t)L * sizeof(pair_t));
        pair_t* om = (pair_t*)malloc((size_t)NW * sizeof(pair_t));
        pair_t* pw = (pair_t*)malloc((size_t)NW * sizeof(pair_t));
        const int ok = s && u && tmp && p && om && pw;
        if (!ok) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t j = 0; j < nt; ++j) {
            if (!ok) continue;
            pair_t a;
            tile_local(x, h, n, j, V, W, NW, s, u, tmp, p, om, pw, &a);
            int64_t q = j / A;
            int64_t Q = q / A2;
            pair_t c = segop(cc[Q], pw_pairs(g + Q * A2, q - Q * A2));
            pair_t e = segop(c, pw_pairs(agg + q * A, j - q * A));
            for (int64_t t = 0; t < L; ++t) {
                pair_t xt = segop(segop(e, pw[t / W]), p[t]);
                for (int64_t k = 0; k < V; ++k) {
                    int64_t i = j * T + t * V + k;
                    if (i < n) y[i] = segop(xt, s[t * V + k]).v;
                }
            }
        }
        free(s); free(u); free(tmp); free(p); free(om); free(pw);
    }
    free(agg); free(g); free(cc);
    return failed ? OREF_NO_MEM : OREF_OK;
}

/* As oref_scan (the same arguments, checks, flips and shift), with the parallel core. */
int FN(opar_scan)(const DET_T* x, DET_T* y, int64_t n, unsigned flags, const int64_t* offsets,
                  int64_t num_segments, int64_t V, int64_t W, int64_t NW, int64_t A,
                  int64_t A2) {
    if (n < 0 || V < 1 || W < 1 || NW < 1 || A < 1 || A2 < 1 ||
        (flags & ~(OREF_EXCLUSIVE | OREF_REVERSE)))
        return OREF_BAD_ARG;
    if (offsets) {
        if (num_segments < 0 || offsets[0] != 0 || offsets[num_segments] != n) return OREF_BAD_ARG;
        for (int64_t k = 0; k < num_segments; ++k)
            if (offsets[k + 1] < offsets[k]) return OREF_BAD_ARG;
    }
    if (n == 0) return OREF_OK;
    const int rev = (flags & OREF_REVERSE) != 0;
    const int excl = (flags & OREF_EXCLUSIVE) != 0;
    DET_T* xs = (DET_T*)malloc((size_t)n * sizeof(DET_T));
    DET_T* ys = (DET_T*)malloc((size_t)n * sizeof(DET_T));
    unsigned char* h = (unsigned char*)calloc((size_t)n, 1);
    if (!xs || !ys || !h) { free(xs); free(ys); free(h); return OREF_NO_MEM; }
#pragma omp parallel for schedule(static)
    for (int64_t f = 0; f < n; ++f) xs[f] = rev ? x[n - 1 - f] : x[f];
    if (offsets) {
        for (int64_t k = 0; k <= num_segments; ++k) {
            int64_t o = offsets[k];
            if (!rev) {
                if (o < n) h[o] = 1;
            } else {
                if (o > 0) h[n - o] = 1;
            }
        }
    }
    int rc = scan_forward_inclusive_par(xs, h, n, V, W, NW, A, A2, ys);
    if (rc == OREF_OK) {
#pragma omp parallel for schedule(static)
        for (int64_t f = 0; f < n; ++f) {
            DET_T v;
            if (!excl) v = ys[f];
            else v = (f == 0 || h[f]) ? (DET_T)0.0 : ys[f - 1];
            y[rev ? n - 1 - f : f] = v;
        }
    }
    free(xs); free(ys); free(h);
    return rc;
}
