/*
 * detref.c -- plain CPU oracle for reproducible floating-point add-reductions.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load this code.  The GPU library never links, loads or
 * calls it, and the two share no source, header, table or constant.
 *
 * It states the association order as directly as the arithmetic allows:
 * single-threaded loops, one IEEE addition at a time, no blocking, no fusion.
 * The file is compiled twice, once with DET_T=float / DET_SUF=_f32 and once
 * with DET_T=double / DET_SUF=_f64.  Required flags: -O2 -ffp-contract=off,
 * no -ffast-math, SSE2 scalar arithmetic (the x86-64 default), so every "+"
 * below is one binary32 / binary64 addition rounded to nearest-even with
 * subnormals kept.
 *
 * Sources (pages on one subject, cited by title and section):
 *  - "Floating point and reproducibility" (GPU course, day 68), sections
 *    "Twenty answers, none of them wrong" and "Contracts from tolerance to fixed
 *    bits": a sum is one parenthesisation; a fixed bracket over pairs fixes it.
 *  - Warp user guide "Deterministic Execution", sections "Pattern 1: Accumulation",
 *    "Writing Manual Deterministic Code" and "Picking the Right Mode": records are
 *    grouped by destination in a stable order (ascending thread index) and each
 *    group is reduced in a fixed order.
 *  - Warp reference "warp.tile_atomic_add_indexed": row-indexed accumulate along
 *    axis 0, out-of-range destinations skipped, previous values returned.
 *  - drjit-core pull request "Make CUDA floating-point prefix sums deterministic",
 *    sections "Implementation" and "Validation": single-pass look-back where the
 *    carry only passes through fixed anchor intervals, for inclusive/exclusive,
 *    forward/reverse, full and segmented scans.
 *
 * Where the pages leave a step open, this file takes these readings:
 *  R1  PW(v): pad v with the identity to a power of two, then repeatedly replace
 *      the list by the sums of adjacent pairs (v0+v1, v2+v3, ...) until one value
 *      remains.  PW of an empty list is the identity.
 *  R2  The identity is -0.0: (-0.0) + a == a for every a, including +0.0.
 *  R3  sum(x) = PW(x) for n >= 1 and +0.0 for n == 0.
 *  R4  scatter-add: for destination r and column c, M = the contributions in
 *      ascending source index; if M is non-empty out = out_init + PW(M), else out
 *      is left untouched.  Indices outside [0, num_out) are skipped and counted.
 *      prev[i] is out_init at i's destination (snapshot before the call).
 *  R5  scan tile / wave / lane / anchor layout, see scan_forward_inclusive below
 *      (V, W, NW, A, A2 are parameters so tiny instances can be checked by hand and by
 *      brute force).  Anchors are two-level: every interval of A tiles publishes its
 *      total, every super-interval of A2 intervals carries the running prefix.
 *  R6  exclusive = inclusive shifted by one with +0.0 entering at every segment
 *      head; reverse = flip, forward scan, flip; segments via head flags and the
 *      standard segmented operator (flag_a|flag_b, flag_b ? b : a+b).
 *  R7  running prev (what a loop of atomic adds in ascending source index would hand
 *      back, with the sums it holds formed in a fixed order): lay the members of every
 *      destination (ascending source index, R4) end to end in destination order, one
 *      segment per destination, and scan each column of that array exclusively (R5/R6,
 *      forward).  The member at position g with source row i and destination r gets
 *      prev[i][c] = out_init[r][c] when g is its destination's first position, else
 *      out_init[r][c] + E[g].  out is updated as in R4.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef DET_T
#error "compile with -DDET_T=float|double -DDET_SUF=_f32|_f64"
#endif

#define CAT2(a, b) a##b
#define CAT(a, b) CAT2(a, b)
#define FN(name) CAT(name, DET_SUF)

/* Return codes of the oracle (its own, unrelated to the GPU library's). */
#define OREF_OK 0
#define OREF_BAD_ARG (-1)
#define OREF_NO_MEM (-2)

#define OREF_EXCLUSIVE 1u
#define OREF_REVERSE 2u

static DET_T identity(void) { return (DET_T)(-0.0); }

/* ---------------------------------------------------------------- R1: PW */

/* Pairwise tree over v[0..m): pad to the next power of two with the identity,
 * then halve by adjacent pairs until one value remains. */
DET_T FN(oref_pw)(const DET_T* v, int64_t m) {
    if (m <= 0) return identity();
    if (m == 1) return v[0];
    int64_t p = 1;
    while (p < m) p *= 2;
    /* first level read straight from v, so the buffer is half the padded size */
    int64_t h = p / 2;
    DET_T* buf = (DET_T*)malloc((size_t)h * sizeof(DET_T));
    if (!buf) abort();
    for (int64_t i = 0; i < h; ++i) {
        DET_T a = (2 * i < m) ? v[2 * i] : identity();
        DET_T b = (2 * i + 1 < m) ? v[2 * i + 1] : identity();
        buf[i] = a + b;
    }
    for (int64_t len = h; len > 1; len /= 2)
        for (int64_t i = 0; i < len / 2; ++i) buf[i] = buf[2 * i] + buf[2 * i + 1];
    DET_T r = buf[0];
    free(buf);
    return r;
}

/* ---------------------------------------------------------------- R3: sum */

DET_T FN(oref_sum)(const DET_T* x, int64_t n) {
    if (n <= 0) return (DET_T)0.0; /* +0.0 */
    return FN(oref_pw)(x, n);
}

/* ---------------------------------------------------------------- R4: scatter-add */

/* values: [n * row_len] row-major; index: [n]; out: [num_out * row_len], updated in
 * place; prev: NULL or [n * row_len].  Returns the number of skipped source rows,
 * or a negative error code. */
int64_t FN(oref_scatter_add)(const DET_T* values, const int32_t* index, int64_t n,
                             int64_t row_len, DET_T* out, int64_t num_out, DET_T* prev) {
    if (n < 0 || row_len < 1 || num_out < 0) return OREF_BAD_ARG;
    int64_t skipped = 0;
    int64_t* start = (int64_t*)calloc((size_t)num_out + 1, sizeof(int64_t));
    if (!start) return OREF_NO_MEM;
    /* count members per destination */
    for (int64_t i = 0; i < n; ++i) {
        int64_t b = index[i];
        if (b < 0 || b >= num_out) { ++skipped; continue; }
        start[b + 1] += 1;
    }
    for (int64_t b = 0; b < num_out; ++b) start[b + 1] += start[b];
    /* stable grouping: members of each destination in ascending source index */
    int64_t valid = n - skipped;
    int64_t* order = (int64_t*)malloc((size_t)(valid > 0 ? valid : 1) * sizeof(int64_t));
    int64_t* fill = (int64_t*)malloc((size_t)(num_out > 0 ? num_out : 1) * sizeof(int64_t));
    if (!order || !fill) { free(start); free(order); free(fill); return OREF_NO_MEM; }
    for (int64_t b = 0; b < num_out; ++b) fill[b] = start[b];
    for (int64_t i = 0; i < n; ++i) {
        int64_t b = index[i];
        if (b < 0 || b >= num_out) continue;
        order[fill[b]++] = i;
    }
    /* snapshot of the destination before any addition */
    if (prev) {
        for (int64_t i = 0; i < n; ++i) {
            int64_t b = index[i];
            if (b < 0 || b >= num_out) continue;
            for (int64_t c = 0; c < row_len; ++c) prev[i * row_len + c] = out[b * row_len + c];
        }
    }
    int64_t maxm = 0;
    for (int64_t b = 0; b < num_out; ++b)
        if (start[b + 1] - start[b] > maxm) maxm = start[b + 1] - start[b];
    DET_T* col = (DET_T*)malloc((size_t)(maxm > 0 ? maxm : 1) * sizeof(DET_T));
    if (!col) { free(start); free(order); free(fill); return OREF_NO_MEM; }
    for (int64_t b = 0; b < num_out; ++b) {
        int64_t m = start[b + 1] - start[b];
        if (m == 0) continue; /* untouched */
        for (int64_t c = 0; c < row_len; ++c) {
            for (int64_t k = 0; k < m; ++k) col[k] = values[order[start[b] + k] * row_len + c];
            out[b * row_len + c] = out[b * row_len + c] + FN(oref_pw)(col, m);
        }
    }
    free(col); free(start); free(order); free(fill);
    return skipped;
}

/* ---------------------------------------------------------------- R5/R6: scan */

/* A scan element: head flag and value.  Unsegmented scans have every flag 0,
 * and then the operator below is plain addition. */
typedef struct { int f; DET_T v; } pair_t;

static pair_t pair_identity(void) { pair_t r; r.f = 0; r.v = identity(); return r; }

/* Segmented operator, left operand = lower index. */
static pair_t segop(pair_t a, pair_t b) {
    pair_t r;
    r.f = a.f | b.f;
    r.v = b.f ? b.v : a.v + b.v;
    return r;
}

/* R1 applied to a list of pairs. */
static pair_t pw_pairs(const pair_t* v, int64_t m) {
    if (m <= 0) return pair_identity();
    int64_t p = 1;
    while (p < m) p *= 2;
    pair_t* buf = (pair_t*)malloc((size_t)p * sizeof(pair_t));
    if (!buf) abort();
    for (int64_t i = 0; i < p; ++i) buf[i] = (i < m) ? v[i] : pair_identity();
    for (int64_t len = p; len > 1; len /= 2)
        for (int64_t i = 0; i < len / 2; ++i) buf[i] = segop(buf[2 * i], buf[2 * i + 1]);
    pair_t r = buf[0];
    free(buf);
    return r;
}

/* Local part of tile j.  A tile is NW waves of W lanes; lane t (= w*W + l) owns a run of
 * V consecutive elements.
 *   s[t*V+k]  lane-serial inclusive prefix of lane t's run;
 *   p[t]      exclusive prefix of lane t inside its wave: a Kogge-Stone scan over the W lane
 *             totals of the wave (offsets 1, 2, 4, ... < W, each step using the previous
 *             step's values), shifted by one lane;
 *   pw[w]     exclusive prefix of wave w inside the tile: the same Kogge-Stone rule over the
 *             NW wave totals (offsets 1, 2, ... < NW), shifted by one wave;
 *   *agg      the tile total (last wave-level Kogge-Stone value).
 * Positions at or past n are identity leaves. */
static void tile_local(const DET_T* x, const unsigned char* h, int64_t n, int64_t j,
                       int64_t V, int64_t W, int64_t NW, pair_t* s, pair_t* u, pair_t* tmp,
                       pair_t* p, pair_t* om, pair_t* pw, pair_t* agg) {
    int64_t L = W * NW;
    int64_t T = V * L;
    for (int64_t t = 0; t < L; ++t) {
        for (int64_t k = 0; k < V; ++k) {
            int64_t i = j * T + t * V + k;
            pair_t leaf = pair_identity();
            if (i < n) { leaf.f = h[i]; leaf.v = x[i]; }
            s[t * V + k] = (k == 0) ? leaf : segop(s[t * V + k - 1], leaf);
        }
        u[t] = s[t * V + V - 1];
    }
    for (int64_t d = 1; d < W; d *= 2) {
        for (int64_t t = 0; t < L; ++t) tmp[t] = (t % W >= d) ? segop(u[t - d], u[t]) : u[t];
        memcpy(u, tmp, (size_t)L * sizeof(pair_t));
    }
    for (int64_t t = 0; t < L; ++t) p[t] = (t % W == 0) ? pair_identity() : u[t - 1];
    for (int64_t w = 0; w < NW; ++w) om[w] = u[w * W + W - 1];
    for (int64_t d = 1; d < NW; d *= 2) {
        for (int64_t w = 0; w < NW; ++w) tmp[w] = (w >= d) ? segop(om[w - d], om[w]) : om[w];
        memcpy(om, tmp, (size_t)NW * sizeof(pair_t));
    }
    for (int64_t w = 0; w < NW; ++w) pw[w] = (w == 0) ? pair_identity() : om[w - 1];
    *agg = om[NW - 1];
}

/* Forward inclusive scan of (x, h) into y with constants V, W, NW, A, A2.
 *   Agg_j        tile totals;
 *   interval q   = tiles [qA, qA+A);            G_q = PW(Agg of every tile of interval q);
 *   super-interval Q = intervals [Q*A2, Q*A2+A2);  H_Q = PW(G of every interval of Q);
 *   CC_0 = id,   CC_{Q+1} = CC_Q (+) H_Q        (the carry through super-anchor Q);
 *   C_q          = CC_Q (+) PW(G_{Q*A2}, ..., G_{q-1})   (the carry into interval q);
 *   W_j          = PW(Agg_{qA}, ..., Agg_{j-1})  (identity for the interval's first tile);
 *   E_j          = C_q (+) W_j;
 *   y            = ((E_j (+) pw[w]) (+) p[t]) (+) s[t*V+k]. */
static int scan_forward_inclusive(const DET_T* x, const unsigned char* h, int64_t n,
                                  int64_t V, int64_t W, int64_t NW, int64_t A, int64_t A2,
                                  DET_T* y) {
    if (n == 0) return OREF_OK;
    int64_t L = W * NW;
    int64_t T = V * L;
    int64_t nt = (n + T - 1) / T;
    int64_t nq = (nt + A - 1) / A;
    int64_t nQ = (nq + A2 - 1) / A2;
    int64_t big = L > NW ? L : NW;
    pair_t* agg = (pair_t*)malloc((size_t)nt * sizeof(pair_t));
    pair_t* g = (pair_t*)malloc((size_t)nq * sizeof(pair_t));
    pair_t* cc = (pair_t*)malloc((size_t)(nQ + 1) * sizeof(pair_t));
    pair_t* s = (pair_t*)malloc((size_t)T * sizeof(pair_t));
    pair_t* u = (pair_t*)malloc((size_t)L * sizeof(pair_t));
    pair_t* tmp = (pair_t*)malloc((size_t)big * sizeof(pair_t));
    pair_t* p = (pair_t*)malloc((size_t)L * sizeof(pair_t));
    pair_t* om = (pair_t*)malloc((size_t)NW * sizeof(pair_t));
    pair_t* pw = (pair_t*)malloc((size_t)NW * sizeof(pair_t));
    if (!agg || !g || !cc || !s || !u || !tmp || !p || !om || !pw) {
        free(agg); free(g); free(cc); free(s); free(u); free(tmp); free(p); free(om); free(pw);
        return OREF_NO_MEM;
    }
    for (int64_t j = 0; j < nt; ++j) tile_local(x, h, n, j, V, W, NW, s, u, tmp, p, om, pw, &agg[j]);
    for (int64_t q = 0; q < nq; ++q) {
        int64_t cnt = (nt - q * A < A) ? nt - q * A : A;
        g[q] = pw_pairs(agg + q * A, cnt);
    }
    cc[0] = pair_identity();
    for (int64_t Q = 0; Q < nQ; ++Q) {
        int64_t cnt = (nq - Q * A2 < A2) ? nq - Q * A2 : A2;
        cc[Q + 1] = segop(cc[Q], pw_pairs(g + Q * A2, cnt));
    }
    for (int64_t j = 0; j < nt; ++j) {
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
    free(agg); free(g); free(cc); free(s); free(u); free(tmp); free(p); free(om); free(pw);
    return OREF_OK;
}

/* Scan with flags (bit 0 exclusive, bit 1 reverse) and optional segment offsets
 * offsets[0..S] with offsets[0] == 0 <= ... <= offsets[S] == n.  x and y must not
 * overlap.  Returns OREF_OK or an error code. */
int FN(oref_scan)(const DET_T* x, DET_T* y, int64_t n, unsigned flags, const int64_t* offsets,
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
    int rev = (flags & OREF_REVERSE) != 0;
    int excl = (flags & OREF_EXCLUSIVE) != 0;
    /* working copies in scan order (flipped for reverse) */
    DET_T* xs = (DET_T*)malloc((size_t)n * sizeof(DET_T));
    DET_T* ys = (DET_T*)malloc((size_t)n * sizeof(DET_T));
    unsigned char* h = (unsigned char*)calloc((size_t)n, 1);
    if (!xs || !ys || !h) { free(xs); free(ys); free(h); return OREF_NO_MEM; }
    for (int64_t f = 0; f < n; ++f) xs[f] = rev ? x[n - 1 - f] : x[f];
    if (offsets) {
        for (int64_t k = 0; k <= num_segments; ++k) {
            int64_t o = offsets[k];
            if (!rev) {
                if (o < n) h[o] = 1;          /* a segment starts at o */
            } else {
                if (o > 0) h[n - o] = 1;      /* original o-1 ends a segment */
            }
        }
    }
    int rc = scan_forward_inclusive(xs, h, n, V, W, NW, A, A2, ys);
    if (rc == OREF_OK) {
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

/* ---------------------------------------------------------------- R7: running prev */

/* Arguments as for oref_scatter_add; prev is required and receives the running value of R7
 * (rows of skipped sources are not written); V, W, NW, A, A2 are the scan's constants.
 * Returns the number of skipped source rows, or a negative error code. */
int64_t FN(oref_scatter_add_running)(const DET_T* values, const int32_t* index, int64_t n,
                                     int64_t row_len, DET_T* out, int64_t num_out, DET_T* prev,
                                     int64_t V, int64_t W, int64_t NW, int64_t A, int64_t A2) {
    if (n < 0 || row_len < 1 || num_out < 0 || !prev) return OREF_BAD_ARG;
    int64_t* start = (int64_t*)calloc((size_t)num_out + 1, sizeof(int64_t));
    if (!start) return OREF_NO_MEM;
    int64_t valid = 0;
    for (int64_t i = 0; i < n; ++i) {
        int64_t b = index[i];
        if (b < 0 || b >= num_out) continue;
        start[b + 1] += 1;
        ++valid;
    }
    for (int64_t b = 0; b < num_out; ++b) start[b + 1] += start[b];
    /* G: position g holds source row src[g] of destination dst[g] */
    int64_t* src = (int64_t*)malloc((size_t)(valid > 0 ? valid : 1) * sizeof(int64_t));
    int64_t* dst = (int64_t*)malloc((size_t)(valid > 0 ? valid : 1) * sizeof(int64_t));
    int64_t* fill = (int64_t*)malloc((size_t)(num_out > 0 ? num_out : 1) * sizeof(int64_t));
    DET_T* g_col = (DET_T*)malloc((size_t)(valid > 0 ? valid : 1) * sizeof(DET_T));
    DET_T* e_col = (DET_T*)malloc((size_t)(valid > 0 ? valid : 1) * sizeof(DET_T));
    int rc = OREF_OK;
    if (!src || !dst || !fill || !g_col || !e_col) rc = OREF_NO_MEM;
    if (rc == OREF_OK) {
        for (int64_t b = 0; b < num_out; ++b) fill[b] = start[b];
        for (int64_t i = 0; i < n; ++i) {
            int64_t b = index[i];
            if (b < 0 || b >= num_out) continue;
            src[fill[b]] = i;
            dst[fill[b]] = b;
            fill[b] += 1;
        }
        for (int64_t c = 0; c < row_len && rc == OREF_OK; ++c) {
            for (int64_t g = 0; g < valid; ++g) g_col[g] = values[src[g] * row_len + c];
            rc = FN(oref_scan)(g_col, e_col, valid, OREF_EXCLUSIVE, start, num_out, V, W, NW, A,
                               A2);
            if (rc != OREF_OK) break;
            for (int64_t g = 0; g < valid; ++g) {
                const DET_T init = out[dst[g] * row_len + c];
                prev[src[g] * row_len + c] = (g == start[dst[g]]) ? init : init + e_col[g];
            }
        }
    }
    free(start); free(src); free(dst); free(fill); free(g_col); free(e_col);
    if (rc != OREF_OK) return rc;
    return FN(oref_scatter_add)(values, index, n, row_len, out, num_out, NULL);
}
