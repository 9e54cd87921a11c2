/*
 * CPU oracle for the neighbour-graph attention hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file defines what the path computes, in
 * plain, slow, obviously correct C with fp64 arithmetic.  Only the tests,
 * the package's smoke check and the benchmark's CPU-baseline leg may load
 * it; the GPU library never does, and the two share no code.
 *
 * Sources (web pages; cited by title and section):
 *   [P1] deepmd-kit issue "perf: DPA4 .pt2 LAMMPS (C++ AOTI) inference 3-6x
 *        slower than Python (ASE) due to CPU-side edge construction and data
 *        marshalling".
 *   [P2] deepmd-kit issue "perf: NeighborGraph attention is 4-9x slower than
 *        dense and OOM-prone -- move to block-dense attention via the
 *        destination CSR".
 *
 * Readings taken where the pages are silent (each is listed with its reason
 * in the design notes of the repository):
 *   - all periodic images within rcut are neighbours, not only the minimum
 *     image (the diamond boxes of [P2] "Measurements" are smaller than
 *     2*rcut); the image shift n is stored per edge and the edge vector is
 *     d = (x_j - x_i) + n*L, neighbour image minus centre;
 *   - the distance is r2 = (dx*dx + dy*dy) + dz*dz in IEEE fp64 with no
 *     fused multiply-add, and the cutoff test is strict, r2 < rcut*rcut;
 *   - a row keeps the sel nearest neighbours, ordered by the total key
 *     (r2, j, n_x, n_y, n_z) ascending; a row with fewer neighbours within
 *     rcut is shorter (ragged), never filled past rcut;
 *   - attention heads are contiguous column blocks of width d = c/H, the
 *     score scale is 1/sqrt(d), each query attends to every edge of its
 *     centre including itself, and there are no biases, residuals or norms;
 *     stacked layers compose, x <- y.
 *
 * Build: gcc -O3 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Neighbour list: brute force over every atom and every periodic image.     */
/* ------------------------------------------------------------------------ */

typedef struct {
    double r2;
    int32_t j;
    int32_t n[3];
    double d[3];
} orc_cand;

/* Total order of [P2] "Proposed fix" rows: nearest first, ties by neighbour
 * index, then by image shift. */
static int orc_cand_cmp(const void* pa, const void* pb)
{
    const orc_cand* a = (const orc_cand*)pa;
    const orc_cand* b = (const orc_cand*)pb;
    if (a->r2 < b->r2) return -1;
    if (a->r2 > b->r2) return 1;
    if (a->j != b->j) return a->j < b->j ? -1 : 1;
    for (int t = 0; t < 3; ++t)
        if (a->n[t] != b->n[t]) return a->n[t] < b->n[t] ? -1 : 1;
    return 0;
}

/* Number of images to try per side along one axis: every image with
 * |n| * L < rcut + L is reachable, so |n| <= floor(rcut / L) + 1 suffices. */
static int orc_image_range(double rcut, double side)
{
    return (int)floor(rcut / side) + 1;
}

/*
 * One centre's neighbour row ([P1] "Root cause analysis": the edge list of
 * the periodic system; [P2] "Proposed fix": one destination row per centre).
 *
 * Every atom j and every image n in [-K, K]^3 is tried; the self pair
 * (j == i, n == 0) is skipped.  Kept candidates are sorted by the total key
 * and the first min(sel, count) are returned.  Returns the number written;
 * *n_within receives the number within rcut before truncation.  Returns -1
 * if out of memory.  col: [sel], shift: [sel][3], vec: [sel][3] (nullable),
 * r2out: [sel] (nullable).
 */
int64_t orc_nl_row(const double* pos, int64_t n_atoms, const double* box, double rcut,
                   int32_t sel, int64_t i, int32_t* col, int32_t* shift, double* vec,
                   double* r2out, int64_t* n_within)
{
    const double rc2 = rcut * rcut;
    int K[3];
    for (int a = 0; a < 3; ++a) K[a] = orc_image_range(rcut, box[a]);

    size_t cap = 256, cnt = 0;
    orc_cand* cand = (orc_cand*)malloc(cap * sizeof(orc_cand));
    if (!cand) return -1;

    /* An image whose component |d_a| along one axis is already >= rcut is
     * skipped before the other axes are tried: d_a*d_a then rounds to at
     * least rcut*rcut (rounding is monotonic) and adding the other,
     * non-negative squares cannot bring r2 back below it, so the full test
     * would reject it too.  The kept set is exactly that of the full test. */
    const double* xi = pos + 3 * i;
    for (int64_t j = 0; j < n_atoms; ++j) {
        const double* xj = pos + 3 * j;
        for (int nx = -K[0]; nx <= K[0]; ++nx) {
            const double dx = (xj[0] - xi[0]) + (double)nx * box[0];
            if (fabs(dx) >= rcut) continue;
            for (int ny = -K[1]; ny <= K[1]; ++ny) {
                const double dy = (xj[1] - xi[1]) + (double)ny * box[1];
                if (fabs(dy) >= rcut) continue;
                for (int nz = -K[2]; nz <= K[2]; ++nz) {
                    if (j == i && nx == 0 && ny == 0 && nz == 0) continue;
                    const double dz = (xj[2] - xi[2]) + (double)nz * box[2];
                    const int nn[3] = {nx, ny, nz};
                    const double d[3] = {dx, dy, dz};
                    double sxy = d[0] * d[0] + d[1] * d[1];
                    double r2 = sxy + d[2] * d[2];
                    if (!(r2 < rc2)) continue;
                    if (cnt == cap) {
                        cap *= 2;
                        orc_cand* grown = (orc_cand*)realloc(cand, cap * sizeof(orc_cand));
                        if (!grown) { free(cand); return -1; }
                        cand = grown;
                    }
                    orc_cand* c = &cand[cnt++];
                    c->r2 = r2;
                    c->j = (int32_t)j;
                    for (int a = 0; a < 3; ++a) { c->n[a] = nn[a]; c->d[a] = d[a]; }
                }
            }
        }
    }
    qsort(cand, cnt, sizeof(orc_cand), orc_cand_cmp);
    int64_t keep = (int64_t)cnt < (int64_t)sel ? (int64_t)cnt : (int64_t)sel;
    for (int64_t k = 0; k < keep; ++k) {
        col[k] = cand[k].j;
        for (int a = 0; a < 3; ++a) {
            shift[3 * k + a] = cand[k].n[a];
            if (vec) vec[3 * k + a] = cand[k].d[a];
        }
        if (r2out) r2out[k] = cand[k].r2;
    }
    if (n_within) *n_within = (int64_t)cnt;
    free(cand);
    return keep;
}

/*
 * Rows of a list of centres (OpenMP over the list): counts[n_list], and for
 * list entry t its row in col[t*sel ..], shift[(t*sel)*3 ..], vec (nullable).
 * Returns 0, or -1 if memory runs out.
 */
int orc_nl_rows(const double* pos, int64_t n_atoms, const double* box, double rcut, int32_t sel,
                const int64_t* centres, int64_t n_list, int64_t* counts, int32_t* col,
                int32_t* shift, double* vec)
{
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int64_t t = 0; t < n_list; ++t) {
        int64_t k = orc_nl_row(pos, n_atoms, box, rcut, sel, centres[t], col + (size_t)t * sel,
                               shift + (size_t)t * sel * 3, vec ? vec + (size_t)t * sel * 3 : NULL,
                               NULL, NULL);
        if (k < 0) failed = 1;
        counts[t] = k < 0 ? 0 : k;
    }
    return failed ? -1 : 0;
}

/*
 * Whole destination CSR for all centres: row_ptr[n_atoms+1], col[e_cap],
 * shift[e_cap][3], vec[e_cap][3] (nullable).  Returns E, or -1 if E would
 * exceed e_cap or memory runs out.  Rows are built independently (OpenMP
 * over centres) into padded scratch and then concatenated in centre order.
 */
int64_t orc_nl_full(const double* pos, int64_t n_atoms, const double* box, double rcut,
                    int32_t sel, int64_t* row_ptr, int32_t* col, int32_t* shift, double* vec,
                    int64_t e_cap)
{
    int32_t* pcol = (int32_t*)malloc((size_t)n_atoms * sel * sizeof(int32_t));
    int32_t* pshift = (int32_t*)malloc((size_t)n_atoms * sel * 3 * sizeof(int32_t));
    double* pvec = (double*)malloc((size_t)n_atoms * sel * 3 * sizeof(double));
    int64_t* cnt = (int64_t*)malloc((size_t)n_atoms * sizeof(int64_t));
    int failed = 0;
    if (!pcol || !pshift || !pvec || !cnt) failed = 1;
    if (!failed) {
#pragma omp parallel for schedule(dynamic, 4) reduction(| : failed)
        for (int64_t i = 0; i < n_atoms; ++i) {
            int64_t k = orc_nl_row(pos, n_atoms, box, rcut, sel, i, pcol + (size_t)i * sel,
                                   pshift + (size_t)i * sel * 3, pvec + (size_t)i * sel * 3,
                                   NULL, NULL);
            if (k < 0) failed = 1;
            cnt[i] = k < 0 ? 0 : k;
        }
    }
    int64_t e = 0;
    if (!failed) {
        row_ptr[0] = 0;
        for (int64_t i = 0; i < n_atoms; ++i) row_ptr[i + 1] = row_ptr[i] + cnt[i];
        e = row_ptr[n_atoms];
        if (e > e_cap) failed = 1;
    }
    if (!failed) {
        for (int64_t i = 0; i < n_atoms; ++i) {
            int64_t base = row_ptr[i];
            for (int64_t k = 0; k < cnt[i]; ++k) {
                col[base + k] = pcol[(size_t)i * sel + k];
                for (int a = 0; a < 3; ++a) {
                    shift[3 * (base + k) + a] = pshift[((size_t)i * sel + k) * 3 + a];
                    if (vec) vec[3 * (base + k) + a] = pvec[((size_t)i * sel + k) * 3 + a];
                }
            }
        }
    }
    free(pcol); free(pshift); free(pvec); free(cnt);
    return failed ? -1 : e;
}

/* ------------------------------------------------------------------------ */
/* Attention: naive loops, one centre at a time.                             */
/* ------------------------------------------------------------------------ */

/* y[n][c] = x[n][c] . W[c][c]  (y = x W, W row-major [c_in][c_out]).
 * Each y[a][u] starts at 0 and adds x[a][t] * W[t][u] for t = 0, 1, ...,
 * c-1 in that order; the loop over u is innermost only so that W's rows are
 * read contiguously. */
static void orc_matmul(const double* x, int64_t n, int32_t c, const double* W, double* y)
{
    for (int64_t a = 0; a < n; ++a) {
        double* ya = y + a * c;
        for (int32_t u = 0; u < c; ++u) ya[u] = 0.0;
        for (int32_t t = 0; t < c; ++t) {
            const double xt = x[a * c + t];
            const double* Wt = W + (int64_t)t * c;
            for (int32_t u = 0; u < c; ++u) ya[u] += xt * Wt[u];
        }
    }
}

/*
 * One attention layer on one centre's block X[n][c] -> Y[n][c]
 * ([P2] "Proposed fix: block-dense attention on the graph": dense attention
 * math on the per-centre (nnei, c) block; "Graph-native alternatives":
 * per-center self-attention among the center's edges).
 *
 *   q = X Wq, k = X Wk, v = X Wv
 *   for head h (columns h*d .. h*d+d-1) and query row a:
 *     s_b = (q_a . k_b)_h / sqrt(d)  for every row b of the block
 *     m = max_b s_b, p_b = exp(s_b - m), Z = sum_b p_b
 *     o_a[h cols] = (sum_b p_b v_b[h cols]) / Z
 *   Y = o Wo
 * W points at the layer's [4][c][c] weights (q, k, v, o).  scratch holds
 * 5*n*c + n doubles.
 *
 * Smooth attention ([P2] "Graph-native alternatives": the occupancy-modified
 * weights are w_j = softmax_j * (sum_j e_j / D~), a per-segment scalar
 * rescale of the vanilla softmax, with D~ computed outside the attention):
 * when log_dt is not NULL it holds ln D~ for each block row a and head h at
 * log_dt[a*heads + h], e_j = exp(s_j) is the unnormalised weight of the
 * segment (query row a, head h), and
 *     o_a[h cols] = (vanilla o_a[h cols]) * (sum_j e_j / D~),
 * with sum_j e_j = exp(m) * Z, the factor evaluated as exp(m + ln Z - ln D~).
 */
static void orc_layer_block(const double* X, int64_t n, int32_t c, int32_t heads,
                            const double* W, const double* log_dt, double* Y, double* scratch)
{
    const int64_t cc = (int64_t)c * c;
    const int32_t d = c / heads;
    const double scale = 1.0 / sqrt((double)d);
    double* q = scratch;
    double* k = q + n * c;
    double* v = k + n * c;
    double* o = v + n * c;
    double* s = o + n * c;
    double* kt = s + n;  /* head h's keys transposed: kt[t][b] = k[b][h*d + t] */
    orc_matmul(X, n, c, W + 0 * cc, q);
    orc_matmul(X, n, c, W + 1 * cc, k);
    orc_matmul(X, n, c, W + 2 * cc, v);
    for (int32_t h = 0; h < heads; ++h) {
        const int32_t c0 = h * d;
        for (int64_t b = 0; b < n; ++b)
            for (int32_t t = 0; t < d; ++t) kt[t * n + b] = k[b * c + c0 + t];
        for (int64_t a = 0; a < n; ++a) {
            /* s_b = (sum over t = 0, 1, ..., d-1 of q_a[t] k_b[t]) * scale, each
             * sum accumulated in t order; b innermost reads kt's rows contiguously. */
            for (int64_t b = 0; b < n; ++b) s[b] = 0.0;
            for (int32_t t = 0; t < d; ++t) {
                const double qt = q[a * c + c0 + t];
                const double* kr = kt + (int64_t)t * n;
                for (int64_t b = 0; b < n; ++b) s[b] += qt * kr[b];
            }
            double m = -INFINITY;
            for (int64_t b = 0; b < n; ++b) {
                s[b] = s[b] * scale;
                if (s[b] > m) m = s[b];
            }
            double z = 0.0;
            for (int64_t b = 0; b < n; ++b) {
                s[b] = exp(s[b] - m);
                z += s[b];
            }
            const double factor = log_dt ? exp(m + log(z) - log_dt[a * heads + h]) : 1.0;
            /* o_a[t] = (sum over b = 0, 1, ..., n-1 of p_b v_b[t]) / Z, each sum
             * accumulated in b order; t innermost reads v's rows contiguously. */
            double* oa = o + a * c + c0;
            for (int32_t t = 0; t < d; ++t) oa[t] = 0.0;
            for (int64_t b = 0; b < n; ++b)
                for (int32_t t = 0; t < d; ++t) oa[t] += s[b] * v[b * c + c0 + t];
            for (int32_t t = 0; t < d; ++t) oa[t] = oa[t] / z * factor;
        }
    }
    orc_matmul(o, n, c, W + 3 * cc, Y);
}

static int64_t orc_edge_of(const int64_t* row_ptr, const int32_t* order, int64_t i, int64_t a)
{
    int64_t slot = row_ptr[i] + a;
    return order ? (int64_t)order[slot] : slot;
}

static int64_t orc_max_row(const int64_t* row_ptr, int64_t n_centres)
{
    int64_t m = 0;
    for (int64_t i = 0; i < n_centres; ++i) {
        int64_t n = row_ptr[i + 1] - row_ptr[i];
        if (n > m) m = n;
    }
    return m;
}

/*
 * Stacked attention layers over the whole edge axis, layer by layer: each
 * layer gathers every centre's block through the destination CSR
 * (row_ptr, optional order permutation), runs orc_layer_block and scatters
 * the rows back; then x <- y for the next layer.
 * x, y: [n_edges][c] fp64; w: [layers][4][c][c] fp64; log_dt: NULL, or
 * ln D~ as [layers][n_edges][heads] keyed by the query edge's row of x.
 * Returns 0, or -1 on bad arguments / out of memory.
 */
static int orc_attn_layers(const int64_t* row_ptr, const int32_t* order, int64_t n_centres,
                           int64_t n_edges, int32_t c, int32_t heads, int32_t layers,
                           const double* w, const double* x, const double* log_dt, double* y)
{
    if (c < 1 || heads < 1 || c % heads != 0 || layers < 1) return -1;
    const int64_t nmax = orc_max_row(row_ptr, n_centres);
    double* cur = (double*)malloc((size_t)(n_edges > 0 ? n_edges : 1) * c * sizeof(double));
    if (!cur) return -1;
    memcpy(cur, x, (size_t)n_edges * c * sizeof(double));
    int failed = 0;
    for (int32_t l = 0; l < layers && !failed; ++l) {
        const double* W = w + (size_t)l * 4 * c * c;
#pragma omp parallel reduction(| : failed)
        {
            double* Xb = (double*)malloc((size_t)(nmax + 1) * c * sizeof(double));
            double* Yb = (double*)malloc((size_t)(nmax + 1) * c * sizeof(double));
            double* sc = (double*)malloc(((size_t)5 * (nmax + 1) * c + nmax + 1) * sizeof(double));
            double* Lb = (double*)malloc((size_t)(nmax + 1) * heads * sizeof(double));
            if (!Xb || !Yb || !sc || !Lb) failed = 1;
#pragma omp for schedule(dynamic, 8)
            for (int64_t i = 0; i < n_centres; ++i) {
                if (failed) continue;
                int64_t n = row_ptr[i + 1] - row_ptr[i];
                if (n <= 0) continue;
                for (int64_t a = 0; a < n; ++a) {
                    const int64_t e = orc_edge_of(row_ptr, order, i, a);
                    memcpy(Xb + a * c, cur + e * c, (size_t)c * sizeof(double));
                    if (log_dt)
                        memcpy(Lb + a * heads, log_dt + ((size_t)l * n_edges + e) * heads,
                               (size_t)heads * sizeof(double));
                }
                orc_layer_block(Xb, n, c, heads, W, log_dt ? Lb : NULL, Yb, sc);
                for (int64_t a = 0; a < n; ++a)
                    memcpy(y + orc_edge_of(row_ptr, order, i, a) * c, Yb + a * c,
                           (size_t)c * sizeof(double));
            }
            free(Xb); free(Yb); free(sc); free(Lb);
        }
        if (l + 1 < layers) memcpy(cur, y, (size_t)n_edges * c * sizeof(double));
    }
    free(cur);
    return failed ? -1 : 0;
}

int orc_attn_naive(const int64_t* row_ptr, const int32_t* order, int64_t n_centres,
                   int64_t n_edges, int32_t c, int32_t heads, int32_t layers,
                   const double* w, const double* x, double* y)
{
    return orc_attn_layers(row_ptr, order, n_centres, n_edges, c, heads, layers, w, x, NULL, y);
}

/* Smooth attention: the same layers with the per-segment rescale by
 * sum_j e_j / D~ (orc_layer_block); log_dt [layers][n_edges][heads]. */
int orc_attn_smooth(const int64_t* row_ptr, const int32_t* order, int64_t n_centres,
                    int64_t n_edges, int32_t c, int32_t heads, int32_t layers,
                    const double* w, const double* x, const double* log_dt, double* y)
{
    if (!log_dt) return -1;
    return orc_attn_layers(row_ptr, order, n_centres, n_edges, c, heads, layers, w, x, log_dt,
                           y);
}

/*
 * The same stacked layers for a chosen list of centres only.  An edge
 * belongs to exactly one destination row and a centre's attention reads only
 * its own rows, so each listed centre can be carried through all layers on
 * its own.  Only the rows of the listed centres are written to y.
 */
int orc_attn_naive_centres(const int64_t* row_ptr, const int32_t* order,
                           const int64_t* centres, int64_t n_list, int32_t c, int32_t heads,
                           int32_t layers, const double* w, const double* x, double* y)
{
    if (c < 1 || heads < 1 || c % heads != 0 || layers < 1) return -1;
    int failed = 0;
#pragma omp parallel reduction(| : failed)
    {
        double* Xb = NULL; double* Yb = NULL; double* sc = NULL;
        int64_t have = -1;
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < n_list; ++t) {
            if (failed) continue;
            int64_t i = centres[t];
            int64_t n = row_ptr[i + 1] - row_ptr[i];
            if (n <= 0) continue;
            if (n > have) {
                free(Xb); free(Yb); free(sc);
                Xb = (double*)malloc((size_t)n * c * sizeof(double));
                Yb = (double*)malloc((size_t)n * c * sizeof(double));
                sc = (double*)malloc(((size_t)5 * n * c + n) * sizeof(double));
                have = n;
                if (!Xb || !Yb || !sc) { failed = 1; have = -1; continue; }
            }
            for (int64_t a = 0; a < n; ++a)
                memcpy(Xb + a * c, x + orc_edge_of(row_ptr, order, i, a) * c,
                       (size_t)c * sizeof(double));
            for (int32_t l = 0; l < layers; ++l) {
                orc_layer_block(Xb, n, c, heads, w + (size_t)l * 4 * c * c, NULL, Yb, sc);
                memcpy(Xb, Yb, (size_t)n * c * sizeof(double));
            }
            for (int64_t a = 0; a < n; ++a)
                memcpy(y + orc_edge_of(row_ptr, order, i, a) * c, Xb + a * c,
                       (size_t)c * sizeof(double));
        }
        free(Xb); free(Yb); free(sc);
    }
    return failed ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Attention: the ragged pair-axis form ([P2] "Root cause").                 */
/* ------------------------------------------------------------------------ */

/*
 * The same layers computed the way [P2] "Root cause" describes the ragged
 * route: project every edge, enumerate the P = sum_i n_i^2 (centre, query
 * edge, key edge) pairs, score each pair per head, take the segment max and
 * segment sum over the pairs that share a query edge (segment softmax),
 * normalise each pair's weight, and index_add w_p * v[key edge] into the
 * query edge's output row; then apply Wo per edge.  Serial, so the
 * index_add order is fixed.  Returns 0, or -1 on bad arguments / out of
 * memory.
 */
int orc_attn_pairaxis(const int64_t* row_ptr, const int32_t* order, int64_t n_centres,
                      int64_t n_edges, int32_t c, int32_t heads, int32_t layers,
                      const double* w, const double* x, double* y)
{
    if (c < 1 || heads < 1 || c % heads != 0 || layers < 1) return -1;
    const int32_t d = c / heads;
    const double scale = 1.0 / sqrt((double)d);
    const int64_t cc = (int64_t)c * c;
    int64_t P = 0;
    for (int64_t i = 0; i < n_centres; ++i) {
        int64_t n = row_ptr[i + 1] - row_ptr[i];
        P += n * n;
    }
    const size_t ne = (size_t)(n_edges > 0 ? n_edges : 1);
    const size_t np = (size_t)(P > 0 ? P : 1);
    int64_t* qe = (int64_t*)malloc(np * sizeof(int64_t));
    int64_t* ke = (int64_t*)malloc(np * sizeof(int64_t));
    double* s = (double*)malloc(np * heads * sizeof(double));
    double* cur = (double*)malloc(ne * c * sizeof(double));
    double* q = (double*)malloc(ne * c * sizeof(double));
    double* k = (double*)malloc(ne * c * sizeof(double));
    double* v = (double*)malloc(ne * c * sizeof(double));
    double* out = (double*)malloc(ne * c * sizeof(double));
    double* segmax = (double*)malloc(ne * heads * sizeof(double));
    double* segsum = (double*)malloc(ne * heads * sizeof(double));
    int rc = 0;
    if (!qe || !ke || !s || !cur || !q || !k || !v || !out || !segmax || !segsum) {
        rc = -1;
        goto done;
    }
    /* Pair enumeration: p -> (query edge, key edge) of the same centre. */
    {
        int64_t p = 0;
        for (int64_t i = 0; i < n_centres; ++i) {
            int64_t n = row_ptr[i + 1] - row_ptr[i];
            for (int64_t a = 0; a < n; ++a)
                for (int64_t b = 0; b < n; ++b) {
                    qe[p] = orc_edge_of(row_ptr, order, i, a);
                    ke[p] = orc_edge_of(row_ptr, order, i, b);
                    ++p;
                }
        }
    }
    memcpy(cur, x, (size_t)n_edges * c * sizeof(double));
    for (int32_t l = 0; l < layers; ++l) {
        const double* W = w + (size_t)l * 4 * cc;
        orc_matmul(cur, n_edges, c, W + 0 * cc, q);
        orc_matmul(cur, n_edges, c, W + 1 * cc, k);
        orc_matmul(cur, n_edges, c, W + 2 * cc, v);
        for (int64_t p = 0; p < P; ++p)
            for (int32_t h = 0; h < heads; ++h) {
                double dot = 0.0;
                for (int32_t t = 0; t < d; ++t)
                    dot += q[qe[p] * c + h * d + t] * k[ke[p] * c + h * d + t];
                s[p * heads + h] = dot * scale;
            }
        for (size_t e = 0; e < (size_t)n_edges * heads; ++e) {
            segmax[e] = -INFINITY;
            segsum[e] = 0.0;
        }
        for (int64_t p = 0; p < P; ++p)                      /* segment max */
            for (int32_t h = 0; h < heads; ++h)
                if (s[p * heads + h] > segmax[qe[p] * heads + h])
                    segmax[qe[p] * heads + h] = s[p * heads + h];
        for (int64_t p = 0; p < P; ++p)                      /* exp, segment sum */
            for (int32_t h = 0; h < heads; ++h) {
                s[p * heads + h] = exp(s[p * heads + h] - segmax[qe[p] * heads + h]);
                segsum[qe[p] * heads + h] += s[p * heads + h];
            }
        memset(out, 0, (size_t)n_edges * c * sizeof(double));
        for (int64_t p = 0; p < P; ++p)                      /* normalise, index_add */
            for (int32_t h = 0; h < heads; ++h) {
                double wp = s[p * heads + h] / segsum[qe[p] * heads + h];
                for (int32_t t = 0; t < d; ++t)
                    out[qe[p] * c + h * d + t] += wp * v[ke[p] * c + h * d + t];
            }
        orc_matmul(out, n_edges, c, W + 3 * cc, y);
        if (l + 1 < layers) memcpy(cur, y, (size_t)n_edges * c * sizeof(double));
    }
done:
    free(qe); free(ke); free(s); free(cur); free(q); free(k); free(v); free(out);
    free(segmax); free(segsum);
    return rc;
}

/*
 * LocalAtten: attention with the centres as queries and each centre's edges
 * as keys and values, one query per segment ([P2] "Graph-native
 * alternatives": LocalAtten maps directly to varlen attention with queries =
 * centers, keys = edges; [P2] "Measurements" names it among the DPA-2 graph
 * attention ops).  For each layer l with weights (Wq, Wk, Wv, Wo) and each
 * centre i with edges e_0 .. e_{n-1} (order-mapped as in orc_attn_naive):
 *   q = xc_i Wq,  k_a = x_{e_a} Wk,  v_a = x_{e_a} Wv
 *   head h (columns h*d .. h*d+d-1):
 *     s_a = (q . k_a)_h / sqrt(d),  m = max_a s_a,  p_a = exp(s_a - m),
 *     o[h cols] = (sum_a p_a v_a[h cols]) / sum_a p_a
 *   yc_i = o Wo
 * Stacked layers update the centre features only, xc <- yc; the edge
 * features x are the keys and values of every layer.  A centre with no edges
 * has no softmax; its output is o = 0, so yc_i = 0.
 * xc, yc: [n_centres][c]; x: [n_edges][c]; w: [layers][4][c][c].
 * Returns 0, or -1 on bad arguments / out of memory.
 */
int orc_local_atten(const int64_t* row_ptr, const int32_t* order, int64_t n_centres,
                    int64_t n_edges, int32_t c, int32_t heads, int32_t layers,
                    const double* w, const double* xc, const double* x, double* yc)
{
    if (c < 1 || heads < 1 || c % heads != 0 || layers < 1 || n_centres < 0 || n_edges < 0)
        return -1;
    const int64_t cc = (int64_t)c * c;
    const int32_t d = c / heads;
    const double scale = 1.0 / sqrt((double)d);
    const int64_t nmax = orc_max_row(row_ptr, n_centres);
    double* cur = (double*)malloc((size_t)(n_centres > 0 ? n_centres : 1) * c * sizeof(double));
    if (!cur) return -1;
    memcpy(cur, xc, (size_t)n_centres * c * sizeof(double));
    int failed = 0;
    for (int32_t l = 0; l < layers && !failed; ++l) {
        const double* W = w + (size_t)l * 4 * cc;
#pragma omp parallel reduction(| : failed)
        {
            double* Xb = (double*)malloc((size_t)(nmax + 1) * c * sizeof(double));
            double* k = (double*)malloc((size_t)(nmax + 1) * c * sizeof(double));
            double* v = (double*)malloc((size_t)(nmax + 1) * c * sizeof(double));
            double* s = (double*)malloc((size_t)(nmax + 1) * sizeof(double));
            double* q = (double*)malloc((size_t)c * sizeof(double));
            double* o = (double*)malloc((size_t)c * sizeof(double));
            if (!Xb || !k || !v || !s || !q || !o) failed = 1;
#pragma omp for schedule(dynamic, 16)
            for (int64_t i = 0; i < n_centres; ++i) {
                if (failed) continue;
                const int64_t n = row_ptr[i + 1] - row_ptr[i];
                for (int32_t t = 0; t < c; ++t) o[t] = 0.0;
                if (n > 0) {
                    for (int64_t a = 0; a < n; ++a)
                        memcpy(Xb + a * c, x + orc_edge_of(row_ptr, order, i, a) * c,
                               (size_t)c * sizeof(double));
                    orc_matmul(cur + i * c, 1, c, W + 0 * cc, q);
                    orc_matmul(Xb, n, c, W + 1 * cc, k);
                    orc_matmul(Xb, n, c, W + 2 * cc, v);
                    for (int32_t h = 0; h < heads; ++h) {
                        const int32_t c0 = h * d;
                        double m = -INFINITY;
                        for (int64_t a = 0; a < n; ++a) {
                            double dot = 0.0;
                            for (int32_t t = 0; t < d; ++t) dot += q[c0 + t] * k[a * c + c0 + t];
                            s[a] = dot * scale;
                            if (s[a] > m) m = s[a];
                        }
                        double z = 0.0;
                        for (int64_t a = 0; a < n; ++a) {
                            s[a] = exp(s[a] - m);
                            z += s[a];
                        }
                        for (int32_t t = 0; t < d; ++t) {
                            double acc = 0.0;
                            for (int64_t a = 0; a < n; ++a) acc += s[a] * v[a * c + c0 + t];
                            o[c0 + t] = acc / z;
                        }
                    }
                }
                orc_matmul(o, 1, c, W + 3 * cc, yc + i * c);
            }
            free(Xb); free(k); free(v); free(s); free(q); free(o);
        }
        if (l + 1 < layers) memcpy(cur, yc, (size_t)n_centres * c * sizeof(double));
    }
    free(cur);
    return failed ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Block gather / scatter through the destination CSR.                       */
/* ------------------------------------------------------------------------ */

/*
 * The padded per-centre block of [P2] "Proposed fix: block-dense attention
 * on the graph": for every centre i with n_i = row_ptr[i+1] - row_ptr[i]
 * edges, block[i][k][:] = x[e_k][:] for k < n_i (e_k = order ? order[row_ptr[i]
 * + k] : row_ptr[i] + k) and block[i][k][:] = 0 for n_i <= k < cap, the
 * (nloc, nnei_max, c) tensor.  Elements are copied as bytes of width es
 * (8 or 4), so the copy is exact for any dtype.  Returns 0, or -1 if a row
 * is longer than cap or an index is out of range.
 */
int orc_block_gather(const int64_t* row_ptr, const int32_t* order, int64_t n_centres,
                     int64_t n_edges, int32_t cap, int32_t c, int32_t es, const void* x,
                     void* block)
{
    const char* xs = (const char*)x;
    char* bs = (char*)block;
    const size_t row = (size_t)c * es;
    for (int64_t i = 0; i < n_centres; ++i) {
        const int64_t n = row_ptr[i + 1] - row_ptr[i];
        if (n < 0 || n > cap) return -1;
        for (int64_t k = 0; k < cap; ++k) {
            char* dst = bs + ((size_t)i * cap + k) * row;
            if (k < n) {
                const int64_t e = orc_edge_of(row_ptr, order, i, k);
                if (e < 0 || e >= n_edges) return -1;
                memcpy(dst, xs + (size_t)e * row, row);
            } else {
                memset(dst, 0, row);
            }
        }
    }
    return 0;
}

/*
 * The inverse scatter back to the edge axis ([P2] "Proposed fix": scatter
 * back): y[e_k][:] = block[i][k][:] for every centre i and k < n_i; rows of
 * y that belong to no centre are left as they are, padding rows are not
 * read.  Returns 0, or -1 as orc_block_gather.
 */
int orc_block_scatter(const int64_t* row_ptr, const int32_t* order, int64_t n_centres,
                      int64_t n_edges, int32_t cap, int32_t c, int32_t es, const void* block,
                      void* y)
{
    const char* bs = (const char*)block;
    char* ys = (char*)y;
    const size_t row = (size_t)c * es;
    for (int64_t i = 0; i < n_centres; ++i) {
        const int64_t n = row_ptr[i + 1] - row_ptr[i];
        if (n < 0 || n > cap) return -1;
        for (int64_t k = 0; k < n; ++k) {
            const int64_t e = orc_edge_of(row_ptr, order, i, k);
            if (e < 0 || e >= n_edges) return -1;
            memcpy(ys + (size_t)e * row, bs + ((size_t)i * cap + k) * row, row);
        }
    }
    return 0;
}

/* Threads the OpenMP loops above use (1 without OpenMP). */
int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
