/*
 * vq_oracle.c -- the CPU oracle for Hessian/salience-weighted vector quantization.
 *
 * TEST INFRASTRUCTURE.  This file is the plain, slow, obviously-correct
 * reference that the HIP library is checked against.  Only the test suite,
 * the package smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or helper with the HIP library, and the
 * library never calls it.
 *
 * Arithmetic: float64 for every distance, sum and scale; float32 for the
 * state (matrix, centroids, scales), as the weighted K-means of the VPTQ page
 * holds fp state.  Build with -ffp-contract=off so that no multiply-add is
 * fused (each line below rounds exactly as written).
 *
 * Notation (VPTQ page, "The Second-Order Optimization Framework"):
 *   W is [M x N] row-major, M outputs by N inputs.  The diagonal Hessian proxy
 *   h has one entry per input column.  Sub-vector s = (row i, block b) holds
 *   W[i, b*d .. b*d+d-1] and has id s = i*(N/d) + b, so W read as [n_sub x d]
 *   is contiguous.  keep[i*N+j] in {0,1} multiplies the weight of element
 *   (i,j): 0 on the salient positions that the sparse correction holds exactly.
 *   omega(i,j) = keep * hcol[j] * rho[i]; without bi-normalization hcol = h and
 *   rho = 1.
 *
 * Distance (VPTQ page, "Hessian-Weighted Centroid Initialization": the
 * diagonal term sum_j h_jj ||dW_:,j||^2 of the decomposed objective, taken
 * one row sub-vector at a time):
 *   D(s,k) = sum_t omega(s,t) * (x(s,t) - C(k,t))^2
 * Objective J = sum_s D(s, a_s).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* Salient count: nnz = floor(p * M * N), the product taken in float64. */
long long orc_nnz(long long M, long long N, double p)
{
    return (long long)floor(p * (double)(M * N));
}

/* ------------------------------------------------------------------ */
/* Salience selection (HAS-VQ abstract: Hessian-Masked Decoupling isolates the
 * second-order-sensitive weights and holds them exactly; SCVQ summary: every
 * exactly held weight in one CSR).  Score of element (i,j): s = h_j * (w_ij * w_ij)
 * in fp32, taken on the original W and h.  The nnz largest scores are selected,
 * ties broken by the smaller linear index i*N+j.  Output: CSR (row_ptr[M+1],
 * col[nnz] ascending within a row, val[nnz] = the exact W value) and keep[M*N]
 * (0 on selected positions, 1 elsewhere). */
typedef struct {
    float score;
    long long lin;
} orc_scored;

static int orc_scored_cmp(const void* a, const void* b)
{
    const orc_scored* x = (const orc_scored*)a;
    const orc_scored* y = (const orc_scored*)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    if (x->lin < y->lin) return -1;
    if (x->lin > y->lin) return 1;
    return 0;
}

int orc_select(const float* W, const float* h, long long M, long long N, long long nnz,
               int* row_ptr, int* col, float* val, unsigned char* keep)
{
    long long total = M * N;
    if (nnz < 0 || nnz > total) return 2;
    orc_scored* all = (orc_scored*)malloc(sizeof(orc_scored) * (size_t)(total > 0 ? total : 1));
    if (!all) return 3;
    for (long long i = 0; i < M; ++i) {
        for (long long j = 0; j < N; ++j) {
            float w = W[i * N + j];
            float sq = w * w;
            float s = h[j] * sq;
            all[i * N + j].score = s;
            all[i * N + j].lin = i * N + j;
        }
    }
    qsort(all, (size_t)total, sizeof(orc_scored), orc_scored_cmp);
    for (long long e = 0; e < total; ++e) keep[e] = 1;
    for (long long e = 0; e < nnz; ++e) keep[all[e].lin] = 0;
    free(all);
    long long pos = 0;
    row_ptr[0] = 0;
    for (long long i = 0; i < M; ++i) {
        for (long long j = 0; j < N; ++j) {
            if (keep[i * N + j] == 0) {
                col[pos] = (int)j;
                val[pos] = W[i * N + j];
                ++pos;
            }
        }
        row_ptr[i + 1] = (int)pos;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* The unified sparse correction (SCVQ summary: a single sparse matrix
 * carries every exactly-held weight, namely the salient elements, whole
 * sub-vectors of high salience and the positions where quantization left the
 * biggest error).  keep[M*N] marks the correction: 0 = held exactly.
 *
 * Salient sub-vectors: score of sub-vector s = (row i, block b) is
 *   S_s = sum over t = 0..d-1, in that order, of h_j * (w_j * w_j), j = b*d+t,
 * each product and the running sum rounded to fp32.  The n_sel largest
 * (ties: smaller s) have all d positions set to 0 in keep. */
int orc_select_subvectors(const float* W, const float* h, long long M, long long N, int d,
                          long long n_sel, unsigned char* keep)
{
    long long nb = N / d, n_sub = M * nb;
    if (n_sel < 0 || n_sel > n_sub) return 2;
    orc_scored* all = (orc_scored*)malloc(sizeof(orc_scored) * (size_t)(n_sub > 0 ? n_sub : 1));
    if (!all) return 3;
    for (long long s = 0; s < n_sub; ++s) {
        long long i = s / nb, b = s % nb;
        float acc = 0.0f;
        for (int t = 0; t < d; ++t) {
            long long j = b * d + t;
            float w = W[i * N + j];
            float sq = w * w;
            float term = h[j] * sq;
            acc = acc + term;
        }
        all[s].score = acc;
        all[s].lin = s;
    }
    qsort(all, (size_t)n_sub, sizeof(orc_scored), orc_scored_cmp);
    for (long long e = 0; e < n_sel; ++e) {
        long long s = all[e].lin;
        for (int t = 0; t < d; ++t) keep[s * d + t] = 0;
    }
    free(all);
    return 0;
}

/* Largest quantization residuals: among the positions still kept
 * (keep == 1), score r_ij = h_j * ((w_ij - what_ij) * (w_ij - what_ij)) in
 * fp32 (difference, square, scale).  The min(n_sel, #kept) largest (ties:
 * smaller linear index) are set to 0 in keep. */
int orc_select_residual(const float* W, const float* What, const float* h, long long M, long long N,
                        long long n_sel, unsigned char* keep)
{
    long long total = M * N, n = 0;
    if (n_sel < 0) return 2;
    orc_scored* all = (orc_scored*)malloc(sizeof(orc_scored) * (size_t)(total > 0 ? total : 1));
    if (!all) return 3;
    for (long long e = 0; e < total; ++e) {
        if (keep[e] == 0) continue;
        float r = W[e] - What[e];
        float sq = r * r;
        all[n].score = h[e % N] * sq;
        all[n].lin = e;
        ++n;
    }
    qsort(all, (size_t)n, sizeof(orc_scored), orc_scored_cmp);
    for (long long e = 0; e < n_sel && e < n; ++e) keep[all[e].lin] = 0;
    free(all);
    return 0;
}

/* The CSR of every position with keep == 0, row by row, columns ascending,
 * values the exact W entries; returns the count. */
long long orc_keep_to_csr(const float* W, const unsigned char* keep, long long M, long long N,
                          int* row_ptr, int* col, float* val)
{
    long long pos = 0;
    row_ptr[0] = 0;
    for (long long i = 0; i < M; ++i) {
        for (long long j = 0; j < N; ++j) {
            if (keep[i * N + j] == 0) {
                col[pos] = (int)j;
                val[pos] = W[i * N + j];
                ++pos;
            }
        }
        row_ptr[i + 1] = (int)pos;
    }
    return pos;
}

/* ------------------------------------------------------------------ */
/* Bi-normalization (SCVQ summary: weights bi-normalized across rows and
 * columns before clustering).  One pass of RMS scaling, rows first:
 *   r_i = sqrt(sum_j W_ij^2 / N)            (sum in fp64; r = 1 if 0)
 *   Wt_ij = W_ij / r_i                      (fp32 division)
 *   c_j = sqrt(sum_i Wt_ij^2 / M)           (sum in fp64; c = 1 if 0)
 *   W'_ij = Wt_ij / c_j                     (fp32 division)
 * The weights are folded so that the objective stays the original-space
 * objective: (W - What)_ij = r_i c_j (W' - W'hat)_ij, hence
 *   hcol_j = h_j * c_j^2,  rho_i = r_i^2   (products in fp64, stored fp32). */
void orc_binorm(const float* W, const float* h, long long M, long long N,
                float* Wp, float* r, float* c, float* hcol, float* rho)
{
    for (long long i = 0; i < M; ++i) {
        double acc = 0.0;
        for (long long j = 0; j < N; ++j) {
            double w = (double)W[i * N + j];
            acc += w * w;
        }
        float ri = (float)sqrt(acc / (double)N);
        if (ri == 0.0f) ri = 1.0f;
        r[i] = ri;
        for (long long j = 0; j < N; ++j) Wp[i * N + j] = W[i * N + j] / ri;
    }
    for (long long j = 0; j < N; ++j) {
        double acc = 0.0;
        for (long long i = 0; i < M; ++i) {
            double w = (double)Wp[i * N + j];
            acc += w * w;
        }
        float cj = (float)sqrt(acc / (double)M);
        if (cj == 0.0f) cj = 1.0f;
        c[j] = cj;
    }
    for (long long i = 0; i < M; ++i)
        for (long long j = 0; j < N; ++j) Wp[i * N + j] = Wp[i * N + j] / c[j];
    for (long long j = 0; j < N; ++j) {
        double cj = (double)c[j];
        hcol[j] = (float)((double)h[j] * cj * cj);
    }
    for (long long i = 0; i < M; ++i) {
        double ri = (double)r[i];
        rho[i] = (float)(ri * ri);
    }
}

/* ------------------------------------------------------------------ */
/* Codebook seeding: walk the permutation and take the first K sub-vectors
 * whose d floats are not bitwise equal to one already taken.  A plain
 * open-addressing hash set over the raw bytes finds repeats.
 * Returns the number of centroids taken (K on success). */
static uint64_t orc_fnv1a(const unsigned char* p, size_t n)
{
    uint64_t x = 1469598103934665603ULL;
    for (size_t i = 0; i < n; ++i) {
        x ^= (uint64_t)p[i];
        x *= 1099511628211ULL;
    }
    return x;
}

int orc_init(const float* X, long long n_sub, int d, const int* perm, int K, float* C)
{
    size_t cap = 16;
    while (cap < (size_t)K * 2 + 2) cap <<= 1;
    int* slot = (int*)malloc(sizeof(int) * cap);
    if (!slot) return -1;
    for (size_t i = 0; i < cap; ++i) slot[i] = -1;
    size_t bytes = sizeof(float) * (size_t)d;
    int taken = 0;
    for (long long e = 0; e < n_sub && taken < K; ++e) {
        const float* v = X + (size_t)perm[e] * (size_t)d;
        size_t pos = (size_t)(orc_fnv1a((const unsigned char*)v, bytes) & (cap - 1));
        int dup = 0;
        while (slot[pos] >= 0) {
            if (memcmp(C + (size_t)slot[pos] * (size_t)d, v, bytes) == 0) { dup = 1; break; }
            pos = (pos + 1) & (cap - 1);
        }
        if (dup) continue;
        memcpy(C + (size_t)taken * (size_t)d, v, bytes);
        slot[pos] = taken;
        ++taken;
    }
    free(slot);
    return taken;
}

/* ------------------------------------------------------------------ */
/* Weight of element t of sub-vector s (fp64; the product of two fp32 values
 * is exact in fp64). */
static double orc_omega(const float* hcol, const float* rho, const unsigned char* keep,
                        long long N, int d, long long s, int t)
{
    long long nb = N / d;
    long long i = s / nb;
    long long j = (s % nb) * d + t;
    if (keep && keep[i * N + j] == 0) return 0.0;
    double w = (double)hcol[j];
    if (rho) w = w * (double)rho[i];
    return w;
}

/* D(s,k) in the direct form, fp64, terms added in t order. */
static double orc_dist(const float* x, const float* ck, const double* om, int d)
{
    double acc = 0.0;
    for (int t = 0; t < d; ++t) {
        double diff = (double)x[t] - (double)ck[t];
        double sq = diff * diff;
        acc += om[t] * sq;
    }
    return acc;
}

/* Assignment (VPTQ page, "The Core Algorithm": Q_V picks the nearest centroid;
 * here under the diagonal-Hessian-weighted distance D).  Exhaustive search;
 * ties go to the lowest centroid index.  subset (nullable) lists the
 * sub-vector ids to assign; idx/dist are indexed by position in that list.
 * dist (nullable) receives the winning D. */
void orc_assign(const float* X, const float* hcol, const float* rho, const unsigned char* keep,
                long long M, long long N, int d, const float* C, int K,
                const long long* subset, long long n_subset,
                unsigned short* idx, double* dist, int nthreads)
{
    long long n = subset ? n_subset : (M * N / d);
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 64)
    for (long long e = 0; e < n; ++e) {
        long long s = subset ? subset[e] : e;
        double om[64];
        for (int t = 0; t < d; ++t) om[t] = orc_omega(hcol, rho, keep, N, d, s, t);
        const float* x = X + (size_t)s * (size_t)d;
        double best = orc_dist(x, C, om, d);
        int arg = 0;
        for (int k = 1; k < K; ++k) {
            double v = orc_dist(x, C + (size_t)k * (size_t)d, om, d);
            if (v < best) { best = v; arg = k; }
        }
        idx[e] = (unsigned short)arg;
        if (dist) dist[e] = best;
    }
}

/* Objective J = sum_s D(s, a_s), fp64, s ascending. */
double orc_objective(const float* X, const float* hcol, const float* rho, const unsigned char* keep,
                     long long M, long long N, int d, const float* C, const unsigned short* idx)
{
    long long n_sub = M * N / d;
    double J = 0.0;
    double om[64];
    for (long long s = 0; s < n_sub; ++s) {
        for (int t = 0; t < d; ++t) om[t] = orc_omega(hcol, rho, keep, N, d, s, t);
        J += orc_dist(X + (size_t)s * (size_t)d, C + (size_t)idx[s] * (size_t)d, om, d);
    }
    return J;
}

/* Centroid update (VPTQ page, "Hessian-Weighted Centroid Initialization":
 * each centroid becomes the Hessian-weighted mean of its members).  With a
 * weight per element the exact minimizer of J for fixed assignments is the
 * per-dimension weighted mean
 *   C(k,t) = sum_{a_s = k} omega(s,t) x(s,t) / sum_{a_s = k} omega(s,t)
 * (fp64 sums over members in ascending s, one rounding to fp32); when the
 * weight sum is 0 the old value is kept.  Returns J against the input C.
 * counts (nullable) receives the member count of each centroid. */
double orc_update(const float* X, const float* hcol, const float* rho, const unsigned char* keep,
                  long long M, long long N, int d, const unsigned short* idx, int K,
                  float* C, int* counts)
{
    long long n_sub = M * N / d;
    double J = orc_objective(X, hcol, rho, keep, M, N, d, C, idx);
    /* counting sort of the sub-vector ids by centroid, stable (ascending s) */
    long long* start = (long long*)calloc((size_t)K + 1, sizeof(long long));
    long long* order = (long long*)malloc(sizeof(long long) * (size_t)(n_sub > 0 ? n_sub : 1));
    long long* fill = (long long*)malloc(sizeof(long long) * (size_t)K);
    for (long long s = 0; s < n_sub; ++s) start[idx[s] + 1] += 1;
    for (int k = 0; k < K; ++k) start[k + 1] += start[k];
    for (int k = 0; k < K; ++k) fill[k] = start[k];
    for (long long s = 0; s < n_sub; ++s) order[fill[idx[s]]++] = s;
    for (int k = 0; k < K; ++k) {
        if (counts) counts[k] = (int)(start[k + 1] - start[k]);
        for (int t = 0; t < d; ++t) {
            double num = 0.0, den = 0.0;
            for (long long e = start[k]; e < start[k + 1]; ++e) {
                long long s = order[e];
                double w = orc_omega(hcol, rho, keep, N, d, s, t);
                num += w * (double)X[(size_t)s * (size_t)d + (size_t)t];
                den += w;
            }
            if (den > 0.0) C[(size_t)k * (size_t)d + (size_t)t] = (float)(num / den);
        }
    }
    free(start);
    free(order);
    free(fill);
    return J;
}

/* ------------------------------------------------------------------ */
/* Residual (VPTQ page, "Residual Vector Quantization": v_res = v - Q(v)),
 * fp32 subtraction per element. */
void orc_residual(const float* X, long long n_sub, int d, const float* C,
                  const unsigned short* idx, float* R)
{
    for (long long s = 0; s < n_sub; ++s)
        for (int t = 0; t < d; ++t)
            R[s * d + t] = X[s * d + t] - C[(size_t)idx[s] * (size_t)d + (size_t)t];
}

/* Reconstruction (VPTQ page, "Residual Vector Quantization": decode
 * v_hat = C[i1] + Cres[i2]; HAS-VQ abstract: exact reconstruction of the
 * salient weights).  In fp32:
 *   w_hat_ij = ((C1[a1]_t + C2[a2]_t) * c_j) * r_i
 * (stage-2 and scale terms dropped when absent), then w_hat_ij = W_ij at
 * every CSR position. */
void orc_reconstruct(long long M, long long N, int d,
                     const float* C1, const unsigned short* idx1,
                     const float* C2, const unsigned short* idx2,
                     const float* r, const float* c,
                     const int* row_ptr, const int* col, const float* val, float* What)
{
    long long nb = N / d;
    for (long long i = 0; i < M; ++i) {
        for (long long j = 0; j < N; ++j) {
            long long s = i * nb + j / d;
            int t = (int)(j % d);
            float v = C1[(size_t)idx1[s] * (size_t)d + (size_t)t];
            if (C2) v = v + C2[(size_t)idx2[s] * (size_t)d + (size_t)t];
            if (c) v = v * c[j];
            if (r) v = v * r[i];
            What[i * N + j] = v;
        }
        if (row_ptr)
            for (int e = row_ptr[i]; e < row_ptr[i + 1]; ++e) What[i * N + col[e]] = val[e];
    }
}

/* ------------------------------------------------------------------ */
/* The product of the compressed matrix with B activation vectors (VPTQ page,
 * "End-to-End Quantization Pipeline": at inference the weights are decoded by
 * codebook lookup inside the matrix-vector product; SCVQ summary: the sparse
 * correction takes part in that product).  By definition
 *   Y[b, i] = sum_j What[i, j] * X[b, j]
 * with What exactly as orc_reconstruct writes it (float32), the products and
 * the sum taken in float64, j ascending.  X is [B x N], Y is [B x M]. */
int orc_qgemv(long long M, long long N, int d,
              const float* C1, const unsigned short* idx1,
              const float* C2, const unsigned short* idx2,
              const float* r, const float* c,
              const int* row_ptr, const int* col, const float* val,
              const float* X, long long B, double* Y)
{
    float* What = (float*)malloc((size_t)M * (size_t)N * sizeof(float));
    if (!What) return 1;
    orc_reconstruct(M, N, d, C1, idx1, C2, idx2, r, c, row_ptr, col, val, What);
    for (long long b = 0; b < B; ++b) {
        const float* x = X + b * N;
        for (long long i = 0; i < M; ++i) {
            double acc = 0.0;
            for (long long j = 0; j < N; ++j) acc += (double)What[i * N + j] * (double)x[j];
            Y[b * M + i] = acc;
        }
    }
    free(What);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Column groups (VPTQ page, "Outlier Elimination": the columns with the
 * largest Hessian diagonal are held apart with their own codebook, shorter
 * vectors and more centroids; "Interaction with group partitioning": the
 * remaining columns may be split into groups with independent codebooks).
 *
 * Column order: the n_out columns with the largest h (ties: smaller j), in
 * ascending j, then every other column in ascending j.  Groups: group 0 =
 * the first n_out columns of that order (vector length d0, K0 centroids, T0
 * Lloyd iterations, no residual stage) when n_out > 0; then the other
 * N - n_out columns in n_groups contiguous runs of w = ceil(nb/n_groups)*d
 * columns (nb = (N - n_out)/d; the last run may be shorter), each a full
 * two-stage fit (d, K1, T1, K2, T2).  Selection of the salient weights and
 * bi-normalization are done once on the whole matrix, as in orc_fit; each
 * group quantizes the gathered columns of the (bi-normalized) matrix with the
 * gathered column weights, masks and column scales; its reconstruction is
 * written back to its columns and the salient values overwrite at the end.
 * Per-group arrays are concatenated in group order: idx_all holds a group's
 * stage-1 indices then its stage-2 indices; cb_all its C1 then C2; J_all its
 * T+1 (then T2+1) objectives; perm1_all / perm2_all its seeding orders. */
static void orc_lloyd(const float* X, const float* hcol, const float* rho, const unsigned char* keep,
                      long long M, long long N, int d, float* C, int K, int T,
                      unsigned short* idx, double* J, int nthreads);

static int orc_h_desc_cmp(const void* a, const void* b)
{
    const orc_scored* x = (const orc_scored*)a;
    const orc_scored* y = (const orc_scored*)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->lin > y->lin) - (x->lin < y->lin);
}

static int orc_int_cmp(const void* a, const void* b)
{
    int x = *(const int*)a, y = *(const int*)b;
    return (x > y) - (x < y);
}

int orc_column_order(const float* h, long long N, long long n_out, int* cols)
{
    if (n_out < 0 || n_out > N) return 2;
    orc_scored* all = (orc_scored*)malloc(sizeof(orc_scored) * (size_t)N);
    unsigned char* out = (unsigned char*)calloc((size_t)N, 1);
    if (!all || !out) { free(all); free(out); return 3; }
    for (long long j = 0; j < N; ++j) { all[j].score = h[j]; all[j].lin = j; }
    qsort(all, (size_t)N, sizeof(orc_scored), orc_h_desc_cmp);
    for (long long e = 0; e < n_out; ++e) { cols[e] = (int)all[e].lin; out[all[e].lin] = 1; }
    qsort(cols, (size_t)n_out, sizeof(int), orc_int_cmp);
    long long pos = n_out;
    for (long long j = 0; j < N; ++j)
        if (!out[j]) cols[pos++] = (int)j;
    free(all);
    free(out);
    return 0;
}

int orc_fit_grouped(const float* W, const float* h, long long M, long long N, int d,
                    int K1, int T1, int K2, int T2, double p, int binorm, int mask_outliers,
                    long long n_out, int d0, int K0, int T0, int n_groups,
                    const int* perm1_all, const int* perm2_all, int nthreads,
                    int* cols, unsigned short* idx_all, float* cb_all,
                    int* row_ptr, int* col, float* val, unsigned char* keep,
                    float* What, double* J_all)
{
    if (M <= 0 || N <= 0 || d <= 0 || N % d || n_out < 0 || n_out % d || n_groups < 1) return 2;
    if (n_out > 0 && (d0 <= 0 || n_out % d0 || K0 < 1)) return 2;
    long long nb_main = (N - n_out) / d;
    long long w = (nb_main + n_groups - 1) / n_groups * d;
    if (nb_main < 1 || (long long)(n_groups - 1) * w >= N - n_out) return 2;
    long long nnz = orc_nnz(M, N, p);
    int rc = orc_select(W, h, M, N, nnz, row_ptr, col, val, keep);
    if (rc) return rc;
    float* Wp = (float*)malloc(sizeof(float) * (size_t)(M * N));
    float* r = (float*)malloc(sizeof(float) * (size_t)M);
    float* c = (float*)malloc(sizeof(float) * (size_t)N);
    float* hcol = (float*)malloc(sizeof(float) * (size_t)N);
    float* rho = (float*)malloc(sizeof(float) * (size_t)M);
    if (!Wp || !r || !c || !hcol || !rho) return 3;
    if (binorm) orc_binorm(W, h, M, N, Wp, r, c, hcol, rho);
    else memcpy(Wp, W, sizeof(float) * (size_t)(M * N));
    const float* hc = binorm ? hcol : h;
    rc = orc_column_order(h, N, n_out, cols);
    if (rc) return rc;
    long long oi = 0, oc = 0, oj = 0, op1 = 0, op2 = 0;
    int n_all = n_groups + (n_out > 0 ? 1 : 0);
    for (int g = 0; g < n_all && rc == 0; ++g) {
        int outlier = (n_out > 0 && g == 0);
        long long c0 = outlier ? 0 : n_out + (long long)(g - (n_out > 0 ? 1 : 0)) * w;
        long long c1 = outlier ? n_out : (c0 + w < N ? c0 + w : N);
        long long Ng = c1 - c0;
        int dg = outlier ? d0 : d, Kg = outlier ? K0 : K1, Tg = outlier ? T0 : T1;
        int K2g = outlier ? 0 : K2;
        long long nsg = M * Ng / dg;
        float* Xg = (float*)malloc(sizeof(float) * (size_t)(M * Ng));
        float* hg = (float*)malloc(sizeof(float) * (size_t)Ng);
        float* cg = (float*)malloc(sizeof(float) * (size_t)Ng);
        unsigned char* kg = (unsigned char*)malloc((size_t)(M * Ng));
        float* Wg = (float*)malloc(sizeof(float) * (size_t)(M * Ng));
        float* Rg = (float*)malloc(sizeof(float) * (size_t)(M * Ng));
        if (!Xg || !hg || !cg || !kg || !Wg || !Rg) return 3;
        for (long long q = 0; q < Ng; ++q) {
            long long j = cols[c0 + q];
            hg[q] = hc[j];
            cg[q] = c[j];
            for (long long i = 0; i < M; ++i) {
                Xg[i * Ng + q] = Wp[i * N + j];
                kg[i * Ng + q] = keep[i * N + j];
            }
        }
        if (Kg > nsg || K2g > nsg) rc = 2;
        unsigned short* i1 = idx_all + oi;
        float* C1 = cb_all + oc;
        if (!rc && orc_init(Xg, nsg, dg, perm1_all + op1, Kg, C1) != Kg) rc = 1;
        if (!rc) orc_lloyd(Xg, hg, binorm ? rho : NULL, mask_outliers ? kg : NULL, M, Ng, dg, C1, Kg, Tg, i1,
                           J_all + oj, nthreads);
        oi += nsg; oc += (long long)Kg * dg; oj += Tg + 1; op1 += nsg;
        unsigned short* i2 = NULL;
        float* C2 = NULL;
        if (!rc && K2g > 0) {
            i2 = idx_all + oi;
            C2 = cb_all + oc;
            orc_residual(Xg, nsg, dg, C1, i1, Rg);
            if (orc_init(Rg, nsg, dg, perm2_all + op2, K2g, C2) != K2g) rc = 1;
            if (!rc) orc_lloyd(Rg, hg, binorm ? rho : NULL, mask_outliers ? kg : NULL, M, Ng, dg, C2, K2g, T2, i2,
                               J_all + oj, nthreads);
            oi += nsg; oc += (long long)K2g * dg; oj += T2 + 1; op2 += nsg;
        }
        if (!rc) {
            orc_reconstruct(M, Ng, dg, C1, i1, C2, i2, binorm ? r : NULL, binorm ? cg : NULL, NULL, NULL, NULL, Wg);
            for (long long q = 0; q < Ng; ++q)
                for (long long i = 0; i < M; ++i) What[i * N + cols[c0 + q]] = Wg[i * Ng + q];
        }
        free(Xg); free(hg); free(cg); free(kg); free(Wg); free(Rg);
    }
    if (!rc)
        for (long long i = 0; i < M; ++i)
            for (int e = row_ptr[i]; e < row_ptr[i + 1]; ++e) What[i * N + col[e]] = val[e];
    free(Wp); free(r); free(c); free(hcol); free(rho);
    return rc;
}

/* ------------------------------------------------------------------ */
/* Second-order error propagation with column sub-vectors (VPTQ page, "The
 * Core Algorithm", Algorithm 1).  W [M x N] is quantized one column at a
 * time, left to right, in blocks of B columns.  Column n is cut into M/V
 * sub-vectors W[m:m+V, n]; each is replaced by its nearest codebook row under
 * the plain Euclidean distance (fp64, lowest index on ties).  The column's
 * error E[:,n] = (W[:,n] - What[:,n]) / U[n,n] is subtracted, scaled by
 * U[n,j], from the block's later columns j; at the end of a block the
 * block's errors are subtracted from every later column through
 * U[s:s+B, s+B:].  U [N x N] is the matrix the algorithm reads where the page
 * writes H^-1 (GPTQ's upper Cholesky factor of the inverse Hessian, or the
 * inverse itself; the algorithm is the same).  The working copy of W is
 * fp64.  Outputs: idx[n*(M/V) + v] (column n, sub-vector v), What [M x N],
 * E [M x N] (fp64) and gap[n*(M/V) + v] = (second - best) / second, the
 * relative margin of each decision (0 when second == 0, 1 when K == 1). */
int orc_vptq(const float* W, const float* U, long long M, long long N, int V, const float* C, int K,
             int B, unsigned short* idx, float* What, double* E, double* gap)
{
    long long nv = M / V;
    double* Wk = (double*)malloc(sizeof(double) * (size_t)(M * N));
    if (!Wk) return 3;
    for (long long e = 0; e < M * N; ++e) Wk[e] = (double)W[e];
    for (long long s = 0; s < N; s += B) {
        long long s_end = s + B < N ? s + B : N;
        for (long long n = s; n < s_end; ++n) {
#pragma omp parallel for schedule(static)
            for (long long v = 0; v < nv; ++v) {
                double best = INFINITY, second = INFINITY;
                int arg = 0;
                for (int k = 0; k < K; ++k) {
                    double dist = 0.0;
                    for (int t = 0; t < V; ++t) {
                        double diff = Wk[(v * V + t) * N + n] - (double)C[(size_t)k * (size_t)V + (size_t)t];
                        dist += diff * diff;
                    }
                    if (dist < best) { second = best; best = dist; arg = k; }
                    else if (dist < second) second = dist;
                }
                idx[n * nv + v] = (unsigned short)arg;
                gap[n * nv + v] = isinf(second) ? 1.0 : (second > 0.0 ? (second - best) / second : 0.0);
                for (int t = 0; t < V; ++t)
                    What[(v * V + t) * N + n] = C[(size_t)arg * (size_t)V + (size_t)t];
            }
            double unn = (double)U[n * N + n];
            for (long long m = 0; m < M; ++m) E[m * N + n] = (Wk[m * N + n] - (double)What[m * N + n]) / unn;
            for (long long j = n + 1; j < s_end; ++j) {
                double unj = (double)U[n * N + j];
                for (long long m = 0; m < M; ++m) Wk[m * N + j] -= E[m * N + n] * unj;
            }
        }
        for (long long m = 0; m < M; ++m) {
            for (long long j = s_end; j < N; ++j) {
                double acc = 0.0;
                for (long long n = s; n < s_end; ++n) acc += E[m * N + n] * (double)U[n * N + j];
                Wk[m * N + j] -= acc;
            }
        }
    }
    free(Wk);
    return 0;
}

/* ------------------------------------------------------------------ */
/* One stage of weighted K-means (Lloyd): T times (assign, update), then a
 * final assign, so the returned indices are the argmin for the returned
 * codebook.  J[0..T] receives the objective of each (codebook, assignment)
 * pair in order (VPTQ page, "Hessian-Weighted Centroid Initialization":
 * weighted K-means; its Lloyd iterations never raise J). */
static void orc_lloyd(const float* X, const float* hcol, const float* rho, const unsigned char* keep,
                      long long M, long long N, int d, float* C, int K, int T,
                      unsigned short* idx, double* J, int nthreads)
{
    for (int it = 0; it < T; ++it) {
        orc_assign(X, hcol, rho, keep, M, N, d, C, K, NULL, 0, idx, NULL, nthreads);
        J[it] = orc_update(X, hcol, rho, keep, M, N, d, idx, K, C, NULL);
    }
    orc_assign(X, hcol, rho, keep, M, N, d, C, K, NULL, 0, idx, NULL, nthreads);
    J[T] = orc_objective(X, hcol, rho, keep, M, N, d, C, idx);
}

/* The whole per-matrix pipeline: select -> (bi-normalize) -> seed -> Lloyd
 * -> residual -> seed -> Lloyd -> reconstruct.  (HAS-VQ abstract: decouple,
 * VQ of the dense body, exact sparse feedback; VPTQ page, "End-to-End
 * Quantization Pipeline": main codebook, then a residual codebook on W - What.)
 * K2 = 0 skips the residual stage.  mask_outliers = 0 keeps the salient
 * positions in the clustering (they are still overwritten on reconstruct).
 * Returns 0 on success, 1 when a stage finds fewer than K distinct
 * sub-vectors, 2 on invalid sizes, 3 on allocation failure. */
int orc_fit(const float* W, const float* h, long long M, long long N, int d,
            int K1, int T1, int K2, int T2, double p, int binorm, int mask_outliers,
            const int* perm1, const int* perm2, int nthreads,
            unsigned short* idx1, float* C1, unsigned short* idx2, float* C2,
            int* row_ptr, int* col, float* val, unsigned char* keep,
            float* Wp, float* r, float* c, float* hcol, float* rho,
            float* What, double* J_hist)
{
    if (M <= 0 || N <= 0 || d <= 0 || d > 64 || N % d != 0 || K1 < 1 || K2 < 0) return 2;
    long long n_sub = M * N / d;
    if (K1 > n_sub || K2 > n_sub || K1 > 65536 || K2 > 65536) return 2;
    long long nnz = orc_nnz(M, N, p);
    int rc = orc_select(W, h, M, N, nnz, row_ptr, col, val, keep);
    if (rc) return rc;
    const unsigned char* km = mask_outliers ? keep : NULL;
    const float* hc = h;
    const float* rh = NULL;
    if (binorm) {
        orc_binorm(W, h, M, N, Wp, r, c, hcol, rho);
        hc = hcol;
        rh = rho;
    } else {
        memcpy(Wp, W, sizeof(float) * (size_t)(M * N));
    }
    if (orc_init(Wp, n_sub, d, perm1, K1, C1) != K1) return 1;
    orc_lloyd(Wp, hc, rh, km, M, N, d, C1, K1, T1, idx1, J_hist, nthreads);
    if (K2 > 0) {
        float* R = (float*)malloc(sizeof(float) * (size_t)(M * N));
        if (!R) return 3;
        orc_residual(Wp, n_sub, d, C1, idx1, R);
        if (orc_init(R, n_sub, d, perm2, K2, C2) != K2) { free(R); return 1; }
        orc_lloyd(R, hc, rh, km, M, N, d, C2, K2, T2, idx2, J_hist + T1 + 1, nthreads);
        free(R);
    }
    orc_reconstruct(M, N, d, C1, idx1, K2 > 0 ? C2 : NULL, idx2,
                    binorm ? r : NULL, binorm ? c : NULL, row_ptr, col, val, What);
    return 0;
}
