/*
 * vq.h -- C ABI of libvq: Hessian/salience-weighted vector quantization of
 * one LLM weight matrix on an AMD Instinct MI355X (gfx950).
 *
 * The method (sources are the pages' titles and sections):
 *   - HAS-VQ abstract: salient weights, scored by second-order sensitivity,
 *     are decoupled from the bulk (its Hessian-Masked Decoupling) and
 *     reconstructed exactly through a sparse correction; the dense remainder
 *     is vector quantized.
 *   - VPTQ page, "Hessian-Weighted Centroid Initialization": with a diagonal
 *     Hessian the objective is a weighted K-means problem; centroids are
 *     weighted means.
 *   - VPTQ page, "Residual Vector Quantization": a second codebook quantizes
 *     the first stage's error; decode adds the two centroids.
 *   - SCVQ summary: weights bi-normalized across rows and columns, salience-
 *     weighted K-means, every exactly held weight in one CSR.
 *
 * Conventions (all entry points):
 *   - W is [M x N] row-major float32, M outputs by N inputs.  h (the diagonal
 *     Hessian proxy) has one float32 entry per input column j.
 *   - A sub-vector s = (row i, block b) holds W[i, b*d .. b*d+d-1]; its id is
 *     s = i*(N/d) + b, so a matrix read as [n_sub x d] is contiguous.
 *     n_sub = M*N/d.  1 <= d <= 8 and N % d == 0.
 *   - Element weight omega(i,j) = m_ij * hcol[j] * rho[i]; m_ij = 0 on the
 *     salient positions (when masking is on), 1 elsewhere; rho = 1 when NULL.
 *   - Distance D(s,k) = sum_t omega(s,t) (x(s,t) - C(k,t))^2; objective
 *     J = sum_s D(s, a_s).
 *   - Indices are uint16 (1 <= K <= 65536); codebooks are [K x d] float32.
 *   - mask is one byte per sub-vector: bit t set <=> element t is salient
 *     (weight 0 in clustering).  A NULL mask means no salient positions.
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns and
 *     allocates every buffer, including the workspace; the library never
 *     allocates device memory in these calls and never frees caller memory.
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).  Step
 *     calls enqueue work and return without synchronizing; vq_init and vq_fit
 *     synchronize the stream (they read device data on the host).
 *   - Every call validates its arguments on the host before any launch and
 *     returns a vq_status; vq_last_error() (thread-local) describes the last
 *     failure.  Finite floating-point inputs and non-negative weights (h,
 *     hcol, rho) are preconditions, unchecked by default.  With the
 *     environment variable VQ_CHECK=1 (read at every call), every
 *     entry point first counts on the device the non-finite values of each
 *     floating-point input array it is given (of the weight arrays: also the
 *     values with the sign bit set) and returns VQ_ERR_INVALID naming the
 *     array if any is found.  That mode reads every input once more and
 *     synchronizes the stream per checked array.
 */
#ifndef VQ_H
#define VQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    VQ_OK = 0,
    VQ_ERR_INVALID = 1,     /* bad argument: null pointer, size or range */
    VQ_ERR_WORKSPACE = 2,   /* ws_bytes below what the call needs */
    VQ_ERR_INIT = 3,        /* fewer than K bitwise-distinct sub-vectors */
    VQ_ERR_DEVICE = 4,      /* a HIP runtime call failed (message attached) */
    VQ_ERR_UNSUPPORTED = 5  /* no gfx950 device current */
} vq_status;

/* Library version string (static storage). */
const char* vq_version(void);

/* Description of the last failure on this thread ("" if none). */
const char* vq_last_error(void);

/* Salient count of a fit: nnz = floor(p * M * N), the product taken in
 * float64 (M*N exact as an integer first).  -1 if M or N is not positive or p
 * is outside [0, 1].  Host arithmetic. */
int64_t vq_nnz(int64_t M, int64_t N, double p);

/* Workspace bytes sufficient for every call below with these sizes
 * (K2 = 0: no residual stage; nnz = number of salient weights). */
size_t vq_workspace_bytes(int64_t M, int64_t N, int d, int K1, int K2, int64_t nnz);

/* Salience selection into the exact sparse correction.
 * HAS-VQ abstract (Hessian-Masked Decoupling; exact reconstruction of the
 * salient weights); SCVQ summary (every exactly held weight in one CSR).
 * Score s_ij = h_j * (w_ij * w_ij) in float32 (no fused multiply-add).  The
 * nnz largest scores are selected, ties broken by the smaller linear index
 * i*N+j.  Outputs: row_ptr int32[M+1], col int32[nnz] (ascending within each
 * row), val float32[nnz] (the exact W values), mask uint8[n_sub] (bit t of
 * byte s set <=> element t of sub-vector s is selected).  Bitwise
 * deterministic.  0 <= nnz <= min(M*N, 2^31-1); scores must be >= +0. */
vq_status vq_sparse_select(const float* W, const float* h, int64_t M, int64_t N, int d,
                           int64_t nnz, int32_t* row_ptr, int32_t* col, float* val,
                           uint8_t* mask, void* ws, size_t ws_bytes, void* stream);

/* The unified sparse correction (SCVQ summary: a single sparse matrix
 * carries every exactly-held weight, namely the salient elements, whole
 * sub-vectors of high salience and the positions where quantization left the
 * biggest error).  The mask (one byte per sub-vector, bit t =
 * element t held exactly) is the correction set; these calls OR new positions
 * into it and vq_mask_to_csr writes its CSR.  Keys below are float32 scores,
 * which must be >= +0 (h >= 0); ties go to the smaller id.  Bitwise
 * deterministic.  Workspace: vq_workspace_bytes for these sizes.
 *
 * Salient sub-vectors: S_s = sum over t in order of h_j * (w_j * w_j), each
 * product and partial sum rounded to float32 (no fused multiply-add); the
 * n_sel largest get every mask bit set.  0 <= n_sel <= n_sub. */
vq_status vq_select_subvectors(const float* W, const float* h, int64_t M, int64_t N, int d,
                               int64_t n_sel, uint8_t* mask, void* ws, size_t ws_bytes, void* stream);

/* Largest quantization residuals: among positions whose mask bit is clear,
 * r_ij = h_j * ((w_ij - what_ij) * (w_ij - what_ij)) in float32 (difference,
 * square, scale); the min(n_sel, #clear) largest get their bit set.  W_hat is
 * the quantized matrix [M x N] (vq_reconstruct without a sparse part). */
vq_status vq_select_residual(const float* W, const float* W_hat, const float* h, int64_t M, int64_t N,
                             int d, int64_t n_sel, uint8_t* mask, void* ws, size_t ws_bytes, void* stream);

/* CSR of every position whose mask bit is set: row_ptr int32[M+1], col
 * ascending within each row, val = the exact W value.  At most nnz_cap entries
 * are written; row_ptr[M] is the full count (> nnz_cap: the CSR was cut).
 * M*N <= 2^31-1. */
vq_status vq_mask_to_csr(const float* W, const uint8_t* mask, int64_t M, int64_t N, int d,
                         int64_t nnz_cap, int32_t* row_ptr, int32_t* col, float* val,
                         void* ws, size_t ws_bytes, void* stream);

/* Bi-normalization (SCVQ summary: rows and columns bi-normalized before
 * clustering), one pass of RMS scaling, rows first:
 *   r_i = sqrt(sum_j W_ij^2 / N) (fp64 sum; 1 if zero), Wt = W / r_i (fp32),
 *   c_j = sqrt(sum_i Wt_ij^2 / M) (fp64 sum; 1 if zero), Wp = Wt / c_j (fp32),
 *   hcol_j = h_j c_j^2 and rho_i = r_i^2 (fp64 products, stored fp32),
 * so that the weighted objective on Wp equals the original-space objective.
 * Outputs Wp [M x N], r [M], c [N], hcol [N], rho [M]. */
vq_status vq_binorm(const float* W, const float* h, int64_t M, int64_t N,
                    float* Wp, float* r, float* c, float* hcol, float* rho,
                    void* ws, size_t ws_bytes, void* stream);

/* Codebook seeding: walk perm (host int32[n_sub], a permutation of the
 * sub-vector ids) and copy the first K sub-vectors of X whose d floats are
 * not bitwise equal to one already taken into C [K x d].  Returns
 * VQ_ERR_INIT if fewer than K distinct sub-vectors exist.  Synchronizes. */
vq_status vq_init(const float* X, int64_t M, int64_t N, int d, const int32_t* perm,
                  int K, float* C, void* ws, size_t ws_bytes, void* stream);

/* Assignment (VPTQ page, "The Core Algorithm": nearest centroid; here under
 * the weighted distance D).  idx[s] = argmin_k D(s,k), ties to the lowest k.
 * The result equals the exact (float64, direct form) argmin: the expanded
 * form runs on the fp16 matrix cores with every fp32 operand split into two
 * fp16 parts (fp32 accumulation), each winner is certified against a
 * rigorous rounding bound, and uncertified sub-vectors are re-searched
 * exactly in float64.  With more than 2048 centroids and a workspace of
 * vq_workspace_bytes (64 bytes per sub-vector beyond the minimum), the search
 * runs in two passes: a coarse pass (one fp16 product per term) with a
 * derived bound names each sub-vector's candidate groups of 1024 centroids,
 * and only those are searched as above; with a smaller workspace it runs in
 * one pass.  The results are the same.  X = the matrix being quantized ([M x N] f32),
 * hcol [N], rho [M] (nullable), mask (nullable), C [K x d].  Outputs
 * idx uint16[n_sub] and, if dist != NULL, dist float32[n_sub] = D(s, idx[s])
 * computed in float64 and rounded. */
vq_status vq_assign(const float* X, const float* hcol, const float* rho, const uint8_t* mask,
                    int64_t M, int64_t N, int d, const float* C, int K,
                    uint16_t* idx, float* dist, void* ws, size_t ws_bytes, void* stream);

/* vq_assign without a workspace argument, for callers that cannot allocate
 * device memory (code under stream capture, serving loops, harnesses that
 * forbid allocation).  Same arguments and results as vq_assign; its scratch
 * (the prepared codebook, the re-search and per-sub-vector lists) lives in one
 * library-held device array of 64 MiB per GPU, allocated when the library is
 * loaded and held until the process ends.  Needs 64*ceil(K/256)*256 +
 * 9*n_sub bytes plus about 2 KiB: K = 65536 allows n_sub up to about 6.99
 * million (the two-pass search of long codebooks runs where the array also
 * holds its 64 bytes per sub-vector, else the one-pass search).  Larger sizes return VQ_ERR_INVALID before any launch.  The call
 * allocates nothing.  Every call on one GPU shares that GPU's array (each call
 * clears what it needs), so calls that overlap in time on one GPU race; the
 * vq_assign_exact_* diagnostics do not see this array. */
vq_status vq_assign_noalloc(const float* X, const float* hcol, const float* rho, const uint8_t* mask,
                            int64_t M, int64_t N, int d, const float* C, int K,
                            uint16_t* idx, float* dist, void* stream);

/* Diagnostics: number of sub-vectors that the last vq_assign call on this
 * workspace (same n_sub and K) sent to the exact float64 re-search because
 * their winner could not be certified.  Synchronizes the stream; -1 on error. */
int vq_assign_exact_count(void* ws, size_t ws_bytes, int64_t n_sub, int K, void* stream);

/* Diagnostics: the ids of those sub-vectors.  Copies up to cap of them (in no
 * particular order) into list (host int32[cap]) and returns their number (may
 * exceed cap); -1 on error.  Synchronizes the stream. */
int64_t vq_assign_exact_list(void* ws, size_t ws_bytes, int64_t n_sub, int K, int32_t* list, int64_t cap,
                             void* stream);

/* Centroid update (VPTQ page, "Hessian-Weighted Centroid Initialization":
 * weighted-mean centroids; with one weight per element this is the
 * per-dimension weighted mean, the exact minimizer of J for fixed indices):
 *   C(k,t) = sum_{idx_s=k} omega x / sum_{idx_s=k} omega   (fp64 sums, one
 *   rounding to fp32); a zero weight sum keeps the old value.
 * C is read and overwritten in place.  counts (nullable) receives int32[K]
 * member counts; J (nullable, device double[1]) receives the objective of
 * the INPUT codebook with these indices.  Members are grouped by a stable
 * bucket scatter and per-bucket counting sorts, and every sum is taken in a
 * fixed order without floating-point atomics, so the result is bitwise
 * deterministic.  Every idx[s] must be < K: an index >= K never causes an
 * out-of-bounds access, but the centroids it lands on are then unspecified. */
vq_status vq_update(const float* X, const float* hcol, const float* rho, const uint8_t* mask,
                    int64_t M, int64_t N, int d, const uint16_t* idx, int K,
                    float* C, int32_t* counts, double* J, void* ws, size_t ws_bytes, void* stream);

/* Objective J = sum_s D(s, idx[s]) (fp64, fixed reduction order) into the
 * device double J[0]. */
vq_status vq_objective(const float* X, const float* hcol, const float* rho, const uint8_t* mask,
                       int64_t M, int64_t N, int d, const float* C, int K, const uint16_t* idx,
                       double* J, void* ws, size_t ws_bytes, void* stream);

/* Residual (VPTQ page, "Residual Vector Quantization": v_res = v - Q(v)):
 * R = X - C[idx] elementwise in float32.  R may not alias X. */
vq_status vq_residual(const float* X, int64_t M, int64_t N, int d, const float* C, int K,
                      const uint16_t* idx, float* R, void* stream);

/* Reconstruction (VPTQ page, "Residual Vector Quantization": decode
 * C[i1] + Cres[i2]; HAS-VQ abstract: salient weights reconstructed exactly):
 *   W_hat_ij = ((C1[idx1]_t + C2[idx2]_t) * cscale_j) * rscale_i   (fp32)
 * with the stage-2 term skipped when C2 == NULL and each scale skipped when
 * NULL; then W_hat_ij = val at every CSR position (row_ptr/col/val may be
 * NULL for no sparse part).  Bitwise deterministic. */
vq_status vq_reconstruct(int64_t M, int64_t N, int d, const float* C1, int K1, const uint16_t* idx1,
                         const float* C2, int K2, const uint16_t* idx2,
                         const float* rscale, const float* cscale,
                         const int32_t* row_ptr, const int32_t* col, const float* val,
                         float* W_hat, void* stream);

/* Fused dequantize-and-multiply (VPTQ page, "End-to-End Quantization
 * Pipeline": at inference the centroids are looked up inside the
 * matrix-vector product so the full weight matrix is never written; SCVQ
 * summary: the sparse correction takes part in the product):
 *   Y[b, i] = sum_j W_hat[i, j] * X[b, j],   b < B, i < M,
 * where W_hat is what vq_reconstruct writes for the same arguments; W_hat is
 * never materialized.  X is [B x N] and Y is [B x M], float32 row-major, Y
 * may not alias X.  Arithmetic: float32.  The kernel multiplies the decoded
 * C1 (+ C2) value by x_j * cscale_j, sums with fused multiply-adds, scales the
 * row sum by rscale_i, and for a salient entry takes the decoded term back out
 * and adds val * x_j.  Error bound against the exact product: with
 * u = 2^-24 and
 *   T[b,i] = sum_j |Wd[i,j] x[b,j]| + sum_{salient (i,j)} (|Wd[i,j]| + |val|) |x[b,j]|
 * (Wd = W_hat without the sparse overwrite),
 *   |Y[b,i] - exact| <= (N/32 + nnz_i + 40) * u * T[b,i],
 * nnz_i the salient count of row i.  Salient columns must be distinct within
 * a row.  Results are bitwise reproducible for fixed arguments.  B = 0 is a
 * no-op.  ws: at least vq_qgemv_workspace_bytes(M, N, d, B) bytes (may be 0,
 * then ws may be NULL). */
size_t vq_qgemv_workspace_bytes(int64_t M, int64_t N, int d, int64_t B);
vq_status vq_qgemv(int64_t M, int64_t N, int d, const float* C1, int K1, const uint16_t* idx1,
                   const float* C2, int K2, const uint16_t* idx2,
                   const float* rscale, const float* cscale,
                   const int32_t* row_ptr, const int32_t* col, const float* val,
                   const float* X, int64_t B, float* Y, void* ws, size_t ws_bytes, void* stream);

/* The matrix the second-order error propagation below reads where the VPTQ
 * page ("The Core Algorithm") writes H^-1, in GPTQ's form (the page says the
 * technique is inherited from it): U [N x N], upper triangular with positive
 * diagonal, U^T U = (H + damp * mean(diag H) * I)^-1.  Computed in float64 as
 * U = P L^-1 P, where P reverses the order and L is the Cholesky factor of
 * P (H + damp * mean(diag H) * I) P; stored float32 with the strict lower
 * triangle zero.  H [N x N] float32 symmetric (read in full); the damped
 * matrix must be positive definite (else U holds NaN).  Workspace:
 * vq_hessian_factor_workspace_bytes(N) (two N x N float64 matrices). */
size_t vq_hessian_factor_workspace_bytes(int64_t N);
vq_status vq_hessian_factor(const float* H, int64_t N, double damp, float* U, void* ws, size_t ws_bytes,
                            void* stream);

/* Second-order error propagation with column sub-vectors (VPTQ page, "The
 * Core Algorithm", Algorithm 1).  Columns of W [M x N] are quantized left to
 * right in blocks of B: each of a column's M/V sub-vectors W[m:m+V, n] takes
 * its nearest row of C [K x V] under the plain Euclidean distance (the
 * lowest index among equal distances); the column's error
 * E[:,n] = (W[:,n] - What[:,n]) / U[n,n] is subtracted, times U[n,j], from the
 * block's later columns j, and at the block's end E[:, s:s+B] U[s:s+B, s+B:]
 * is subtracted from every later column.  U [N x N] row-major is the matrix
 * the algorithm reads where the page writes H^-1; only its upper triangle is
 * read (GPTQ's upper Cholesky factor of the damped inverse Hessian, or the
 * inverse itself).  W is not modified.  Outputs: idx uint16 [N x M/V]
 * (idx[n*(M/V) + v] for sub-vector v of column n), W_hat [M x N] (codebook
 * rows), E [M x N] (nullable; the float64 errors rounded to float32).
 * Arithmetic: the working matrix and the errors are float64, each in-block
 * update is taken as w - e*u (product rounded, then the difference) column
 * after column, and the block's end update forms each sum of e*u over the
 * block's columns in column order (each product rounded, then added) before
 * subtracting it; every decision equals the exact float64 direct-form one
 * (V = 8 with C 16-byte aligned and M % 4 == 0: the expanded form |c|^2/2 -
 * <c, x> on the fp16 matrix cores with split operands, each winner certified
 * against a rounding bound and the uncertified searched again in float64;
 * otherwise the float64 direct form throughout).  The results are therefore
 * those of the float64 algorithm as written, bit for bit.  1 <= V <= 8 with
 * M % V == 0; 1 <= K <= 65536; 1 <= B <= 128.  Workspace:
 * vq_vptq_workspace_bytes(M, N, V) (two float64 and one float32 transposed
 * M x N matrices, the split codebook, per-column keys and chunk results).
 * With timing on, the record "vptq_exact_searches" counts (as launches) the
 * decisions that took the exact search. */
size_t vq_vptq_workspace_bytes(int64_t M, int64_t N, int V);
vq_status vq_vptq(const float* W, const float* U, int64_t M, int64_t N, int V, const float* C, int K, int B,
                  uint16_t* idx, float* W_hat, float* E, void* ws, size_t ws_bytes, void* stream);

/* The whole per-matrix pipeline (HAS-VQ abstract; VPTQ page, "End-to-End
 * Quantization Pipeline": main codebook, then a residual codebook on
 * W - W_hat):
 *   [bi-normalize] -> select -> seed C1 -> iters1 x (assign, update) -> assign
 *   -> residual -> seed C2 -> iters2 x (assign, update) -> assign -> reconstruct.
 * Salient scores are taken on the original W and h. */
typedef struct {
    int64_t M, N;
    int d;
    int K1, iters1;
    int K2, iters2;        /* K2 = 0: no residual stage */
    double outlier_frac;   /* p; nnz = floor(p * M * N) */
    int binorm;            /* 1: bi-normalize before clustering */
    int mask_outliers;     /* 1: salient weights get weight 0 in clustering */
} vq_fit_params;

typedef struct {
    const float* W;        /* [M x N] */
    const float* h;        /* [N] */
    const int32_t* perm1;  /* host int32[n_sub]: seeding order, stage 1 */
    const int32_t* perm2;  /* host int32[n_sub]: seeding order, stage 2 */
    const float* C1_init;  /* nullable [K1 x d]: replaces stage-1 seeding (resume) */
    const float* C2_init;  /* nullable [K2 x d]: replaces stage-2 seeding */
} vq_fit_inputs;

typedef struct {
    uint16_t* idx1; float* C1;     /* [n_sub], [K1 x d] */
    uint16_t* idx2; float* C2;     /* [n_sub], [K2 x d] (unused when K2 = 0) */
    int32_t* row_ptr; int32_t* col; float* val;   /* CSR: [M+1], [nnz], [nnz] */
    uint8_t* mask;                 /* [n_sub] */
    float* Wp;                     /* [M x N] bi-normalized matrix (binorm only) */
    float* rscale; float* cscale;  /* [M], [N] (binorm only) */
    float* hcol; float* rho;       /* [N], [M] (binorm only) */
    float* W_hat;                  /* [M x N] */
    double* J_hist;                /* host double[iters1+1 (+ iters2+1)] */
    double* bpw;                   /* host double[1], b_cb = 32 (nullable) */
    int64_t* empty_hist;           /* host int64[iters1 (+ iters2)] (nullable): after each
                                      update, the number of centroids with no member (they
                                      keep their previous value) */
} vq_fit_outputs;

vq_status vq_fit(const vq_fit_params* p, const vq_fit_inputs* in, vq_fit_outputs* out,
                 void* ws, size_t ws_bytes, void* stream);

/* Column groups (VPTQ page, "Outlier Elimination": the columns with the
 * largest Hessian diagonal are held apart, quantized with a separate codebook
 * of shorter vectors and more centroids; "Interaction with group
 * partitioning": the other columns may be split into groups with independent
 * codebooks).  The whole pipeline of vq_fit with its vector-quantization part
 * run per column group:
 *   select (on W, h) and bi-normalization, both on the whole matrix;
 *   column order cols [N]: the n_out columns with the largest h (ties: the
 *     smaller index) ascending, then the other columns ascending;
 *   groups, in order: the outlier group cols[0, n_out) (d0, K0, iters0, one
 *     stage) when n_out > 0; then the other columns in n_groups contiguous
 *     runs of w = ceil(((N - n_out)/d) / n_groups) * d columns of the order
 *     (the last may be shorter), each a two-stage fit with fit.d, K1, iters1,
 *     K2, iters2;
 *   each group gathers its columns of the (bi-normalized) matrix, column
 *     weights, salient bits and column scales, is seeded from its own
 *     permutation, runs its Lloyd stages, and is reconstructed (with the
 *     scales, without the sparse part) back into its columns; the salient
 *     values overwrite at the end.
 * n_out must be a multiple of fit.d and of d0 (1 <= d0 <= 8).  Per-group
 * arrays are concatenated in group order: idx = a group's stage-1 indices then
 * its stage-2 indices (sub-vector ids of the group's own M x N_g matrix);
 * codebooks = its C1 [K x d_g] then C2; J_hist its iters+1 (then iters2+1)
 * objectives; perm1 (host) its stage-1 seeding order, perm2 (host) the
 * stage-2 orders of the main groups.  vq_grouped_sizes returns the workspace
 * bytes (0 when the sizes do not split) and the lengths of those arrays.
 * Synchronizes. */
typedef struct {
    vq_fit_params fit;      /* the main groups and the salient selection */
    int64_t n_out;          /* outlier columns; 0 = none */
    int d0, K0, iters0;     /* the outlier group */
    int n_groups;           /* groups of the other columns, >= 1 */
} vq_grouped_params;

typedef struct {
    const float* W;         /* [M x N] */
    const float* h;         /* [N] */
    const int32_t* perm1;   /* host */
    const int32_t* perm2;   /* host (unused when K2 = 0) */
} vq_grouped_inputs;

typedef struct {
    int32_t* cols;          /* [N] column order */
    uint16_t* idx;
    float* codebooks;
    int32_t* row_ptr; int32_t* col; float* val;   /* salient CSR, [M+1], [nnz], [nnz] */
    uint8_t* mask;          /* [M*N/fit.d], the whole matrix's salient bits */
    float* W_hat;           /* [M x N] */
    double* J_hist;         /* host */
    double* bpw;            /* host, nullable */
} vq_grouped_outputs;

size_t vq_grouped_sizes(const vq_grouped_params* p, int64_t* n_idx, int64_t* n_codebook, int64_t* n_J,
                        int64_t* n_perm1, int64_t* n_perm2);
vq_status vq_fit_grouped(const vq_grouped_params* p, const vq_grouped_inputs* in, vq_grouped_outputs* out,
                         void* ws, size_t ws_bytes, void* stream);
/* Bits per weight of a grouped fit: every group's index bits and 32-bit
 * codebooks, 64 bits per salient weight plus the int32 row pointer, the
 * scales (bi-normalization) and one int32 per outlier column, over M*N. */
double vq_bits_per_weight_grouped(const vq_grouped_params* p);


/* Bits per weight of the stored result (host arithmetic; VPTQ page,
 * "End-to-End Quantization Pipeline", compression ratio: index bits plus
 * codebook bits, extended by the sparse part and the scales):
 *   n_sub*(ceil(log2 K1) + ceil(log2 K2)) + d*(K1+K2)*cb_bits + 64*nnz
 *   + 32*(M+1) [nnz > 0] + 32*(M+N) [binorm], divided by M*N. */
double vq_bits_per_weight(int64_t M, int64_t N, int d, int K1, int K2, int64_t nnz,
                          int cb_bits, int binorm);

/* Diagnostics: GPU time per step.  vq_timing_enable(1) clears the records
 * and makes every later step call bracket its kernels with HIP events
 * recorded on that call's stream; vq_timing_enable(0) stops recording.
 * Records are keyed by (step name, K); names: "assign_search" (the matrix-core
 * search kernel alone), "assign" (the whole vq_assign), "update", "objective",
 * "select", "binorm", "residual", "reconstruct", "init".  vq_timing_count()
 * waits for the recorded events and returns the number of records;
 * vq_timing_get(i, ...) fills record i (name into a caller buffer of
 * name_len bytes): launches, total, min and max milliseconds.  Returns 0 on
 * success, 1 if i is out of range. */
void vq_timing_enable(int on);
int vq_timing_count(void);
int vq_timing_get(int i, char* name, int name_len, int* K, int64_t* launches, double* total_ms,
                  double* min_ms, double* max_ms);

#ifdef __cplusplus
}
#endif
#endif /* VQ_H */
