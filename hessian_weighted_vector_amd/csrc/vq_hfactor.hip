// The matrix that the second-order error propagation reads where the VPTQ
// page ("The Core Algorithm") writes H^-1, in GPTQ's form (the technique the
// page says it inherits): U, the upper-triangular factor with positive
// diagonal and U^T U = Hd^-1, Hd = H + damp * mean(diag H) * I.
//
// Route, all in float64: with P the reversal permutation, G = P Hd P has the
// ordinary Cholesky factor L (G = L L^T), so Hd = (P L P)(P L P)^T with P L P
// upper triangular and U = (P L P)^-1 = P L^-1 P.  Both L and L^-1 are formed
// by right-looking blocked algorithms over panels of kNb columns:
//   Cholesky:  factor the diagonal block in LDS (one workgroup), solve the
//              panel below it (one thread per row), subtract the panel's
//              outer product from the trailing lower triangle (GEMM);
//   inverse:   X = I, then per block row i: X_i = L_ii^-1 X_i (one thread per
//              column), and X_{i+1:} -= L_{i+1:, i} X_i over the columns X_i
//              can be non-zero in (GEMM).
// The GEMM is a 64 x 64-tile float64 kernel on the vector units (MI355X's
// float64 vector and matrix rates are equal); each thread holds 4 x 4 sums.
#include "vq_internal.h"

namespace vq {
namespace {

constexpr int kNb = 32;       // panel width
constexpr int kGt = 64;       // GEMM output tile
constexpr int kGk = 16;       // GEMM k chunk

// G[i][j] = H[N-1-i][N-1-j] in float64, plus damp * mean(diag H) on the
// diagonal; mean from a fixed-order sum (one block).
__global__ __launch_bounds__(256) void k_diag_mean(const float* __restrict__ H, int64_t N, double* __restrict__ mean)
{
    __shared__ double sh[256];
    double acc = 0.0;
    for (int64_t i = threadIdx.x; i < N; i += 256) acc += (double)H[i * N + i];
    sh[threadIdx.x] = acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) *mean = sh[0] / (double)N;
}

__global__ __launch_bounds__(256) void k_build_g(const float* __restrict__ H, int64_t N, double damp,
                                                 const double* __restrict__ mean, double* __restrict__ G)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= N * N) return;
    const int64_t i = e / N, j = e - i * N;
    double v = (double)H[(N - 1 - i) * N + (N - 1 - j)];
    if (i == j) v += damp * *mean;
    G[e] = v;
}

__global__ __launch_bounds__(256) void k_identity(double* __restrict__ X, int64_t N)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= N * N) return;
    const int64_t i = e / N;
    X[e] = (i == e - i * N) ? 1.0 : 0.0;
}

// U[i][j] = X[N-1-i][N-1-j] (X = L^-1 lower, so U is upper), float32.
__global__ __launch_bounds__(256) void k_reverse_out(const double* __restrict__ X, int64_t N, float* __restrict__ U)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= N * N) return;
    const int64_t i = e / N, j = e - i * N;
    U[e] = j >= i ? (float)X[(N - 1 - i) * N + (N - 1 - j)] : 0.0f;
}

// Cholesky of the kb x kb diagonal block at (k0, k0), in place (lower).
__global__ __launch_bounds__(256) void k_potrf_diag(double* __restrict__ A, int64_t N, int64_t k0, int kb)
{
    __shared__ double a[kNb][kNb + 1];
    for (int q = threadIdx.x; q < kb * kb; q += 256) {
        const int i = q / kb, j = q - i * kb;
        a[i][j] = j <= i ? A[(k0 + i) * N + k0 + j] : 0.0;
    }
    __syncthreads();
    for (int j = 0; j < kb; ++j) {
        if (threadIdx.x == 0) a[j][j] = sqrt(a[j][j]);
        __syncthreads();
        for (int i = j + 1 + (int)threadIdx.x; i < kb; i += 256) a[i][j] = a[i][j] / a[j][j];
        __syncthreads();
        const int rem = kb - j - 1;
        for (int q = threadIdx.x; q < rem * rem; q += 256) {
            const int i = j + 1 + q / rem, k = j + 1 + q % rem;
            if (k <= i) a[i][k] = fma(-a[i][j], a[k][j], a[i][k]);
        }
        __syncthreads();
    }
    for (int q = threadIdx.x; q < kb * kb; q += 256) {
        const int i = q / kb, j = q - i * kb;
        if (j <= i) A[(k0 + i) * N + k0 + j] = a[i][j];
    }
}

// Rows i >= k0 + kb of the panel: l_i L11^T = a_i (forward substitution).
__global__ __launch_bounds__(256) void k_trsm_panel(double* __restrict__ A, int64_t N, int64_t k0, int kb)
{
    __shared__ double l[kNb][kNb + 1];
    for (int q = threadIdx.x; q < kb * kb; q += 256) {
        const int i = q / kb, j = q - i * kb;
        l[i][j] = j <= i ? A[(k0 + i) * N + k0 + j] : 0.0;
    }
    __syncthreads();
    const int64_t i = k0 + kb + (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= N) return;
    double x[kNb];
    double* row = A + i * N + k0;
#pragma unroll
    for (int t = 0; t < kNb; ++t) x[t] = t < kb ? row[t] : 0.0;
#pragma unroll
    for (int j = 0; j < kNb; ++j) {
        if (j < kb) {
            double s = x[j];
#pragma unroll
            for (int t = 0; t < j; ++t) s = fma(-x[t], l[j][t], s);
            x[j] = s / l[j][j];
        }
    }
#pragma unroll
    for (int t = 0; t < kNb; ++t)
        if (t < kb) row[t] = x[t];
}

// Columns c < ncols of block row i0: X_i = L_ii^-1 X_i (forward substitution).
__global__ __launch_bounds__(256) void k_trsm_rows(double* __restrict__ X, const double* __restrict__ L, int64_t N,
                                                   int64_t i0, int ib, int64_t ncols)
{
    __shared__ double l[kNb][kNb + 1];
    for (int q = threadIdx.x; q < ib * ib; q += 256) {
        const int i = q / ib, j = q - i * ib;
        l[i][j] = j <= i ? L[(i0 + i) * N + i0 + j] : 0.0;
    }
    __syncthreads();
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= ncols) return;
    double x[kNb];
#pragma unroll
    for (int r = 0; r < kNb; ++r) x[r] = r < ib ? X[(i0 + r) * N + c] : 0.0;
#pragma unroll
    for (int r = 0; r < kNb; ++r) {
        if (r < ib) {
            double s = x[r];
#pragma unroll
            for (int t = 0; t < r; ++t) s = fma(-l[r][t], x[t], s);
            x[r] = s / l[r][r];
        }
    }
#pragma unroll
    for (int r = 0; r < kNb; ++r)
        if (r < ib) X[(i0 + r) * N + c] = x[r];
}

// C[m x n] -= A[m x k] * op(B); op(B)[kk][j] = B[j*ldb + kk] (TB) or
// B[kk*ldb + j].  lower: only tiles whose columns start at or before the
// tile's last row (the lower triangle of a square C).
template <bool TB>
__global__ __launch_bounds__(256) void k_gemm64(double* __restrict__ C, int64_t ldc, const double* __restrict__ A,
                                                int64_t lda, const double* __restrict__ B, int64_t ldb, int64_t m,
                                                int64_t n, int k, bool lower)
{
    __shared__ double As[kGk][kGt + 1];
    __shared__ double Bs[kGk][kGt + 1];
    const int64_t i0 = (int64_t)blockIdx.y * kGt, j0 = (int64_t)blockIdx.x * kGt;
    if (lower && j0 > i0 + kGt - 1) return;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    double acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
    for (int k0 = 0; k0 < k; k0 += kGk) {
        for (int q = threadIdx.x; q < kGk * kGt; q += 256) {
            const int r = q / kGk, kk = q - r * kGk;           // A: row r, column kk
            const int64_t gi = i0 + r;
            As[kk][r] = (gi < m && k0 + kk < k) ? A[gi * lda + k0 + kk] : 0.0;
            if (TB) {
                const int64_t gj = j0 + r;
                Bs[kk][r] = (gj < n && k0 + kk < k) ? B[gj * ldb + k0 + kk] : 0.0;
            }
        }
        if (!TB) {
            for (int q = threadIdx.x; q < kGk * kGt; q += 256) {
                const int kk = q / kGt, c = q - kk * kGt;
                const int64_t gj = j0 + c;
                Bs[kk][c] = (gj < n && k0 + kk < k) ? B[(int64_t)(k0 + kk) * ldb + gj] : 0.0;
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kGk; ++kk) {
            double av[4], bv[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) av[a] = As[kk][ty * 4 + a];
#pragma unroll
            for (int b = 0; b < 4; ++b) bv[b] = Bs[kk][tx * 4 + b];
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) acc[a][b] = fma(av[a], bv[b], acc[a][b]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int64_t gi = i0 + ty * 4 + a;
        if (gi >= m) continue;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int64_t gj = j0 + tx * 4 + b;
            if (gj < n) C[gi * ldc + gj] -= acc[a][b];
        }
    }
}

}  // namespace

size_t ws_hfactor(int64_t N)
{
    return 2 * align_up((size_t)N * (size_t)N * sizeof(double)) + align_up(sizeof(double));
}

vq_status hfactor_launch(const float* H, int64_t N, double damp, float* U, void* ws, size_t ws_bytes, hipStream_t st)
{
    Carver cv(ws, ws_bytes);
    double* G = cv.take<double>((size_t)(N * N));
    double* X = cv.take<double>((size_t)(N * N));
    double* mean = cv.take<double>(1);
    if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "vq_hessian_factor: workspace too small");
    TimedRegion tr("hessian_factor", 0, st);
    const unsigned ge = grid_for(N * N, 256);
    hipLaunchKernelGGL(k_diag_mean, dim3(1), dim3(256), 0, st, H, N, mean);
    VQ_LAUNCHED("k_diag_mean");
    hipLaunchKernelGGL(k_build_g, dim3(ge), dim3(256), 0, st, H, N, damp, mean, G);
    VQ_LAUNCHED("k_build_g");
    // Cholesky, lower, in place
    for (int64_t k0 = 0; k0 < N; k0 += kNb) {
        const int kb = (int)(N - k0 < kNb ? N - k0 : kNb);
        hipLaunchKernelGGL(k_potrf_diag, dim3(1), dim3(256), 0, st, G, N, k0, kb);
        VQ_LAUNCHED("k_potrf_diag");
        const int64_t rest = N - k0 - kb;
        if (rest <= 0) break;
        hipLaunchKernelGGL(k_trsm_panel, dim3(grid_for(rest, 256)), dim3(256), 0, st, G, N, k0, kb);
        VQ_LAUNCHED("k_trsm_panel");
        double* T = G + (k0 + kb) * N + (k0 + kb);
        const double* P = G + (k0 + kb) * N + k0;
        hipLaunchKernelGGL((k_gemm64<true>), dim3(grid_for(rest, kGt), grid_for(rest, kGt)), dim3(256), 0, st, T, N, P,
                           N, P, N, rest, rest, kb, true);
        VQ_LAUNCHED("k_gemm64");
    }
    // X = L^-1
    hipLaunchKernelGGL(k_identity, dim3(ge), dim3(256), 0, st, X, N);
    VQ_LAUNCHED("k_identity");
    for (int64_t i0 = 0; i0 < N; i0 += kNb) {
        const int ib = (int)(N - i0 < kNb ? N - i0 : kNb);
        const int64_t ncols = i0 + ib;
        hipLaunchKernelGGL(k_trsm_rows, dim3(grid_for(ncols, 256)), dim3(256), 0, st, X, G, N, i0, ib, ncols);
        VQ_LAUNCHED("k_trsm_rows");
        const int64_t rest = N - i0 - ib;
        if (rest <= 0) break;
        hipLaunchKernelGGL((k_gemm64<false>), dim3(grid_for(ncols, kGt), grid_for(rest, kGt)), dim3(256), 0, st,
                           X + (i0 + ib) * N, N, G + (i0 + ib) * N + i0, N, X + i0 * N, N, rest, ncols, ib, false);
        VQ_LAUNCHED("k_gemm64");
    }
    hipLaunchKernelGGL(k_reverse_out, dim3(ge), dim3(256), 0, st, X, N, U);
    VQ_LAUNCHED("k_reverse_out");
    return VQ_OK;
}

}  // namespace vq
