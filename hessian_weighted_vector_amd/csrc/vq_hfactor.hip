// The matrix that the second-order error propagation reads where the VPTQ
// page ("The Core Algorithm") writes H^-1, in GPTQ's form (the technique the
// page says it inherits): U, the upper-triangular factor with positive
// diagonal and U^T U = Hd^-1, Hd = H + damp * mean(diag H) * I.
//
// Route, all in float64: with P the reversal permutation, G = P Hd P has the
// ordinary Cholesky factor L (G = L L^T), so Hd = (P L P)(P L P)^T with P L P
// upper triangular and U = (P L P)^-1 = P L^-1 P.  Both L and L^-1 are formed
// by right-looking blocked algorithms over panels of kNo = 256 columns, each
// worked as kNb = 32-column sub-panels:
//   Cholesky:  factor the sub-panel's diagonal block in LDS (one workgroup),
//              solve the sub-panel below it (one thread per row), subtract
//              its outer product from the rest of the panel (GEMM); after the
//              panel, one rank-256 update of the trailing lower triangle;
//   inverse:   X = I, then per sub-block row: X_i = L_ii^-1 X_i (one thread
//              per column) and X_{rows below in the block row} -= L X_i; after
//              the block row, one rank-256 update of every row below over the
//              columns the block row can be non-zero in.
// The GEMMs run on the float64 matrix cores (128 x 128 workgroup tiles).
#include "vq_internal.h"

namespace vq {
namespace {

constexpr int kNb = 32;       // sub-panel width (factored in LDS)
constexpr int kNo = 256;      // panel width (one trailing update per panel)

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

// C[m x n] -= A[m x k] * op(B) on the float64 matrix cores
// (v_mfma_f64_16x16x4f64).  op(B)[kk][j] = B[j*ldb + kk] (TB) or
// B[kk*ldb + j].  Workgroup tile 128 x 128, eight wavefronts: wavefront w
// owns rows 32(w%4) .. +31 and columns 64(w/4) .. +63 as 2 x 4 blocks of
// 16 x 16; k moves through LDS in chunks of 16 (double buffered, one barrier
// per chunk).  Operand layout of one MFMA:
// lane l supplies A[l%16][l/16] and B[l/16][l%16]; it holds
// D[l/16 + 4r][l%16] in element r of its accumulator (checked on the device
// against a host product).  lower: only tiles
// whose columns start at or before the tile's last row.
constexpr int kDm = 128, kDn = 128, kDk = 16;
typedef double f64x4 __attribute__((ext_vector_type(4)));

template <bool TB>
__global__ __launch_bounds__(512) void k_dgemm(double* __restrict__ C, int64_t ldc, const double* __restrict__ A,
                                               int64_t lda, const double* __restrict__ B, int64_t ldb, int64_t m,
                                               int64_t n, int k, bool lower)
{
    __shared__ double As[2][kDk][kDm + 2];
    __shared__ double Bs[2][kDk][kDn + 2];
    const int64_t i0 = (int64_t)blockIdx.y * kDm, j0 = (int64_t)blockIdx.x * kDn;
    if (lower && j0 > i0 + kDm - 1) return;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int wr = (w & 3) * 32, wc = (w >> 2) * 64;
    // staging: A row ar, k ak..ak+3; B (TB) column bc, k bk..bk+3, or (!TB) k bkk, columns bj..bj+3
    const int ar = t >> 2, ak = (t & 3) * 4;
    const int bc = t >> 2, bk = (t & 3) * 4;
    const int bkk = t >> 5, bj = (t & 31) * 4;
    double ra[4], rb[4];
    auto load = [&](int k0) {
        const int64_t gi = i0 + ar;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int kk = k0 + ak + q;
            ra[q] = (gi < m && kk < k) ? A[gi * lda + kk] : 0.0;
        }
        if (TB) {
            const int64_t gj = j0 + bc;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int kk = k0 + bk + q;
                rb[q] = (gj < n && kk < k) ? B[gj * ldb + kk] : 0.0;
            }
        } else {
            const int kk = k0 + bkk;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t gj = j0 + bj + q;
                rb[q] = (gj < n && kk < k) ? B[(int64_t)kk * ldb + gj] : 0.0;
            }
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int q = 0; q < 4; ++q) As[buf][ak + q][ar] = ra[q];
        if (TB) {
#pragma unroll
            for (int q = 0; q < 4; ++q) Bs[buf][bk + q][bc] = rb[q];
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) Bs[buf][bkk][bj + q] = rb[q];
        }
    };
    f64x4 acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = (f64x4){0.0, 0.0, 0.0, 0.0};
    const int nk = (k + kDk - 1) / kDk;
    load(0);
    store(0);
    __syncthreads();
    const int lr = lane & 15, lk = lane >> 4;
    for (int c = 0; c < nk; ++c) {
        const int buf = c & 1;
        if (c + 1 < nk) load((c + 1) * kDk);
#pragma unroll
        for (int ks = 0; ks < kDk; ks += 4) {
            double av[2], bv[4];
#pragma unroll
            for (int a = 0; a < 2; ++a) av[a] = As[buf][ks + lk][wr + a * 16 + lr];
#pragma unroll
            for (int b = 0; b < 4; ++b) bv[b] = Bs[buf][ks + lk][wc + b * 16 + lr];
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[b], acc[a][b], 0, 0, 0);
        }
        if (c + 1 < nk) store(buf ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t gi = i0 + wr + a * 16 + lk + 4 * r;
                const int64_t gj = j0 + wc + b * 16 + lr;
                if (gi < m && gj < n) C[gi * ldc + gj] -= acc[a][b][r];
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
    auto dgemm = [&](bool tb, double* Cp, const double* Ap, const double* Bp, int64_t m, int64_t n, int k,
                     bool lower) {
        const dim3 grid(grid_for(n, kDn), grid_for(m, kDm));
        if (tb)
            hipLaunchKernelGGL((k_dgemm<true>), grid, dim3(512), 0, st, Cp, N, Ap, N, Bp, N, m, n, k, lower);
        else
            hipLaunchKernelGGL((k_dgemm<false>), grid, dim3(512), 0, st, Cp, N, Ap, N, Bp, N, m, n, k, lower);
    };
    // Cholesky, lower, in place: panels of kNo columns, each factored as
    // kNb-column sub-panels whose updates stay inside the panel; then one
    // rank-kNo update of the trailing lower triangle.
    for (int64_t K0 = 0; K0 < N; K0 += kNo) {
        const int64_t K1 = K0 + kNo < N ? K0 + kNo : N;
        for (int64_t k0 = K0; k0 < K1; k0 += kNb) {
            const int kb = (int)(K1 - k0 < kNb ? K1 - k0 : kNb);
            hipLaunchKernelGGL(k_potrf_diag, dim3(1), dim3(256), 0, st, G, N, k0, kb);
            VQ_LAUNCHED("k_potrf_diag");
            const int64_t rest = N - k0 - kb;
            if (rest <= 0) break;
            hipLaunchKernelGGL(k_trsm_panel, dim3(grid_for(rest, 256)), dim3(256), 0, st, G, N, k0, kb);
            VQ_LAUNCHED("k_trsm_panel");
            const int64_t wr = K1 - (k0 + kb);          // panel columns right of this sub-panel
            if (wr > 0) {
                const double* P = G + (k0 + kb) * N + k0;
                dgemm(true, G + (k0 + kb) * N + (k0 + kb), P, P, rest, wr, kb, true);
                VQ_LAUNCHED("k_dgemm");
            }
        }
        const int64_t rest = N - K1;
        if (rest <= 0) break;
        const double* P = G + K1 * N + K0;
        dgemm(true, G + K1 * N + K1, P, P, rest, rest, (int)(K1 - K0), true);
        VQ_LAUNCHED("k_dgemm");
    }
    // X = L^-1: block rows of kNo, each solved as kNb-row sub-blocks whose
    // updates stay inside the block row; then one rank-kNo update of the rows
    // below over the columns the block row can be non-zero in.
    hipLaunchKernelGGL(k_identity, dim3(ge), dim3(256), 0, st, X, N);
    VQ_LAUNCHED("k_identity");
    for (int64_t I0 = 0; I0 < N; I0 += kNo) {
        const int64_t I1 = I0 + kNo < N ? I0 + kNo : N;
        for (int64_t i0 = I0; i0 < I1; i0 += kNb) {
            const int ib = (int)(I1 - i0 < kNb ? I1 - i0 : kNb);
            const int64_t ncols = i0 + ib;
            hipLaunchKernelGGL(k_trsm_rows, dim3(grid_for(ncols, 256)), dim3(256), 0, st, X, G, N, i0, ib, ncols);
            VQ_LAUNCHED("k_trsm_rows");
            const int64_t rr = I1 - i0 - ib;                // block-row rows below this sub-block
            if (rr > 0) {
                dgemm(false, X + (i0 + ib) * N, G + (i0 + ib) * N + i0, X + i0 * N, rr, ncols, ib, false);
                VQ_LAUNCHED("k_dgemm");
            }
        }
        const int64_t rest = N - I1;
        if (rest <= 0) break;
        dgemm(false, X + I1 * N, G + I1 * N + I0, X + I0 * N, rest, I1, (int)(I1 - I0), false);
        VQ_LAUNCHED("k_dgemm");
    }
    hipLaunchKernelGGL(k_reverse_out, dim3(ge), dim3(256), 0, st, X, N, U);
    VQ_LAUNCHED("k_reverse_out");
    return VQ_OK;
}

}  // namespace vq
