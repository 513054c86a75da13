// Column groups (VPTQ page, "Outlier Elimination": the columns with the
// largest Hessian diagonal are held apart with their own codebook; "group
// partitioning": the other columns may be split into groups with independent
// codebooks).  The pieces the grouped fit adds to the plain fit:
//   k_col_rank / k_col_order  the column order: the n_out columns with the
//                             largest h (ties: smaller index) ascending, then
//                             the rest ascending (partial ranks by comparison
//                             against LDS tiles of h over slices of the
//                             columns, their sums, then one block's scans);
//   k_gather_cols             a group's columns of a matrix (or of h, c);
//   k_gather_mask             a group's salient bits, in its own sub-vector
//                             layout (d_g bits per byte);
//   k_scatter_cols            a group's reconstruction back into its columns.
#include "vq_internal.h"

namespace vq {
namespace {

constexpr int kRankTile = 1024;
constexpr int kRankSlicesMax = 32;

// Partial ranks: slice blockIdx.y of the columns k compares its h[k] with
// every h[j] of this block; part[slice * N + j] counts the k that come before
// j (larger h, or equal h and smaller index).  Slicing the k range gives the
// launch enough workgroups to fill the chip for N of a few thousand.
__global__ __launch_bounds__(256) void k_col_rank(const float* __restrict__ h, int64_t N, int64_t chunk,
                                                  int32_t* __restrict__ part)
{
    __shared__ float th[kRankTile];
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const float hj = j < N ? h[j] : 0.0f;
    const int64_t ka = (int64_t)blockIdx.y * chunk;
    const int64_t kb = ka + chunk < N ? ka + chunk : N;
    int32_t r = 0;
    for (int64_t k0 = ka; k0 < kb; k0 += kRankTile) {
        const int kn = (int)(kb - k0 < kRankTile ? kb - k0 : kRankTile);
        __syncthreads();
        for (int q = threadIdx.x; q < kn; q += 256) th[q] = h[k0 + q];
        __syncthreads();
        for (int q = 0; q < kn; ++q) {
            const float hk = th[q];
            r += (hk > hj) || (hk == hj && k0 + q < j);
        }
    }
    if (j < N) part[(int64_t)blockIdx.y * N + j] = r;
}

// Rank of column j = the sum of its slices' partial ranks; the n_out columns
// of rank < n_out are flagged.
__global__ __launch_bounds__(256) void k_col_flag(const int32_t* __restrict__ part, int nslice, int64_t N,
                                                  int64_t n_out, uint8_t* __restrict__ flag)
{
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= N) return;
    int64_t r = 0;
    for (int q = 0; q < nslice; ++q) r += part[(int64_t)q * N + j];
    flag[j] = r < n_out ? 1 : 0;
}

// cols = [flagged columns ascending, unflagged columns ascending]; one block.
__global__ __launch_bounds__(1024) void k_col_order(const uint8_t* __restrict__ flag, int64_t N,
                                                    int32_t* __restrict__ cols)
{
    __shared__ int64_t sh[1024];
    const int64_t per = (N + 1023) / 1024;
    const int64_t j0 = threadIdx.x * per;
    const int64_t j1 = j0 + per < N ? j0 + per : N;
    int64_t cnt = 0;
    for (int64_t j = j0; j < j1; ++j) cnt += flag[j];
    sh[threadIdx.x] = cnt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int64_t add = (int)threadIdx.x >= off ? sh[threadIdx.x - off] : 0;
        __syncthreads();
        sh[threadIdx.x] += add;
        __syncthreads();
    }
    const int64_t total = sh[1023];
    int64_t before = sh[threadIdx.x] - cnt;        // flagged columns before j0
    int64_t rest = (j0 < N ? j0 : N) - before;      // unflagged columns before j0
    for (int64_t j = j0; j < j1; ++j) {
        if (flag[j]) cols[before++] = (int32_t)j;
        else cols[total + rest++] = (int32_t)j;
    }
}

__global__ __launch_bounds__(256) void k_gather_cols(const float* __restrict__ X, int64_t M, int64_t N,
                                                     const int32_t* __restrict__ cols, int64_t Ng,
                                                     float* __restrict__ Y)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= M * Ng) return;
    const int64_t i = e / Ng, q = e - i * Ng;
    Y[e] = X[i * N + cols[q]];
}

__global__ __launch_bounds__(256) void k_scatter_cols(const float* __restrict__ Y, int64_t M, int64_t Ng,
                                                      const int32_t* __restrict__ cols, float* __restrict__ X,
                                                      int64_t N)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= M * Ng) return;
    const int64_t i = e / Ng, q = e - i * Ng;
    X[i * N + cols[q]] = Y[e];
}

__global__ __launch_bounds__(256) void k_gather_mask(const uint8_t* __restrict__ mask, int64_t M, int64_t N, int d,
                                                     const int32_t* __restrict__ cols, int64_t Ng, int dg,
                                                     uint8_t* __restrict__ mg)
{
    const int64_t nbg = Ng / dg;
    const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (s >= M * nbg) return;
    const int64_t i = s / nbg, b = s - i * nbg;
    const int64_t nb = N / d;
    unsigned m = 0;
    for (int t = 0; t < dg; ++t) {
        const int64_t j = cols[b * dg + t];
        const int64_t jb = j / d;
        m |= ((unsigned)(mask[i * nb + jb] >> (int)(j - jb * d)) & 1u) << t;
    }
    mg[s] = (uint8_t)m;
}

}  // namespace

int column_order_slices(int64_t N)
{
    const int64_t s = (N + 1023) / 1024 * 4;   // about 256 columns of k per slice
    return (int)(s < 1 ? 1 : (s > kRankSlicesMax ? kRankSlicesMax : s));
}

vq_status column_order_launch(const float* h, int64_t N, int64_t n_out, int32_t* cols, uint8_t* flag, int32_t* part,
                              hipStream_t st)
{
    const int ns = column_order_slices(N);
    const int64_t chunk = (N + ns - 1) / ns;
    hipLaunchKernelGGL(k_col_rank, dim3(grid_for(N, 256), ns), dim3(256), 0, st, h, N, chunk, part);
    VQ_LAUNCHED("k_col_rank");
    hipLaunchKernelGGL(k_col_flag, dim3(grid_for(N, 256)), dim3(256), 0, st, part, ns, N, n_out, flag);
    VQ_LAUNCHED("k_col_flag");
    hipLaunchKernelGGL(k_col_order, dim3(1), dim3(1024), 0, st, flag, N, cols);
    VQ_LAUNCHED("k_col_order");
    return VQ_OK;
}

vq_status gather_cols_launch(const float* X, int64_t M, int64_t N, const int32_t* cols, int64_t Ng, float* Y,
                             hipStream_t st)
{
    hipLaunchKernelGGL(k_gather_cols, dim3(grid_for(M * Ng, 256)), dim3(256), 0, st, X, M, N, cols, Ng, Y);
    VQ_LAUNCHED("k_gather_cols");
    return VQ_OK;
}

vq_status scatter_cols_launch(const float* Y, int64_t M, int64_t Ng, const int32_t* cols, float* X, int64_t N,
                              hipStream_t st)
{
    hipLaunchKernelGGL(k_scatter_cols, dim3(grid_for(M * Ng, 256)), dim3(256), 0, st, Y, M, Ng, cols, X, N);
    VQ_LAUNCHED("k_scatter_cols");
    return VQ_OK;
}

vq_status gather_mask_launch(const uint8_t* mask, int64_t M, int64_t N, int d, const int32_t* cols, int64_t Ng,
                             int dg, uint8_t* mg, hipStream_t st)
{
    hipLaunchKernelGGL(k_gather_mask, dim3(grid_for(M * (Ng / dg), 256)), dim3(256), 0, st, mask, M, N, d, cols, Ng,
                       dg, mg);
    VQ_LAUNCHED("k_gather_mask");
    return VQ_OK;
}

}  // namespace vq
