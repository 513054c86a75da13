// Salience selection into the exact sparse correction.
//
// Method: HAS-VQ abstract ("Hessian-Masked Decoupling" isolates the weights
// with the largest second-order sensitivity; they are held exactly) and the
// SCVQ summary (one sparse correction matrix).  Score of element (i,j):
// s_ij = h_j * (w_ij * w_ij) in float32 (two roundings, no fused
// multiply-add).  The nnz largest scores are selected, ties broken by the
// smaller linear index i*N + j.
//
// Design (bitwise deterministic; integer atomics only, which commute):
//   1. radix select of the threshold tau on the uint32 bits of the scores
//      (non-negative floats order like their bit patterns): three passes of
//      11/11/10-bit digits, each a histogram over the elements that still
//      match the known high bits, then one block picks the digit;
//   2. per row: count of scores > tau and == tau;
//   3. one block scans the rows: the first (nnz - #{> tau}) ties in linear
//      order are taken, which gives each row's count and the CSR row pointer;
//   4. per row, a block walks the row in column order and writes col/val and
//      the per-sub-vector mask bytes (stable block-wide prefix sums).
#include "vq_internal.h"

#include <algorithm>

namespace vq {
namespace {

constexpr int kBins = 2048;
constexpr int kHistBlocks = 2048;
constexpr int kRowThreads = 256;
constexpr int kScanThreads = 1024;

struct SelState {
    uint32_t prefix;    // known high bits of tau
    uint32_t pad;
    int64_t remaining;  // elements still to take among those matching prefix
};

__device__ inline uint32_t score_bits(const float* W, const float* h, int64_t e, int64_t N)
{
    const float w = W[e];
    const float sq = w * w;
    const float s = h[e % N] * sq;
    return __float_as_uint(s);
}

__global__ void k_sel_init(SelState* st, int64_t nnz, int* hist)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t == 0) { st->prefix = nnz > 0 ? 0u : 0xFFFFFFFFu; st->pad = 0u; st->remaining = nnz; }
    if (t < kBins) hist[t] = 0;
}

__global__ __launch_bounds__(256) void k_sel_hist(const float* __restrict__ W,
                                                  const float* __restrict__ h, int64_t total,
                                                  int64_t N, const SelState* __restrict__ st,
                                                  uint32_t pmask, int shift, int* __restrict__ hist)
{
    __shared__ int cnt[kBins];
    for (int q = threadIdx.x; q < kBins; q += blockDim.x) cnt[q] = 0;
    __syncthreads();
    const uint32_t prefix = st->prefix;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
        const uint32_t b = score_bits(W, h, e, N);
        if ((b & pmask) == prefix) atomicAdd(&cnt[(b >> shift) & (kBins - 1)], 1);
    }
    __syncthreads();
    for (int q = threadIdx.x; q < kBins; q += blockDim.x)
        if (cnt[q]) atomicAdd(&hist[q], cnt[q]);
}

// Picks the digit holding the remaining-th largest element; clears hist.
// 256 threads, kBins / 256 consecutive bins each: a suffix sum of the
// per-thread totals (from the highest digit down) locates the one thread
// whose bins hold the crossing, which walks them from the top.
__global__ __launch_bounds__(256) void k_sel_pick(SelState* st, int* hist, int shift, int nbins)
{
    constexpr int kPer = kBins / 256;
    __shared__ int64_t suf[257];
    const int t = threadIdx.x;
    const int64_t rem = st->remaining;   // read before any thread can update it (barriers follow)
    int64_t c[kPer];
    int64_t tot = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int b = t * kPer + u;
        c[u] = b < nbins ? (int64_t)hist[b] : 0;
        tot += c[u];
    }
    suf[t] = tot;
    if (t == 0) suf[256] = 0;
    __syncthreads();
    // inclusive suffix sums over threads: suf[t] = sum of totals of threads >= t
    for (int off = 1; off < 256; off <<= 1) {
        const int64_t add = (t + off < 256) ? suf[t + off] : 0;
        __syncthreads();
        suf[t] += add;
        __syncthreads();
    }
    const int64_t above = suf[t + 1];    // suf[256] = 0
    if (above < rem && rem <= suf[t]) {
        int64_t cum = above;
        for (int u = kPer - 1; u >= 0; --u) {
            if (cum + c[u] >= rem) {
                st->prefix |= ((uint32_t)(t * kPer + u)) << shift;
                st->remaining = rem - cum;
                break;
            }
            cum += c[u];
        }
    }
    __syncthreads();
    for (int q = t; q < kBins; q += 256) hist[q] = 0;
}

// Per row: number of scores > tau and == tau.
__global__ __launch_bounds__(kRowThreads) void k_sel_row_count(
    const float* __restrict__ W, const float* __restrict__ h, int64_t N,
    const SelState* __restrict__ st, int* __restrict__ cgt, int* __restrict__ ceq)
{
    __shared__ int sg[kRowThreads], se[kRowThreads];
    const int64_t i = blockIdx.x;
    const uint32_t tau = st->prefix;
    int g = 0, q = 0;
    for (int64_t j = threadIdx.x; j < N; j += kRowThreads) {
        const uint32_t b = score_bits(W, h, i * N + j, N);
        g += b > tau;
        q += b == tau;
    }
    sg[threadIdx.x] = g;
    se[threadIdx.x] = q;
    __syncthreads();
    for (int w = kRowThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) {
            sg[threadIdx.x] += sg[threadIdx.x + w];
            se[threadIdx.x] += se[threadIdx.x + w];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) { cgt[i] = sg[0]; ceq[i] = se[0]; }
}

// Inclusive block scan (1024 threads) of one int64 per thread.
__device__ inline int64_t scan1024(int64_t v, int64_t* sh)
{
    sh[threadIdx.x] = v;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
        const int64_t add = (int)threadIdx.x >= off ? sh[threadIdx.x - off] : 0;
        __syncthreads();
        sh[threadIdx.x] += add;
        __syncthreads();
    }
    const int64_t r = sh[threadIdx.x];
    __syncthreads();
    return r;
}

// One block over all rows: ties taken in linear order; row pointers.
__global__ __launch_bounds__(kScanThreads) void k_sel_rows(const SelState* __restrict__ st,
                                                           int64_t M, const int* __restrict__ cgt,
                                                           const int* __restrict__ ceq,
                                                           int* __restrict__ take,
                                                           int32_t* __restrict__ row_ptr)
{
    __shared__ int64_t sh[kScanThreads];
    const int64_t per = (M + kScanThreads - 1) / kScanThreads;
    const int64_t r0 = threadIdx.x * per;
    const int64_t r1 = r0 + per < M ? r0 + per : M;
    const int64_t need = st->remaining;   // ties to take, in linear order
    int64_t eq_local = 0;
    for (int64_t i = r0; i < r1; ++i) eq_local += ceq[i];
    int64_t eq_before = scan1024(eq_local, sh) - eq_local;
    int64_t sel_local = 0;
    for (int64_t i = r0; i < r1; ++i) {
        int64_t t = need - eq_before;
        t = t < 0 ? 0 : (t > ceq[i] ? ceq[i] : t);
        take[i] = (int)t;
        eq_before += ceq[i];
        sel_local += cgt[i] + t;
    }
    int64_t run = scan1024(sel_local, sh) - sel_local;
    for (int64_t i = r0; i < r1; ++i) {
        row_ptr[i] = (int32_t)run;
        run += cgt[i] + take[i];
    }
    if (threadIdx.x == kScanThreads - 1) row_ptr[M] = (int32_t)run;
}

// Inclusive scan of one int per thread over a 256-thread block.
__device__ inline int scan256(int v, int* sh)
{
    // inclusive scan within each wavefront by shuffles, then the totals of
    // the earlier wavefronts (4 per block) from LDS
    static_assert(kRowThreads == 256, "four wavefronts");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) sh[wave] = x;
    __syncthreads();
    int add = 0;
    for (int w = 0; w < wave; ++w) add += sh[w];
    __syncthreads();   // sh is reused by the next call
    return x + add;
}

// Per row: walk sub-vectors in column order, write CSR entries and masks.
__global__ __launch_bounds__(kRowThreads) void k_sel_compact(
    const float* __restrict__ W, const float* __restrict__ h, int64_t N, int d,
    const SelState* __restrict__ st, const int* __restrict__ take,
    const int32_t* __restrict__ row_ptr, int64_t nnz, int32_t* __restrict__ col,
    float* __restrict__ val, uint8_t* __restrict__ mask)
{
    __shared__ int sh[kRowThreads];
    __shared__ int tot_eq, tot_sel;
    const int64_t i = blockIdx.x;
    const int64_t nb = N / d;
    const uint32_t tau = st->prefix;
    const int row_take = take[i];
    int eq_run = 0;        // ties seen earlier in this row
    int pos_run = row_ptr[i];
    for (int64_t b0 = 0; b0 < nb; b0 += kRowThreads) {
        const int64_t b = b0 + threadIdx.x;
        uint32_t bits[8];
        int n_eq = 0;
        if (b < nb) {
            for (int t = 0; t < d; ++t) {
                bits[t] = score_bits(W, h, i * N + b * d + t, N);
                n_eq += bits[t] == tau;
            }
        }
        const int eq_incl = scan256(n_eq, sh);
        int eq_rank = eq_run + eq_incl - n_eq;
        unsigned mb = 0;
        int n_sel = 0;
        if (b < nb) {
            for (int t = 0; t < d; ++t) {
                bool s = bits[t] > tau;
                if (bits[t] == tau) { s = eq_rank < row_take; ++eq_rank; }
                if (s) { mb |= 1u << t; ++n_sel; }
            }
        }
        // chunk totals (the last thread's inclusive values)
        if (threadIdx.x == kRowThreads - 1) tot_eq = eq_incl;
        const int sel_incl = scan256(n_sel, sh);
        if (threadIdx.x == kRowThreads - 1) tot_sel = sel_incl;
        if (b < nb) {
            int p = pos_run + sel_incl - n_sel;
            for (int t = 0; t < d; ++t) {
                if (((mb >> t) & 1u) && p < nnz) {
                    col[p] = (int32_t)(b * d + t);
                    val[p] = W[i * N + b * d + t];
                    ++p;
                }
            }
            mask[i * nb + b] = (uint8_t)mb;
        }
        __syncthreads();
        eq_run += tot_eq;
        pos_run += tot_sel;
        __syncthreads();
    }
}

}  // namespace

size_t ws_select(int64_t M, int64_t N)
{
    (void)N;
    return align_up(sizeof(SelState)) + align_up(kBins * sizeof(int)) + 3 * align_up((size_t)M * sizeof(int));
}

vq_status select_launch(const float* W, const float* h, int64_t M, int64_t N, int d, int64_t nnz,
                        int32_t* row_ptr, int32_t* col, float* val, uint8_t* mask, void* ws,
                        size_t ws_bytes, hipStream_t st)
{
    Carver cv(ws, ws_bytes);
    SelState* state = cv.take<SelState>(1);
    int* hist = cv.take<int>(kBins);
    int* cgt = cv.take<int>((size_t)M);
    int* ceq = cv.take<int>((size_t)M);
    int* take = cv.take<int>((size_t)M);
    if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "vq_sparse_select: workspace too small");
    const int64_t total = M * N;
    TimedRegion tr("select", 0, st);

    // nnz == 0 skips the threshold search: the initial threshold pattern
    // 0xFFFFFFFF lies above every non-negative score, so nothing is taken.
    hipLaunchKernelGGL(k_sel_init, dim3(grid_for(kBins, 256)), dim3(256), 0, st, state, nnz, hist);
    VQ_LAUNCHED("k_sel_init");
    if (nnz > 0) {
        const int shifts[3] = {21, 10, 0};
        const int nbins[3] = {2048, 2048, 1024};
        const uint32_t pmasks[3] = {0u, 0xFFE00000u, 0xFFFFFC00u};
        const unsigned hb = (unsigned)std::min<int64_t>(kHistBlocks, grid_for(total, 256 * 16));
        for (int p = 0; p < 3; ++p) {
            hipLaunchKernelGGL(k_sel_hist, dim3(hb), dim3(256), 0, st, W, h, total, N, state, pmasks[p],
                               shifts[p], hist);
            VQ_LAUNCHED("k_sel_hist");
            hipLaunchKernelGGL(k_sel_pick, dim3(1), dim3(256), 0, st, state, hist, shifts[p], nbins[p]);
            VQ_LAUNCHED("k_sel_pick");
        }
    }
    hipLaunchKernelGGL(k_sel_row_count, dim3((unsigned)M), dim3(kRowThreads), 0, st, W, h, N, state, cgt,
                       ceq);
    VQ_LAUNCHED("k_sel_row_count");
    hipLaunchKernelGGL(k_sel_rows, dim3(1), dim3(kScanThreads), 0, st, state, M, cgt, ceq, take, row_ptr);
    VQ_LAUNCHED("k_sel_rows");
    hipLaunchKernelGGL(k_sel_compact, dim3((unsigned)M), dim3(kRowThreads), 0, st, W, h, N, d, state,
                       take, row_ptr, nnz, col, val, mask);
    VQ_LAUNCHED("k_sel_compact");
    return VQ_OK;
}

}  // namespace vq
