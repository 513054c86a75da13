// Centroid update as a weighted segmented reduction (VPTQ page,
// "Hessian-Weighted Centroid Initialization": each centroid becomes the
// Hessian-weighted mean of its members; with one weight per element the
// exact minimizer of the objective is the per-dimension weighted mean).
//
// Design (no floating-point atomics; bitwise deterministic):
//   1. binning: stable LSD radix sort of (index, sub-vector id) pairs, 8-bit
//      digits (one pass when K <= 256, else two).  Per-block digit counts use
//      LDS integer atomics (exact), block offsets come from a scan, and
//      ranks inside a block come from wavefront ballots, so equal indices
//      keep ascending sub-vector order;
//   2. segment starts by binary search of the sorted indices;
//   3. each segment is cut into pieces of at most kPiece members; one
//      wavefront reduces a piece (float64 sums of omega*x and omega per
//      dimension, lane-strided then a fixed xor butterfly);
//   4. one thread per centroid adds its pieces in order and divides once.
#include "vq_internal.h"

namespace vq {
namespace {

constexpr int kSortThreads = 256;
constexpr int kSortItems = 16;
constexpr int kSortTile = kSortThreads * kSortItems;   // elements per sort block
constexpr int kPiece = 256;                             // members per wavefront piece
constexpr int kScanThreads = 1024;

// Inclusive scan of one int per thread over a 256-thread block.
__device__ inline int block_incl_scan_256(int v, int* sh)
{
    sh[threadIdx.x] = v;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        int add = (int)threadIdx.x >= off ? sh[threadIdx.x - off] : 0;
        __syncthreads();
        sh[threadIdx.x] += add;
        __syncthreads();
    }
    int r = sh[threadIdx.x];
    __syncthreads();
    return r;
}

// Per-block digit histogram: hist[digit * nblk + block].
__global__ __launch_bounds__(kSortThreads) void k_sort_hist(const uint16_t* __restrict__ keys,
                                                            int64_t n, int shift,
                                                            int* __restrict__ hist, int nblk)
{
    __shared__ int cnt[256];
    cnt[threadIdx.x] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kSortTile;
    for (int q = threadIdx.x; q < kSortTile; q += kSortThreads) {
        const int64_t e = base + q;
        if (e < n) atomicAdd(&cnt[(keys[e] >> shift) & 255], 1);
    }
    __syncthreads();
    hist[(int64_t)threadIdx.x * nblk + blockIdx.x] = cnt[threadIdx.x];
}

// One block per digit: exclusive scan of its per-block counts, in place;
// digit_total[digit] = the digit's count.
__global__ __launch_bounds__(256) void k_scan_digit(int* __restrict__ hist, int nblk,
                                                    int* __restrict__ digit_total)
{
    __shared__ int sh[256];
    int* row = hist + (int64_t)blockIdx.x * nblk;
    int carry = 0;
    for (int c0 = 0; c0 < nblk; c0 += 256) {
        const int q = c0 + threadIdx.x;
        const int v = q < nblk ? row[q] : 0;
        const int inc = block_incl_scan_256(v, sh);   // leaves the inclusive sums in sh
        const int chunk_total = sh[255];
        if (q < nblk) row[q] = carry + inc - v;
        carry += chunk_total;
        __syncthreads();
    }
    if (threadIdx.x == 0) digit_total[blockIdx.x] = carry;
}

// Stable scatter of one block by the digit at `shift`.
// vals_in == nullptr means the values are the element positions.
__global__ __launch_bounds__(kSortThreads) void k_sort_scatter(
    const uint16_t* __restrict__ keys_in, const int32_t* __restrict__ vals_in, int64_t n, int shift,
    const int* __restrict__ hist, const int* __restrict__ digit_total, int nblk,
    uint16_t* __restrict__ keys_out, int32_t* __restrict__ vals_out)
{
    __shared__ int sh[256];
    __shared__ int base[256];
    __shared__ int running[256];
    __shared__ int wcnt[4][256];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // global start of each digit for this block
    const int tot = digit_total[tid];
    const int incl = block_incl_scan_256(tot, sh);
    base[tid] = (incl - tot) + hist[(int64_t)tid * nblk + blockIdx.x];
    running[tid] = 0;
    __syncthreads();

    const int64_t blk0 = (int64_t)blockIdx.x * kSortTile;
    const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int r = 0; r < kSortItems; ++r) {
        const int64_t e = blk0 + (int64_t)r * kSortThreads + tid;
        const bool valid = e < n;
        uint16_t key = 0;
        int32_t val = 0;
        int dg = 0;
        if (valid) {
            key = keys_in[e];
            val = vals_in ? vals_in[e] : (int32_t)e;
            dg = (key >> shift) & 255;
        }
        for (int q = tid; q < 4 * 256; q += kSortThreads) (&wcnt[0][0])[q] = 0;
        __syncthreads();
        // lanes of this wavefront holding the same digit
        unsigned long long peers = __ballot(valid);
        for (int bit = 0; bit < 8; ++bit) {
            const unsigned long long bal = __ballot(valid && ((dg >> bit) & 1));
            peers &= ((dg >> bit) & 1) ? bal : ~bal;
        }
        const int wrank = __popcll(peers & lt_mask);
        if (valid && wrank == 0) wcnt[wave][dg] = __popcll(peers);
        __syncthreads();
        if (valid) {
            int off = running[dg] + wrank;
            for (int w = 0; w < wave; ++w) off += wcnt[w][dg];
            const int64_t pos = (int64_t)base[dg] + off;
            keys_out[pos] = key;
            vals_out[pos] = val;
        }
        __syncthreads();
        running[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
        __syncthreads();
    }
}

// start[k] = first position of key k in the sorted keys (k = 0..K).
__global__ void k_seg_start(const uint16_t* __restrict__ skeys, int64_t n, int K,
                            int* __restrict__ start)
{
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k > K) return;
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if ((int)skeys[mid] < k) lo = mid + 1; else hi = mid;
    }
    start[k] = (int)lo;
}

// Single-block exclusive scan of the per-centroid piece counts:
// poff[k] = pieces before centroid k, poff[K] = total.
__global__ __launch_bounds__(kScanThreads) void k_piece_scan(const int* __restrict__ start, int K,
                                                             int* __restrict__ poff)
{
    __shared__ int sh[kScanThreads];
    const int per = (K + kScanThreads - 1) / kScanThreads;
    const int k0 = threadIdx.x * per;
    int local = 0;
    for (int k = k0; k < k0 + per && k < K; ++k) local += (start[k + 1] - start[k] + kPiece - 1) / kPiece;
    sh[threadIdx.x] = local;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
        int add = (int)threadIdx.x >= off ? sh[threadIdx.x - off] : 0;
        __syncthreads();
        sh[threadIdx.x] += add;
        __syncthreads();
    }
    int run = sh[threadIdx.x] - local;
    for (int k = k0; k < k0 + per && k < K; ++k) {
        poff[k] = run;
        run += (start[k + 1] - start[k] + kPiece - 1) / kPiece;
    }
    if (threadIdx.x == kScanThreads - 1) poff[K] = sh[kScanThreads - 1];
}

// One wavefront per piece: float64 sums of omega*x and omega per dimension.
__global__ __launch_bounds__(256) void k_seg_reduce(
    const float* __restrict__ X, const float* __restrict__ hcol, const float* __restrict__ rho,
    const uint8_t* __restrict__ mask, int64_t nb, int d, const int32_t* __restrict__ svals,
    const int* __restrict__ start, const int* __restrict__ poff, int K,
    double* __restrict__ part)
{
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int total = poff[K];
    if (w >= total) return;
    // centroid owning piece w: last k with poff[k] <= w
    int lo = 0, hi = K;   // poff[lo] <= w < poff[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (poff[mid] <= w) lo = mid; else hi = mid;
    }
    const int k = lo;
    const int64_t j = w - poff[k];
    const int64_t e0 = start[k] + j * kPiece;
    const int64_t e1 = min((int64_t)start[k + 1], e0 + kPiece);
    double num[8], den[8];
    for (int t = 0; t < 8; ++t) { num[t] = 0.0; den[t] = 0.0; }
    for (int64_t e = e0 + lane; e < e1; e += 64) {
        const int64_t s = svals[e];
        const int64_t i = s / nb;
        const int64_t b = s - i * nb;
        const unsigned mb = mask ? mask[s] : 0u;
        const double rr = rho ? (double)rho[i] : 1.0;
        for (int t = 0; t < d; ++t) {
            double wt = (double)hcol[b * d + t];
            if (rho) wt = wt * rr;
            if ((mb >> t) & 1u) wt = 0.0;
            num[t] = num[t] + wt * (double)X[s * d + t];
            den[t] = den[t] + wt;
        }
    }
    for (int off = 32; off > 0; off >>= 1) {
        for (int t = 0; t < 8; ++t) {
            num[t] = num[t] + __shfl_xor(num[t], off);
            den[t] = den[t] + __shfl_xor(den[t], off);
        }
    }
    if (lane == 0) {
        double* p = part + w * 16;
        for (int t = 0; t < 8; ++t) { p[t] = num[t]; p[8 + t] = den[t]; }
    }
}

// One thread per centroid: add its pieces in order; C = num/den rounded once,
// kept where the weight sum is 0.
__global__ void k_seg_finish(const double* __restrict__ part, const int* __restrict__ start,
                             const int* __restrict__ poff, int K, int d, float* __restrict__ C,
                             int32_t* __restrict__ counts)
{
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= K) return;
    if (counts) counts[k] = start[k + 1] - start[k];
    double num[8], den[8];
    for (int t = 0; t < 8; ++t) { num[t] = 0.0; den[t] = 0.0; }
    for (int p = poff[k]; p < poff[k + 1]; ++p) {
        const double* q = part + (int64_t)p * 16;
        for (int t = 0; t < 8; ++t) { num[t] = num[t] + q[t]; den[t] = den[t] + q[8 + t]; }
    }
    for (int t = 0; t < d; ++t)
        if (den[t] > 0.0) C[(size_t)k * d + t] = (float)(num[t] / den[t]);
}

struct UpdateWs {
    uint16_t *k1, *k2;
    int32_t *v1, *v2;
    int *hist, *dtot, *start, *poff;
    double* part;
};

int64_t piece_bound(int64_t n_sub, int K) { return (n_sub + kPiece - 1) / kPiece + K; }

UpdateWs carve_update(Carver& cv, int64_t n_sub, int K)
{
    UpdateWs w;
    const int64_t nblk = (n_sub + kSortTile - 1) / kSortTile;
    w.k1 = cv.take<uint16_t>(n_sub);
    w.k2 = cv.take<uint16_t>(n_sub);
    w.v1 = cv.take<int32_t>(n_sub);
    w.v2 = cv.take<int32_t>(n_sub);
    w.hist = cv.take<int>((size_t)256 * nblk);
    w.dtot = cv.take<int>(256);
    w.start = cv.take<int>((size_t)K + 1);
    w.poff = cv.take<int>((size_t)K + 1);
    w.part = cv.take<double>((size_t)piece_bound(n_sub, K) * 16);
    return w;
}

}  // namespace

size_t ws_update(int64_t n_sub, int K)
{
    Carver cv(nullptr, 0);
    cv.base = reinterpret_cast<char*>(kAlign);   // size-only pass
    cv.cap = SIZE_MAX / 2;
    carve_update(cv, n_sub, K);
    return cv.used;
}

vq_status update_launch(const float* X, const float* hcol, const float* rho, const uint8_t* mask,
                        int64_t M, int64_t N, int d, const uint16_t* idx, int K, float* C,
                        int32_t* counts, void* ws, size_t ws_bytes, hipStream_t st)
{
    const int64_t n_sub = M * N / d;
    const int nblk = (int)((n_sub + kSortTile - 1) / kSortTile);
    Carver cv(ws, ws_bytes);
    UpdateWs w = carve_update(cv, n_sub, K);
    if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "vq_update: workspace too small");

    TimedRegion tr("update", K, st);
    const int passes = K > 256 ? 2 : 1;
    const uint16_t* kin = idx;
    const int32_t* vin = nullptr;
    uint16_t* kout = w.k1;
    int32_t* vout = w.v1;
    for (int p = 0; p < passes; ++p) {
        const int shift = 8 * p;
        hipLaunchKernelGGL(k_sort_hist, dim3(nblk), dim3(kSortThreads), 0, st, kin, n_sub, shift, w.hist,
                           nblk);
        VQ_LAUNCHED("k_sort_hist");
        hipLaunchKernelGGL(k_scan_digit, dim3(256), dim3(256), 0, st, w.hist, nblk, w.dtot);
        VQ_LAUNCHED("k_scan_digit");
        hipLaunchKernelGGL(k_sort_scatter, dim3(nblk), dim3(kSortThreads), 0, st, kin, vin, n_sub, shift,
                           w.hist, w.dtot, nblk, kout, vout);
        VQ_LAUNCHED("k_sort_scatter");
        kin = kout;
        vin = vout;
        kout = (kout == w.k1) ? w.k2 : w.k1;
        vout = (vout == w.v1) ? w.v2 : w.v1;
    }
    const uint16_t* skeys = kin;
    const int32_t* svals = vin;
    hipLaunchKernelGGL(k_seg_start, dim3(grid_for((int64_t)K + 1, 256)), dim3(256), 0, st, skeys, n_sub, K,
                       w.start);
    VQ_LAUNCHED("k_seg_start");
    hipLaunchKernelGGL(k_piece_scan, dim3(1), dim3(kScanThreads), 0, st, w.start, K, w.poff);
    VQ_LAUNCHED("k_piece_scan");
    const int64_t bound = piece_bound(n_sub, K);
    hipLaunchKernelGGL(k_seg_reduce, dim3(grid_for(bound, 4)), dim3(256), 0, st, X, hcol, rho, mask,
                       N / d, d, svals, w.start, w.poff, K, w.part);
    VQ_LAUNCHED("k_seg_reduce");
    hipLaunchKernelGGL(k_seg_finish, dim3(grid_for(K, 256)), dim3(256), 0, st, w.part, w.start, w.poff, K,
                       d, C, counts);
    VQ_LAUNCHED("k_seg_finish");
    return VQ_OK;
}

}  // namespace vq
