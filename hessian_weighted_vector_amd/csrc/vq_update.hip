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
//   3. the sorted array is cut into fixed chunks; 8 lanes (one per
//      dimension) walk a chunk in order with float64 sums of omega*x and
//      omega, finishing the segments that lie inside it and leaving partial
//      sums for the two that cross its ends;
//   4. 8 lanes per crossing centroid add those partials in chunk order and
//      divide once.
#include "vq_internal.h"

namespace vq {
namespace {

constexpr int kSortThreads = 256;
constexpr int kSortItems = 16;
constexpr int kSortTile = kSortThreads * kSortItems;   // elements per sort block
constexpr int kChunk = 64;                              // sorted members per 8-lane group

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
// vals_in == nullptr means the values are the element positions; the tag
// bytes (the sub-vector's mask, nullable) travel with the values.
// Each wavefront ranks its own contiguous sub-tile of kSortItems*64 elements
// (ballot match of equal digits, wave-private LDS counters), then one
// cross-wave prefix per digit gives every element its position.
__global__ __launch_bounds__(kSortThreads) void k_sort_scatter(
    const uint16_t* __restrict__ keys_in, const int32_t* __restrict__ vals_in, const uint8_t* __restrict__ tag_in,
    int64_t n, int shift, const int* __restrict__ hist, const int* __restrict__ digit_total, int nblk,
    uint16_t* __restrict__ keys_out, int32_t* __restrict__ vals_out, uint8_t* __restrict__ tag_out)
{
    __shared__ int sh[256];
    __shared__ int base[256];
    __shared__ int wcnt[4][256];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // global start of each digit for this block
    const int tot = digit_total[tid];
    const int incl = block_incl_scan_256(tot, sh);
    base[tid] = (incl - tot) + hist[(int64_t)tid * nblk + blockIdx.x];
    for (int w = 0; w < 4; ++w) wcnt[w][tid] = 0;
    __syncthreads();

    const int64_t wave0 = (int64_t)blockIdx.x * kSortTile + (int64_t)wave * (kSortItems * 64);
    const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint16_t key[kSortItems];
    int32_t val[kSortItems];
    uint8_t tag[kSortItems];
    int rank[kSortItems];
#pragma unroll
    for (int r = 0; r < kSortItems; ++r) {
        const int64_t e = wave0 + (int64_t)r * 64 + lane;
        const bool valid = e < n;
        key[r] = valid ? keys_in[e] : (uint16_t)0;
        val[r] = valid ? (vals_in ? vals_in[e] : (int32_t)e) : 0;
        tag[r] = (valid && tag_in) ? tag_in[e] : (uint8_t)0;
        const int dg = (key[r] >> shift) & 255;
        unsigned long long peers = __ballot(valid);
        for (int bit = 0; bit < 8; ++bit) {
            const unsigned long long bal = __ballot(valid && ((dg >> bit) & 1));
            peers &= ((dg >> bit) & 1) ? bal : ~bal;
        }
        const int wrank = __popcll(peers & lt_mask);
        int run = 0;
        if (valid) run = wcnt[wave][dg];
        rank[r] = valid ? run + wrank : -1;
        if (valid && wrank == 0) wcnt[wave][dg] = run + __popcll(peers);
    }
    __syncthreads();
    // offsets of each wavefront's part of each digit: prefix over the waves
    {
        int acc = 0;
        for (int w = 0; w < 4; ++w) {
            const int c = wcnt[w][tid];
            wcnt[w][tid] = acc;
            acc += c;
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kSortItems; ++r) {
        if (rank[r] >= 0) {
            const int dg = (key[r] >> shift) & 255;
            const int64_t pos = (int64_t)base[dg] + wcnt[wave][dg] + rank[r];
            keys_out[pos] = key[r];
            vals_out[pos] = val[r];
            if (tag_out) tag_out[pos] = tag[r];
        }
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

// Weight and value of element t of sub-vector s, float64 (weight = hcol,
// times rho if present; 0 when masked).
__device__ inline void member_term(const float* __restrict__ X, const float* __restrict__ hcol,
                                   const float* __restrict__ rho, unsigned mb,
                                   uint32_t s, uint32_t nb, int d, int t, double& w, double& x)
{
    const uint32_t i = s / nb;
    const uint32_t b = s - i * nb;
    double wt = (double)hcol[(size_t)b * d + t];
    if (rho) wt = wt * (double)rho[i];
    if ((mb >> t) & 1u) wt = 0.0;
    w = wt;
    x = (double)X[(size_t)s * d + t];
}

// Chunked segmented reduction over the sorted (index, sub-vector) pairs.
// The sorted array is cut into fixed chunks of kChunk members; a group of 8
// lanes owns one chunk (lane t = dimension t) and walks it in order with
// float64 sums of omega*x and omega.  A segment (all members of one
// centroid) that lies inside the chunk is finished here; the segment that
// enters the chunk from the left leaves a "head" partial and the one that
// leaves to the right a "tail" partial, added in chunk order later.
__global__ __launch_bounds__(256) void k_seg_chunks(
    const float* __restrict__ X, const float* __restrict__ hcol, const float* __restrict__ rho,
    const uint8_t* __restrict__ smask, uint32_t nb, int d, const uint16_t* __restrict__ skeys,
    const int32_t* __restrict__ svals, const int* __restrict__ start, int64_t n, int64_t nchunks,
    float* __restrict__ C, int32_t* __restrict__ counts, double* __restrict__ head,
    double* __restrict__ tail)
{
    constexpr int kBatch = 8;   // members whose loads are issued together
    const int t = threadIdx.x & 7;
    const int64_t ch = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
    if (ch >= nchunks) return;
    const int64_t c0 = ch * kChunk;
    const int64_t c1 = c0 + kChunk < n ? c0 + kChunk : n;
    int k = skeys[c0];
    double num = 0.0, den = 0.0;
    for (int64_t e0 = c0; e0 < c1; e0 += kBatch) {
        int kk[kBatch];
        double wv[kBatch], xv[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int64_t e = e0 + q;
            kk[q] = -1;
            wv[q] = 0.0;
            xv[q] = 0.0;
            if (e < c1) {
                kk[q] = skeys[e];
                if (t < d)
                    member_term(X, hcol, rho, smask ? smask[e] : 0u, (uint32_t)svals[e], nb, d, t, wv[q], xv[q]);
            }
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            if (kk[q] < 0) break;
            if (kk[q] != k) {
                // segment k ends inside this chunk
                if (start[k] < c0) {
                    if (t < d) { head[ch * 16 + t] = num; head[ch * 16 + 8 + t] = den; }
                } else {
                    if (t < d && den > 0.0) C[(size_t)k * d + t] = (float)(num / den);
                    if (t == 0 && counts) counts[k] = start[k + 1] - start[k];
                }
                k = kk[q];
                num = 0.0;
                den = 0.0;
            }
            num = num + wv[q] * xv[q];
            den = den + wv[q];
        }
    }
    // the last segment of the chunk
    const bool from_left = start[k] < c0;
    const bool to_right = start[k + 1] > c1;
    if (to_right) {
        // continues in the next chunk: a tail, or a head when it also came from the left
        double* dst = from_left ? head : tail;
        if (t < d) { dst[ch * 16 + t] = num; dst[ch * 16 + 8 + t] = den; }
    } else if (from_left) {
        if (t < d) { head[ch * 16 + t] = num; head[ch * 16 + 8 + t] = den; }
    } else {
        if (t < d && den > 0.0) C[(size_t)k * d + t] = (float)(num / den);
        if (t == 0 && counts) counts[k] = start[k + 1] - start[k];
    }
}

// Segments that cross chunk boundaries: the tail of the first chunk plus the
// heads of the following ones.  One wavefront per centroid: lane q adds
// chunks j0+1+q, j0+1+q+64, ... in order, then a fixed xor butterfly over
// the lanes; 16 values per chunk (8 sums of omega*x, 8 of omega).  Empty
// centroids get a zero count and keep their value.
__global__ __launch_bounds__(64) void k_seg_cross(const int* __restrict__ start, int K, int d,
                                                  const double* __restrict__ head,
                                                  const double* __restrict__ tail,
                                                  float* __restrict__ C, int32_t* __restrict__ counts)
{
    const int k = blockIdx.x;
    const int lane = threadIdx.x;
    const int s0 = start[k], s1 = start[k + 1];
    if (s1 == s0) {
        if (lane == 0 && counts) counts[k] = 0;
        return;
    }
    const int64_t j0 = s0 / kChunk, j1 = (int64_t)(s1 - 1) / kChunk;
    if (j0 == j1) return;   // finished inside its chunk
    if (lane == 0 && counts) counts[k] = s1 - s0;
    double acc[16];
    for (int v = 0; v < 16; ++v) acc[v] = 0.0;
    for (int64_t j = j0 + 1 + lane; j <= j1; j += 64)
        for (int v = 0; v < 16; ++v) acc[v] = acc[v] + head[j * 16 + v];
    for (int off = 32; off > 0; off >>= 1)
        for (int v = 0; v < 16; ++v) acc[v] = acc[v] + __shfl_xor(acc[v], off);
    if (lane < d) {
        double num = tail[j0 * 16 + lane], den = tail[j0 * 16 + 8 + lane];
        for (int v = 0; v < 8; ++v) {   // select this lane's dimension without dynamic indexing
            if (v == lane) { num = num + acc[v]; den = den + acc[8 + v]; }
        }
        if (den > 0.0) C[(size_t)k * d + lane] = (float)(num / den);
    }
}

struct UpdateWs {
    uint16_t *k1, *k2;
    int32_t *v1, *v2;
    uint8_t *g1, *g2;
    int *hist, *dtot, *start;
    double *head, *tail;
};

int64_t n_chunks(int64_t n_sub) { return (n_sub + kChunk - 1) / kChunk; }

UpdateWs carve_update(Carver& cv, int64_t n_sub, int K)
{
    UpdateWs w;
    const int64_t nblk = (n_sub + kSortTile - 1) / kSortTile;
    w.k1 = cv.take<uint16_t>(n_sub);
    w.k2 = cv.take<uint16_t>(n_sub);
    w.v1 = cv.take<int32_t>(n_sub);
    w.v2 = cv.take<int32_t>(n_sub);
    w.g1 = cv.take<uint8_t>(n_sub);
    w.g2 = cv.take<uint8_t>(n_sub);
    w.hist = cv.take<int>((size_t)256 * nblk);
    w.dtot = cv.take<int>(256);
    w.start = cv.take<int>((size_t)K + 1);
    w.head = cv.take<double>((size_t)n_chunks(n_sub) * 16);
    w.tail = cv.take<double>((size_t)n_chunks(n_sub) * 16);
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
    const uint8_t* gin = mask;
    uint16_t* kout = w.k1;
    int32_t* vout = w.v1;
    uint8_t* gout = mask ? w.g1 : nullptr;
    for (int p = 0; p < passes; ++p) {
        const int shift = 8 * p;
        hipLaunchKernelGGL(k_sort_hist, dim3(nblk), dim3(kSortThreads), 0, st, kin, n_sub, shift, w.hist,
                           nblk);
        VQ_LAUNCHED("k_sort_hist");
        hipLaunchKernelGGL(k_scan_digit, dim3(256), dim3(256), 0, st, w.hist, nblk, w.dtot);
        VQ_LAUNCHED("k_scan_digit");
        hipLaunchKernelGGL(k_sort_scatter, dim3(nblk), dim3(kSortThreads), 0, st, kin, vin, gin, n_sub, shift,
                           w.hist, w.dtot, nblk, kout, vout, gout);
        VQ_LAUNCHED("k_sort_scatter");
        kin = kout;
        vin = vout;
        gin = gout;
        kout = (kout == w.k1) ? w.k2 : w.k1;
        vout = (vout == w.v1) ? w.v2 : w.v1;
        gout = mask ? ((gout == w.g1) ? w.g2 : w.g1) : nullptr;
    }
    const uint16_t* skeys = kin;
    const int32_t* svals = vin;
    const uint8_t* smask = gin;
    hipLaunchKernelGGL(k_seg_start, dim3(grid_for((int64_t)K + 1, 256)), dim3(256), 0, st, skeys, n_sub, K,
                       w.start);
    VQ_LAUNCHED("k_seg_start");
    const int64_t nch = n_chunks(n_sub);
    hipLaunchKernelGGL(k_seg_chunks, dim3(grid_for(nch, 32)), dim3(256), 0, st, X, hcol, rho, smask,
                       (uint32_t)(N / d), d, skeys, svals, w.start, n_sub, nch, C, counts, w.head, w.tail);
    VQ_LAUNCHED("k_seg_chunks");
    hipLaunchKernelGGL(k_seg_cross, dim3((unsigned)K), dim3(64), 0, st, w.start, K, d, w.head, w.tail, C, counts);
    VQ_LAUNCHED("k_seg_cross");
    return VQ_OK;
}

}  // namespace vq
