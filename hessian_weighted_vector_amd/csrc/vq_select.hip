// Salience selection into the exact sparse correction.
//
// Method: HAS-VQ abstract ("Hessian-Masked Decoupling" isolates the weights
// with the largest second-order sensitivity; they are held exactly) and the
// SCVQ summary (every exactly held weight lives in one CSR).  Score of element (i,j):
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

__device__ inline uint32_t score_of(float w, float hj)
{
    const float sq = w * w;
    return __float_as_uint(hj * sq);
}

// Scores of row i, columns j .. j+3 (vec: N % 4 == 0 and W, h 16-byte aligned).
__device__ inline void score4(const float* __restrict__ W, const float* __restrict__ h, int64_t i, int64_t N,
                              int64_t j, uint32_t (&b)[4])
{
    const float4 w = *reinterpret_cast<const float4*>(W + i * N + j);
    const float4 hh = *reinterpret_cast<const float4*>(h + j);
    b[0] = score_of(w.x, hh.x);
    b[1] = score_of(w.y, hh.y);
    b[2] = score_of(w.z, hh.z);
    b[3] = score_of(w.w, hh.w);
}

__global__ void k_sel_init(SelState* st, int64_t nnz, int* hist)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t == 0) { st->prefix = nnz > 0 ? 0u : 0xFFFFFFFFu; st->pad = 0u; st->remaining = nnz; }
    if (t < kBins) hist[t] = 0;
}

// Workgroups take whole rows (row, then columns: no index division), four
// columns per thread per step with 16-byte loads where vec; each wavefront
// counts into its own LDS copy of the histogram (less contention on the
// few crowded bins of the first digit), summed at the end.
__global__ __launch_bounds__(256) void k_sel_hist(const float* __restrict__ W,
                                                  const float* __restrict__ h, int64_t M,
                                                  int64_t N, bool vec, const SelState* __restrict__ st,
                                                  uint32_t pmask, int shift, uint32_t dmask,
                                                  int* __restrict__ hist)
{
    __shared__ int cnt[4][kBins];
    for (int q = threadIdx.x; q < 4 * kBins; q += blockDim.x) (&cnt[0][0])[q] = 0;
    __syncthreads();
    const uint32_t prefix = st->prefix;
    int* my = cnt[threadIdx.x >> 6];
    for (int64_t i = blockIdx.x; i < M; i += gridDim.x) {
        if (vec) {
            for (int64_t j = (int64_t)threadIdx.x * 4; j < N; j += 4 * (int64_t)blockDim.x) {
                uint32_t b[4];
                score4(W, h, i, N, j, b);
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if ((b[u] & pmask) == prefix) atomicAdd(&my[(b[u] >> shift) & dmask], 1);
            }
        } else {
            for (int64_t j = threadIdx.x; j < N; j += blockDim.x) {
                const uint32_t b = score_of(W[i * N + j], h[j]);
                if ((b & pmask) == prefix) atomicAdd(&my[(b >> shift) & dmask], 1);
            }
        }
    }
    __syncthreads();
    for (int q = threadIdx.x; q < kBins; q += blockDim.x) {
        const int c = cnt[0][q] + cnt[1][q] + cnt[2][q] + cnt[3][q];
        if (c) atomicAdd(&hist[q], c);
    }
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
    const float* __restrict__ W, const float* __restrict__ h, int64_t N, bool vec,
    const SelState* __restrict__ st, int* __restrict__ cgt, int* __restrict__ ceq)
{
    __shared__ int sg[kRowThreads], se[kRowThreads];
    const int64_t i = blockIdx.x;
    const uint32_t tau = st->prefix;
    int g = 0, q = 0;
    if (vec) {
        for (int64_t j = (int64_t)threadIdx.x * 4; j < N; j += 4 * kRowThreads) {
            uint32_t b[4];
            score4(W, h, i, N, j, b);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                g += b[u] > tau;
                q += b[u] == tau;
            }
        }
    } else {
        for (int64_t j = threadIdx.x; j < N; j += kRowThreads) {
            const uint32_t b = score_of(W[i * N + j], h[j]);
            g += b > tau;
            q += b == tau;
        }
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
    if (row_ptr == nullptr) return;   // uniform: the selection only needs take[]
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
    const float* __restrict__ W, const float* __restrict__ h, int64_t N, int d, bool vec8,
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
            if (vec8) {
                score4(W, h, i, N, b * 8, *reinterpret_cast<uint32_t(*)[4]>(&bits[0]));
                score4(W, h, i, N, b * 8 + 4, *reinterpret_cast<uint32_t(*)[4]>(&bits[4]));
            } else {
                for (int t = 0; t < d; ++t) bits[t] = score_of(W[i * N + b * d + t], h[b * d + t]);
            }
            for (int t = 0; t < d; ++t) n_eq += bits[t] == tau;
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

// ---- the unified sparse correction ---------------------------------------
// SCVQ summary: a single sparse matrix carries every exactly-held weight:
// the salient elements, whole sub-vectors of high salience and the positions
// where quantization left the biggest error.  The two extra
// selections mark the mask (bit t of byte s = element t of sub-vector s is
// held exactly); vq_mask_to_csr turns the mask into the CSR.
//
// Keys are uint32: 0 = not eligible, otherwise the score's float bits + 1
// (non-negative floats order like their bits), so the same radix select
// (k_sel_init / k_sel_pick / k_sel_rows) finds the n-th largest key; a
// threshold of 0 means fewer eligible keys than asked, and then every
// eligible key is taken and no tie is.  The unit of work is one sub-vector
// (contiguous d floats of W); a functor yields its keys in linear order.

// One key per sub-vector: S_s = sum over t of h_j * (w_j * w_j), fp32, t in
// order, no fused multiply-add.
struct KeySubvector {
    const float* W;
    const float* h;
    uint32_t nb;
    int d;
    bool vec;   // d == 8 with 16-byte aligned W and h
    static constexpr int kKeys = 1;
    __device__ int count() const { return 1; }
    __device__ void keys(int64_t s, uint32_t* k) const
    {
        const uint32_t b = (uint32_t)s % nb;
        float acc = 0.0f;
        if (vec) {
            const float4* w4 = reinterpret_cast<const float4*>(W + s * 8);
            const float4* h4 = reinterpret_cast<const float4*>(h + (size_t)b * 8);
            const float4 wa = w4[0], wb = w4[1], ha = h4[0], hb = h4[1];
            const float w[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
            const float hh[8] = {ha.x, ha.y, ha.z, ha.w, hb.x, hb.y, hb.z, hb.w};
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float sq = w[t] * w[t];
                const float term = hh[t] * sq;
                acc = acc + term;
            }
        } else {
            const float* w = W + s * d;
            const float* hh = h + (size_t)b * d;
            for (int t = 0; t < d; ++t) {
                const float x = w[t];
                const float sq = x * x;
                const float term = hh[t] * sq;
                acc = acc + term;
            }
        }
        k[0] = __float_as_uint(acc) + 1u;
    }
};

// One key per element: r = h_j * ((w - what) * (w - what)), fp32, not
// eligible where the mask bit is already set.
struct KeyResidual {
    const float* W;
    const float* Wh;
    const float* h;
    const uint8_t* mask;
    uint32_t nb;
    int d;
    bool vec;   // d == 8 with 16-byte aligned W, W_hat and h
    static constexpr int kKeys = 8;
    __device__ int count() const { return d; }
    __device__ void keys(int64_t s, uint32_t* k) const
    {
        const uint32_t b = (uint32_t)s % nb;
        const unsigned mb = mask[s];
        if (vec) {
            const float4* w4 = reinterpret_cast<const float4*>(W + s * 8);
            const float4* q4 = reinterpret_cast<const float4*>(Wh + s * 8);
            const float4* h4 = reinterpret_cast<const float4*>(h + (size_t)b * 8);
            const float4 wa = w4[0], wb = w4[1], qa = q4[0], qb = q4[1], ha = h4[0], hb = h4[1];
            const float w[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
            const float q[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
            const float hh[8] = {ha.x, ha.y, ha.z, ha.w, hb.x, hb.y, hb.z, hb.w};
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float r = w[t] - q[t];
                const float sq = r * r;
                const float sc = hh[t] * sq;
                k[t] = ((mb >> t) & 1u) ? 0u : __float_as_uint(sc) + 1u;
            }
            return;
        }
        const float* w = W + s * d;
        const float* wh = Wh + s * d;
        const float* hh = h + (size_t)b * d;
        for (int t = 0; t < d; ++t) {
            const float r = w[t] - wh[t];
            const float sq = r * r;
            const float sc = hh[t] * sq;
            k[t] = ((mb >> t) & 1u) ? 0u : __float_as_uint(sc) + 1u;
        }
    }
};

template <class F>
__global__ __launch_bounds__(256) void k_key_hist(F f, int64_t n_units, const SelState* __restrict__ st,
                                                  uint32_t pmask, int shift, uint32_t dmask,
                                                  int* __restrict__ hist)
{
    __shared__ int cnt[kBins];
    for (int q = threadIdx.x; q < kBins; q += blockDim.x) cnt[q] = 0;
    __syncthreads();
    const uint32_t prefix = st->prefix;
    const int g = f.count();
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; s < n_units; s += stride) {
        uint32_t k[F::kKeys];
        f.keys(s, k);
        for (int t = 0; t < g; ++t)
            if ((k[t] & pmask) == prefix) atomicAdd(&cnt[(k[t] >> shift) & dmask], 1);
    }
    __syncthreads();
    for (int q = threadIdx.x; q < kBins; q += blockDim.x)
        if (cnt[q]) atomicAdd(&hist[q], cnt[q]);
}

// Per row (units [i*upr, (i+1)*upr)): keys above the threshold, and ties
// (none when the threshold is 0).
template <class F>
__global__ __launch_bounds__(kRowThreads) void k_key_row_count(F f, int64_t upr, const SelState* __restrict__ st,
                                                               int* __restrict__ cgt, int* __restrict__ ceq)
{
    __shared__ int sg[kRowThreads], se[kRowThreads];
    const int64_t i = blockIdx.x;
    const uint32_t tau = st->prefix;
    const int g_n = f.count();
    int g = 0, q = 0;
    for (int64_t u = threadIdx.x; u < upr; u += kRowThreads) {
        uint32_t k[F::kKeys];
        f.keys(i * upr + u, k);
        for (int t = 0; t < g_n; ++t) {
            g += k[t] > tau;
            q += (k[t] == tau) && tau != 0u;
        }
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

// Per row: walk the units in order, decide each key (above the threshold, or
// one of the row's first take[i] ties), and OR the decisions into the mask:
// bit t per element key, or every bit of the sub-vector for a sub-vector key.
template <class F>
__global__ __launch_bounds__(kRowThreads) void k_key_mark(F f, int64_t upr, int d, const SelState* __restrict__ st,
                                                          const int* __restrict__ take, uint8_t* __restrict__ mask)
{
    __shared__ int sh[kRowThreads];
    __shared__ int tot_eq;
    const int64_t i = blockIdx.x;
    const uint32_t tau = st->prefix;
    const int row_take = take[i];
    const int g_n = f.count();
    const unsigned all_bits = (1u << d) - 1u;
    int eq_run = 0;
    for (int64_t u0 = 0; u0 < upr; u0 += kRowThreads) {
        const int64_t u = u0 + threadIdx.x;
        uint32_t k[F::kKeys];
        int n_eq = 0;
        if (u < upr) {
            f.keys(i * upr + u, k);
            for (int t = 0; t < g_n; ++t) n_eq += (k[t] == tau) && tau != 0u;
        }
        const int eq_incl = scan256(n_eq, sh);
        if (threadIdx.x == kRowThreads - 1) tot_eq = eq_incl;
        if (u < upr) {
            int eq_rank = eq_run + eq_incl - n_eq;
            unsigned mb = 0;
            for (int t = 0; t < g_n; ++t) {
                bool sel = k[t] > tau;
                if (k[t] == tau && tau != 0u) { sel = eq_rank < row_take; ++eq_rank; }
                if (sel) mb |= (F::kKeys == 1) ? all_bits : (1u << t);
            }
            if (mb) {
                const int64_t s = i * upr + u;
                mask[s] = (uint8_t)(mask[s] | mb);
            }
        }
        __syncthreads();
        eq_run += tot_eq;
        __syncthreads();
    }
}

// mask -> CSR: per-row counts, one block scans the rows, then per row a
// block writes the held positions in column order (at most cap entries).
__global__ __launch_bounds__(kRowThreads) void k_mask_row_count(const uint8_t* __restrict__ mask, int64_t nb, int d,
                                                                int* __restrict__ cnt)
{
    __shared__ int sh[kRowThreads];
    const int64_t i = blockIdx.x;
    const unsigned all_bits = (1u << d) - 1u;
    int c = 0;
    for (int64_t b = threadIdx.x; b < nb; b += kRowThreads) c += __popc(mask[i * nb + b] & all_bits);
    sh[threadIdx.x] = c;
    __syncthreads();
    for (int w = kRowThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) cnt[i] = sh[0];
}

__global__ __launch_bounds__(kScanThreads) void k_mask_rows(int64_t M, const int* __restrict__ cnt,
                                                            int32_t* __restrict__ row_ptr)
{
    __shared__ int64_t sh[kScanThreads];
    const int64_t per = (M + kScanThreads - 1) / kScanThreads;
    const int64_t r0 = threadIdx.x * per;
    const int64_t r1 = r0 + per < M ? r0 + per : M;
    int64_t local = 0;
    for (int64_t i = r0; i < r1; ++i) local += cnt[i];
    int64_t run = scan1024(local, sh) - local;
    for (int64_t i = r0; i < r1; ++i) {
        row_ptr[i] = (int32_t)run;
        run += cnt[i];
    }
    if (threadIdx.x == kScanThreads - 1) row_ptr[M] = (int32_t)run;
}

__global__ __launch_bounds__(kRowThreads) void k_mask_compact(const float* __restrict__ W,
                                                              const uint8_t* __restrict__ mask, int64_t N, int d,
                                                              const int32_t* __restrict__ row_ptr, int64_t cap,
                                                              int32_t* __restrict__ col, float* __restrict__ val)
{
    __shared__ int sh[kRowThreads];
    __shared__ int tot;
    const int64_t i = blockIdx.x;
    const int64_t nb = N / d;
    const unsigned all_bits = (1u << d) - 1u;
    int64_t pos_run = row_ptr[i];
    for (int64_t b0 = 0; b0 < nb; b0 += kRowThreads) {
        const int64_t b = b0 + threadIdx.x;
        const unsigned mb = b < nb ? (mask[i * nb + b] & all_bits) : 0u;
        const int n = __popc(mb);
        const int incl = scan256(n, sh);
        if (threadIdx.x == kRowThreads - 1) tot = incl;
        int64_t p = pos_run + incl - n;
        for (int t = 0; t < d; ++t) {
            if (((mb >> t) & 1u) && p < cap) {
                col[p] = (int32_t)(b * d + t);
                val[p] = W[i * N + b * d + t];
                ++p;
            }
        }
        __syncthreads();
        pos_run += tot;
        __syncthreads();
    }
}

// Radix select of the n-th largest key, then per-row counts, ties and marks.
template <class F>
vq_status key_select_launch(const F& f, int64_t M, int64_t upr, int d, int64_t n, uint8_t* mask, void* ws,
                            size_t ws_bytes, const char* what, hipStream_t st)
{
    Carver cv(ws, ws_bytes);
    SelState* state = cv.take<SelState>(1);
    int* hist = cv.take<int>(kBins);
    int* cgt = cv.take<int>((size_t)M);
    int* ceq = cv.take<int>((size_t)M);
    int* take = cv.take<int>((size_t)M);
    if (!cv.ok) return fail(VQ_ERR_WORKSPACE, std::string(what) + ": workspace too small");
    const int64_t n_units = M * upr;
    hipLaunchKernelGGL(k_sel_init, dim3(grid_for(kBins, 256)), dim3(256), 0, st, state, n, hist);
    VQ_LAUNCHED("k_sel_init");
    if (n > 0) {
        const int shifts[3] = {21, 10, 0};
        const int nbins[3] = {2048, 2048, 1024};
        const uint32_t pmasks[3] = {0u, 0xFFE00000u, 0xFFFFFC00u};
        const unsigned hb = (unsigned)std::min<int64_t>(kHistBlocks, grid_for(n_units, 256 * 4));
        for (int p = 0; p < 3; ++p) {
            hipLaunchKernelGGL((k_key_hist<F>), dim3(hb), dim3(256), 0, st, f, n_units, state, pmasks[p], shifts[p],
                               (uint32_t)(nbins[p] - 1), hist);
            VQ_LAUNCHED("k_key_hist");
            hipLaunchKernelGGL(k_sel_pick, dim3(1), dim3(256), 0, st, state, hist, shifts[p], nbins[p]);
            VQ_LAUNCHED("k_sel_pick");
        }
    }
    hipLaunchKernelGGL((k_key_row_count<F>), dim3((unsigned)M), dim3(kRowThreads), 0, st, f, upr, state, cgt, ceq);
    VQ_LAUNCHED("k_key_row_count");
    hipLaunchKernelGGL(k_sel_rows, dim3(1), dim3(kScanThreads), 0, st, state, M, cgt, ceq, take,
                       static_cast<int32_t*>(nullptr));
    VQ_LAUNCHED("k_sel_rows");
    hipLaunchKernelGGL((k_key_mark<F>), dim3((unsigned)M), dim3(kRowThreads), 0, st, f, upr, d, state, take, mask);
    VQ_LAUNCHED("k_key_mark");
    return VQ_OK;
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
    (void)total;
    // 16-byte loads of W's rows and of h: rows of whole float4 groups
    const bool vec = N % 4 == 0 && ((reinterpret_cast<uintptr_t>(W) | reinterpret_cast<uintptr_t>(h)) & 15u) == 0;
    TimedRegion tr("select", 0, st);

    // nnz == 0 skips the threshold search: the initial threshold pattern
    // 0xFFFFFFFF lies above every non-negative score, so nothing is taken.
    hipLaunchKernelGGL(k_sel_init, dim3(grid_for(kBins, 256)), dim3(256), 0, st, state, nnz, hist);
    VQ_LAUNCHED("k_sel_init");
    if (nnz > 0) {
        const int shifts[3] = {21, 10, 0};
        const int nbins[3] = {2048, 2048, 1024};
        const uint32_t pmasks[3] = {0u, 0xFFE00000u, 0xFFFFFC00u};
        const unsigned hb = (unsigned)std::min<int64_t>(kHistBlocks, M);
        for (int p = 0; p < 3; ++p) {
            hipLaunchKernelGGL(k_sel_hist, dim3(hb), dim3(256), 0, st, W, h, M, N, vec, state, pmasks[p],
                               shifts[p], (uint32_t)(nbins[p] - 1), hist);
            VQ_LAUNCHED("k_sel_hist");
            hipLaunchKernelGGL(k_sel_pick, dim3(1), dim3(256), 0, st, state, hist, shifts[p], nbins[p]);
            VQ_LAUNCHED("k_sel_pick");
        }
    }
    hipLaunchKernelGGL(k_sel_row_count, dim3((unsigned)M), dim3(kRowThreads), 0, st, W, h, N, vec, state, cgt,
                       ceq);
    VQ_LAUNCHED("k_sel_row_count");
    hipLaunchKernelGGL(k_sel_rows, dim3(1), dim3(kScanThreads), 0, st, state, M, cgt, ceq, take, row_ptr);
    VQ_LAUNCHED("k_sel_rows");
    hipLaunchKernelGGL(k_sel_compact, dim3((unsigned)M), dim3(kRowThreads), 0, st, W, h, N, d, vec && d == 8,
                       state, take, row_ptr, nnz, col, val, mask);
    VQ_LAUNCHED("k_sel_compact");
    return VQ_OK;
}

vq_status subvector_select_launch(const float* W, const float* h, int64_t M, int64_t N, int d, int64_t n_sel,
                                  uint8_t* mask, void* ws, size_t ws_bytes, hipStream_t st)
{
    TimedRegion tr("select_subvectors", 0, st);
    const bool vec = d == 8 && aligned16(W) && aligned16(h);
    const KeySubvector f{W, h, (uint32_t)(N / d), d, vec};
    return key_select_launch(f, M, N / d, d, n_sel, mask, ws, ws_bytes, "vq_select_subvectors", st);
}

vq_status residual_select_launch(const float* W, const float* Wh, const float* h, int64_t M, int64_t N, int d,
                                 int64_t n_sel, uint8_t* mask, void* ws, size_t ws_bytes, hipStream_t st)
{
    TimedRegion tr("select_residual", 0, st);
    const bool vec = d == 8 && aligned16(W) && aligned16(Wh) && aligned16(h);
    const KeyResidual f{W, Wh, h, mask, (uint32_t)(N / d), d, vec};
    return key_select_launch(f, M, N / d, d, n_sel, mask, ws, ws_bytes, "vq_select_residual", st);
}

vq_status mask_to_csr_launch(const float* W, const uint8_t* mask, int64_t M, int64_t N, int d, int64_t cap,
                             int32_t* row_ptr, int32_t* col, float* val, void* ws, size_t ws_bytes, hipStream_t st)
{
    Carver cv(ws, ws_bytes);
    int* cnt = cv.take<int>((size_t)M);
    if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "vq_mask_to_csr: workspace too small");
    TimedRegion tr("mask_to_csr", 0, st);
    hipLaunchKernelGGL(k_mask_row_count, dim3((unsigned)M), dim3(kRowThreads), 0, st, mask, N / d, d, cnt);
    VQ_LAUNCHED("k_mask_row_count");
    hipLaunchKernelGGL(k_mask_rows, dim3(1), dim3(kScanThreads), 0, st, M, cnt, row_ptr);
    VQ_LAUNCHED("k_mask_rows");
    hipLaunchKernelGGL(k_mask_compact, dim3((unsigned)M), dim3(kRowThreads), 0, st, W, mask, N, d, row_ptr, cap, col,
                       val);
    VQ_LAUNCHED("k_mask_compact");
    return VQ_OK;
}

}  // namespace vq
