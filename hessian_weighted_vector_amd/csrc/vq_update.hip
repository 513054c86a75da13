// Centroid update as a weighted segmented reduction (VPTQ page,
// "Hessian-Weighted Centroid Initialization": each centroid becomes the
// Hessian-weighted mean of its members; with one weight per element the
// exact minimizer of the objective is the per-dimension weighted mean).
//
// Design (no floating-point atomics; bitwise deterministic):
//   1. buckets (K > 256 only): one stable scatter by idx >> 7 moves whole
//      records (the sub-vector's d values and a word holding its id, mask
//      byte and idx & 127) into 128-centroid buckets, so no sub-vector is
//      gathered at random later.  Each 2048-record tile is ordered by bucket
//      in LDS first (ranks from wavefront ballots: stable), then written out
//      as contiguous runs.  Tile digit counts use LDS integer atomics
//      (exact) and tile offsets come from a scan.  With K <= 256 the whole
//      matrix is one bucket of up to 256 centroids, read in place;
//   2. each bucket is cut into fixed pieces; a workgroup streams its piece
//      through LDS in sub-chunks of 1024 records, stages each record's x,
//      its column weights (zero where masked) and its row weight, counting-
//      sorts the sub-chunk by centroid (stable), and 8-lane groups that own
//      fixed centroids add their members in order into float64 sums of
//      omega*x and omega kept in registers.  A bucket that fits one piece
//      is finished there (members in ascending sub-vector order, the order
//      of a plain sequential sum);
//   3. buckets with several pieces: one pass adds the pieces' partial sums
//      in a fixed order and divides once.
#include "vq_internal.h"

#include <algorithm>

namespace vq {
namespace {

constexpr int kTile = 2048;          // records per scatter tile
constexpr int kTileThreads = 1024;   // two records per thread
constexpr int kMaxBuckets = 512;     // K <= 65536, 128 centroids per bucket
constexpr int kBucketShift = 7;
constexpr int kSub = 1024;           // records per LDS sub-chunk (one per thread)
constexpr int kRedThreads = 1024;
constexpr int kPieceMax = 32768;     // records per piece in bucket mode
constexpr int kDirectPieces = 512;   // target piece count with one bucket

// Per-tile bucket histogram: hist[bucket * ntile + tile].
__global__ __launch_bounds__(256) void k_bucket_hist(const uint16_t* __restrict__ idx, int64_t n, int nbk,
                                                     int* __restrict__ hist, int ntile)
{
    __shared__ int cnt[kMaxBuckets];
    for (int q = threadIdx.x; q < kMaxBuckets; q += 256) cnt[q] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kTile;
    for (int q = threadIdx.x; q < kTile; q += 256) {
        const int64_t e = base + q;
        if (e < n) {
            const int bk = idx[e] >> kBucketShift;
            if (bk < nbk) atomicAdd(&cnt[bk], 1);
        }
    }
    __syncthreads();
    for (int q = threadIdx.x; q < nbk; q += 256) hist[(int64_t)q * ntile + blockIdx.x] = cnt[q];
}

// One block per bucket: exclusive scan of its per-tile counts, in place;
// total[bucket] = the bucket's size.  1024 threads: a wavefront-shuffle
// scan, the 16 wavefront totals from LDS, a running carry per 1024 tiles.
__global__ __launch_bounds__(1024) void k_bucket_scan(int* __restrict__ hist, int ntile, int* __restrict__ total)
{
    __shared__ int wsum[16];
    __shared__ int carry_sh;
    int* row = hist + (int64_t)blockIdx.x * ntile;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (threadIdx.x == 0) carry_sh = 0;
    __syncthreads();
    for (int c0 = 0; c0 < ntile; c0 += 1024) {
        const int q = c0 + threadIdx.x;
        const int v = q < ntile ? row[q] : 0;
        int x = v;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) wsum[wave] = x;
        __syncthreads();
        int before = carry_sh;
        for (int w = 0; w < wave; ++w) before += wsum[w];
        if (q < ntile) row[q] = before + x - v;
        __syncthreads();
        if (threadIdx.x == 0) {
            int t = 0;
            for (int w = 0; w < 16; ++w) t += wsum[w];
            carry_sh += t;
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) total[blockIdx.x] = carry_sh;
}

// Bucket starts and piece numbering (one wavefront, nbk <= 512): bucket b
// holds records [bstart[b], bstart[b+1]) and is cut into ceil(size / piece)
// pieces, numbered from poff[b].  total == nullptr: one bucket of n records.
__global__ __launch_bounds__(64) void k_piece_setup(const int* __restrict__ total, int nbk, int64_t n, int piece,
                                                    int64_t* __restrict__ bstart, int* __restrict__ poff)
{
    const int lane = threadIdx.x;
    const int per = (nbk + 63) / 64;
    int64_t sz[8];
    int64_t s_sum = 0;
    int p_sum = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int q = lane * per + u;
        sz[u] = (u < per && q < nbk) ? (total ? (int64_t)total[q] : n) : 0;
        s_sum += sz[u];
        p_sum += (int)((sz[u] + piece - 1) / piece);
    }
    int64_t s_inc = s_sum;
    int p_inc = p_sum;
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t so = __shfl_up(s_inc, off);
        const int po = __shfl_up(p_inc, off);
        if (lane >= off) { s_inc += so; p_inc += po; }
    }
    int64_t srun = s_inc - s_sum;
    int prun = p_inc - p_sum;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int q = lane * per + u;
        if (u < per && q < nbk) {
            bstart[q] = srun;
            poff[q] = prun;
        }
        srun += sz[u];
        prun += (int)((sz[u] + piece - 1) / piece);
    }
    if (lane == 63) {
        bstart[nbk] = srun;
        poff[nbk] = prun;
    }
}

// Stable ranks of up to 64 keys (< 2^bits) across one wavefront: peers =
// lanes holding the same key; returns the lane's rank among its peers.
__device__ inline int wave_peer_rank(int key, bool valid, int bits, unsigned long long lt_mask,
                                     unsigned long long& peers)
{
    peers = __ballot(valid);
    for (int bit = 0; bit < bits; ++bit) {
        const unsigned long long bal = __ballot(valid && ((key >> bit) & 1));
        peers &= ((key >> bit) & 1) ? bal : ~bal;
    }
    return __popcll(peers & lt_mask);
}

// Exclusive scan of cnt[0..n) (n <= 512) by the first wavefront, into out;
// out[n] = total.  Callers synchronize around it.
template <class T>
__device__ inline void wave_excl_scan(const int* cnt, int n, T* out)
{
    const int lane = threadIdx.x;
    if (lane >= 64) return;
    const int per = (n + 63) / 64;
    int s = 0;
    for (int u = 0; u < per; ++u) {
        const int q = lane * per + u;
        s += q < n ? cnt[q] : 0;
    }
    int inc = s;
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(inc, off);
        if (lane >= off) inc += o;
    }
    int run = inc - s;
    for (int u = 0; u < per; ++u) {
        const int q = lane * per + u;
        if (q < n) { out[q] = (T)run; run += cnt[q]; }
    }
    if (lane == 63) out[n] = (T)run;
}

// Stable scatter of whole records into buckets.  A tile of kTile records is
// ranked by bucket (wavefront ballots + a prefix over the wavefronts), laid
// out in bucket order in LDS, and written to its place in each bucket as
// contiguous runs: rx gets the d values, rw the word
//   id | (idx & 127) << 32 | mask << 40.
__global__ __launch_bounds__(kTileThreads) void k_bucket_scatter(
    const uint16_t* __restrict__ idx, const uint8_t* __restrict__ mask, const float* __restrict__ X, int d,
    int64_t n, int nbk, const int* __restrict__ hist, int ntile, const int64_t* __restrict__ bstart,
    float* __restrict__ rx, uint64_t* __restrict__ rw)
{
    __shared__ __align__(16) float sxr[kTile * 8];
    __shared__ uint64_t sw[kTile];
    __shared__ uint16_t sdg[kTile];
    __shared__ uint16_t wcnt[kTileThreads / 64][kMaxBuckets];
    __shared__ int tcnt[kMaxBuckets];
    __shared__ int tstart[kMaxBuckets + 1];
    __shared__ int64_t gbase[kMaxBuckets];

    // Workgroups are dealt to the 8 XCDs in turn; numbering tiles so that
    // each XCD takes a contiguous range lets one L2 merge the partial lines
    // that neighbouring tiles write into the same bucket run.
    const int tiles_per_xcd = (ntile + 7) / 8;
    const int tile = (int)(blockIdx.x % 8) * tiles_per_xcd + (int)(blockIdx.x / 8);
    if (tile >= ntile) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t e0 = (int64_t)tile * kTile;
    const int m = (int)min((int64_t)kTile, n - e0);
    for (int q = tid; q < (kTileThreads / 64) * kMaxBuckets; q += kTileThreads) (&wcnt[0][0])[q] = 0;
    for (int q = tid; q < nbk; q += kTileThreads)
        gbase[q] = bstart[q] + hist[(int64_t)q * ntile + tile];
    __syncthreads();
    const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int bits = 0;
    while ((1 << bits) < nbk) ++bits;
    int dg[2], rank[2], r_of[2];
    uint16_t iv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = wave * 128 + h * 64 + lane;
        r_of[h] = r;
        iv[h] = r < m ? idx[e0 + r] : (uint16_t)0;
        const bool valid = r < m && (iv[h] >> kBucketShift) < nbk;
        dg[h] = valid ? (iv[h] >> kBucketShift) : 0;
        unsigned long long peers;
        const int wr = wave_peer_rank(dg[h], valid, bits, lt_mask, peers);
        int run = 0;
        if (valid) run = wcnt[wave][dg[h]];
        rank[h] = valid ? run + wr : -1;
        if (valid && wr == 0) wcnt[wave][dg[h]] = (uint16_t)(run + __popcll(peers));
    }
    __syncthreads();
    for (int q = tid; q < nbk; q += kTileThreads) {
        int acc = 0;
        for (int w = 0; w < kTileThreads / 64; ++w) {
            const int c = wcnt[w][q];
            wcnt[w][q] = (uint16_t)acc;
            acc += c;
        }
        tcnt[q] = acc;
    }
    __syncthreads();
    wave_excl_scan(tcnt, nbk, tstart);
    __syncthreads();
    const bool vec = (d == 8) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (rank[h] < 0) continue;
        const int lp = tstart[dg[h]] + wcnt[wave][dg[h]] + rank[h];
        const int64_t e = e0 + r_of[h];
        if (vec) {
            const float4* src = reinterpret_cast<const float4*>(X + e * 8);
            float4* dst = reinterpret_cast<float4*>(sxr + lp * 8);
            dst[0] = src[0];
            dst[1] = src[1];
        } else {
            for (int t = 0; t < d; ++t) sxr[lp * 8 + t] = X[e * d + t];
        }
        const uint64_t mk = mask ? (uint64_t)mask[e] : 0ull;
        sw[lp] = (uint64_t)(uint32_t)e | ((uint64_t)(iv[h] & 127) << 32) | (mk << 40);
        sdg[lp] = (uint16_t)dg[h];
    }
    __syncthreads();
    const int mv = tstart[nbk];   // records with a valid bucket
    for (int lp = tid; lp < mv; lp += kTileThreads) {
        const int b = sdg[lp];
        const int64_t pos = gbase[b] + (lp - tstart[b]);
        if (d == 8) {
            const float4* src = reinterpret_cast<const float4*>(sxr + lp * 8);
            float4* dst = reinterpret_cast<float4*>(rx + pos * 8);
            dst[0] = src[0];
            dst[1] = src[1];
        } else {
            for (int t = 0; t < d; ++t) rx[pos * d + t] = sxr[lp * 8 + t];
        }
        rw[pos] = sw[lp];
    }
}

// One workgroup per piece.  The piece goes through LDS in sub-chunks of
// kSub records, one per thread: the thread stages the record's x, its
// column weights hcol (zero where the mask bit is set) and its row weight
// rho, and ranks it by centroid within the sub-chunk (stable counting
// sort).  Then 8-lane group g (lane t = dimension t) walks the members of
// its centroids (g, and g + 128 when a bucket spans 256 centroids) in record
// order, adding omega_t x_t and omega_t (omega = hcol * rho in float64, the
// product of two floats, exact) into float64 sums kept in registers.
// rx == nullptr: one bucket of up to 256 centroids read in place from X,
// idx and mask.
__global__ __launch_bounds__(kRedThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void k_piece_reduce(
    const float* __restrict__ rx, const uint64_t* __restrict__ rw, const float* __restrict__ X,
    const uint16_t* __restrict__ idx, const uint8_t* __restrict__ mask, const float* __restrict__ hcol,
    const float* __restrict__ rho, uint32_t nb, int d, int K, int nbk, int piece,
    const int64_t* __restrict__ bstart, const int* __restrict__ poff, float* __restrict__ C,
    int32_t* __restrict__ counts, double* __restrict__ partial)
{
    __shared__ __align__(16) float sx[kSub * 8];
    __shared__ __align__(16) float shv[kSub * 8];
    __shared__ float srho[kSub];
    __shared__ uint16_t perm[kSub];
    __shared__ uint16_t wcnt[kRedThreads / 64][256];
    __shared__ uint16_t cstart[257];
    __shared__ int ccount[256];

    const int j = blockIdx.x;
    if (j >= poff[nbk]) return;
    int bk = 0;
    {
        int lo = 0, hi = nbk;   // poff[lo] <= j < poff[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (poff[mid] <= j) lo = mid; else hi = mid;
        }
        bk = lo;
    }
    const bool direct = (rx == nullptr);
    const int width = direct ? 256 : 128;     // centroids per bucket
    const int kbits = direct ? 8 : 7;
    const int q = j - poff[bk];
    const int npieces = poff[bk + 1] - poff[bk];
    const int64_t p0 = bstart[bk] + (int64_t)q * piece;
    const int64_t p1 = min(bstart[bk + 1], p0 + (int64_t)piece);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int t = tid & 7;
    const int g = tid >> 3;            // 128 groups
    const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const bool vx = (d == 8) && ((reinterpret_cast<uintptr_t>(direct ? X : rx) & 15) == 0);
    const bool vh = (d == 8) && ((reinterpret_cast<uintptr_t>(hcol) & 15) == 0);
    double num[2] = {0.0, 0.0}, den[2] = {0.0, 0.0};
    int count[2] = {0, 0};

    // Raw fields of record tid of a sub-chunk (the next one is loaded while
    // the current one is reduced).
    auto load_raw = [&](int64_t c0, bool& valid, int& key, uint32_t& sv, uint32_t& mk, float4& xa, float4& xb) {
        const int m = (int)min((int64_t)kSub, p1 - c0);
        valid = c0 < p1 && tid < m;
        key = 0; sv = 0; mk = 0;
        xa = make_float4(0.f, 0.f, 0.f, 0.f);
        xb = xa;
        if (!valid) return;
        const int64_t e = c0 + tid;
        if (direct) {
            sv = (uint32_t)e;
            mk = mask ? mask[e] : 0u;
            key = idx[e] & 255;
        } else {
            const uint64_t wd = rw[e];
            sv = (uint32_t)wd;
            key = (int)((wd >> 32) & 127);
            mk = (uint32_t)((wd >> 40) & 255);
        }
        const float* xs = direct ? X + e * d : rx + e * d;
        if (vx) {
            xa = reinterpret_cast<const float4*>(xs)[0];
            xb = reinterpret_cast<const float4*>(xs)[1];
        } else {
            float tmp[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) tmp[u] = u < d ? xs[u] : 0.0f;
            xa = make_float4(tmp[0], tmp[1], tmp[2], tmp[3]);
            xb = make_float4(tmp[4], tmp[5], tmp[6], tmp[7]);
        }
    };
    bool valid;
    int key;
    uint32_t sv, mk;
    float4 xa, xb;
    load_raw(p0, valid, key, sv, mk, xa, xb);

    for (int64_t c0 = p0; c0 < p1; c0 += kSub) {
        // ---- stage record tid: x now, weights requested (used after the ranking) ----
        const int r = tid;
        float4 ha = make_float4(0.f, 0.f, 0.f, 0.f), hb = ha;
        float rhov = 1.0f;
        if (valid) {
            const uint32_t i = sv / nb;
            const uint32_t b = sv - i * nb;
            if (rho) rhov = rho[i];
            const float* hs = hcol + (size_t)b * d;
            if (vh) {
                ha = reinterpret_cast<const float4*>(hs)[0];
                hb = reinterpret_cast<const float4*>(hs)[1];
            } else {
                float tmp[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) tmp[u] = u < d ? hs[u] : 0.0f;
                ha = make_float4(tmp[0], tmp[1], tmp[2], tmp[3]);
                hb = make_float4(tmp[4], tmp[5], tmp[6], tmp[7]);
            }
            reinterpret_cast<float4*>(sx + r * 8)[0] = xa;
            reinterpret_cast<float4*>(sx + r * 8)[1] = xb;
        }
        for (int v = tid; v < (kRedThreads / 64) * 256; v += kRedThreads) (&wcnt[0][0])[v] = 0;
        __syncthreads();
        // ---- stable rank of record tid by centroid ----
        unsigned long long peers;
        const int wr = wave_peer_rank(key, valid, kbits, lt_mask, peers);
        int rnk = -1;
        {
            int run = 0;
            if (valid) run = wcnt[wave][key];
            if (valid) rnk = run + wr;
            if (valid && wr == 0) wcnt[wave][key] = (uint16_t)(run + __popcll(peers));
        }
        __syncthreads();
        if (tid < width) {
            int acc = 0;
            for (int w = 0; w < kRedThreads / 64; ++w) {
                const int c = wcnt[w][tid];
                wcnt[w][tid] = (uint16_t)acc;
                acc += c;
            }
            ccount[tid] = acc;
        }
        __syncthreads();
        wave_excl_scan(ccount, width, cstart);
        __syncthreads();
        if (valid) {
            perm[cstart[key] + wcnt[wave][key] + rnk] = (uint16_t)r;
            srho[r] = rhov;
            shv[r * 8 + 0] = (mk & 1u) ? 0.0f : ha.x;
            shv[r * 8 + 1] = (mk & 2u) ? 0.0f : ha.y;
            shv[r * 8 + 2] = (mk & 4u) ? 0.0f : ha.z;
            shv[r * 8 + 3] = (mk & 8u) ? 0.0f : ha.w;
            shv[r * 8 + 4] = (mk & 16u) ? 0.0f : hb.x;
            shv[r * 8 + 5] = (mk & 32u) ? 0.0f : hb.y;
            shv[r * 8 + 6] = (mk & 64u) ? 0.0f : hb.z;
            shv[r * 8 + 7] = (mk & 128u) ? 0.0f : hb.w;
        }
        // next sub-chunk's raw fields, in flight during the sums below
        load_raw(c0 + kSub, valid, key, sv, mk, xa, xb);
        __syncthreads();
        // ---- per owned centroid, members in record order ----
#pragma unroll
        for (int o = 0; o < 2; ++o) {
            const int c = g + o * 128;
            if (c >= width) break;
            const int b0 = cstart[c], b1 = cstart[c + 1];
            count[o] += b1 - b0;
            int e = b0;
            for (; e + 2 <= b1; e += 2) {
                double w[2], x[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int rr = perm[e + u];
                    w[u] = (double)shv[rr * 8 + t] * (double)srho[rr];
                    x[u] = (double)sx[rr * 8 + t];
                }
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    num[o] = num[o] + w[u] * x[u];
                    den[o] = den[o] + w[u];
                }
            }
            for (; e < b1; ++e) {
                const int rr = perm[e];
                const double w = (double)shv[rr * 8 + t] * (double)srho[rr];
                num[o] = num[o] + w * (double)sx[rr * 8 + t];
                den[o] = den[o] + w;
            }
        }
        __syncthreads();
    }
    // ---- results ----
#pragma unroll
    for (int o = 0; o < 2; ++o) {
        const int c = g + o * 128;
        if (c >= width) break;
        const int k = bk * width + c;
        if (k >= K) continue;
        if (npieces == 1) {
            if (t < d && den[o] > 0.0) C[(size_t)k * d + t] = (float)(num[o] / den[o]);
            if (t == 0 && counts) counts[k] = count[o];
        } else {
            double* pp = partial + ((int64_t)j * 256 + c) * 17;
            pp[t] = t < d ? num[o] : 0.0;
            pp[8 + t] = t < d ? den[o] : 0.0;
            if (t == 0) pp[16] = (double)count[o];
        }
    }
}

// Buckets with several pieces (and empty buckets, whose counts are zeroed):
// one wavefront per centroid (grid-stride);
// lane = (group q, dimension t); group q adds pieces q, q + 8, ... in order,
// then the 8 group sums are combined by a fixed butterfly and divided once.
__global__ __launch_bounds__(64) void k_piece_finish(const int* __restrict__ poff, int nbk, int width, int K,
                                                     int d, const double* __restrict__ partial,
                                                     float* __restrict__ C, int32_t* __restrict__ counts)
{
    const int lane = threadIdx.x;
    const int t = lane & 7, qg = lane >> 3;
    for (int k = blockIdx.x; k < K; k += gridDim.x) {
        const int bk = k / width, c = k - bk * width;
        if (bk >= nbk) break;
        const int j0 = poff[bk], j1 = poff[bk + 1];
        if (j1 - j0 == 1) continue;   // finished inside its piece
        if (j1 == j0) {                // empty bucket: no members, C kept
            if (lane == 0 && counts) counts[k] = 0;
            continue;
        }
        double num = 0.0, den = 0.0, cntd = 0.0;
        for (int jj = j0 + qg; jj < j1; jj += 8) {
            const double* pp = partial + ((int64_t)jj * 256 + c) * 17;
            num = num + pp[t];
            den = den + pp[8 + t];
            cntd = cntd + pp[16];
        }
#pragma unroll
        for (int off = 8; off < 64; off <<= 1) {
            num = num + __shfl_xor(num, off);
            den = den + __shfl_xor(den, off);
            cntd = cntd + __shfl_xor(cntd, off);
        }
        if (qg == 0) {
            if (t < d && den > 0.0) C[(size_t)k * d + t] = (float)(num / den);
            if (t == 0 && counts) counts[k] = (int32_t)cntd;
        }
    }
}

struct UpdateWs {
    int *hist, *total, *poff;
    int64_t* bstart;
    float* rx;
    uint64_t* rw;
    double* partial;
};

// Records per piece: bucket mode kPieceMax; one bucket: about kDirectPieces
// pieces, a multiple of kSub.
int piece_size(int64_t n_sub, int K)
{
    if (K > 256) return kPieceMax;
    int64_t p = (n_sub + kDirectPieces - 1) / kDirectPieces;
    p = (p + kSub - 1) / kSub * kSub;
    return (int)std::max<int64_t>(kSub, std::min<int64_t>(kPieceMax, p));
}

int64_t max_pieces(int64_t n_sub, int K)
{
    const int nbk = K > 256 ? (K + 127) / 128 : 1;
    return (n_sub + piece_size(n_sub, K) - 1) / piece_size(n_sub, K) + nbk;
}

UpdateWs carve_update(Carver& cv, int64_t n_sub, int K, int d)
{
    UpdateWs w = {};
    const int64_t ntile = (n_sub + kTile - 1) / kTile;
    w.hist = cv.take<int>((size_t)kMaxBuckets * ntile);
    w.total = cv.take<int>(kMaxBuckets);
    w.poff = cv.take<int>(kMaxBuckets + 1);
    w.bstart = cv.take<int64_t>(kMaxBuckets + 1);
    if (K > 256) {
        w.rx = cv.take<float>((size_t)n_sub * d);
        w.rw = cv.take<uint64_t>(n_sub);
    }
    w.partial = cv.take<double>((size_t)max_pieces(n_sub, K) * 256 * 17);
    return w;
}

}  // namespace

size_t ws_update(int64_t n_sub, int K)
{
    Carver cv(nullptr, 0);
    cv.base = reinterpret_cast<char*>(kAlign);   // size-only pass
    cv.cap = SIZE_MAX / 2;
    carve_update(cv, n_sub, K, 8);
    return cv.used;
}

vq_status update_launch(const float* X, const float* hcol, const float* rho, const uint8_t* mask,
                        int64_t M, int64_t N, int d, const uint16_t* idx, int K, float* C,
                        int32_t* counts, void* ws, size_t ws_bytes, hipStream_t st)
{
    const int64_t n_sub = M * N / d;
    Carver cv(ws, ws_bytes);
    UpdateWs w = carve_update(cv, n_sub, K, d);
    if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "vq_update: workspace too small");
    if (n_sub > (int64_t)UINT32_MAX) return fail(VQ_ERR_UNSUPPORTED, "vq_update: more than 2^32 sub-vectors");
    TimedRegion tr("update", K, st);
    const bool bucketed = K > 256;
    const int nbk = bucketed ? (K + 127) / 128 : 1;
    const int width = bucketed ? 128 : 256;
    const int piece = piece_size(n_sub, K);
    if (bucketed) {
        const int ntile = (int)((n_sub + kTile - 1) / kTile);
        hipLaunchKernelGGL(k_bucket_hist, dim3(ntile), dim3(256), 0, st, idx, n_sub, nbk, w.hist, ntile);
        VQ_LAUNCHED("k_bucket_hist");
        hipLaunchKernelGGL(k_bucket_scan, dim3(nbk), dim3(1024), 0, st, w.hist, ntile, w.total);
        VQ_LAUNCHED("k_bucket_scan");
        hipLaunchKernelGGL(k_piece_setup, dim3(1), dim3(64), 0, st, w.total, nbk, n_sub, piece, w.bstart, w.poff);
        VQ_LAUNCHED("k_piece_setup");
        hipLaunchKernelGGL(k_bucket_scatter, dim3((ntile + 7) / 8 * 8), dim3(kTileThreads), 0, st, idx, mask, X, d, n_sub, nbk,
                           w.hist, ntile, w.bstart, w.rx, w.rw);
        VQ_LAUNCHED("k_bucket_scatter");
    } else {
        hipLaunchKernelGGL(k_piece_setup, dim3(1), dim3(64), 0, st, nullptr, 1, n_sub, piece, w.bstart, w.poff);
        VQ_LAUNCHED("k_piece_setup");
    }
    hipLaunchKernelGGL(k_piece_reduce, dim3((unsigned)max_pieces(n_sub, K)), dim3(kRedThreads), 0, st,
                       bucketed ? w.rx : nullptr, w.rw, X, idx, mask, hcol, rho, (uint32_t)(N / d), d, K, nbk, piece,
                       w.bstart, w.poff, C, counts, w.partial);
    VQ_LAUNCHED("k_piece_reduce");
    hipLaunchKernelGGL(k_piece_finish, dim3((unsigned)std::min(K, 4096)), dim3(64), 0, st, w.poff, nbk, width, K, d,
                       w.partial, C, counts);
    VQ_LAUNCHED("k_piece_finish");
    return VQ_OK;
}

}  // namespace vq
