// Centroid update as a weighted segmented reduction (VPTQ page,
// "Hessian-Weighted Centroid Initialization": each centroid becomes the
// Hessian-weighted mean of its members; with one weight per element the
// exact minimizer of the objective is the per-dimension weighted mean).
//
// Design (no floating-point atomics; bitwise deterministic):
//   1. buckets (K > 256 only): one stable scatter by idx >> 8 moves whole
//      records (the sub-vector's d values and a word holding its id, mask
//      byte and idx & 255) into 256-centroid buckets, so no sub-vector is
//      gathered at random later.  Each 2048-record tile is ordered by bucket
//      in LDS first (ranks from wavefront ballots: stable), then written out
//      as contiguous runs.  Tile digit counts use LDS integer atomics
//      (exact) and tile offsets come from a scan.  With K <= 256 the whole
//      matrix is one bucket of up to 256 centroids, read in place;
//   2. each bucket is cut into fixed pieces; a workgroup streams its piece
//      through LDS in sub-chunks of 1024 records (the next sub-chunk's loads
//      in flight meanwhile), stages each record's x, its column weights
//      (zero where masked) and its row weight, counting-sorts the sub-chunk
//      by centroid (stable), and the lanes that own a centroid (a few
//      dimensions each) add its members in order into float64 sums of
//      omega*x and omega kept in registers, each product and sum rounded on
//      its own as in a plain sequential loop.  A bucket that fits one piece
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
constexpr int kMaxBuckets = 256;     // K <= 65536, 256 centroids per bucket
constexpr int kBucketShift = 8;
constexpr int kWidth = 1 << kBucketShift;
constexpr int kSub = 1024;           // records per LDS sub-chunk
constexpr int kRedThreads = 512;     // two records per thread
constexpr int kPieceMax = 32768;     // records per piece in bucket mode
constexpr int kDirectPieces = 512;   // target piece count with one bucket
constexpr int kMinPieces = 256;      // target piece count with few buckets

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
    peers = __ballot(valid);   // invalid lanes drop out here; their key bits do not matter
    for (int bit = 0; bit < bits; ++bit) {
        const int m = -((key >> bit) & 1);                       // 0 or all ones
        const unsigned long long bal = __ballot(m != 0);
        peers &= ~(bal ^ (unsigned long long)(long long)m);      // lanes whose bit equals this lane's
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
//   id | (idx & 255) << 32 | mask << 40.
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
    const bool vec = (d == 8) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
    // every global load of the tile is issued first: the records' x and mask
    // bytes arrive while the indices are ranked
    int dg[2], rank[2], r_of[2];
    uint16_t iv[2];
    uint32_t mkv[2];
    float4 xa[2], xb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = wave * 128 + h * 64 + lane;
        r_of[h] = r;
        iv[h] = 0;
        mkv[h] = 0;
        xa[h] = make_float4(0.f, 0.f, 0.f, 0.f);
        xb[h] = xa[h];
        if (r < m) {
            iv[h] = idx[e0 + r];
            if (mask) mkv[h] = mask[e0 + r];
            if (vec) {
                const float4* src = reinterpret_cast<const float4*>(X + (e0 + r) * 8);
                xa[h] = src[0];
                xb[h] = src[1];
            }
        }
    }
    for (int q = tid; q < (kTileThreads / 64) * kMaxBuckets; q += kTileThreads) (&wcnt[0][0])[q] = 0;
    for (int q = tid; q < nbk; q += kTileThreads)
        gbase[q] = bstart[q] + hist[(int64_t)q * ntile + tile];
    __syncthreads();
    const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int bits = 0;
    while ((1 << bits) < nbk) ++bits;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = r_of[h];
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
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (rank[h] < 0) continue;
        const int lp = tstart[dg[h]] + wcnt[wave][dg[h]] + rank[h];
        const int64_t e = e0 + r_of[h];
        if (vec) {
            float4* dst = reinterpret_cast<float4*>(sxr + lp * 8);
            dst[0] = xa[h];
            dst[1] = xb[h];
        } else {
            for (int t = 0; t < d; ++t) sxr[lp * 8 + t] = X[e * d + t];
        }
        const uint64_t mk = (uint64_t)mkv[h];
        sw[lp] = (uint64_t)(uint32_t)e | ((uint64_t)(iv[h] & (kWidth - 1)) << 32) | (mk << 40);
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

// Adds one member's term of one dimension into float64 sums in the oracle's
// operation order: omega = hcol * rho (the product of two floats, exact in
// float64), then num + omega * x and den + omega, each rounded on its own
// (no fused multiply-add).
__device__ inline void add_term(double& num, double& den, float h, float x, double rd)
{
#pragma clang fp contract(off)
    const double w = (double)h * rd;
    num = num + w * (double)x;
    den = den + w;
}

// One workgroup per piece; the piece goes through LDS in sub-chunks of kSub
// records, kPer per thread (record r = u * kRedThreads + tid).  Each thread
// stages its records' x, column weights hcol (zero where the mask bit is
// set) and row weight rho, and ranks them by centroid among the records of
// its wavefront in the same pass u (ballots: stable).  Per-key counts of the
// kSegs (pass, wavefront) segments, taken in record order, give a stable
// counting sort of the sub-chunk.  Then the owner lanes walk their
// centroid's members in record order, lane = (centroid, part of the
// dimensions): two lanes per centroid, four dimensions each (W = 256), or
// four lanes per centroid, two dimensions each (W = 128).  DIRECT: one
// bucket read in place from X, idx and mask; otherwise the scattered
// buckets rx/rw.
// Sums stay in registers across the piece.
constexpr int kPer = kSub / kRedThreads;
constexpr int kSegs = kPer * (kRedThreads / 64);

template <int W, bool DIRECT>
__global__ __launch_bounds__(kRedThreads) void k_piece_reduce(
    const float* __restrict__ rx, const uint64_t* __restrict__ rw, const float* __restrict__ X,
    const uint16_t* __restrict__ idx, const uint8_t* __restrict__ mask, const float* __restrict__ hcol,
    const float* __restrict__ rho, uint32_t nb, int d, int K, int nbk, int piece,
    const int64_t* __restrict__ bstart, const int* __restrict__ poff, float* __restrict__ C,
    int32_t* __restrict__ counts, double* __restrict__ partial)
{
    constexpr bool kDirect = DIRECT;
    constexpr int KB = W == 256 ? 8 : 7;           // key bits
    constexpr int DP = 8 * W / kRedThreads;        // dimensions per owner lane
    static_assert(DP == 4 || DP == 2, "owner layout");
    __shared__ __align__(16) float sx[kSub * 8];
    __shared__ __align__(16) float sh[kSub * 8];
    __shared__ float srho[kSub];
    __shared__ uint16_t perm[kSub];
    __shared__ __align__(16) uint16_t scnt[kSegs][W];
    __shared__ int cstart[W + 1];
    __shared__ int wsum[kRedThreads / 64];

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
    const int q = j - poff[bk];
    const int npieces = poff[bk + 1] - poff[bk];
    const int64_t p0 = bstart[bk] + (int64_t)q * piece;
    const int64_t p1 = min(bstart[bk + 1], p0 + (int64_t)piece);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const bool vx = (d == 8) && ((reinterpret_cast<uintptr_t>(kDirect ? X : rx) & 15) == 0);
    const bool vh = (d == 8) && ((reinterpret_cast<uintptr_t>(hcol) & 15) == 0);
    const int oc = tid % W;                 // owned centroid within the bucket
    const int oq = tid / W;                 // owned dimension part
    double num[DP], den[DP];
#pragma unroll
    for (int t = 0; t < DP; ++t) { num[t] = 0.0; den[t] = 0.0; }
    int count = 0;

    // Raw fields of record u * kRedThreads + tid of the sub-chunk at c0.  The
    // loads of the next sub-chunk stay in flight across the sums of the
    // current one: nothing reads their registers (no masking, shifting or
    // selecting) until that sub-chunk is staged.
    struct Raw {
        float4 xa, xb, ha, hb;
        float rv;
        uint64_t wd;        // scattered record word (not DIRECT)
        uint32_t sv, kraw, mk;
        bool valid;
    };
    // Row and column block of sub-vector sv: the quotient by nb from a float64
    // reciprocal (off by at most one for sv < 2^32), then corrected exactly.
    const double rnb = 1.0 / (double)nb;
    auto load_weights = [&](Raw& R) {
        uint32_t i = (uint32_t)((double)R.sv * rnb);
        int64_t rem = (int64_t)R.sv - (int64_t)i * nb;
        if (rem < 0) { --i; rem += nb; }
        else if (rem >= (int64_t)nb) { ++i; rem -= nb; }
        const uint32_t b = (uint32_t)rem;
        const float* hs = hcol + (size_t)b * d;
        if (vh) {
            R.ha = reinterpret_cast<const float4*>(hs)[0];
            R.hb = reinterpret_cast<const float4*>(hs)[1];
        } else {
            float tmp[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) tmp[t] = t < d ? hs[t] : 0.0f;
            R.ha = make_float4(tmp[0], tmp[1], tmp[2], tmp[3]);
            R.hb = make_float4(tmp[4], tmp[5], tmp[6], tmp[7]);
        }
        if (rho) R.rv = rho[i];
    };
    auto load_raw = [&](int64_t c0, int u, Raw& R) {
        const int64_t e = c0 + (int64_t)u * kRedThreads + tid;
        R.valid = e < p1;
        R.sv = 0; R.kraw = 0; R.mk = 0; R.wd = 0;
        R.xa = make_float4(0.f, 0.f, 0.f, 0.f);
        R.xb = R.xa;
        R.ha = R.xa;
        R.hb = R.xa;
        R.rv = 1.0f;
        if (!R.valid) return;
        if (kDirect) {
            R.sv = (uint32_t)e;
            if (mask) R.mk = mask[e];
            R.kraw = idx[e];
        } else {
            R.wd = rw[e];
        }
        const float* xs = (kDirect ? X : rx) + e * d;
        if (vx) {
            R.xa = reinterpret_cast<const float4*>(xs)[0];
            R.xb = reinterpret_cast<const float4*>(xs)[1];
        } else {
            float tmp[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) tmp[t] = t < d ? xs[t] : 0.0f;
            R.xa = make_float4(tmp[0], tmp[1], tmp[2], tmp[3]);
            R.xb = make_float4(tmp[4], tmp[5], tmp[6], tmp[7]);
        }
        if (kDirect) load_weights(R);   // the id is known before the record arrives
    };
    Raw cur[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) load_raw(p0, u, cur[u]);

    for (int64_t c0 = p0; c0 < p1; c0 += kSub) {
        // ---- stage x, the masked column weights and rho; clear the segment counts ----
        int key[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            if (!kDirect && cur[u].valid) {
                cur[u].sv = (uint32_t)cur[u].wd;
                cur[u].kraw = (uint32_t)(cur[u].wd >> 32);
                cur[u].mk = (uint32_t)(cur[u].wd >> 40) & 255u;
                load_weights(cur[u]);
            }
            key[u] = (int)(cur[u].kraw & (uint32_t)(W - 1));
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int r = u * kRedThreads + tid;
            if (!cur[u].valid) continue;
            float4 ha = cur[u].ha, hb = cur[u].hb;
            const uint32_t mk = cur[u].mk;
            if (mk) {   // masked element: weight +0 (bit t of mk, sign-extended, clears the float)
                auto zap = [mk](float v, int t) {
                    return __uint_as_float(__float_as_uint(v) & ~(uint32_t)(-(int32_t)((mk >> t) & 1u)));
                };
                ha.x = zap(ha.x, 0);
                ha.y = zap(ha.y, 1);
                ha.z = zap(ha.z, 2);
                ha.w = zap(ha.w, 3);
                hb.x = zap(hb.x, 4);
                hb.y = zap(hb.y, 5);
                hb.z = zap(hb.z, 6);
                hb.w = zap(hb.w, 7);
            }
            reinterpret_cast<float4*>(sx + r * 8)[0] = cur[u].xa;
            reinterpret_cast<float4*>(sx + r * 8)[1] = cur[u].xb;
            reinterpret_cast<float4*>(sh + r * 8)[0] = ha;
            reinterpret_cast<float4*>(sh + r * 8)[1] = hb;
            srho[r] = cur[u].rv;
        }
        for (int v = tid; v < kSegs * W / 8; v += kRedThreads)
            reinterpret_cast<uint4*>(&scnt[0][0])[v] = make_uint4(0u, 0u, 0u, 0u);
        __syncthreads();
        // ---- stable ranks within each (pass, wavefront) segment ----
        int wr[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            unsigned long long peers;
            wr[u] = wave_peer_rank(key[u], cur[u].valid, KB, lt_mask, peers);
            if (cur[u].valid && wr[u] == 0) scnt[u * (kRedThreads / 64) + wave][key[u]] = (uint16_t)__popcll(peers);
        }
        __syncthreads();
        // ---- per key: exclusive scan over the segments; then over the keys ----
        int tot = 0;
        if (tid < W) {
#pragma unroll
            for (int s = 0; s < kSegs; ++s) {
                const int c = scnt[s][tid];
                scnt[s][tid] = (uint16_t)tot;
                tot += c;
            }
        }
        int inc = tot;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(inc, off);
            if (lane >= off) inc += o;
        }
        if (lane == 63) wsum[wave] = inc;
        __syncthreads();
        {
            int carry = 0;
            for (int w2 = 0; w2 < wave; ++w2) carry += wsum[w2];
            if (tid < W) cstart[tid] = carry + inc - tot;
            if (tid == W - 1) cstart[W] = carry + inc;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            if (!cur[u].valid) continue;
            const int k = key[u];
            perm[cstart[k] + scnt[u * (kRedThreads / 64) + wave][k] + wr[u]] = (uint16_t)(u * kRedThreads + tid);
        }
        // next sub-chunk's raw fields, in flight during the sums below
#pragma unroll
        for (int u = 0; u < kPer; ++u) load_raw(c0 + kSub, u, cur[u]);
        __syncthreads();
        // ---- owner lanes: members in record order ----
        {
            const int e0 = cstart[oc], e1 = cstart[oc + 1];
            count += e1 - e0;
            // software pipelined: the next member's fields are read from LDS
            // while the current member's terms are added
            auto fetch = [&](int r_, float (&xv)[DP], float (&hv)[DP], float& rv_) {
                const int o = r_ * 8 + oq * DP;
                if constexpr (DP == 4) {
                    const float4 a = *reinterpret_cast<const float4*>(sx + o);
                    const float4 b = *reinterpret_cast<const float4*>(sh + o);
                    xv[0] = a.x; xv[1] = a.y; xv[2] = a.z; xv[3] = a.w;
                    hv[0] = b.x; hv[1] = b.y; hv[2] = b.z; hv[3] = b.w;
                } else {
                    const float2 a = *reinterpret_cast<const float2*>(sx + o);
                    const float2 b = *reinterpret_cast<const float2*>(sh + o);
                    xv[0] = a.x; xv[1] = a.y;
                    hv[0] = b.x; hv[1] = b.y;
                }
                rv_ = srho[r_];
            };
            if (e0 < e1) {
                float ax[DP], ah[DP], ar;
                fetch(perm[e0], ax, ah, ar);
                for (int e = e0; e < e1; ++e) {
                    float bx[DP], bh[DP], br;
                    fetch(perm[min(e + 1, e1 - 1)], bx, bh, br);
                    const double rd = (double)ar;
#pragma unroll
                    for (int t = 0; t < DP; ++t) {
                        add_term(num[t], den[t], ah[t], ax[t], rd);
                        ax[t] = bx[t];
                        ah[t] = bh[t];
                    }
                    ar = br;
                }
            }
        }
        __syncthreads();
    }
    // ---- results ----
    const int k = bk * W + oc;
    if (k >= K) return;
    const int t0 = oq * DP;
    if (npieces == 1) {
#pragma unroll
        for (int t = 0; t < DP; ++t)
            if (t0 + t < d && den[t] > 0.0) C[(size_t)k * d + t0 + t] = (float)(num[t] / den[t]);
        if (oq == 0 && counts) counts[k] = count;
    } else {
        double* pp = partial + ((int64_t)j * 256 + oc) * 17;
#pragma unroll
        for (int t = 0; t < DP; ++t) {
            pp[t0 + t] = num[t];
            pp[8 + t0 + t] = den[t];
        }
        if (oq == 0) pp[16] = (double)count;
    }
}

// Buckets with several pieces (and empty buckets, whose counts are zeroed):
// one workgroup per cpb centroids of one bucket; thread = (group q of 32,
// dimension t).  Group q adds pieces q, q + 32, ... in order, four loads in
// flight; the 32 group sums are then combined in a fixed pattern (a
// butterfly within each wavefront, the four wavefront sums in order) and
// divided once.
__global__ __launch_bounds__(256) void k_piece_finish(const int* __restrict__ poff, int nbk, int width, int cpb,
                                                      int K, int d, const double* __restrict__ partial,
                                                      float* __restrict__ C, int32_t* __restrict__ counts)
{
    __shared__ double wnum[4][8], wden[4][8], wcntd[4];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int t = tid & 7, qg = tid >> 3;
    // workgroup: centroids [k0, k0 + cpb) of one bucket; a bucket finished
    // inside its piece ends the workgroup at once
    const int k0 = blockIdx.x * cpb;
    if (k0 >= K || k0 / width >= nbk) return;
    if (poff[k0 / width + 1] - poff[k0 / width] == 1) return;
    for (int k = k0; k < min(k0 + cpb, K); ++k) {
        const int bk = k / width, c = k - bk * width;
        const int j0 = poff[bk], j1 = poff[bk + 1];
        if (j1 == j0) {                // empty bucket: no members, C kept
            if (tid == 0 && counts) counts[k] = 0;
            continue;
        }
        double num = 0.0, den = 0.0, cntd = 0.0;
        int jj = j0 + qg;
        for (; jj + 96 < j1; jj += 128) {
            double a[4], b[4], n4[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const double* pp = partial + ((int64_t)(jj + 32 * u) * 256 + c) * 17;
                a[u] = pp[t];
                b[u] = pp[8 + t];
                n4[u] = pp[16];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                num = num + a[u];
                den = den + b[u];
                cntd = cntd + n4[u];
            }
        }
        for (; jj < j1; jj += 32) {
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
        if (lane < 8) {
            wnum[wave][t] = num;
            wden[wave][t] = den;
            if (t == 0) wcntd[wave] = cntd;
        }
        __syncthreads();
        if (tid < 8) {
            double sn = wnum[0][t], sd = wden[0][t], sc = wcntd[0];
#pragma unroll
            for (int w2 = 1; w2 < 4; ++w2) {
                sn = sn + wnum[w2][t];
                sd = sd + wden[w2][t];
                sc = sc + wcntd[w2];
            }
            if (t < d && sd > 0.0) C[(size_t)k * d + t] = (float)(sn / sd);
            if (t == 0 && counts) counts[k] = (int32_t)sc;
        }
        __syncthreads();
    }
}

struct UpdateWs {
    int *hist, *total, *poff;
    int64_t* bstart;
    float* rx;
    uint64_t* rw;
    double* partial;
};

// Records per piece, a multiple of kSub: bucket mode kPieceMax when there
// are enough buckets to fill the device (a bucket then usually stays one
// piece, with no merge), else about kMinPieces pieces in all; one bucket:
// about kDirectPieces pieces.
int piece_size(int64_t n_sub, int K)
{
    if (K > 256) {
        const int nbk = (K + kWidth - 1) / kWidth;
        if (nbk >= kMinPieces) return kPieceMax;
        int64_t p = (n_sub + kMinPieces - 1) / kMinPieces;
        p = (p + kSub - 1) / kSub * kSub;
        return (int)std::max<int64_t>(kSub, std::min<int64_t>(kPieceMax, p));
    }
    int64_t p = (n_sub + kDirectPieces - 1) / kDirectPieces;
    p = (p + kSub - 1) / kSub * kSub;
    return (int)std::max<int64_t>(kSub, std::min<int64_t>(kPieceMax, p));
}

int64_t max_pieces(int64_t n_sub, int K)
{
    const int nbk = K > 256 ? (K + kWidth - 1) / kWidth : 1;
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
    const int nbk = bucketed ? (K + kWidth - 1) / kWidth : 1;
    const int width = bucketed ? kWidth : 256;
    // the merge: per workgroup 16 centroids of one bucket when there are
    // many buckets (a workgroup per centroid would mostly exit at once)
    const int cpb = bucketed ? 16 : 1;
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
    if (bucketed)
        hipLaunchKernelGGL((k_piece_reduce<kWidth, false>), dim3((unsigned)max_pieces(n_sub, K)), dim3(kRedThreads), 0, st, w.rx,
                           w.rw, X, idx, mask, hcol, rho, (uint32_t)(N / d), d, K, nbk, piece, w.bstart, w.poff, C,
                           counts, w.partial);
    else
        hipLaunchKernelGGL((k_piece_reduce<256, true>), dim3((unsigned)max_pieces(n_sub, K)), dim3(kRedThreads), 0, st,
                           nullptr, w.rw, X, idx, mask, hcol, rho, (uint32_t)(N / d), d, K, nbk, piece, w.bstart,
                           w.poff, C, counts, w.partial);
    VQ_LAUNCHED("k_piece_reduce");
    hipLaunchKernelGGL(k_piece_finish, dim3((unsigned)((K + cpb - 1) / cpb)), dim3(256), 0, st, w.poff, nbk, width,
                       cpb, K, d, w.partial, C, counts);
    VQ_LAUNCHED("k_piece_finish");
    return VQ_OK;
}

}  // namespace vq
